"""GPU GEMM parity: the HIP block-scaled GEMM against the CPU oracle.

Bar: |gpu - ref| <= 2^-7 |ref| + 1e-5 sum_k |a_k b_k| + 2^-126 per element,
and bit-exact bf16 where fp32 accumulation is exact in any order.
Operands for the oracle are quantized by the oracle itself from the bf16
inputs; the GPU GEMM consumes the GPU cast's output.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import (say, to_device, bf16_to_f64, assert_gemm_close, assert_gemm_whole, bf16_rne_of_exact,
                      device_ref_blocks)

pytestmark = pytest.mark.gpu


def gpu_nt(a_bits, b_bits, what):
    say("gemm_nt %s M=%d N=%d K=%d" % (what, a_bits.shape[0], b_bits.shape[0], a_bits.shape[1]))
    a = mx.cast(to_device(a_bits))
    b = mx.cast(to_device(b_bits))
    out = mx.gemm_nt(a, b)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def oracle_nt(a_bits, b_bits):
    qa, sa = oracle.cast_rows(a_bits)
    qb, sb = oracle.cast_rows(b_bits)
    return oracle.gemm(qa, sa, qb, sb)


# The device reference of the full-size whole-output checks (oracle-dequantized operands, float64
# torch.matmul on the device) against the oracle's own GEMM: ragged shape, several row blocks, one
# operand with all-zero and subnormal-magnitude blocks.
def test_device_reference_matches_oracle():
    M, N, K = 700, 530, 2080
    a = W.ragged_values((M, K), 41)
    b = W.ragged_values((N, K), 43)
    qa, sa = oracle.cast_rows(a)
    qb, sb = oracle.cast_rows(b)
    ref, absref = oracle.gemm(qa, sa, qb, sb)
    say("device reference %dx%dx%d" % (M, N, K))
    got_ref, got_abs = np.empty_like(ref), np.empty_like(absref)
    for r0, r, ab, _ in device_ref_blocks((qa, sa), (qb, sb), torch.device("cuda:0"), block_rows=256):
        got_ref[r0:r0 + r.shape[0]] = r.cpu().numpy()
        got_abs[r0:r0 + r.shape[0]] = ab.cpu().numpy()
    assert np.all(np.abs(got_ref - ref) <= 1e-12 * absref + 1e-300)
    assert np.all(np.abs(got_abs - absref) <= 1e-12 * absref + 1e-300)


def test_tiny_config():
    a, w, _ = W.projection_inputs("tiny", 0, 256, 256, 256, with_grad=False)
    got = gpu_nt(a, w, "tiny")
    ref, absref = oracle_nt(a, w)
    assert_gemm_close(got, ref, absref, "tiny")


@pytest.mark.parametrize("M,N,K", [(1, 128, 32), (17, 128, 32), (17, 4096 // 16, 4096 // 8), (33, 65, 96),
                                   (64, 64, 64), (100, 200, 288), (129, 257, 544), (256, 96, 1024),
                                   (1, 300, 2048), (70, 33, 320)])
def test_ragged_small(M, N, K):
    a = W.ragged_values((M, K), M * 31 + K)
    b = W.ragged_values((N, K), N * 17 + K)
    got = gpu_nt(a, b, "ragged")
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "ragged %dx%dx%d" % (M, N, K))


# Shapes with at least 128 output tiles of 256 x 256 (the launcher gives fewer to the skinny kernel):
# persistent kernel with one trip per tile (K <= 512, K = 32 included), with several trips and K not a
# multiple of 512, the pipelined kernel for N % 8 != 0; ragged M / N edges and K tails.
# (250, 65784, K): 257 tiles, two rounds on 129 workgroups, the last of which has one tile.
@pytest.mark.parametrize("M,N,K", [(4096, 2048, 32), (2048, 4096, 256), (2100, 4000, 288), (4096, 2056, 800),
                                   (2048, 4100, 1024), (2304, 3840, 1024), (3000, 2568, 1536),
                                   (250, 65784, 288), (250, 65784, 1056)])
def test_tiled_shapes(M, N, K):
    a = W.normal_bf16((M, K), 1.0, M + 7 * K)
    b = W.normal_bf16((N, K), 0.5, N + 11 * K)
    got = gpu_nt(a, b, "tiled")
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "tiled %dx%dx%d" % (M, N, K))


# Outputs too small for the tiled kernels.  Skinny kernel: split of the contraction over the waves of
# a workgroup, 32*MA x 32*NB blocks with (MA, NB) = (1, 1), (1, 2), (1, 4), (2, 2), the smaller side
# taken as A (output written transposed when that is the GEMM's B; small sides of 33..128 rows in
# several 32-row groups), K chunks past the padded code tiles; 2 x 2 blocks in (97, 20000, 1024),
# (65536, 100, 544) and (16384, 128, 4096).  The panel kernel takes
# (1000, 2000, 1024), (1536, 2816, 544) and (2100, 3000, 256); (128, 65536, 512) has enough
# 256 x 256 tiles for the tiled kernels.
@pytest.mark.parametrize("M,N,K", [(1, 4096, 14336), (4096, 32, 8192), (32, 65536, 1024), (128, 65536, 512),
                                   (65536, 100, 544), (17, 300, 2080), (1, 128256, 32), (1000, 2000, 1024),
                                   (48, 3000, 544), (5000, 64, 2080), (4096, 128, 14336), (97, 20000, 1024),
                                   (16384, 128, 4096), (1536, 2816, 544), (2100, 3000, 256)])
def test_skinny_shapes(M, N, K):
    a = W.ragged_values((M, K), 3 * M + K)
    b = W.ragged_values((N, K), 5 * N + K)
    got = gpu_nt(a, b, "skinny")
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "skinny %dx%dx%d" % (M, N, K))


# Panel kernel (both output sides of 128 rows or more, too few 256 x 256 tiles for the tiled kernels):
# 128 x 128 blocks whose 4 waves share the operand panels through LDS.  Taken unsplit for a smaller
# side of 512 rows or more with blocks for half the CUs (1000 x 2100, 2100 x 1000, 1100 x 1900,
# 1024 x 2048), and for 2^20 outputs or more over contractions of 8192 or more (130 x 12500 over 8192,
# 12500 x 130 over 8320: 196 blocks, a 130-row side, i.e. a 64-row partial block with 2 valid rows).
# The output is written transposed when the GEMM's B is the smaller side; K with an odd number of
# 128-wide code tiles (the last chunk's second K tile reads zero: K = 32, 288, 8320).
@pytest.mark.parametrize("M,N,K", [(1000, 2100, 288), (2100, 1000, 416), (1100, 1900, 32), (1024, 2048, 1024),
                                   (130, 12500, 8192), (12500, 130, 8320)])
def test_panel_shapes(M, N, K):
    a = W.ragged_values((M, K), 13 * M + K)
    b = W.ragged_values((N, K), 19 * N + K)
    got = gpu_nt(a, b, "panel")
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "panel %dx%dx%d" % (M, N, K))


# Panel kernel with a workspace: the contraction of each 128 x 128 block split over S workgroups, whose
# fp32 partials of the waves' 64 x 64 blocks the reduction kernel adds in split order.  128 x 8192 over
# 8192 (64 blocks, 4 splits), 130 x 8150 and 8150 x 130 over 8320 (128 blocks, 2 splits, 65 K tiles,
# ragged 64-row partial blocks); full, half and garbage workspace as for the skinny split (half of it
# gives fewer splits, and with them too few workgroups: the skinny kernel takes over), and the same
# bits from the full and the garbage run.
@pytest.mark.parametrize("M,N,K", [(128, 8192, 8192), (130, 8150, 8320), (8150, 130, 8320)])
def test_panel_split(M, N, K):
    a = W.ragged_values((M, K), 23 * M + K)
    b = W.ragged_values((N, K), 29 * N + K)
    need = mx.gemm_workspace_bytes(M, N, K)
    assert need > 0, "the shape should split its contraction"
    ad, bd = mx.cast(to_device(a)), mx.cast(to_device(b))
    ref, absref = oracle_nt(a, b)
    outs = []
    for what, nbytes in (("full", need), ("half", need // 2), ("garbage", need)):
        ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device="cuda:0")
        if what == "garbage":
            ws.fill_(0x7F)
        say("panel gemm_nt_ws %s M=%d N=%d K=%d ws=%d" % (what, M, N, K, nbytes))
        out = mx.gemm_nt(ad, bd, ws=ws)
        torch.cuda.synchronize()
        assert_gemm_close(bf16_to_f64(out), ref, absref, "panel split %s %dx%dx%d" % (what, M, N, K))
        outs.append(out.view(torch.int16).clone())
    assert torch.equal(outs[0], outs[2])


# The largest contraction the boundary accepts, K = 2^23 (65536 code tiles and 32768 scale tiles per
# row): 1 x 32 and 17 x 32 outputs on the skinny kernel, without a workspace (the waves of a workgroup
# split the contraction) and with one (the split over workgroups at its largest chunk counts).
@pytest.mark.parametrize("M,N", [(1, 32), (17, 32)])
def test_max_contraction(M, N):
    K = 1 << 23
    a = W.normal_bf16((M, K), 1.0, 71 + M)
    b = W.normal_bf16((N, K), 1.0, 73 + N)
    ref, absref = oracle_nt(a, b)
    ad, bd = mx.cast(to_device(a)), mx.cast(to_device(b))
    assert mx.gemm_workspace_bytes(M, N, K) > 0
    for ws in (None, mx.gemm_workspace([(M, N, K)], "cuda:0")):
        say("gemm_nt at K = 2^23 M=%d N=%d workspace=%s" % (M, N, ws is not None))
        out = mx.gemm_nt(ad, bd, ws=ws)
        torch.cuda.synchronize()
        assert_gemm_close(bf16_to_f64(out), ref, absref, "K = 2^23 %dx%d ws=%s" % (M, N, ws is not None))


@pytest.mark.parametrize("M,N,K", [(384, 320, 768), (2048, 4096, 1024)])
def test_same_scale_bit_exact(M, N, K):
    # skinny (few tiles) and persistent tiled kernels
    rng = np.random.default_rng(16)
    fa = rng.uniform(-4, 4, (M, K)).astype(np.float32)
    fb = rng.uniform(-4, 4, (N, K)).astype(np.float32)
    fa[:, ::32] = 4.0
    fb[:, ::32] = 4.0
    a, b = W.bf16_bits(fa), W.bf16_bits(fb)
    got = gpu_nt(a, b, "tiled same-scale")
    ref, _ = oracle_nt(a, b)
    assert np.array_equal(got, bf16_rne_of_exact(ref))


def test_k32_is_bit_exact():
    # one block: each output is one integer dot times a power of two -> exact in fp32,
    # so the bf16 result must be the nearest-even rounding of the exact value
    rng = np.random.default_rng(5)
    a = W.normal_bf16((96, 32), 1.0, 11)
    b = W.normal_bf16((160, 32), 3.0, 12)
    got = gpu_nt(a, b, "K=32")
    ref, _ = oracle_nt(a, b)
    assert np.array_equal(got, bf16_rne_of_exact(ref))


def test_same_scale_blocks_bit_exact():
    # every block holds an anchor of magnitude 4 (fixes X = 0) and values in [-4, 4]:
    # products are multiples of 1/4 below 36 and sums stay far below 2^24 units -> exact
    rng = np.random.default_rng(6)
    M, N, K = 80, 72, 512
    fa = rng.uniform(-4, 4, (M, K)).astype(np.float32)
    fb = rng.uniform(-4, 4, (N, K)).astype(np.float32)
    fa[:, ::32] = 4.0
    fb[:, ::32] = -4.0
    a, b = W.bf16_bits(fa), W.bf16_bits(fb)
    got = gpu_nt(a, b, "same-scale")
    ref, _ = oracle_nt(a, b)
    assert np.array_equal(got, bf16_rne_of_exact(ref))


def test_one_hot_rows_pick_dequantized_entries():
    # A row m = e_{k_m}: out[m, n] = dequant(B)[n, k_m] exactly (pins the operand lane layout)
    rng = np.random.default_rng(8)
    M, N, K = 64, 96, 1024
    ks = rng.integers(0, K, M)
    a = np.zeros((M, K), np.uint16)
    a[np.arange(M), ks] = 0x3F80
    b = W.normal_bf16((N, K), 1.0, 21)
    got = gpu_nt(a, b, "one-hot")
    qb, sb = oracle.cast_rows(b)
    db = oracle.dequant(qb, sb)
    expect = bf16_rne_of_exact(db[:, ks].T.copy())
    assert np.array_equal(got, expect)


def test_empty_and_zero_k():
    a = mx.empty_operand(0, 64, "cuda:0")
    b = mx.empty_operand(16, 64, "cuda:0")
    out = mx.gemm_nt(a, b)
    assert out.shape == (0, 16)
    # K = 0 writes zeros: a skinny output, and outputs the panel kernel takes (its descriptors then
    # span no bytes, every load reads zero)
    for M, N in ((8, 16), (1000, 2000), (4096, 4096)):
        say("gemm K=0 M=%d N=%d" % (M, N))
        a0 = mx.empty_operand(M, 0, "cuda:0")
        b0 = mx.empty_operand(N, 0, "cuda:0")
        out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda:0")
        mx.gemm_nt(a0, b0, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0)


def test_nn_form_with_column_copy():
    # out[M, N] = A[M, K] . B[K, N] with B entering through its column copy
    M, K, N = 96, 320, 160
    a = W.normal_bf16((M, K), 1.0, 31)
    bkn = W.normal_bf16((K, N), 1.0, 32)
    say("gemm_nn")
    ag = mx.cast(to_device(a))
    bt = mx.cast_dual(to_device(bkn))
    out = mx.gemm_nn(ag, bt.col)
    torch.cuda.synchronize()
    qa, sa = oracle.cast_rows(a)
    qc, sc = oracle.cast_cols(bkn)
    ref, absref = oracle.gemm(qa, sa, qc, sc)
    assert_gemm_close(bf16_to_f64(out), ref, absref, "nn")


def test_output_leading_dimension():
    M, N, K = 40, 72, 256
    a = W.normal_bf16((M, K), 1.0, 41)
    b = W.normal_bf16((N, K), 1.0, 42)
    big = torch.full((M, 100), -1.0, dtype=torch.bfloat16, device="cuda:0")
    say("gemm ldo")
    mx.gemm_nt(mx.cast(to_device(a)), mx.cast(to_device(b)), out=big[:, 10:10 + N])
    torch.cuda.synchronize()
    ref, absref = oracle_nt(a, b)
    got = bf16_to_f64(big)
    assert_gemm_close(got[:, 10:10 + N], ref, absref, "ldo")
    assert np.all(got[:, :10] == -1.0) and np.all(got[:, 10 + N:] == -1.0)


def test_persistent_multi_round_whole_output():
    # 2048 x 20480: 8 x 80 = 640 tiles of 256 x 256, three rounds of the balanced persistent grid
    # (214 workgroups, 3 tiles each but the last ones), tile rows grouped by 4 (tiles_m = 8 >
    # group_m), K = 1024 (two trips per tile); every output checked
    M, N, K = 2048, 20480, 1024
    a = W.normal_bf16((M, K), 1.0, 71)
    b = W.normal_bf16((N, K), 0.3, 72)
    got = gpu_nt(a, b, "persistent 3 rounds")
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "persistent %dx%dx%d" % (M, N, K))


# Tiled launches (128 tiles of 256 x 256) writing into a wider output buffer: ldo % 8 == 0 and a
# 16-byte aligned start (persistent kernel), ldo % 8 == 4 (pipelined kernel, 8-byte stores), and a
# start 2 bytes past 8-byte alignment (pipelined kernel, 2-byte stores); the columns around the
# window must stay untouched.
@pytest.mark.parametrize("extra,offset,K", [(64, 0, 512), (64, 8, 1536), (4, 0, 512), (64, 1, 512), (4, 1, 1024)],
                         ids=["persist-ldo", "persist-ldo-offset", "pipe-vec-ldo", "pipe-unaligned",
                              "pipe-unaligned-ldo4"])
def test_tiled_output_leading_dimension(extra, offset, K):
    M, N = 2048, 4096
    a = W.normal_bf16((M, K), 1.0, 81 + extra + offset)
    b = W.normal_bf16((N, K), 1.0, 82 + extra + offset)
    ldo = N + extra
    big = torch.full((M, ldo + offset), -1.0, dtype=torch.bfloat16, device="cuda:0")
    view = big.view(-1)[offset:offset + M * ldo].view(M, ldo)[:, :N]
    say("gemm ldo=%d offset=%d K=%d" % (ldo, offset, K))
    mx.gemm_nt(mx.cast(to_device(a)), mx.cast(to_device(b)), out=view)
    torch.cuda.synchronize()
    ref, absref = oracle_nt(a, b)
    flat = bf16_to_f64(big).reshape(-1)
    win = flat[offset:offset + M * ldo].reshape(M, ldo)
    assert_gemm_close(win[:, :N], ref, absref, "ldo %d offset %d" % (ldo, offset))
    assert np.all(win[:, N:] == -1.0) and np.all(flat[:offset] == -1.0) and np.all(flat[offset + M * ldo:] == -1.0)


# Split contraction (mxfp4_gemm_nt_ws): long contractions behind small outputs -- the dA of an LM head
# (1 or 17 x 32 outputs over 128256, 31 splits; 4096 x 32 and 32 x 4096, 2 splits), ragged blocks of a
# row vector and of 33 x 100 and 64 x 96 outputs -- with the full workspace, with half of it (fewer
# splits), and with a workspace full of garbage (the partials need no initialization); against the
# oracle, and the same bits as a second call.
@pytest.mark.parametrize("M,N,K", [(1, 32, 128256), (17, 32, 128256), (4096, 32, 128256), (32, 4096, 128256),
                                   (1, 1000, 100000), (33, 100, 20000), (64, 96, 65536)])
def test_split_contraction(M, N, K):
    a = W.ragged_values((M, K), 7 * M + K)
    b = W.ragged_values((N, K), 9 * N + K)
    need = mx.gemm_workspace_bytes(M, N, K)
    assert need > 0, "the shape should split its contraction"
    ad, bd = mx.cast(to_device(a)), mx.cast(to_device(b))
    ref, absref = oracle_nt(a, b)
    outs = []
    for what, nbytes in (("full", need), ("half", need // 2), ("garbage", need)):
        ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device="cuda:0")
        if what == "garbage":
            ws.fill_(0x7F)  # every partial float starts as a huge value
        say("gemm_nt_ws %s M=%d N=%d K=%d ws=%d" % (what, M, N, K, nbytes))
        out = mx.gemm_nt(ad, bd, ws=ws)
        torch.cuda.synchronize()
        got = bf16_to_f64(out)
        assert_gemm_close(got, ref, absref, "split %s %dx%dx%d" % (what, M, N, K))
        outs.append(out.view(torch.int16).clone())
    assert torch.equal(outs[0], outs[2])  # same split, same order: same bits


# Two products in one call (mxfp4_gemm_nt_pair_ws), as the training backward runs dA and dB.  Paired
# launches (one persistent grid, XCDs 0..s-1 on the first product, the rest on the second): the dA /
# dB shapes of a 2048 x 4096 x 2048 step (4 + 4 XCDs), one trip per tile (K = 512 and 256), a
# ragged pair (9 x 16 tiles each, K = 1056 and 2080: 3 + 5 XCDs, so the slot mapping runs over 3
# and 5 XCDs), a partial last tile column (N = 4032), and the remaining splits 1 + 7, 2 + 6, 5 + 3,
# 6 + 2 and 7 + 1 at K = 640 (two trips per tile, the second half past K; the smaller product's
# grid leaves part of its XCDs' workgroups idle).  Two launches: a skinny product beside a tiled
# one (with its split contraction in ws), tiled products whose trip structures differ (one trip per
# tile against two), and an uneven pair the cost model keeps apart.  Every output against the device
# reference of the oracle's copies, and bit for bit against its own mxfp4_gemm_nt_ws call.
PAIRS = [((2048, 4096, 4096), (4096, 4096, 2048), 4), ((2048, 4096, 512), (4096, 2048, 256), 4),
         ((2100, 4000, 1056), (4000, 2056, 2080), 3), ((2048, 4032, 1024), (2048, 4096, 1024), 4),
         ((2048, 4000, 640), (6144, 8192, 640), 1), ((2048, 4000, 640), (2100, 6144, 640), 2),
         ((2100, 8192, 640), (2048, 4000, 640), 5), ((6144, 4000, 640), (2048, 4000, 640), 6),
         ((8192, 8192, 640), (2048, 4000, 640), 7),
         ((17, 4096, 4096), (4096, 4096, 1024), 0), ((2048, 4096, 512), (4096, 2048, 1024), 0),
         ((4096, 4096, 1024), (2048, 4096, 8192), 0)]


@pytest.mark.parametrize("s0,s1,split", PAIRS, ids=["step", "one-trip", "ragged-3-5", "partial-col", "xcds-1-7",
                                                    "xcds-2-6", "xcds-5-3", "xcds-6-2", "xcds-7-1", "skinny-tiled",
                                                    "trips-differ", "uneven-apart"])
def test_gemm_pair(s0, s1, split):
    assert mx.gemm_pair_split(*s0, *s1) == split
    ops, copies = [], []
    for i, (M, N, K) in enumerate((s0, s1)):
        a = W.ragged_values((M, K), 37 * M + K + i)
        b = W.ragged_values((N, K), 41 * N + K + i)
        ops.append((mx.cast(to_device(a)), mx.cast(to_device(b))))
        copies.append((oracle.cast_rows(a), oracle.cast_rows(b)))
    ws = mx.gemm_workspace([s0, s1], "cuda:0")
    say("gemm_nt_pair %s + %s split %d" % (s0, s1, split))
    out0, out1 = mx.gemm_nt_pair(ops[0][0], ops[0][1], ops[1][0], ops[1][1], ws=ws)
    torch.cuda.synchronize()
    for i, out in enumerate((out0, out1)):
        alone = mx.gemm_nt(ops[i][0], ops[i][1], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), alone.view(torch.int16)), "product %d differs from its own call" % i
        assert_gemm_whole(out, copies[i][0], copies[i][1], "pair %s + %s, product %d" % (s0, s1, i))


# Paired outputs inside wider buffers: ldo % 8 == 0 with 16-byte aligned starts (the paired launch),
# and the second output at ldo % 8 == 4 (the pipelined kernel: two launches); columns around the
# windows untouched.
@pytest.mark.parametrize("extra1", [72, 4], ids=["paired", "second-ldo4"])
def test_gemm_pair_output_leading_dimension(extra1):
    shapes = ((2048, 4096, 1024), (4096, 2048, 1536))
    ops, copies, bigs, views = [], [], [], []
    for i, ((M, N, K), extra) in enumerate(zip(shapes, (64, extra1))):
        a = W.normal_bf16((M, K), 1.0, 91 + i)
        b = W.normal_bf16((N, K), 1.0, 93 + i)
        ops.append((mx.cast(to_device(a)), mx.cast(to_device(b))))
        copies.append((oracle.cast_rows(a), oracle.cast_rows(b)))
        big = torch.full((M, N + extra + 8), -1.0, dtype=torch.bfloat16, device="cuda:0")
        bigs.append(big)
        views.append(big[:, 8:8 + N])
    say("gemm_nt_pair ldo %d / %d" % (views[0].stride(0), views[1].stride(0)))
    mx.gemm_nt_pair(ops[0][0], ops[0][1], ops[1][0], ops[1][1], out0=views[0], out1=views[1])
    torch.cuda.synchronize()
    for i, ((M, N, K), big, view) in enumerate(zip(shapes, bigs, views)):
        assert_gemm_whole(view, copies[i][0], copies[i][1], "pair ldo, product %d" % i)
        got = big.view(torch.int16)
        minus1 = torch.tensor(-1.0, dtype=torch.bfloat16).view(torch.int16).item()
        assert bool((got[:, :8] == minus1).all()) and bool((got[:, 8 + N:] == minus1).all())


# Non-finite inputs: a 32-block holding Inf or NaN gets the scale byte 0xFF (the E8M0 NaN) and zero
# codes, and every output whose dot product touches such a block is NaN; the other outputs are
# unaffected.  One Inf in a row of A and one NaN in a row of B, in K blocks that a skinny, a panel, a
# persistent and a pipelined launch each reach (N % 8 != 0 for the last).
@pytest.mark.parametrize("M,N,K", [(17, 300, 2080), (1000, 2100, 288), (2048, 4096, 1024), (2048, 4100, 1024)],
                         ids=["skinny", "panel", "persistent", "pipelined"])
def test_non_finite_blocks_give_nan_outputs(M, N, K):
    a = W.normal_bf16((M, K), 1.0, 101 + M)
    b = W.normal_bf16((N, K), 1.0, 103 + N)
    ia, ka = M // 3, K - 40          # +Inf in A's last-but-one block of row ia
    ib, kb = (2 * N) // 3, 70        # NaN in B's third block of row ib
    a[ia, ka] = 0x7F80
    b[ib, kb] = 0x7FC1
    qa, sa = oracle.cast_rows(a)
    qb, sb = oracle.cast_rows(b)
    assert sa[ia, ka // 32] == 0xFF and sb[ib, kb // 32] == 0xFF
    got = gpu_nt(a, b, "non-finite")
    nan_mask = np.zeros((M, N), bool)
    nan_mask[ia, :] = True
    nan_mask[:, ib] = True
    assert np.all(np.isnan(got[nan_mask])), "outputs touching a non-finite block must be NaN"
    assert np.all(np.isfinite(got[~nan_mask]))
    a2, b2 = a.copy(), b.copy()
    a2[ia, :] = 0
    b2[ib, :] = 0
    ref, absref = oracle_nt(a2, b2)  # the finite outputs do not depend on the non-finite rows
    keep = ~nan_mask
    assert_gemm_close(np.where(keep, got, 0.0), np.where(keep, ref, 0.0), absref, "non-finite %dx%dx%d" % (M, N, K))


# Outputs past 2^31 elements (the row offset m * ldo past 32 bits): 32768 x 66560 on the persistent kernel
# (N % 8 == 0; 33280 tiles of 256 x 256 in 130 rounds) and 32768 x 66564 on the pipelined one (N % 8 == 4,
# 8-byte stores), K = 32 (one block per output: the launch is output-bound); every output against the
# device reference of the oracle's copies.
@pytest.mark.slow
@pytest.mark.parametrize("N", [66560, 66564], ids=["persistent", "pipelined"])
def test_gemm_output_past_2_31_elements(N):
    M, K = 32768, 32
    assert M * N > 2 ** 31
    a = W.ragged_values((M, K), 111)
    b = W.ragged_values((N, K), 113 + N)
    say("gemm_nt output past 2^31 elements M=%d N=%d K=%d" % (M, N, K))
    out = mx.gemm_nt(mx.cast(to_device(a)), mx.cast(to_device(b)))
    torch.cuda.synchronize()
    assert_gemm_whole(out, oracle.cast_rows(a), oracle.cast_rows(b), "output past 2^31 %dx%d" % (M, N))


# A seeded draw of shapes across the launch-selection boundaries (numpy default_rng(2024): a small side
# below 128, both sides 128..1500, both 1500..5000, and odd N; K a multiple of 32 up to 2528; half of
# them transposed), each through mxfp4_gemm_nt_ws with the workspace its split needs; every output
# against the device reference of the oracle's copies.
RANDOM_SHAPES = [(4055, 31, 256), (422, 1374, 2048), (1997, 1774, 2208), (5655, 1236, 928), (3532, 59, 2048),
                 (797, 974, 1440), (2209, 3127, 192), (4063, 3926, 1536), (1238, 17, 1952), (1117, 735, 2240),
                 (2459, 2787, 2048), (2259, 3421, 704), (100, 2803, 2464), (490, 973, 736), (2772, 3205, 1248),
                 (2965, 2404, 2272), (41, 1471, 1632), (1242, 381, 1408), (1749, 4418, 224), (2495, 2046, 608),
                 (4177, 24, 1376), (1486, 590, 704), (3495, 3499, 2336), (2001, 4429, 512)]


@pytest.mark.parametrize("M,N,K", RANDOM_SHAPES)
def test_random_shapes_whole_output(M, N, K):
    a = W.ragged_values((M, K), 7 * M + 3 * K)
    b = W.ragged_values((N, K), 11 * N + 5 * K)
    ws = mx.gemm_workspace([(M, N, K)], "cuda:0")
    say("gemm_nt_ws random shape M=%d N=%d K=%d" % (M, N, K))
    out = mx.gemm_nt(mx.cast(to_device(a)), mx.cast(to_device(b)), ws=ws)
    torch.cuda.synchronize()
    assert_gemm_whole(out, oracle.cast_rows(a), oracle.cast_rows(b), "random %dx%dx%d" % (M, N, K))


# One trip per tile with every count of K tiles that hold data (the kernel leaves out the MFMAs and
# register reads of the K tiles wholly past K): K = 32 and 128 (1 of 4), 160 and 256 (2), 288 and 384
# (3), 416 and 512 (4), on 2048 x 4096 outputs (128 tiles) and, paired, beside a product with fewer
# live K tiles (the pair runs the larger count; the other product's extra K tiles add zeros).
@pytest.mark.parametrize("K", [32, 128, 160, 256, 288, 384, 416, 512])
def test_one_trip_live_k_tiles(K):
    M, N = 2048, 4096
    a = W.ragged_values((M, K), 51 + K)
    b = W.ragged_values((N, K), 53 + K)
    got = gpu_nt(a, b, "one trip, K = %d" % K)
    ref, absref = oracle_nt(a, b)
    assert_gemm_close(got, ref, absref, "one trip %dx%dx%d" % (M, N, K))
    # paired with a 32-deep product: K tiles beyond the shorter product's own count add zeros
    a2 = W.ragged_values((M, 32), 55 + K)
    b2 = W.ragged_values((N, 32), 57 + K)
    ops = [(mx.cast(to_device(a)), mx.cast(to_device(b))), (mx.cast(to_device(a2)), mx.cast(to_device(b2)))]
    assert mx.gemm_pair_split(M, N, K, M, N, 32) in (0, 4)
    say("gemm_nt_pair one trip K = %d and 32" % K)
    o0, o1 = mx.gemm_nt_pair(ops[0][0], ops[0][1], ops[1][0], ops[1][1])
    torch.cuda.synchronize()
    assert_gemm_close(bf16_to_f64(o0), ref, absref, "paired one trip K = %d" % K)
    ref2, absref2 = oracle_nt(a2, b2)
    assert_gemm_close(bf16_to_f64(o1), ref2, absref2, "paired one trip K = 32 beside K = %d" % K)
