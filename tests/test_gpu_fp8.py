"""GPU parity of the MXFP8 (E4M3) path -- the FP8 dB variant -- against the CPU oracle.

Casts: bit for bit (scales, codes and zero padding), for the MXFP8 row copy, the MXFP8
dual cast and the mixed cast (MXFP4 row copy + MXFP8 column copy).  They also pin the
hardware's scaled FP8 conversion (rounding, saturation through the clamp, subnormal codes,
subnormal scales) against the oracle's exact rounding.
GEMMs: the block-scaled bar of the MXFP4 GEMM tests plus the in-group truncation the FP8
scaled MFMA performs (measured: groups of 8 products, each truncated toward zero to 13 bits
below the group's largest exponent sum; fp8_truncation_bound); bit-exact bf16 where every
product is exact on that grid and the fp32 accumulation is exact in any order.
The step with the FP8 wgrad option: forward and dA against the MXFP4 oracle, dB against the
MXFP8 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import (say, to_device, operand_rowmajor, operand_padding, bf16_to_f64, assert_gemm_close,
                      bf16_rne_of_exact, fp8_truncation_bound, device_ref_blocks)

pytestmark = pytest.mark.gpu


def check(op, ref, what):
    q_ref, s_ref = ref
    q, s = operand_rowmajor(op)
    assert np.array_equal(s, s_ref), "%s: scales differ at %s" % (what, np.argwhere(s != s_ref)[:5].tolist())
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, "%s: codes differ at %s (got %s want %s)" % (
        what, bad[:5].tolist(), [hex(q[tuple(i)]) for i in bad[:5]], [hex(q_ref[tuple(i)]) for i in bad[:5]])
    assert np.all(operand_padding(op) == 0), "%s: padding not zero" % what


def run_casts(x_bits, what):
    x = to_device(x_bits)
    say("mxfp8 casts %s %s" % (what, x_bits.shape))
    r8 = mx.cast_fp8(x)
    d8 = mx.cast_fp8_dual(x)
    mixed = mx.cast_dual_fp8col(x)
    torch.cuda.synchronize()
    row8 = oracle.cast_rows_fp8(x_bits)
    col8 = oracle.cast_cols_fp8(x_bits)
    check(r8, row8, what + " row (mxfp8_cast)")
    check(d8.row, row8, what + " row (mxfp8_cast_dual)")
    check(d8.col, col8, what + " col (mxfp8_cast_dual)")
    check(mixed.row, oracle.cast_rows(x_bits), what + " MXFP4 row (mixed)")
    check(mixed.col, col8, what + " col (mixed)")


@pytest.mark.parametrize("R,C", [(1, 32), (17, 96), (64, 256), (100, 800), (257, 2080), (300, 4096)])
def test_ragged_values(R, C):
    run_casts(W.ragged_values((R, C), 41 * R + C), "ragged")


def test_every_bf16_pattern():
    # all 65536 bit patterns (Inf / NaN blocks included), in rows and down columns
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(2048, 32)
    run_casts(x, "all patterns")
    run_casts(np.ascontiguousarray(x.reshape(64, 1024)), "all patterns, wide")


def test_saturation_and_ties():
    # blocks whose amax mantissa is near 2 (x / 2^X in [448, 512): clamped to 448), every bf16
    # mantissa at a fixed exponent beside an anchor (all E4M3 ties of the top binades), and
    # tiny blocks (scale byte 0: subnormal fp32 scale, E4M3 subnormal codes)
    rng = np.random.default_rng(3)
    rows = []
    for e in (-100, -3, 0, 5, 60, 120):
        for m in range(128):
            anchor = (127 + e) << 7 | 0x7F                      # 1.9921875 * 2^e
            blk = rng.integers(0, 128, 32).astype(np.uint16) | ((127 + e) << 7)
            blk[0] = anchor
            blk[1] = ((127 + e) << 7) | m                        # every mantissa in the amax binade
            blk |= (rng.integers(0, 2, 32).astype(np.uint16) << 15)
            rows.append(blk)
    tiny = rng.integers(1, 0x0100, (64, 32)).astype(np.uint16)   # subnormal and min-normal bf16
    tiny |= (rng.integers(0, 2, (64, 32)).astype(np.uint16) << 15)
    x = np.concatenate([np.array(rows, np.uint16), tiny])
    run_casts(x, "saturation/ties/tiny")


def test_normal_values_with_outliers():
    run_casts(W.activations_with_outliers(512, 1024, 91, 92), "normal+outliers")


# ---- GEMM

def gpu_nt8(a_bits, b_bits, what):
    say("gemm_fp8_nt %s M=%d N=%d K=%d" % (what, a_bits.shape[0], b_bits.shape[0], a_bits.shape[1]))
    a = mx.cast_fp8(to_device(a_bits))
    b = mx.cast_fp8(to_device(b_bits))
    out = mx.gemm_fp8_nt(a, b)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def oracle_nt8(a_bits, b_bits):
    """(ref, absref, truncation allowance) of out = A . B^T on the oracle's MXFP8 operands."""
    qa, sa = oracle.cast_rows_fp8(a_bits)
    qb, sb = oracle.cast_rows_fp8(b_bits)
    ref, absref = oracle.gemm_fp8(qa, sa, qb, sb)
    return ref, absref, fp8_truncation_bound(qa, sa, qb, sb)


# The device reference of the full-size whole-output FP8 check against the oracle: the oracle-dequantized
# MXFP8 operands' float64 product equals the oracle's MXFP8 GEMM (to 1e-12 of sum|ab|), and the
# envelope allowance (one matrix product of per-group exponent maxima) is never below the per-group
# truncation bound of fp8_truncation_bound.
def test_device_reference_fp8_matches_oracle():
    M, N, K = 300, 260, 1056
    a = W.ragged_values((M, K), 61)
    b = W.ragged_values((N, K), 67)
    qa, sa = oracle.cast_rows_fp8(a)
    qb, sb = oracle.cast_rows_fp8(b)
    ref, absref = oracle.gemm_fp8(qa, sa, qb, sb)
    tight = fp8_truncation_bound(qa, sa, qb, sb)
    say("fp8 device reference %dx%dx%d" % (M, N, K))
    got_ref, got_abs, got_extra = np.empty_like(ref), np.empty_like(absref), np.empty_like(ref)
    for r0, r, ab, ex in device_ref_blocks((qa, sa), (qb, sb), torch.device("cuda:0"), block_rows=128, fmt=8):
        got_ref[r0:r0 + r.shape[0]] = r.cpu().numpy()
        got_abs[r0:r0 + r.shape[0]] = ab.cpu().numpy()
        got_extra[r0:r0 + r.shape[0]] = ex.cpu().numpy()
    assert np.all(np.abs(got_ref - ref) <= 1e-12 * absref + 1e-300)
    assert np.all(np.abs(got_abs - absref) <= 1e-12 * absref + 1e-300)
    assert np.all(got_extra >= tight)


@pytest.mark.parametrize("M,N,K", [(1, 128, 32), (17, 128, 32), (33, 65, 96), (64, 64, 64), (100, 200, 288),
                                   (129, 257, 544), (256, 96, 1024), (1, 300, 2048), (70, 33, 320)])
def test_ragged_small(M, N, K):
    a = W.ragged_values((M, K), M * 37 + K)
    b = W.ragged_values((N, K), N * 19 + K)
    ref, absref, trunc = oracle_nt8(a, b)
    assert_gemm_close(gpu_nt8(a, b, "ragged"), ref, absref, "fp8 ragged %dx%dx%d" % (M, N, K), trunc)


# at least 128 output tiles of 256 x 256: persistent kernel with one trip per tile (K <= 256: four
# 64-wide K tiles, of which K = 32, 128, 192 and 256 fill 1, 2, 3 and 4), several trips with a K tail
# (K not a multiple of 256), the pipelined kernel (N % 8 != 0), ragged M / N edges
@pytest.mark.parametrize("M,N,K", [(4096, 2048, 32), (2048, 4096, 128), (2048, 4096, 192), (2048, 4096, 256),
                                   (2100, 4000, 288), (4096, 2056, 800), (2048, 4100, 1024), (2304, 3840, 1024),
                                   (3000, 2568, 1568)])
def test_tiled_shapes(M, N, K):
    a = W.normal_bf16((M, K), 1.0, M + 5 * K)
    b = W.normal_bf16((N, K), 0.5, N + 13 * K)
    ref, absref, trunc = oracle_nt8(a, b)
    assert_gemm_close(gpu_nt8(a, b, "tiled"), ref, absref, "fp8 tiled %dx%dx%d" % (M, N, K), trunc)


# skinny kernel: split contraction, NB = 1 and 2 (FP8 stops at 2), the smaller side as A (also in
# two 32-row groups)
@pytest.mark.parametrize("M,N,K", [(1, 4096, 14336), (4096, 32, 8192), (32, 65536, 1024), (65536, 100, 544),
                                   (17, 300, 2080), (1000, 2000, 1024), (48, 3000, 544), (5000, 64, 2080)])
def test_skinny_shapes(M, N, K):
    a = W.ragged_values((M, K), 7 * M + K)
    b = W.ragged_values((N, K), 11 * N + K)
    ref, absref, trunc = oracle_nt8(a, b)
    assert_gemm_close(gpu_nt8(a, b, "skinny"), ref, absref, "fp8 skinny %dx%dx%d" % (M, N, K), trunc)


def integer_blocks(M, K, seed):
    """bf16 values v / 64 with one anchor v = 256 per block (fixes X = -6), zeros beside it in
    its group of 8, and integers |v| <= 16 elsewhere: every code is exact, no product falls
    below its group's truncation grid (2^(E-13) with E <= 8 away from the anchors), every
    product is an integer / 4096, and any fp32 sum of them over K <= 512 stays an integer
    multiple of 2^-12 below 2^24 units -- exact in any order."""
    rng = np.random.default_rng(seed)
    v = rng.integers(-16, 17, (M, K)).astype(np.float32)
    v[:, (np.arange(K) % 32) < 8] = 0.0
    v[:, ::32] = 256.0
    return W.bf16_bits(v / 64.0)


@pytest.mark.parametrize("M,N,K", [(96, 160, 32), (384, 320, 512), (2048, 4096, 512), (4096, 2048, 32)])
def test_exact_sums_are_bit_exact(M, N, K):
    a, b = integer_blocks(M, K, 1), integer_blocks(N, K, 2)
    ref, _, _ = oracle_nt8(a, b)
    assert np.array_equal(gpu_nt8(a, b, "exact"), bf16_rne_of_exact(ref))


def test_one_hot_rows_pick_dequantized_entries():
    # A row m = e_{k_m}: out[m, n] = dequant(B)[n, k_m] exactly (pins the FP8 operand lane layout)
    rng = np.random.default_rng(9)
    for M, N, K in ((64, 96, 1024), (512, 4096, 1024)):
        ks = rng.integers(0, K, M)
        a = np.zeros((M, K), np.uint16)
        a[np.arange(M), ks] = 0x3F80
        b = W.normal_bf16((N, K), 1.0, 23)
        got = gpu_nt8(a, b, "one-hot")
        db = oracle.dequant_fp8(*oracle.cast_rows_fp8(b))
        assert np.array_equal(got, bf16_rne_of_exact(db[:, ks].T.copy()))


def test_empty_and_zero_k():
    a = mx.empty_operand(0, 64, "cuda:0", 8)
    b = mx.empty_operand(8, 64, "cuda:0", 8)
    assert mx.gemm_fp8_nt(a, b).shape == (0, 8)
    a = mx.empty_operand(300, 0, "cuda:0", 8)
    b = mx.empty_operand(40, 0, "cuda:0", 8)
    out = mx.gemm_fp8_nt(a, b)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()).item() == 0


def test_formats_must_match():
    x = to_device(W.normal_bf16((64, 64), 1.0, 3))
    with pytest.raises(ValueError):
        mx.gemm_fp8_nt(mx.cast(x), mx.cast_fp8(x))
    with pytest.raises(ValueError):
        mx.gemm_nt(mx.cast_fp8(x), mx.cast_fp8(x))


# ---- the step with the FP8 wgrad

def oracle_step_fp8_wgrad(a, w, dout):
    f = oracle.gemm(*oracle.cast_rows(a), *oracle.cast_rows(w))
    d = oracle.gemm(*oracle.cast_rows(dout), *oracle.cast_cols(w))
    qg, sg = oracle.cast_cols_fp8(dout)
    qa, sa = oracle.cast_cols_fp8(a)
    g = oracle.gemm_fp8(qg, sg, qa, sa) + (fp8_truncation_bound(qg, sg, qa, sa),)
    return f, d, g


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (17, 128, 32), (100, 160, 320), (300, 64, 544),
                                   (2048, 4096, 1024)])
def test_step_with_fp8_wgrad_matches_oracle(M, N, K):
    a = W.ragged_values((M, K), 3 * M + K + 2)
    w = W.ragged_values((N, K), 5 * N + K + 2)
    dout = W.ragged_values((M, N), 7 * M + N + 2)
    say("gemm_fp4_bf16 fp8 wgrad step M=%d N=%d K=%d" % (M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt, fp8_wgrad=True)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    (f, fa), (d, da_abs), (g, ga, gt) = oracle_step_fp8_wgrad(a, w, dout)
    assert_gemm_close(bf16_to_f64(out.detach()), f, fa, "fwd")
    assert_gemm_close(bf16_to_f64(at.grad), d, da_abs, "dA")
    assert_gemm_close(bf16_to_f64(wt.grad), g, ga, "dB (MXFP8)", gt)


def test_fp8_wgrad_with_cached_weight_is_identical():
    M, N, K = 256, 512, 1024
    a = W.ragged_values((M, K), 61)
    w = W.ragged_values((N, K), 62)
    dout = W.ragged_values((M, N), 63)
    say("gemm_fp4_bf16 fp8 wgrad, cached weight")
    w_dev = to_device(w)
    outs = []
    for cached in (False, True):
        at = to_device(a).requires_grad_(True)
        wt = w_dev.clone().requires_grad_(True)
        w_fp4 = mx.MXFP4Quantizer.for_weight().quantize(w_dev) if cached else None
        out = mx.gemm_fp4_bf16(at, wt, w_fp4=w_fp4, fp8_wgrad=True)
        out.backward(to_device(dout))
        torch.cuda.synchronize()
        outs.append((out.detach().cpu(), at.grad.cpu(), wt.grad.cpu()))
    for x, y in zip(*outs):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    with pytest.raises(ValueError):
        mx.gemm_fp4_bf16(to_device(a).requires_grad_(True), w_dev, hadamard_grad=True, fp8_wgrad=True)


def test_fp8_wgrad_is_more_accurate():
    # against the exact product of the bf16 inputs, dB from MXFP8 operands (3 mantissa bits)
    # carries well under half the RMS error of dB from MXFP4 operands (1 mantissa bit)
    M, N, K = 1024, 512, 256
    a = W.normal_bf16((M, K), 1.0, 31)
    w = W.normal_bf16((N, K), 1.0, 32)
    g = W.normal_bf16((M, N), 1.0, 33)
    exact = bf16_to_f64(to_device(g)).T @ bf16_to_f64(to_device(a))
    errs = []
    for f8 in (False, True):
        say("dB error, fp8_wgrad=%s" % f8)
        wt = to_device(w).requires_grad_(True)
        out = mx.gemm_fp4_bf16(to_device(a), wt, fp8_wgrad=f8)
        out.backward(to_device(g))
        torch.cuda.synchronize()
        errs.append(np.sqrt(np.mean((bf16_to_f64(wt.grad) - exact) ** 2)))
    assert errs[1] < 0.5 * errs[0], errs


def test_mfma_group_truncation_model():
    # the arithmetic fp8_truncation_bound assumes, on single-product probes: A = ones, each B row
    # holds +1, -1 at K 0, 1 (their products cancel) and one small product s = 2^-gap
    K = 256
    rows, expect = [], []
    for gap in (12, 13, 14, 15):
        s = 2.0 ** -gap
        for k, sign in ((7, 1), (2, -1), (8, 1), (40, 1), (128, 1)):
            b = np.zeros(K, np.float32)
            b[0], b[1], b[k] = 1.0, -1.0, sign * s
            rows.append(b)
            # in the group of K 0..7 (exponent sum 0) a product below 2^-13 truncates to zero;
            # in any other group it is the group's largest and stays exact
            expect.append(0.0 if (k < 8 and gap > 13) else sign * s)
    # truncation toward zero on the 2^-13 grid
    for v in (1.5, -1.5, 3.75, -3.75):
        b = np.zeros(K, np.float32)
        b[0], b[1], b[2] = 1.0, -1.0, v * 2.0 ** -13
        rows.append(b)
        expect.append(np.trunc(v) * 2.0 ** -13)
    vals = np.array(rows, np.float32)
    B = W.bf16_bits(vals)
    A = W.bf16_bits(np.ones((1, K), np.float32))
    # the probes are exact in bf16 and in MXFP8
    assert np.array_equal(oracle.dequant_fp8(*oracle.cast_rows_fp8(B)), vals.astype(np.float64))
    got = gpu_nt8(A, B, "truncation probes")[0]
    assert np.array_equal(got, np.array(expect)), list(zip(got, expect))
