"""GPU cast parity: the HIP row and dual casts must equal the CPU oracle bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, operand_rowmajor, operand_padding, assert_operand_equal

pytestmark = pytest.mark.gpu


def check_row(x_bits, op, what):
    q_ref, s_ref = oracle.cast_rows(x_bits)
    q, s = operand_rowmajor(op)
    assert np.array_equal(s, s_ref), "%s: row scales differ at %s" % (what, np.argwhere(s != s_ref)[:5].tolist())
    assert np.array_equal(q, q_ref), "%s: row codes differ at %s" % (what, np.argwhere(q != q_ref)[:5].tolist())
    assert np.all(operand_padding(op) == 0), "%s: row padding not zero" % what


def check_col(x_bits, op, what):
    q_ref, s_ref = oracle.cast_cols(x_bits)
    q, s = operand_rowmajor(op)
    assert np.array_equal(s, s_ref), "%s: col scales differ at %s" % (what, np.argwhere(s != s_ref)[:5].tolist())
    assert np.array_equal(q, q_ref), "%s: col codes differ at %s" % (what, np.argwhere(q != q_ref)[:5].tolist())
    assert np.all(operand_padding(op) == 0), "%s: col padding not zero" % what


def run_both(x_bits, what):
    x = to_device(x_bits)
    say("cast %s %s" % (what, x_bits.shape))
    op = mx.cast(x)
    say("cast_dual %s %s" % (what, x_bits.shape))
    t = mx.cast_dual(x)
    torch.cuda.synchronize()
    check_row(x_bits, op, what + " cast")
    check_row(x_bits, t.row, what + " dual.row")
    check_col(x_bits, t.col, what + " dual.col")


def test_tiny_config():
    a, w, _ = W.projection_inputs("tiny", 0, 256, 256, 256, with_grad=False)
    run_both(a, "tiny A")
    run_both(w, "tiny B")


def test_hand_block_matrix():
    run_both(W.hand_block_matrix(), "hand blocks")


@pytest.mark.parametrize("R,C", [(1, 32), (17, 32), (1, 4096), (17, 96), (31, 288), (64, 256), (65, 544),
                                 (100, 800), (257, 2080), (300, 256)])
def test_ragged_shapes(R, C):
    run_both(W.ragged_values((R, C), 7 * R + C), "ragged")


def test_every_bf16_pattern_at_every_exponent_band():
    # each row: an anchor fixing the block exponent, then 31 consecutive bf16 patterns;
    # anchors sweep 2^-126 .. 2^127 so every pattern meets many scales
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((pats >> 7) & 0xFF) != 0xFF
    pats = pats[finite]
    nrow = -(-pats.size // 31)
    pats = np.concatenate([pats, np.zeros(nrow * 31 - pats.size, np.uint16)]).reshape(nrow, 31)
    rows = []
    for e in range(1, 255, 9):
        anchor = np.full((nrow, 1), e << 7, np.uint16)
        rows.append(np.concatenate([anchor, pats], 1))
    x = np.concatenate(rows, 0)
    run_both(x, "bf16 sweep")


def test_nonfinite_blocks():
    rng = np.random.default_rng(3)
    x = W.normal_bf16((64, 128), 1.0, 5)
    x[0, 3] = 0x7F80
    x[5, 100] = 0xFF80
    x[40, 64] = 0x7FC0
    x[33, 0:32] = 0x7F81
    run_both(x, "non-finite")


def test_strided_input():
    base = W.normal_bf16((48, 512), 1.0, 9)
    xt = to_device(base)[:, :256]      # leading dimension 512, 256 columns
    say("cast strided")
    op = mx.cast(xt)
    t = mx.cast_dual(xt)
    torch.cuda.synchronize()
    sub = np.ascontiguousarray(base[:, :256])
    check_row(sub, op, "strided cast")
    check_row(sub, t.row, "strided dual.row")
    check_col(sub, t.col, "strided dual.col")


def test_side_stream_ordering():
    # the cast must run on the caller's stream: queue long work first on a side stream,
    # cast on that stream, and read the result after synchronizing only that stream
    x_bits = W.normal_bf16((4096, 4096), 1.0, 77)
    x = to_device(x_bits)
    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda:0")
    torch.cuda.synchronize()
    say("cast on a side stream behind ballast work")
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big.T / 4096.0
        y = x * 1  # produced on the side stream just before the cast
        t = mx.cast_dual(y)
    side.synchronize()
    check_row(x_bits, t.row, "side stream row")
    check_col(x_bits, t.col, "side stream col")


@pytest.mark.parametrize("shape0,shape1", [((65, 544), (257, 2080)), ((8, 256), (300, 256)), ((0, 64), (17, 96)),
                                           ((31, 288), (0, 0)), ((1, 4096), (1, 32))])
def test_dual_pair_equals_two_dual_casts(shape0, shape1):
    # one launch for two tensors: both results bit-equal to the oracle (and to separate launches);
    # the first tensor's grid (padded to a multiple of 8 workgroups) and an empty tensor on either side
    from mxfp4_block_scaled_cast_amd import _native as N
    dev = torch.device("cuda:0")
    xs, rows, cols = [], [], []
    for i, (R, C) in enumerate((shape0, shape1)):
        bits = W.ragged_values((R, C), 11 * R + C + i) if R * C else np.zeros((R, C), dtype=np.uint16)
        xs.append(bits)
    say("cast_dual_pair %s %s" % (shape0, shape1))
    ops = []
    for bits in xs:
        R, C = bits.shape
        x = to_device(bits) if R * C else torch.empty((max(R, 1), max(C, 32)), dtype=torch.bfloat16, device=dev)
        ops.append((x, R, C, mx.empty_operand(R, C, dev), mx.empty_operand(C, -(-R // 32) * 32, dev)))
    args = []
    for x, R, C, row, col in ops:
        args += [x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(), col.q.data_ptr(),
                 col.s.data_ptr()]
    sp = torch.cuda.current_stream(dev).cuda_stream
    N.check(N.lib().mxfp4_cast_dual_pair(*args, sp), "mxfp4_cast_dual_pair")
    torch.cuda.synchronize()
    for bits, (x, R, C, row, col) in zip(xs, ops):
        if R * C == 0:
            continue
        check_row(bits, row, "pair row %dx%d" % (R, C))
        check_col(bits, col, "pair col %dx%d" % (R, C))


def test_python_cast_dual_pair():
    a = W.ragged_values((300, 544), 21)
    b = W.ragged_values((65, 96), 22)
    say("cast_dual_pair (python) %s %s" % (a.shape, b.shape))
    ta, tb = mx.cast_dual_pair(to_device(a), to_device(b))
    torch.cuda.synchronize()
    check_row(a, ta.row, "pair A row")
    check_col(a, ta.col, "pair A col")
    check_row(b, tb.row, "pair B row")
    check_col(b, tb.col, "pair B col")


def test_dual_pair_strided_inputs():
    # row strides larger than the row (views into wider matrices), different for the two tensors
    from mxfp4_block_scaled_cast_amd import _native as N
    dev = torch.device("cuda:0")
    a = W.ragged_values((70, 256), 31)
    b = W.ragged_values((129, 96), 32)
    wide_a = np.zeros((70, 264), dtype=np.uint16)
    wide_a[:, :256] = a
    wide_b = np.zeros((129, 1000), dtype=np.uint16)
    wide_b[:, 8:104] = b
    xa = to_device(wide_a)[:, :256]
    xb = to_device(wide_b)[:, 8:104]
    say("cast_dual_pair strided %s %s" % (a.shape, b.shape))
    outs, args = [], []
    for x, (R, C) in ((xa, a.shape), (xb, b.shape)):
        row, col = mx.empty_operand(R, C, dev), mx.empty_operand(C, -(-R // 32) * 32, dev)
        outs.append((row, col))
        args += [x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(), col.q.data_ptr(),
                 col.s.data_ptr()]
    N.check(N.lib().mxfp4_cast_dual_pair(*args, torch.cuda.current_stream(dev).cuda_stream), "pair")
    torch.cuda.synchronize()
    for bits, (row, col) in zip((a, b), outs):
        check_row(bits, row, "strided pair row")
        check_col(bits, col, "strided pair col")


# A tensor of more than 2^31 elements (16384 x 131104 = 2^31 + 524288, 4.3 GB of bf16): element, code
# and scale offsets past 32 bits in both copies.  Every byte of the row and column copies (padding
# included) against the oracle's casts of the whole input.
@pytest.mark.slow
def test_dual_cast_past_2_31_elements():
    R, C = 16384, 131104
    dev = torch.device("cuda:0")
    x = W.ragged_values_torch((R, C), 8801, dev).view(torch.bfloat16)
    say("cast_dual %d x %d (%d elements)" % (R, C, R * C))
    t = mx.cast_dual(x)
    torch.cuda.synchronize()
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    del x
    q, s = oracle.cast_rows(bits)
    assert_operand_equal(t.row, q, s, "2^31+ row copy")
    del q, s
    q, s = oracle.cast_cols(bits)
    assert_operand_equal(t.col, q, s, "2^31+ column copy")


# Seeded random shapes (numpy default_rng(77), plus two just under the switch) on both sides of the
# launcher's tile switch: casts of up to 4096 tiles of 64 rows take 32-row tiles, larger ones 64-row
# tiles (9224 x 8160: 4640 tiles; 9224 x 7168: 4060; 16138 x 4000: 4048), rows and columns not
# multiples of the tile; row cast and dual cast, every byte of every copy against the oracle.
RANDOM_CAST_SHAPES = [(180, 5024), (1904, 3520), (2386, 1568), (2595, 2144), (2905, 2048), (1073, 2496),
                      (9224, 8160), (5452, 14528), (7367, 10080), (16138, 4480), (9224, 7168), (16138, 4000)]


@pytest.mark.parametrize("R,C", RANDOM_CAST_SHAPES)
def test_random_shapes(R, C):
    run_both(W.ragged_values((R, C), 13 * R + C), "random")


# Pairs in one launch, the switch decided on both tensors' tiles together (1815, 4025 and 926 tiles:
# 32-row tiles for all three).
@pytest.mark.parametrize("shape0,shape1", [((8768, 1056), (7175, 2464)), ((6396, 5600), (4617, 6240)),
                                           ((2636, 4576), (2138, 1216))])
def test_random_shape_pairs(shape0, shape1):
    a = W.ragged_values(shape0, 17 * shape0[0] + shape0[1])
    b = W.ragged_values(shape1, 19 * shape1[0] + shape1[1])
    say("cast_dual_pair random %s %s" % (shape0, shape1))
    ta, tb = mx.cast_dual_pair(to_device(a), to_device(b))
    torch.cuda.synchronize()
    check_row(a, ta.row, "random pair A row")
    check_col(a, ta.col, "random pair A col")
    check_row(b, tb.row, "random pair B row")
    check_col(b, tb.col, "random pair B col")
