"""GPU parity of the Hadamard-transformed casts and of the gemm_fp4_bf16 step with the
Hadamard gradient recipe, against the CPU oracle.

Casts: bit for bit (both sides evaluate the transform with the same binary32 butterflies).
GEMMs: the block-scaled bar of the other GEMM tests, the oracle quantizing every operand
from the bf16 sources with its own Hadamard casts.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, operand_rowmajor, operand_padding, bf16_to_f64, assert_gemm_close

pytestmark = pytest.mark.gpu


def check(op, ref, what):
    q_ref, s_ref = ref
    q, s = operand_rowmajor(op)
    assert np.array_equal(s, s_ref), "%s: scales differ at %s" % (what, np.argwhere(s != s_ref)[:5].tolist())
    assert np.array_equal(q, q_ref), "%s: codes differ at %s" % (what, np.argwhere(q != q_ref)[:5].tolist())
    assert np.all(operand_padding(op) == 0), "%s: padding not zero" % what


def run(x_bits, t_row, t_col, shift, what):
    x = to_device(x_bits)
    say("cast_hadamard %s %s row=%d col=%d shift=%d" % (what, x_bits.shape, t_row, t_col, shift))
    t = mx.cast_hadamard(x, t_row, t_col, shift)
    say("cast_hadamard row-only %s" % what)
    r = mx.cast_hadamard(x, t_row, False, shift, columnwise=False)
    torch.cuda.synchronize()
    row_ref = oracle.cast_rows_hadamard(x_bits, shift) if t_row else oracle.cast_rows(x_bits)
    col_ref = oracle.cast_cols_hadamard(x_bits, shift) if t_col else oracle.cast_cols(x_bits)
    check(t.row, row_ref, what + " row")
    check(t.col, col_ref, what + " col")
    check(r.row, row_ref, what + " row-only")


MODES = [(True, True, 5), (False, True, 0), (True, False, 0), (True, True, 0)]


@pytest.mark.parametrize("mode", MODES, ids=["grad", "colonly", "rowonly", "both-shift0"])
@pytest.mark.parametrize("R,C", [(1, 32), (17, 96), (64, 256), (100, 800), (257, 2080), (300, 4096)])
def test_ragged_values(R, C, mode):
    run(W.ragged_values((R, C), 31 * R + C), *mode, "ragged")


@pytest.mark.parametrize("mode", MODES, ids=["grad", "colonly", "rowonly", "both-shift0"])
def test_normal_values_with_outliers(mode):
    x = W.activations_with_outliers(512, 1024, 71, 72)
    run(x, *mode, "normal+outliers")


def test_every_bf16_pattern():
    # all 65536 bit patterns (Inf / NaN blocks included) in a [2048, 32] matrix
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(2048, 32)
    for mode in MODES:
        run(x, *mode, "all patterns")


def test_overflowing_blocks():
    # 32 values at the bf16 maximum sum past binary32's range: scale 0xFF, codes 0
    x = np.full((64, 64), 0x7F7F, np.uint16)
    x[:, 32:] = W.bf16_bits(np.ones((64, 32), np.float32))
    for mode in MODES:
        run(x, *mode, "overflow")


def oracle_step_hadamard(a, w, dout):
    f = oracle.gemm(*oracle.cast_rows(a), *oracle.cast_rows(w))
    d = oracle.gemm(*oracle.cast_rows_hadamard(dout, 5), *oracle.cast_cols_hadamard(w, 0))
    g = oracle.gemm(*oracle.cast_cols_hadamard(dout, 5), *oracle.cast_cols_hadamard(a, 0))
    return f, d, g


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (17, 128, 32), (100, 160, 320), (300, 64, 544),
                                   (2048, 4096, 1024)])
def test_step_with_hadamard_grad_matches_oracle(M, N, K):
    a = W.ragged_values((M, K), 3 * M + K + 1)
    w = W.ragged_values((N, K), 5 * N + K + 1)
    dout = W.ragged_values((M, N), 7 * M + N + 1)
    say("gemm_fp4_bf16 hadamard step M=%d N=%d K=%d" % (M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt, hadamard_grad=True)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    (f, fa), (d, da_abs), (g, ga) = oracle_step_hadamard(a, w, dout)
    assert_gemm_close(bf16_to_f64(out.detach()), f, fa, "fwd")
    assert_gemm_close(bf16_to_f64(at.grad), d, da_abs, "dA (Hadamard)")
    assert_gemm_close(bf16_to_f64(wt.grad), g, ga, "dB (Hadamard)")


def test_cached_weight_with_hadamard_recipe():
    M, N, K = 256, 512, 1024
    a = W.ragged_values((M, K), 81)
    w = W.ragged_values((N, K), 82)
    dout = W.ragged_values((M, N), 83)
    say("gemm_fp4_bf16 hadamard, cached weight")
    w_dev = to_device(w)
    ws = mx.WeightWorkspace()
    outs = []
    for cached in (False, True):
        at = to_device(a).requires_grad_(True)
        wt = w_dev.clone().requires_grad_(True)
        w_fp4 = ws.get_or_quantize(w_dev, mx.MXFP4Quantizer.for_weight(hadamard=True), "w") if cached else None
        out = mx.gemm_fp4_bf16(at, wt, w_fp4=w_fp4, hadamard_grad=True)
        out.backward(to_device(dout))
        torch.cuda.synchronize()
        outs.append((out.detach().cpu(), at.grad.cpu(), wt.grad.cpu()))
    for x, y in zip(*outs):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # a weight quantized without the transform does not fit the recipe (and vice versa)
    plain = mx.MXFP4Quantizer.for_weight().quantize(w_dev)
    with pytest.raises(ValueError):
        mx.gemm_fp4_bf16(to_device(a).requires_grad_(True), w_dev, w_fp4=plain, hadamard_grad=True)
    transformed = ws.get_or_quantize(w_dev, mx.MXFP4Quantizer.for_weight(hadamard=True), "w")
    assert ws.hits == 1
    with pytest.raises(ValueError):
        mx.gemm_fp4_bf16(to_device(a).requires_grad_(True), w_dev, w_fp4=transformed)


def test_hadamard_recipe_lowers_gradient_error_on_outliers():
    # dOut with one x20 value per 32-block along N: dA's error against the exact product of the
    # bf16 inputs drops with the recipe (the oracle pins the same effect)
    rng = np.random.default_rng(12)
    M, N, K = 512, 1024, 512
    g = rng.standard_normal((M, N)).astype(np.float32)
    g[np.arange(M)[:, None], rng.integers(0, 32, (M, N // 32)) + 32 * np.arange(N // 32)] *= 20
    a = W.normal_bf16((M, K), 1.0, 13)
    w = W.normal_bf16((N, K), 1.0, 14)
    gb = W.bf16_bits(g)
    exact = bf16_to_f64(to_device(gb)) @ bf16_to_f64(to_device(w))
    errs = []
    for had in (False, True):
        say("dA error, hadamard=%s" % had)
        at = to_device(a).requires_grad_(True)
        out = mx.gemm_fp4_bf16(at, to_device(w), hadamard_grad=had)
        out.backward(to_device(gb))
        torch.cuda.synchronize()
        errs.append(np.sqrt(np.mean((bf16_to_f64(at.grad) - exact) ** 2)))
    assert errs[1] < 0.85 * errs[0], errs
