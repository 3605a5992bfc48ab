"""gemm_fp4_bf16 forward + backward (FP4 fwd, FP4 dA, FP4 dB) against the oracle.

The oracle quantizes each operand from the bf16 sources: forward uses the row
copies of A and W, dA the row copy of dOut and the column copy of W, dB the
column copies of dOut and A.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, bf16_to_f64, assert_gemm_close, assert_gemm_whole

pytestmark = pytest.mark.gpu


def oracle_step(a, w, dout):
    qa, sa = oracle.cast_rows(a)
    qw, sw = oracle.cast_rows(w)
    fwd = oracle.gemm(qa, sa, qw, sw)
    qg, sg = oracle.cast_rows(dout)
    qwc, swc = oracle.cast_cols(w)
    da = oracle.gemm(qg, sg, qwc, swc)
    qgc, sgc = oracle.cast_cols(dout)
    qac, sac = oracle.cast_cols(a)
    dw = oracle.gemm(qgc, sgc, qac, sac)
    return fwd, da, dw


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (17, 128, 32), (1, 96, 64), (100, 160, 320), (300, 64, 544)])
def test_step_matches_oracle(M, N, K):
    a = W.ragged_values((M, K), 3 * M + K)
    w = W.ragged_values((N, K), 5 * N + K)
    dout = W.ragged_values((M, N), 7 * M + N)
    say("gemm_fp4_bf16 step M=%d N=%d K=%d" % (M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    (f, fa), (d, da_abs), (g, ga) = oracle_step(a, w, dout)
    assert_gemm_close(bf16_to_f64(out.detach()), f, fa, "fwd")
    assert_gemm_close(bf16_to_f64(at.grad), d, da_abs, "dA")
    assert_gemm_close(bf16_to_f64(wt.grad), g, ga, "dB")


# Steps whose dA and dB run as one paired launch (the XCDs divided between them): 2048 x 2048 x 4096
# (128 tiles each, 4 + 4 XCDs) against the oracle's GEMM, and a ragged 5000 x 3072 x 3104 (dA 240
# tiles over 3072, dB 156 tiles over 5024, M padded to 5024 in the column copies: 3 + 5 XCDs)
# against the device reference of the oracle's copies.
def test_step_paired_backward_matches_oracle():
    M, N, K = 2048, 2048, 4096
    assert mx.gemm_pair_split(M, K, N, N, K, M) == 4, "dA and dB should share one launch"
    test_step_matches_oracle(M, N, K)


def test_ragged_step_paired_backward_whole_output():
    M, N, K = 5000, 3072, 3104
    assert mx.gemm_pair_split(M, K, N, N, K, 5024) == 3, "dA and dB should share one launch"
    a = W.ragged_values((M, K), 31)
    w = W.ragged_values((N, K), 37)
    dout = W.ragged_values((M, N), 41)
    say("gemm_fp4_bf16 ragged paired step M=%d N=%d K=%d" % (M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    assert_gemm_whole(out.detach(), oracle.cast_rows(a), oracle.cast_rows(w), "ragged paired step fwd")
    assert_gemm_whole(at.grad, oracle.cast_rows(dout), oracle.cast_cols(w), "ragged paired step dA")
    assert_gemm_whole(wt.grad, oracle.cast_cols(dout), oracle.cast_cols(a), "ragged paired step dB")


def test_inference_forward_uses_row_copies_only():
    M, N, K = 64, 96, 128
    a = W.normal_bf16((M, K), 1.0, 51)
    w = W.normal_bf16((N, K), 0.02, 52)
    say("gemm_fp4_bf16 inference")
    with torch.no_grad():
        out = mx.gemm_fp4_bf16(to_device(a), to_device(w))
    torch.cuda.synchronize()
    qa, sa = oracle.cast_rows(a)
    qw, sw = oracle.cast_rows(w)
    ref, absref = oracle.gemm(qa, sa, qw, sw)
    assert_gemm_close(bf16_to_f64(out), ref, absref, "inference")
    assert mx.workspace_bytes(M, N, K, training=False) < mx.workspace_bytes(M, N, K, training=True)


def test_only_one_gradient():
    M, N, K = 64, 64, 64
    a = W.normal_bf16((M, K), 1.0, 61)
    w = W.normal_bf16((N, K), 1.0, 62)
    dout = W.normal_bf16((M, N), 1.0, 63)
    at = to_device(a)
    wt = to_device(w).requires_grad_(True)
    say("gemm_fp4_bf16 dW only")
    out = mx.gemm_fp4_bf16(at, wt)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    _, _, (g, ga) = oracle_step(a, w, dout)
    assert at.grad is None
    assert_gemm_close(bf16_to_f64(wt.grad), g, ga, "dB only")


@pytest.mark.parametrize("M,N,K", [(256, 512, 1024), (17, 128, 544), (1000, 2048, 4096)])
def test_cached_weight_matches_uncached(M, N, K):
    # the cached copies are the same casts of the same W, so every output is bit-identical,
    # and the uncached path is the one checked against the oracle above
    a = W.ragged_values((M, K), 11 * M + K)
    w = W.ragged_values((N, K), 13 * N + K)
    dout = W.ragged_values((M, N), 17 * M + N)
    say("gemm_fp4_bf16 cached weight M=%d N=%d K=%d" % (M, N, K))
    ws = mx.WeightWorkspace()
    w_dev = to_device(w)
    outs = []
    for cached in (False, True, True):
        at = to_device(a).requires_grad_(True)
        wt = w_dev.clone().requires_grad_(True)
        w_fp4 = ws.get_or_quantize(w_dev, mx.MXFP4Quantizer.for_weight(), cache_name="w") if cached else None
        out = mx.gemm_fp4_bf16(at, wt, w_fp4=w_fp4)
        out.backward(to_device(dout))
        torch.cuda.synchronize()
        outs.append((out.detach().cpu(), at.grad.cpu(), wt.grad.cpu()))
    assert ws.misses == 1 and ws.hits == 1
    for got in outs[1:]:
        for x, y in zip(outs[0], got):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_cached_weight_inference_and_role_checks():
    M, N, K = 64, 96, 128
    a = to_device(W.normal_bf16((M, K), 1.0, 61))
    w = to_device(W.normal_bf16((N, K), 0.02, 62))
    say("gemm_fp4_bf16 cached weight, inference")
    w_row = mx.MXFP4Quantizer.for_weight(columnwise=False).quantize(w)
    assert w_row.col is None
    with torch.no_grad():
        got = mx.gemm_fp4_bf16(a, w, w_fp4=w_row)
        ref = mx.gemm_fp4_bf16(a, w)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # training needs W's column copy
    with pytest.raises(ValueError):
        mx.gemm_fp4_bf16(a.clone().requires_grad_(True), w, w_fp4=w_row)
    # a stale cache entry is refreshed after an in-place update of W
    ws = mx.WeightWorkspace()
    q1 = ws.get_or_quantize(w, mx.MXFP4Quantizer.for_weight(), cache_name="w")
    w.mul_(2)
    q2 = ws.get_or_quantize(w, mx.MXFP4Quantizer.for_weight(), cache_name="w")
    torch.cuda.synchronize()
    assert q1 is not q2 and ws.misses == 2
    # doubling W moves every nonzero block's scale up by one (codes unchanged)
    assert torch.equal(q1.row.q, q2.row.q)


# Seeded random steps (numpy default_rng(99): M in 1..6000, N and K multiples of 32 up to 5088) through
# the autograd wrapper: fwd, dA and dB (the backward's pair call, which runs these as two launches),
# every output against the device reference of the oracle's copies.
RANDOM_STEPS = [(5749, 2592, 3872), (3390, 928, 2624), (5651, 4960, 4928), (3689, 1600, 2912),
                (3899, 1472, 4896), (3327, 1792, 2400), (639, 3104, 1760), (5582, 1536, 1280),
                (3615, 1600, 1760), (2347, 3520, 1376)]


@pytest.mark.slow
@pytest.mark.parametrize("M,N,K", RANDOM_STEPS)
def test_random_steps_whole_output(M, N, K):
    a = W.ragged_values((M, K), 3 * M + 5 * K)
    w = W.ragged_values((N, K), 7 * N + 11 * K)
    dout = W.ragged_values((M, N), 13 * M + 17 * N)
    say("gemm_fp4_bf16 random step M=%d N=%d K=%d" % (M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt)
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    assert_gemm_whole(out.detach(), oracle.cast_rows(a), oracle.cast_rows(w), "random step fwd")
    assert_gemm_whole(at.grad, oracle.cast_rows(dout), oracle.cast_cols(w), "random step dA")
    assert_gemm_whole(wt.grad, oracle.cast_cols(dout), oracle.cast_cols(a), "random step dB")


# The same kind of seeded random steps with the Hadamard gradient recipe (dA, dB on transformed copies:
# dOut's divided by 32) and with the FP8 wgrad (dB an MXFP8 product, its bar widened by the MFMA's
# in-group truncation envelope); every output against the device reference of the oracle's copies.
@pytest.mark.slow
@pytest.mark.parametrize("M,N,K", RANDOM_STEPS[:5])
@pytest.mark.parametrize("variant", ["hadamard", "fp8wgrad"])
def test_random_variant_steps_whole_output(M, N, K, variant):
    a = W.ragged_values((M, K), 3 * M + 5 * K + 1)
    w = W.ragged_values((N, K), 7 * N + 11 * K + 1)
    dout = W.ragged_values((M, N), 13 * M + 17 * N + 1)
    say("gemm_fp4_bf16 random %s step M=%d N=%d K=%d" % (variant, M, N, K))
    at = to_device(a).requires_grad_(True)
    wt = to_device(w).requires_grad_(True)
    out = mx.gemm_fp4_bf16(at, wt, hadamard_grad=variant == "hadamard", fp8_wgrad=variant == "fp8wgrad")
    out.backward(to_device(dout))
    torch.cuda.synchronize()
    assert_gemm_whole(out.detach(), oracle.cast_rows(a), oracle.cast_rows(w), "random %s fwd" % variant)
    if variant == "hadamard":
        assert_gemm_whole(at.grad, oracle.cast_rows_hadamard(dout, 5), oracle.cast_cols_hadamard(w, 0),
                          "random hadamard dA")
        assert_gemm_whole(wt.grad, oracle.cast_cols_hadamard(dout, 5), oracle.cast_cols_hadamard(a, 0),
                          "random hadamard dB")
    else:
        assert_gemm_whole(at.grad, oracle.cast_rows(dout), oracle.cast_cols(w), "random fp8wgrad dA")
        assert_gemm_whole(wt.grad, oracle.cast_cols_fp8(dout), oracle.cast_cols_fp8(a), "random fp8wgrad dB",
                          fmt=8)
