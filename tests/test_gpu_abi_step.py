"""The composed step's C entry points, called through ctypes on the GPU, against the oracle.

gemm_fp4_bf16_fwd / gemm_fp4_bf16_bwd (inference and training, either gradient alone), and
their pre-quantized-weight forms gemm_fp4_bf16_fwd_qw / gemm_fp4_bf16_bwd_qw fed with W's
copies from mxfp4_cast_dual; and the Python cached-weight path (WeightWorkspace +
gemm_fp4_bf16(w_fp4=...)) checked directly against the oracle's fwd, dA and dB.
Shapes span the skinny kernel, the persistent kernel with one trip per tile (K <= 512) and
with several trips, ragged M / N / K edges and a 32-row padded column copy (M = 17, 1000).
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import _native as native
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, bf16_to_f64, assert_gemm_close

pytestmark = pytest.mark.gpu

SHAPES = [(17, 128, 544), (256, 512, 1024), (1000, 2048, 4096), (2048, 4096, 512), (2304, 4096, 1536)]


def oracle_step(a, w, dout):
    qa, sa = oracle.cast_rows(a)
    qw, sw = oracle.cast_rows(w)
    fwd = oracle.gemm(qa, sa, qw, sw)
    if dout is None:
        return fwd, None, None
    qg, sg = oracle.cast_rows(dout)
    qwc, swc = oracle.cast_cols(w)
    da = oracle.gemm(qg, sg, qwc, swc)
    qgc, sgc = oracle.cast_cols(dout)
    qac, sac = oracle.cast_cols(a)
    dw = oracle.gemm(qgc, sgc, qac, sac)
    return fwd, da, dw


def inputs(M, Nn, K):
    a = W.ragged_values((M, K), 19 * M + K)
    w = W.ragged_values((Nn, K), 23 * Nn + K)
    g = W.ragged_values((M, Nn), 29 * M + Nn)
    return a, w, g


def empty_bf16(r, c):
    return torch.full((r, c), float("nan"), dtype=torch.bfloat16, device="cuda:0")


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plain_entry_points_training(M, N, K):
    a, w, g = inputs(M, N, K)
    L = native.lib()
    nbytes = L.gemm_fp4_bf16_workspace_bytes(M, N, K, 1)
    assert nbytes > 0
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda:0")
    ad, wd, gd = to_device(a), to_device(w), to_device(g)
    out, da, dw = empty_bf16(M, N), empty_bf16(M, K), empty_bf16(N, K)
    say("gemm_fp4_bf16_fwd/_bwd (C ABI) M=%d N=%d K=%d" % (M, N, K))
    native.check(L.gemm_fp4_bf16_fwd(ad.data_ptr(), wd.data_ptr(), M, N, K, out.data_ptr(), ws.data_ptr(), nbytes,
                                1, stream()), "gemm_fp4_bf16_fwd")
    native.check(L.gemm_fp4_bf16_bwd(gd.data_ptr(), M, N, K, ws.data_ptr(), nbytes, da.data_ptr(), dw.data_ptr(),
                                stream()), "gemm_fp4_bf16_bwd")
    torch.cuda.synchronize()
    (f, fa), (d, dab), (e, eab) = oracle_step(a, w, g)
    assert_gemm_close(bf16_to_f64(out), f, fa, "fwd")
    assert_gemm_close(bf16_to_f64(da), d, dab, "dA")
    assert_gemm_close(bf16_to_f64(dw), e, eab, "dB")
    # either gradient alone (the other pointer NULL) gives the same bits
    da2, dw2 = empty_bf16(M, K), empty_bf16(N, K)
    say("gemm_fp4_bf16_bwd dA only, dB only")
    native.check(L.gemm_fp4_bf16_bwd(gd.data_ptr(), M, N, K, ws.data_ptr(), nbytes, da2.data_ptr(), None, stream()),
            "gemm_fp4_bf16_bwd")
    native.check(L.gemm_fp4_bf16_bwd(gd.data_ptr(), M, N, K, ws.data_ptr(), nbytes, None, dw2.data_ptr(), stream()),
            "gemm_fp4_bf16_bwd")
    torch.cuda.synchronize()
    assert torch.equal(da2.view(torch.int16), da.view(torch.int16))
    assert torch.equal(dw2.view(torch.int16), dw.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(1, 96, 64), (17, 130, 544), (2048, 4096, 512)])
def test_plain_forward_inference(M, N, K):
    a, w, _ = inputs(M, N, K)
    L = native.lib()
    nbytes = L.gemm_fp4_bf16_workspace_bytes(M, N, K, 0)
    assert nbytes > 0
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda:0")
    out = empty_bf16(M, N)
    ad, wd = to_device(a), to_device(w)
    say("gemm_fp4_bf16_fwd inference (C ABI) M=%d N=%d K=%d" % (M, N, K))
    native.check(L.gemm_fp4_bf16_fwd(ad.data_ptr(), wd.data_ptr(), M, N, K, out.data_ptr(), ws.data_ptr(), nbytes, 0,
                                stream()), "gemm_fp4_bf16_fwd")
    torch.cuda.synchronize()
    (f, fa), _, _ = oracle_step(a, w, None)
    assert_gemm_close(bf16_to_f64(out), f, fa, "inference fwd")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_quantized_weight_entry_points(M, N, K):
    a, w, g = inputs(M, N, K)
    L = native.lib()
    Wt = mx.cast_dual(to_device(w))  # W's row + column copies, made once (mxfp4_cast_dual)
    nbytes = L.gemm_fp4_bf16_workspace_bytes_qw(M, N, K, 1)
    assert 0 < nbytes < L.gemm_fp4_bf16_workspace_bytes(M, N, K, 1)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda:0")
    ad, gd = to_device(a), to_device(g)
    out, da, dw = empty_bf16(M, N), empty_bf16(M, K), empty_bf16(N, K)
    say("gemm_fp4_bf16_fwd_qw/_bwd_qw (C ABI) M=%d N=%d K=%d" % (M, N, K))
    native.check(L.gemm_fp4_bf16_fwd_qw(ad.data_ptr(), Wt.row.q.data_ptr(), Wt.row.s.data_ptr(), M, N, K,
                                   out.data_ptr(), ws.data_ptr(), nbytes, 1, stream()), "gemm_fp4_bf16_fwd_qw")
    native.check(L.gemm_fp4_bf16_bwd_qw(gd.data_ptr(), Wt.col.q.data_ptr(), Wt.col.s.data_ptr(), M, N, K, ws.data_ptr(),
                                   nbytes, da.data_ptr(), dw.data_ptr(), stream()), "gemm_fp4_bf16_bwd_qw")
    torch.cuda.synchronize()
    (f, fa), (d, dab), (e, eab) = oracle_step(a, w, g)
    assert_gemm_close(bf16_to_f64(out), f, fa, "fwd_qw")
    assert_gemm_close(bf16_to_f64(da), d, dab, "dA_qw")
    assert_gemm_close(bf16_to_f64(dw), e, eab, "dB_qw")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_cached_weight_against_oracle(M, N, K):
    # the WeightWorkspace path of the Python API, twice (a miss, then a hit), each checked
    # against the oracle's fwd, dA and dB of the bf16 inputs
    a, w, g = inputs(M, N, K)
    ref = oracle_step(a, w, g)
    wsp = mx.WeightWorkspace()
    w_dev = to_device(w).requires_grad_(True)
    for it in range(2):
        say("cached-weight step M=%d N=%d K=%d, call %d" % (M, N, K, it))
        w_fp4 = wsp.get_or_quantize(w_dev, mx.MXFP4Quantizer.for_weight(), cache_name="w")
        at = to_device(a).requires_grad_(True)
        out = mx.gemm_fp4_bf16(at, w_dev, w_fp4=w_fp4)
        out.backward(to_device(g))
        torch.cuda.synchronize()
        for got, (r, rab), what in ((out.detach(), ref[0], "fwd"), (at.grad, ref[1], "dA"),
                                    (w_dev.grad, ref[2], "dB")):
            assert_gemm_close(bf16_to_f64(got), r, rab, "cached %s call %d" % (what, it))
        w_dev.grad = None
    assert wsp.misses == 1 and wsp.hits == 1
