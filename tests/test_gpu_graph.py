"""The training step under HIP graph capture, and the autograd wrapper on batched inputs.

The library allocates, frees, synchronizes and memsets nothing, so a captured forward +
backward (caller-owned workspace and outputs) must replay bit-identically to eager calls;
every replay is checked, with eager work and synchronizations in between.  The autograd
wrapper flattens leading dimensions: a [B, T, K] input gives the same bits as the [B*T, K]
call.
"""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import _native as N
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def step_calls(a, w, g, out, ws, da, dw, flags):
    L = N.lib()
    M, K = a.shape
    Nn = w.shape[0]

    def run():
        s = torch.cuda.current_stream().cuda_stream
        N.check(L.gemm_fp4_bf16_fwd_ex(a.data_ptr(), w.data_ptr(), None, None, M, Nn, K, out.data_ptr(),
                                       ws.data_ptr(), ws.numel(), flags, s), "fwd_ex")
        N.check(L.gemm_fp4_bf16_bwd_ex(g.data_ptr(), None, None, M, Nn, K, ws.data_ptr(), ws.numel(),
                                       da.data_ptr(), dw.data_ptr(), flags, s), "bwd_ex")
    return run


@pytest.mark.parametrize("flags", [N.STEP_TRAINING, N.STEP_TRAINING | N.STEP_HADAMARD_GRAD,
                                   N.STEP_TRAINING | N.STEP_FP8_WGRAD], ids=["plain", "hadamard", "fp8wgrad"])
# (17, 32768, 256): dA is 17 x 256 outputs over a contraction of 32768, split across workgroups
# (partials in the workspace, then the reduction kernel) inside the captured graph;
# (128, 8192, 8192): fwd and dA are 128 x 8192 outputs over 8192 on the panel kernel, split likewise;
# (2048, 2048, 4096): dA and dB in one paired persistent launch
@pytest.mark.parametrize("M,Nn,K", [(256, 512, 1024), (17, 4096, 4096), (2048, 4096, 1024), (17, 32768, 256),
                                    (128, 8192, 8192), (2048, 2048, 4096)])
def test_captured_step_replays_like_eager(M, Nn, K, flags):
    a = to_device(W.normal_bf16((M, K), 1.0, 1))
    w = to_device(W.normal_bf16((Nn, K), 0.05, 2))
    g = to_device(W.normal_bf16((M, Nn), 1.0, 3))
    ws = torch.empty(mx.workspace_bytes_ex(M, Nn, K, flags), dtype=torch.uint8, device="cuda:0")
    if (M, Nn, K) == (17, 32768, 256):
        assert mx.gemm_workspace_bytes(M, K, Nn) > 0, "dA should split its contraction"
    if (M, Nn, K) == (128, 8192, 8192):
        assert mx.gemm_workspace_bytes(M, Nn, K) > 0 and mx.gemm_workspace_bytes(M, K, Nn) > 0, \
            "fwd and dA should split their contraction"
    if (M, Nn, K) == (2048, 2048, 4096):
        assert mx.gemm_pair_split(M, K, Nn, Nn, K, M) > 0, "dA and dB should share one launch"
    out = torch.empty((M, Nn), dtype=torch.bfloat16, device="cuda:0")
    da = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    dw = torch.empty((Nn, K), dtype=torch.bfloat16, device="cuda:0")
    run = step_calls(a, w, g, out, ws, da, dw, flags)
    say("graph capture step M=%d N=%d K=%d flags=%d" % (M, Nn, K, flags))
    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (out, da, dw)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run()  # warm up on the side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for t in (out, da, dw):
            t.fill_(float("nan"))
        ws.fill_(0xA5)  # the replay must not depend on what the workspace held
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref, name in zip((out, da, dw), want, ("out", "dA", "dB")):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "replay %d: %s differs" % (rep, name)
        (a.float() @ a.float().t()).sum().item()  # unrelated eager work between replays


def test_batched_input_matches_flat():
    B, T, K, Nn = 3, 40, 512, 256
    a = to_device(W.normal_bf16((B * T, K), 1.0, 7))
    w = to_device(W.normal_bf16((Nn, K), 0.05, 8))
    g = to_device(W.normal_bf16((B * T, Nn), 1.0, 9))
    say("gemm_fp4_bf16 batched input")
    res = []
    for shape in ((B * T, K), (B, T, K)):
        at = a.clone().reshape(shape).requires_grad_(True)
        wt = w.clone().requires_grad_(True)
        out = mx.gemm_fp4_bf16(at, wt)
        assert out.shape == shape[:-1] + (Nn,)
        out.backward(g.reshape(out.shape))
        torch.cuda.synchronize()
        res.append((out.reshape(B * T, Nn), at.grad.reshape(B * T, K), wt.grad))
    for x, y in zip(*res):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
