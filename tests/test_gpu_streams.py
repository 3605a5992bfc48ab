"""Concurrent use of the library: two host threads, each launching casts and GEMMs (single and paired)
on its own stream with its own buffers, must give the bits a serial run gives.  The library keeps no
shared mutable state between such calls (workspaces and outputs are the caller's)."""
import threading

import pytest
import torch

import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def work(x, w, g):
    """A backward-like sequence on the current stream: dual casts, fwd, then dA and dB paired."""
    X, Wt, G = mx.cast_dual(x), mx.cast_dual(w), mx.cast_dual(g)
    M, N, K = x.shape[0], w.shape[0], x.shape[1]
    ws = mx.gemm_workspace([(M, N, K), (M, K, N), (N, K, X.col.k)], x.device)
    out = mx.gemm_nt(X.row, Wt.row, ws=ws)
    da, dw = mx.gemm_nt_pair(G.row, Wt.col, G.col, X.col, ws=ws)
    return out, da, dw


@pytest.mark.parametrize("shapes", [((2048, 2048, 4096), (300, 640, 1024)), ((17, 4096, 4096), (1000, 2048, 544))],
                         ids=["paired+small", "skinny+panel"])
def test_two_threads_two_streams_match_serial(shapes):
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        inputs.append(tuple(to_device(b) for b in (W.normal_bf16((M, K), 1.0, 200 + i),
                                                   W.normal_bf16((N, K), 0.05, 210 + i),
                                                   W.normal_bf16((M, N), 1.0, 220 + i))))
    say("serial reference %s" % (shapes,))
    want = [work(*inp) for inp in inputs]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                res = None
                for _ in range(10):
                    res = work(*inputs[i])
                s.synchronize()
            got[i] = res
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    say("two threads, two streams")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for a, b, name in zip(got[i], want[i], ("out", "dA", "dB")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "thread %d: %s differs" % (i, name)
