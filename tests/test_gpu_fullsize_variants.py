"""Parity of the step variants at the full 8B MLP per-GPU sizes, launched as bench.py launches
them (--fp8-wgrad, --fused-producers), on sampled rows and columns like test_gpu_fullsize:

* FP8 wgrad: the MXFP4 row + MXFP8 column casts of A and dOut (sampled rows / columns bit for
  bit against the oracle) and a block of dB from the MXFP8 GEMM against the oracle's MXFP8 GEMM
  of the sampled columns (MXFP4 bar plus the FP8 MFMA's in-group truncation allowance);
* fused producers: SiLU-and-mul + cast of the 8192 x 28672 gate/up output and RMSNorm (+
  residual) + cast of the 8192 x 4096 block input -- produced values of sampled rows, row copies
  of sampled rows and column copies of sampled columns bit for bit against the oracle producers
  and casts of the same rows / columns.
The oracle only ever sees sampled rows / columns of the bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import layout
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, assert_gemm_close, fp8_truncation_bound

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NS = 24


def sample(n, rng):
    picks = {0, n - 1, min(n - 1, 31), min(n - 1, 32), n // 2}
    picks |= set(int(v) for v in rng.integers(0, n, NS))
    return np.array(sorted(picks), np.int64)


def dev_rows(op, rows):
    """Codes and scales of the given rows of a device operand, in the oracle's row-major form."""
    offs = (layout.code8_offsets if op.fmt == 8 else layout.code_offsets)(op.rows, op.k)[rows]
    co = torch.from_numpy(offs).to(op.q.device)
    so = torch.from_numpy(layout.scale_offsets(op.rows, op.k)[rows]).to(op.s.device)
    return op.q[co].cpu().numpy(), op.s[so].cpu().numpy()


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def same(op, rows, ref, what):
    q, s = dev_rows(op, rows)
    assert np.array_equal(s, ref[1]), what + ": scales differ"
    assert np.array_equal(q, ref[0]), what + ": codes differ"


@pytest.mark.parametrize("index", [0, 1], ids=["gate_up", "down"])
def test_fp8_wgrad_step_full_size(index):
    name, M, Nn, K = W.LLAMA8B_MLP[index]
    a, w, g = W.projection_inputs("llama8b_mlp", index, M, Nn, K)
    say("full-size FP8-wgrad step %s M=%d N=%d K=%d" % (name, M, Nn, K))
    A = mx.cast_dual_fp8col(to_device(a))
    G = mx.cast_dual_fp8col(to_device(g))
    dw = mx.gemm_fp8_nt(G.col, A.col)
    torch.cuda.synchronize()
    rng = np.random.default_rng(300 + index)
    mi, ni, ki = sample(M, rng), sample(Nn, rng), sample(K, rng)
    same(A.row, mi, oracle.cast_rows(np.ascontiguousarray(a[mi])), "A row copy")
    same(G.row, mi, oracle.cast_rows(np.ascontiguousarray(g[mi])), "dOut row copy")
    qa, sa = oracle.cast_cols_fp8(np.ascontiguousarray(a[:, ki]))
    qg, sg = oracle.cast_cols_fp8(np.ascontiguousarray(g[:, ni]))
    same(A.col, ki, (qa, sa), "A MXFP8 column copy")
    same(G.col, ni, (qg, sg), "dOut MXFP8 column copy")
    ref, ab = oracle.gemm_fp8(qg, sg, qa, sa)
    got = dw[torch.from_numpy(ni).cuda()][:, torch.from_numpy(ki).cuda()].float().cpu().numpy()
    assert_gemm_close(got, ref, ab, "full-size FP8 dB " + name, fp8_truncation_bound(qg, sg, qa, sa))


def test_silu_mul_cast_full_size():
    M, F = 8192, 14336
    rng = np.random.default_rng(41)
    dev = torch.device("cuda:0")
    # the gate/up output: gates ~N(0, 2), ups ~N(0, 1), generated on the device
    gen = torch.Generator(device=dev).manual_seed(41)
    x = torch.cat([torch.randn(M, F, device=dev, generator=gen) * 2,
                   torch.randn(M, F, device=dev, generator=gen)], dim=1).to(torch.bfloat16)
    say("full-size silu_mul_cast M=%d F=%d" % (M, F))
    t, y = mx.silu_mul_cast(x, return_y=True)
    torch.cuda.synchronize()
    mi, fi = sample(M, rng), sample(F, rng)
    rows_x = bits(x[torch.from_numpy(mi).cuda()])
    y_rows = oracle.silu_mul(rows_x)
    assert np.array_equal(bits(y[torch.from_numpy(mi).cuda()]), y_rows), "produced values differ"
    same(t.row, mi, oracle.cast_rows(y_rows), "row copy")
    cols = np.concatenate([fi, fi + F])
    y_cols = oracle.silu_mul(bits(x[:, torch.from_numpy(cols).cuda()].contiguous()))
    same(t.col, fi, oracle.cast_cols(y_cols), "column copy")


@pytest.mark.parametrize("with_residual", [False, True])
def test_rmsnorm_cast_full_size(with_residual):
    M, D = 8192, 4096
    a, _, _ = W.projection_inputs("llama8b_mlp", 0, M, 128, D, with_grad=False)
    rng = np.random.default_rng(51)
    gamma = W.bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    res = W.normal_bf16((M, D), 2.0, 52) if with_residual else None
    eps = float(np.float32(1e-5))
    say("full-size rmsnorm_cast M=%d D=%d residual=%s" % (M, D, with_residual))
    t, h, rstd, y = mx.rmsnorm_cast(to_device(a), to_device(gamma[None, :])[0], eps,
                                    residual=to_device(res) if res is not None else None, return_y=True)
    torch.cuda.synchronize()
    mi, di = sample(M, rng), sample(D, rng)
    y_rows, h_rows, r_rows = oracle.rmsnorm(np.ascontiguousarray(a[mi]), gamma, eps,
                                            residual_bits=np.ascontiguousarray(res[mi]) if with_residual else None)
    assert np.array_equal(bits(y[torch.from_numpy(mi).cuda()]), y_rows), "produced values differ"
    assert np.allclose(rstd.cpu().numpy()[mi], r_rows, rtol=1e-14, atol=0)
    if with_residual:
        assert np.array_equal(bits(h[torch.from_numpy(mi).cuda()]), h_rows), "residual sums differ"
    same(t.row, mi, oracle.cast_rows(y_rows), "row copy")
    # a column of y needs every row's rstd: the oracle recomputes all rows, then keeps the sampled columns
    y_all, _, _ = oracle.rmsnorm(a, gamma, eps, residual_bits=res)
    same(t.col, di, oracle.cast_cols(np.ascontiguousarray(y_all[:, di])), "column copy")
