"""Parity of the step variants at the full 8B MLP per-GPU sizes, launched as bench.py launches
them (--fp8-wgrad, --hadamard-grad, --fused-producers), checked whole like test_gpu_fullsize:

* FP8 wgrad: every byte of the MXFP4 row and MXFP8 column copies of A and dOut against the
  oracle's casts of the whole inputs; complete rows (one per 256-row tile row, plus the
  edges) and complete columns (one per 256-column tile column) of dB from the MXFP8 GEMM
  against the oracle's MXFP8 GEMM (MXFP4 bar plus the FP8 MFMA's in-group truncation
  allowance); and every output of dB against the device reference of the oracle's copies
  (dequantized by the oracle, float64 matmul on the device) with the envelope form of that
  allowance (one matrix product; never below the per-group bound);
* Hadamard gradient recipe: the casts as the bench's --hadamard-grad launches them (A and W:
  column copies block-transformed; dOut: both copies transformed and divided by 32), every byte
  of every copy against the oracle's (transformed) casts of the whole inputs, and every output
  of fwd, dA and dB against the device reference of the oracle's copies;
* fused producers: SiLU-and-mul + cast of the 8192 x 28672 gate/up output and RMSNorm (+
  residual) + cast of the 8192 x 4096 block input -- every produced value, residual sum and
  statistic, and every byte of the row and column copies, against the oracle producers and
  the oracle's casts of their whole output.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, assert_gemm_close, assert_gemm_whole, assert_operand_equal, fp8_truncation_bound
from test_gpu_fullsize import tile_picks

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_copies(T, x_bits, col_fmt, what):
    q, s = oracle.cast_rows(x_bits)
    assert_operand_equal(T.row, q, s, what + " row copy")
    q, s = (oracle.cast_cols_fp8 if col_fmt == 8 else oracle.cast_cols)(x_bits)
    assert_operand_equal(T.col, q, s, what + " column copy")
    return q, s


@pytest.mark.parametrize("index", [0, 1], ids=["gate_up", "down"])
def test_fp8_wgrad_step_full_size(index):
    name, M, Nn, K = W.LLAMA8B_MLP[index]
    a, w, g = W.projection_inputs("llama8b_mlp", index, M, Nn, K)
    say("full-size FP8-wgrad step %s M=%d N=%d K=%d" % (name, M, Nn, K))
    A = mx.cast_dual_fp8col(to_device(a))
    G = mx.cast_dual_fp8col(to_device(g))
    dw = mx.gemm_fp8_nt(G.col, A.col)
    torch.cuda.synchronize()
    qa, sa = check_copies(A, a, 8, "A")
    qg, sg = check_copies(G, g, 8, "dOut")
    rng = np.random.default_rng(300 + index)
    rows, cols = tile_picks(Nn, rng), tile_picks(K, rng)
    ref, ab = oracle.gemm_fp8(qg[rows], sg[rows], qa, sa)
    got = dw[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    extra = fp8_truncation_bound(qg[rows], sg[rows], qa, sa, chunk_rows=4)
    assert_gemm_close(got, ref, ab, "full-size FP8 dB rows " + name, extra)
    ref, ab = oracle.gemm_fp8(qg, sg, qa[cols], sa[cols])
    got = dw[:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    extra = fp8_truncation_bound(qg, sg, qa[cols], sa[cols])
    assert_gemm_close(got, ref, ab, "full-size FP8 dB columns " + name, extra)
    assert_gemm_whole(dw, (qg, sg), (qa, sa), "full-size FP8 dB whole output " + name, fmt=8)


@pytest.mark.parametrize("index", [0, 1], ids=["gate_up", "down"])
def test_hadamard_grad_step_full_size(index):
    name, M, Nn, K = W.LLAMA8B_MLP[index]
    a, w, g = W.projection_inputs("llama8b_mlp", index, M, Nn, K)
    dev = torch.device("cuda:0")
    say("full-size Hadamard-grad step %s M=%d N=%d K=%d" % (name, M, Nn, K))
    A = mx.cast_hadamard(to_device(a), False, True, 0)
    Wt = mx.cast_hadamard(to_device(w), False, True, 0)
    G = mx.cast_hadamard(to_device(g), True, True, 5)
    ws = mx.gemm_workspace([(M, Nn, K), (M, K, Nn), (Nn, K, A.col.k)], dev)
    out = mx.gemm_nt(A.row, Wt.row, ws=ws)
    da, dw = mx.gemm_nt_pair(G.row, Wt.col, G.col, A.col, ws=ws)
    torch.cuda.synchronize()
    copies = {}
    for what, T, x, t_row, shift in (("A", A, a, False, 0), ("W", Wt, w, False, 0), ("dOut", G, g, True, 5)):
        row = oracle.cast_rows_hadamard(x, shift) if t_row else oracle.cast_rows(x)
        assert_operand_equal(T.row, row[0], row[1], "Hadamard %s %s row copy" % (name, what))
        col = oracle.cast_cols_hadamard(x, shift)
        assert_operand_equal(T.col, col[0], col[1], "Hadamard %s %s column copy" % (name, what))
        copies[what] = (row, col)
    del a, w, g
    assert_gemm_whole(out, copies["A"][0], copies["W"][0], "Hadamard %s fwd whole output" % name)
    assert_gemm_whole(da, copies["dOut"][0], copies["W"][1], "Hadamard %s dA whole output" % name)
    assert_gemm_whole(dw, copies["dOut"][1], copies["A"][1], "Hadamard %s dB whole output" % name)


def test_silu_mul_cast_full_size():
    M, F = 8192, 14336
    dev = torch.device("cuda:0")
    # the gate/up output: gates ~N(0, 2), ups ~N(0, 1), generated on the device
    gen = torch.Generator(device=dev).manual_seed(41)
    x = torch.cat([torch.randn(M, F, device=dev, generator=gen) * 2,
                   torch.randn(M, F, device=dev, generator=gen)], dim=1).to(torch.bfloat16)
    say("full-size silu_mul_cast M=%d F=%d" % (M, F))
    t, y = mx.silu_mul_cast(x, return_y=True)
    torch.cuda.synchronize()
    y_ref = oracle.silu_mul(bits(x))
    del x
    got = bits(y)
    if not np.array_equal(got, y_ref):
        raise AssertionError("produced values differ at %d of %d elements" % ((got != y_ref).sum(), got.size))
    check_copies(t, y_ref, 4, "silu_mul")


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
    y_ref, h_ref, r_ref = oracle.rmsnorm(a, gamma, eps, residual_bits=res)
    assert np.array_equal(bits(y), y_ref), "produced values differ"
    assert np.allclose(rstd.cpu().numpy(), r_ref, rtol=1e-14, atol=0)
    if with_residual:
        assert np.array_equal(bits(h), h_ref), "residual sums differ"
    check_copies(t, y_ref, 4, "rmsnorm")
