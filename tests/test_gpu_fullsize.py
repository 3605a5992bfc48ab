"""Parity at the full per-GPU sizes, launched as bench.py launches them.

For each projection GEMM of the 8B attention, 8B MLP and 70B configs, and for
every (M, N, K) of the ragged sweep, run the whole training step on the GPU
(dual casts of A, W, dOut; fwd; dA; dB) and check, on sampled rows and
columns (the first and last rows / columns of every dimension plus random
ones):
* the row and column copies of each cast, bit for bit against the oracle;
* a block of outputs of each GEMM against the oracle GEMM of the sampled
  operand rows (tolerance 2^-7 |ref| + 1e-5 sum|ab| + 2^-126).
The oracle only ever sees the sampled rows / columns of the bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import layout
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, assert_gemm_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NS = 24  # sampled indices per dimension


def sample(n, rng):
    picks = {0, n - 1, min(n - 1, 31), min(n - 1, 32), n // 2}
    picks |= set(int(v) for v in rng.integers(0, n, NS))
    return np.array(sorted(picks), np.int64)


def dev_rows(op, rows):
    """Codes [len(rows), k/2] and scales [len(rows), k/32] of the given rows of a device MX operand."""
    co = torch.from_numpy(layout.code_offsets(op.rows, op.k)[rows]).to(op.q.device)
    so = torch.from_numpy(layout.scale_offsets(op.rows, op.k)[rows]).to(op.s.device)
    return op.q[co].cpu().numpy(), op.s[so].cpu().numpy()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_step(a_d, w_d, g_d):
    M, K = a_d.shape
    Nn = w_d.shape[0]
    Mp = -(-M // 32) * 32
    A = mx.cast_dual(a_d)
    Wt = mx.cast_dual(w_d)
    out = mx.gemm_nt(A.row, Wt.row)
    G = mx.cast_dual(g_d)
    da = mx.gemm_nn(G.row, Wt.col)
    dw = mx.gemm_nt(G.col, A.col)
    torch.cuda.synchronize()
    assert A.col.k == Mp and G.col.k == Mp
    return A, Wt, G, out, da, dw


def check_step(a_bits_of, w_bits_of, g_bits_of, dims, A, Wt, G, out, da, dw, rng, what):
    """`x_bits_of(rows=None, cols=None)` returns host bf16 bits of the selected rows or columns."""
    M, Nn, K = dims
    mi, ni, ki = sample(M, rng), sample(Nn, rng), sample(K, rng)
    # casts: row copies of sampled rows, column copies of sampled columns
    for name, op, fetch, rows in (("A.row", A.row, lambda r: a_bits_of(rows=r), mi),
                                  ("W.row", Wt.row, lambda r: w_bits_of(rows=r), ni),
                                  ("G.row", G.row, lambda r: g_bits_of(rows=r), mi)):
        q, s = dev_rows(op, rows)
        qr, sr = oracle.cast_rows(fetch(rows))
        assert np.array_equal(s, sr) and np.array_equal(q, qr), "%s %s cast differs" % (what, name)
    for name, op, fetch, cols in (("A.col", A.col, lambda c: a_bits_of(cols=c), ki),
                                  ("W.col", Wt.col, lambda c: w_bits_of(cols=c), ki),
                                  ("G.col", G.col, lambda c: g_bits_of(cols=c), ni)):
        q, s = dev_rows(op, cols)
        qr, sr = oracle.cast_cols(fetch(cols))
        assert np.array_equal(s, sr) and np.array_equal(q, qr), "%s %s cast differs" % (what, name)
    # GEMMs on the sampled rows: fwd out[mi, ni], dA[mi, ki], dB[ni, ki]
    qa, sa = oracle.cast_rows(a_bits_of(rows=mi))
    qw, sw = oracle.cast_rows(w_bits_of(rows=ni))
    ref, ab = oracle.gemm(qa, sa, qw, sw)
    assert_gemm_close(out[mi][:, ni].float().cpu().numpy(), ref, ab, what + " fwd")
    qg, sg = oracle.cast_rows(g_bits_of(rows=mi))
    qwc, swc = oracle.cast_cols(w_bits_of(cols=ki))
    ref, ab = oracle.gemm(qg, sg, qwc, swc)
    assert_gemm_close(da[mi][:, ki].float().cpu().numpy(), ref, ab, what + " dA")
    qgc, sgc = oracle.cast_cols(g_bits_of(cols=ni))
    qac, sac = oracle.cast_cols(a_bits_of(cols=ki))
    ref, ab = oracle.gemm(qgc, sgc, qac, sac)
    assert_gemm_close(dw[ni][:, ki].float().cpu().numpy(), ref, ab, what + " dB")


def host_getter(bits):
    def get(rows=None, cols=None):
        if rows is not None:
            return np.ascontiguousarray(bits[rows])
        return np.ascontiguousarray(bits[:, cols])
    return get


def device_getter(t):
    def get(rows=None, cols=None):
        if rows is not None:
            return host_bits(t[torch.from_numpy(rows).to(t.device)])
        return host_bits(t[:, torch.from_numpy(cols).to(t.device)].contiguous())
    return get


PROJECTIONS = ([("llama8b_attn", i, p) for i, p in enumerate(W.LLAMA8B_ATTN)] +
               [("llama8b_mlp", i, p) for i, p in enumerate(W.LLAMA8B_MLP)] +
               [("llama70b", i, p) for i, p in enumerate(W.LLAMA70B)])


@pytest.mark.parametrize("config,index,proj", PROJECTIONS, ids=["%s-%s" % (c, p[0]) for c, _, p in PROJECTIONS])
def test_projection_step_full_size(config, index, proj):
    name, M, Nn, K = proj
    a, w, g = W.projection_inputs(config, index, M, Nn, K)
    say("full-size step %s %s M=%d N=%d K=%d" % (config, name, M, Nn, K))
    A, Wt, G, out, da, dw = run_step(to_device(a), to_device(w), to_device(g))
    rng = np.random.default_rng(index + 100 * W.CONFIG_IDS[config])
    check_step(host_getter(a), host_getter(w), host_getter(g), (M, Nn, K), A, Wt, G, out, da, dw, rng,
               "%s %s" % (config, name))


COMBOS = list(enumerate(W.ragged_combos()))


@pytest.mark.parametrize("combo,shape", COMBOS, ids=["M%d-N%d-K%d" % s for _, s in COMBOS])
def test_ragged_step_full_size(combo, shape):
    M, Nn, K = shape
    seed = W.seed_of(W.CONFIG_IDS["ragged"], 0, combo)
    say("full-size ragged step M=%d N=%d K=%d" % (M, Nn, K))
    dev = torch.device("cuda:0")
    a = W.ragged_values_torch((M, K), seed + W.A, dev)
    w = W.ragged_values_torch((Nn, K), seed + W.W, dev)
    g = W.ragged_values_torch((M, Nn), seed + W.DOUT, dev)
    A, Wt, G, out, da, dw = run_step(a.view(torch.bfloat16), w.view(torch.bfloat16), g.view(torch.bfloat16))
    rng = np.random.default_rng(combo)
    check_step(device_getter(a), device_getter(w), device_getter(g), (M, Nn, K), A, Wt, G, out, da, dw, rng,
               "ragged %dx%dx%d" % (M, Nn, K))
    del a, w, g, A, Wt, G, out, da, dw
    torch.cuda.empty_cache()
