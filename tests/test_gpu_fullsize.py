"""Parity at the full per-GPU sizes, launched as bench.py launches them.

For each projection GEMM of the 8B attention, 8B MLP and 70B configs, and for
every (M, N, K) of the ragged sweep, run the whole training step on the GPU
(dual casts of A, W, dOut; fwd; dA and dB in one paired call) and check:
* casts, whole: every byte of the row and column copies of A, W and dOut
  (codes, scales and the zero padding of the tiled layout) against the
  oracle's cast of the whole bf16 input;
* GEMMs, every output: for each of fwd, dA and dB, the whole output against
  the exact product of the oracle's copies (dequantized by the oracle, summed
  in float64 by torch.matmul on the device, a library DGEMM independent of
  the kernels under test), tolerance 2^-7 |ref| + 1e-5 sum|ab| + 2^-126;
* GEMMs against the oracle's own GEMM: one complete output row in every
  256-row tile row (a seeded position in it) plus the first and last rows,
  and one complete output column in every 256-column tile column plus the
  first and last columns, same tolerance.  This pins the device reference:
  every 256 x 256 output tile of every launch has outputs checked against
  both.
The oracle casts the whole bf16 inputs; the GEMM references come from those
oracle copies.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, assert_gemm_close, assert_gemm_whole, assert_operand_equal

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TILE = 256


def tile_picks(n, rng):
    """All of 0..n-1 for n <= 64; else 0, n-1 and one seeded index inside every 256-block."""
    if n <= 64:
        return np.arange(n, dtype=np.int64)
    picks = {0, n - 1}
    for t0 in range(0, n, TILE):
        picks.add(int(t0 + rng.integers(0, min(TILE, n - t0))))
    return np.array(sorted(picks), np.int64)


def run_step(a_d, w_d, g_d):
    M, K = a_d.shape
    Nn = w_d.shape[0]
    Mp = -(-M // 32) * 32
    # the products go through the workspace form, as bench.py launches them (split contraction
    # behind small outputs)
    ws = mx.gemm_workspace([(M, Nn, K), (M, K, Nn), (Nn, K, Mp)], a_d.device)
    A = mx.cast_dual(a_d)
    Wt = mx.cast_dual(w_d)
    out = mx.gemm_nt(A.row, Wt.row, ws=ws)
    G = mx.cast_dual(g_d)
    # dA = dOut . W (the NT kernel on W's column copy) and dB in one call, as the step makes them
    da, dw = mx.gemm_nt_pair(G.row, Wt.col, G.col, A.col, ws=ws)
    torch.cuda.synchronize()
    assert A.col.k == Mp and G.col.k == Mp
    return A, Wt, G, out, da, dw


def check_casts(bits, T, name, what):
    """Whole row and column copies of one operand; returns the oracle's (row, col) copies."""
    row = oracle.cast_rows(bits)
    assert_operand_equal(T.row, row[0], row[1], "%s %s.row" % (what, name))
    col = oracle.cast_cols(bits)
    assert_operand_equal(T.col, col[0], col[1], "%s %s.col" % (what, name))
    return row, col


def check_gemm(out, a, b, rng, what):
    """Complete output rows and columns of out = a . b^T (a, b oracle (q, s) copies) against the
    oracle's GEMM, then every output against the device reference of the same copies."""
    qa, sa = a
    qb, sb = b
    rows = tile_picks(qa.shape[0], rng)
    cols = tile_picks(qb.shape[0], rng)
    dev = out.device
    ref, ab = oracle.gemm(qa[rows], sa[rows], qb, sb)
    got = out[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    assert_gemm_close(got, ref, ab, "%s rows %s" % (what, rows[:8].tolist()))
    ref, ab = oracle.gemm(qa, sa, qb[cols], sb[cols])
    got = out[:, torch.from_numpy(cols).to(dev)].float().cpu().numpy()
    assert_gemm_close(got, ref, ab, "%s columns %s" % (what, cols[:8].tolist()))
    assert_gemm_whole(out, a, b, "%s whole output" % what)


def check_step(a_bits, w_bits, g_bits, A, Wt, G, out, da, dw, rng, what):
    (a_row, a_col) = check_casts(a_bits, A, "A", what)
    del a_bits
    (w_row, w_col) = check_casts(w_bits, Wt, "W", what)
    del w_bits
    (g_row, g_col) = check_casts(g_bits, G, "dOut", what)
    del g_bits
    check_gemm(out, a_row, w_row, rng, what + " fwd")
    del a_row, w_row
    check_gemm(da, g_row, w_col, rng, what + " dA")
    del g_row, w_col
    check_gemm(dw, g_col, a_col, rng, what + " dB")


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


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
    check_step(a, w, g, A, Wt, G, out, da, dw, rng, "%s %s" % (config, name))


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
    a_bits, w_bits, g_bits = host_bits(a), host_bits(w), host_bits(g)
    del a, w, g
    rng = np.random.default_rng(combo)
    check_step(a_bits, w_bits, g_bits, A, Wt, G, out, da, dw, rng, "ragged %dx%dx%d" % (M, Nn, K))
    del A, Wt, G, out, da, dw
    torch.cuda.empty_cache()
