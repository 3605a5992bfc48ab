"""GPU parity of the fused producer + cast kernels (README Supported ops: SiLU-and-Mul,
RMSNorm, Fused Add+RMSNorm feeding the MXFP4 cast) against the CPU oracle.

Bit for bit: the produced BF16 values (y_out) against the oracle's producers (exact value
rounded once), the residual sum, and the MXFP4 / MXFP8 copies against the oracle's casts of
the oracle's producer output.  rstd (fp64, summed in another order) to 1e-14 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, operand_rowmajor, operand_padding

pytestmark = pytest.mark.gpu


def check(op, ref, what):
    q_ref, s_ref = ref
    q, s = operand_rowmajor(op)
    assert np.array_equal(s, s_ref), "%s: scales differ at %s" % (what, np.argwhere(s != s_ref)[:5].tolist())
    assert np.array_equal(q, q_ref), "%s: codes differ at %s" % (what, np.argwhere(q != q_ref)[:5].tolist())
    assert np.all(operand_padding(op) == 0), "%s: padding not zero" % what


def bits_of(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def check_copies(t, y_ref, col_fmt, what):
    check(t.row, oracle.cast_rows(y_ref), what + " row")
    if t.col is not None:
        col_ref = oracle.cast_cols_fp8(y_ref) if col_fmt == 8 else oracle.cast_cols(y_ref)
        check(t.col, col_ref, what + " col (MXFP%d)" % col_fmt)


def silu_inputs(R, F, seed):
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal((R, F)) * 3).astype(np.float32)
    # the far tails of the gate (e^-g overflowing binary32 below -88), exact zeros
    g.flat[rng.integers(0, g.size, max(1, g.size // 200))] = rng.uniform(-120, 120, max(1, g.size // 200))
    g.flat[rng.integers(0, g.size, max(1, g.size // 200))] = 0.0
    up = W.ragged_values((R, F), seed + 1, lo=-50, hi=50)
    return np.concatenate([W.bf16_bits(g), up], axis=1)


@pytest.mark.parametrize("col_fmt", [4, 8])
# the last two drawn at random (rows not a multiple of any tile, F a multiple of 32)
@pytest.mark.parametrize("R,F", [(1, 32), (17, 96), (64, 256), (100, 800), (257, 2080), (1024, 14336), (2777, 1376),
                                 (513, 5056)])
def test_silu_mul_cast(R, F, col_fmt):
    x = silu_inputs(R, F, 7 * R + F)
    say("silu_mul_cast R=%d F=%d col_fmt=%d" % (R, F, col_fmt))
    t, y = mx.silu_mul_cast(to_device(x), col_fmt=col_fmt, return_y=True)
    r, _ = mx.silu_mul_cast(to_device(x), columnwise=False)
    torch.cuda.synchronize()
    y_ref = oracle.silu_mul(x)
    yb = bits_of(y)
    bad = np.argwhere(yb != y_ref)
    assert bad.size == 0, "y differs at %s: got %s want %s" % (
        bad[:5].tolist(), [hex(yb[tuple(i)]) for i in bad[:5]], [hex(y_ref[tuple(i)]) for i in bad[:5]])
    check_copies(t, y_ref, col_fmt, "silu_mul")
    check(r.row, oracle.cast_rows(y_ref), "silu_mul row-only")


def test_silu_mul_cast_strided_input():
    R, F = 70, 160
    x = silu_inputs(R, F, 3)
    wide = np.zeros((R, 2 * F + 64), np.uint16)
    wide[:, :2 * F] = x
    say("silu_mul_cast strided")
    t, _ = mx.silu_mul_cast(to_device(wide)[:, :2 * F])
    torch.cuda.synchronize()
    check_copies(t, oracle.silu_mul(x), 4, "silu_mul strided")


def rms_inputs(R, D, seed):
    rng = np.random.default_rng(seed)
    x = W.activations_with_outliers(R, D, seed, seed + 1) if R >= 2 else W.normal_bf16((R, D), 1.0, seed)
    gamma = W.bf16_bits((1 + 0.2 * rng.standard_normal(D)).astype(np.float32))
    return x, gamma


@pytest.mark.parametrize("col_fmt", [4, 8])
@pytest.mark.parametrize("with_residual", [False, True])
@pytest.mark.parametrize("R,D", [(1, 32), (17, 96), (64, 4096), (300, 800), (1000, 4096), (3001, 2912),
                                 (129, 7168)])
def test_rmsnorm_cast(R, D, with_residual, col_fmt):
    x, gamma = rms_inputs(R, D, 11 * R + D)
    res = W.ragged_values((R, D), R + 5 * D, lo=-20, hi=20) if with_residual else None
    eps = float(np.float32(1e-5))
    say("rmsnorm_cast R=%d D=%d residual=%s col_fmt=%d" % (R, D, with_residual, col_fmt))
    t, h, rstd, y = mx.rmsnorm_cast(to_device(x), to_device(gamma[None, :])[0], eps,
                                    residual=to_device(res) if res is not None else None, col_fmt=col_fmt,
                                    return_y=True)
    torch.cuda.synchronize()
    y_ref, h_ref, rstd_ref = oracle.rmsnorm(x, gamma, eps, residual_bits=res)
    if with_residual:
        assert np.array_equal(bits_of(h), h_ref)
    assert np.allclose(rstd.cpu().numpy(), rstd_ref, rtol=1e-14, atol=0)
    yb = bits_of(y)
    bad = np.argwhere(yb != y_ref)
    assert bad.size == 0, "y differs at %s: got %s want %s" % (
        bad[:5].tolist(), [hex(yb[tuple(i)]) for i in bad[:5]], [hex(y_ref[tuple(i)]) for i in bad[:5]])
    check_copies(t, y_ref, col_fmt, "rmsnorm")


def test_rmsnorm_cast_edge_rows():
    # a zero row (y = 0 with eps > 0), constant rows (rstd a power of two), subnormal rows
    D = 128
    x = np.zeros((64, D), np.uint16)
    x[1] = W.bf16_bits(np.float32(2.0 ** -20))
    x[2] = W.bf16_bits(np.float32(-(2.0 ** 30)))
    x[3:35] = W.ragged_values((32, D), 5, lo=-1e-38, hi=1e-38)
    x[35:] = W.normal_bf16((29, D), 1.0, 6)
    gamma = W.bf16_bits(np.linspace(-2, 2, D).astype(np.float32))
    for eps in (float(np.float32(1e-6)), 0.0):   # the entry point takes eps as binary32
        xx = x if eps > 0 else x[1:]
        say("rmsnorm_cast edge rows eps=%g" % eps)
        t, _, rstd, y = mx.rmsnorm_cast(to_device(xx), to_device(gamma[None, :])[0], eps, return_y=True)
        torch.cuda.synchronize()
        y_ref, _, rstd_ref = oracle.rmsnorm(xx, gamma, eps)
        assert np.array_equal(bits_of(y), y_ref)
        assert np.allclose(rstd.cpu().numpy(), rstd_ref, rtol=1e-14, atol=0)
        check_copies(t, y_ref, 4, "rmsnorm edge eps=%g" % eps)


def test_silu_mul_every_gate_value():
    # every finite bf16 gate value (the binary32 fast path depends on the gate alone up to the
    # last multiplication), each against several up values
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    gates = pats[((pats >> 7) & 0xFF) != 0xFF]
    F = 512
    n = -(-gates.size // F) * F
    g = np.resize(gates, n).reshape(-1, F)
    for seed in range(3):
        up = W.bf16_bits(np.random.default_rng(seed).standard_normal(g.shape).astype(np.float32))
        x = np.concatenate([g, up], axis=1)
        say("silu_mul every gate value, seed %d" % seed)
        t, y = mx.silu_mul_cast(to_device(x), return_y=True)
        torch.cuda.synchronize()
        y_ref = oracle.silu_mul(x)
        yb = bits_of(y)
        bad = np.argwhere(yb != y_ref)
        assert bad.size == 0, "y differs at %s: gate %s got %s want %s" % (
            bad[:5].tolist(), [hex(x[tuple(i)]) for i in bad[:5]], [hex(yb[tuple(i)]) for i in bad[:5]],
            [hex(y_ref[tuple(i)]) for i in bad[:5]])
        check_copies(t, y_ref, 4, "silu_mul every gate")


def near_midpoint_pairs(n_gates, seed, max_units=48):
    """(gate, up) bf16 pairs whose exact silu(gate) * up lies within max_units binary32 units of a
    bf16 rounding midpoint -- where a binary32 evaluation is closest to rounding the wrong way."""
    rng = np.random.default_rng(seed)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = pats[((pats >> 7) & 0xFF) != 0xFF]
    fv = fin.view(np.int16).astype(np.int32) << 16
    vals = fv.astype(np.int32).view(np.float32).astype(np.float64)
    gsel = fin[(np.abs(vals) < 80)]
    gates = rng.choice(gsel, n_gates, replace=False)
    gvals = (gates.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out_g, out_u = [], []
    for gb, g in zip(gates, gvals):
        y = g / (1.0 + np.exp(-g)) * vals
        m, e = np.frexp(np.abs(y))                    # |y| = m 2^e, m in [0.5, 1)
        units = np.ldexp(np.abs(y), 24 - e)           # the significand in binary32 units (2^23 .. 2^24)
        frac = np.mod(units, 2 ** 16)                 # position within a bf16 step (2^16 units)
        near = (np.abs(frac - 2 ** 15) <= max_units) & (np.abs(y) > 2.0 ** -120) & (np.abs(y) < 2.0 ** 120)
        k = np.nonzero(near)[0][:64]
        out_g.append(np.full(k.size, gb, np.uint16))
        out_u.append(fin[k])
    return np.concatenate(out_g), np.concatenate(out_u)


def test_silu_mul_near_midpoints():
    g, u = near_midpoint_pairs(600, 21)
    F = 256
    n = g.size // F * F
    assert n >= 4 * F
    x = np.concatenate([g[:n].reshape(-1, F), u[:n].reshape(-1, F)], axis=1)
    say("silu_mul near bf16 midpoints: %d pairs" % n)
    t, y = mx.silu_mul_cast(to_device(x), return_y=True)
    torch.cuda.synchronize()
    y_ref = oracle.silu_mul(x)
    yb = bits_of(y)
    bad = np.argwhere(yb != y_ref)
    assert bad.size == 0, "y differs at %s" % bad[:5].tolist()
    check_copies(t, y_ref, 4, "silu_mul near midpoints")


def test_add_rmsnorm_in_place_residual():
    # residual_out may be the residual buffer itself (the usual in-place residual update)
    R, D = 96, 512
    x, gamma = rms_inputs(R, D, 5)
    res = W.normal_bf16((R, D), 3.0, 6)
    eps = float(np.float32(1e-6))
    y_ref, h_ref, _ = oracle.rmsnorm(x, gamma, eps, residual_bits=res)
    L = mx._native.lib()
    xd, rd, gd = to_device(x), to_device(res), to_device(gamma[None, :])[0]
    row, col = mx.api._produced_copies(R, D, xd.device, True, 4)
    rstd = torch.empty(R, dtype=torch.float64, device=xd.device)
    say("add_rmsnorm in place")
    st = L.mxfp4_rmsnorm_cast(xd.data_ptr(), rd.data_ptr(), gd.data_ptr(), eps, R, D, row.q.data_ptr(),
                              row.s.data_ptr(), col.q.data_ptr(), col.s.data_ptr(), 4, rd.data_ptr(),
                              rstd.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(rd), h_ref)
    check(row, oracle.cast_rows(y_ref), "in-place row")
    check(col, oracle.cast_cols(y_ref), "in-place col")
