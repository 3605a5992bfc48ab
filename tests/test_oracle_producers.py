"""Pins of the oracle's producers (README "Supported ops": SiLU-and-Mul, RMSNorm, Fused
Add+RMSNorm) and of its single bf16 rounding.

The C oracle evaluates each producer in fp64 and rounds once with ``bf16_round``.  The
checks use what does not share that code: exact rational rounding (``scalar.bf16_round_exact``)
of the same functions written another way (sigmoid through tanh, the norm as a division by
the root mean square), closed forms (large |gate|, constant rows), and invariants (sign
symmetry, power-of-two scaling, the residual sum as the normalized input).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import scalar
from mxfp4_block_scaled_cast_amd import workloads as W


def exact_round(values):
    flat = np.asarray(values, np.float64).reshape(-1)
    out = [scalar.bf16_round_exact(Fraction(float(v)), math.copysign(1.0, v) < 0) for v in flat]
    return np.array(out, np.uint16).reshape(np.shape(values))


def f64(bits):
    return np.array([float(scalar.bf16_value(int(b))) for b in np.asarray(bits).reshape(-1)],
                    np.float64).reshape(np.shape(bits))


# ---- bf16 rounding

def test_bf16_round_random_and_signed_zero():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-44, 39, 3000)
    v = np.concatenate([v, [0.0, -0.0, 1.0, -2.5, 3.3e38, 1e-41, -1e-45]])
    assert np.array_equal(oracle.bf16_round(v), exact_round(v))


def test_bf16_round_ties_go_to_even():
    rng = np.random.default_rng(1)
    m = rng.integers(128, 256, 500)
    e = rng.integers(-126, 128, 500)
    mid = (m + 0.5) * np.ldexp(1.0, e - 7)              # halfway between two adjacent bf16
    got = oracle.bf16_round(mid)
    even = np.where(m % 2 == 0, m, m + 1)              # the neighbour with an even mantissa
    want = exact_round(even * np.ldexp(1.0, e - 7))
    assert np.array_equal(got, want)
    # subnormal midpoints: (k + 1/2) * 2^-133
    k = rng.integers(0, 128, 200)
    got = oracle.bf16_round((k + 0.5) * 2.0 ** -133)
    assert np.array_equal(got, np.where(k % 2 == 0, k, k + 1).astype(np.uint16))


def test_bf16_round_overflow_boundary():
    top = (2 - 2.0 ** -7) * 2.0 ** 127                   # largest finite bf16, 0x7F7F
    half = 2.0 ** 119                                    # half its spacing
    got = oracle.bf16_round(np.array([top, top + half * 0.999, top + half, -(top + half), 2.0 ** 128]))
    assert list(got) == [0x7F7F, 0x7F7F, 0x7F80, 0xFF80, 0x7F80]


# ---- SiLU-and-Mul

def test_silu_mul_matches_tanh_form():
    rng = np.random.default_rng(2)
    R, F = 48, 256
    g = rng.standard_normal((R, F)).astype(np.float32) * 3
    u = rng.standard_normal((R, F)).astype(np.float32)
    x = np.concatenate([W.bf16_bits(g), W.bf16_bits(u)], axis=1)
    y = oracle.silu_mul(x)
    gv, uv = f64(x[:, :F]), f64(x[:, F:])
    # sigmoid(t) = (1 + tanh(t / 2)) / 2: another route to the same real number
    alt = gv * (0.5 * (1.0 + np.tanh(gv / 2))) * uv
    assert np.array_equal(y, exact_round(alt))


def test_silu_mul_closed_forms_and_symmetry():
    rng = np.random.default_rng(3)
    F = 64
    u = W.bf16_bits(rng.standard_normal((4, F)).astype(np.float32))
    big = np.full((4, F), W.bf16_bits(np.float32(128.0)), np.uint16)
    zero = np.zeros((4, F), np.uint16)
    # silu(128) = 128 (1 - e^-128) rounds to exactly 128 * up: the up pattern with exponent + 7
    y = oracle.silu_mul(np.concatenate([big, u], axis=1))
    nz = (u & 0x7FFF) != 0
    assert np.array_equal(y[nz], (u[nz] + (7 << 7)).astype(np.uint16))
    # silu(-128) * up underflows to a zero of sign -sign(up)
    y = oracle.silu_mul(np.concatenate([big | 0x8000, u], axis=1))
    assert np.array_equal(y, ((u ^ 0x8000) & 0x8000).astype(np.uint16))
    # silu(0) = +0: zero with the sign of up
    y = oracle.silu_mul(np.concatenate([zero, u], axis=1))
    assert np.array_equal(y, (u & 0x8000).astype(np.uint16))
    # negating up negates the result bit for bit; the gate half is not interchangeable with up
    g = W.bf16_bits(rng.standard_normal((4, F)).astype(np.float32) * 2)
    a = oracle.silu_mul(np.concatenate([g, u], axis=1))
    b = oracle.silu_mul(np.concatenate([g, u ^ 0x8000], axis=1))
    assert np.array_equal(a ^ 0x8000, b)
    assert not np.array_equal(a, oracle.silu_mul(np.concatenate([u, g], axis=1)))


# ---- RMSNorm and Add+RMSNorm

def test_rmsnorm_constant_rows_give_gamma():
    # rows of +-2^k with eps = 0: mean(h^2) = 4^k, rstd = 2^-k, y = +-gamma exactly
    rng = np.random.default_rng(4)
    D = 96
    gamma = W.bf16_bits(rng.standard_normal(D).astype(np.float32))
    k = rng.integers(-20, 20, 16)
    sign = rng.integers(0, 2, (16, D))
    x = (W.bf16_bits(np.ldexp(1.0, k).astype(np.float32))[:, None] | (sign << 15)).astype(np.uint16)
    y, h, rstd = oracle.rmsnorm(x, gamma, 0.0)
    assert h is None
    assert np.array_equal(rstd, np.ldexp(1.0, -k))
    assert np.array_equal(y, (gamma[None, :] ^ (sign << 15)).astype(np.uint16))


def test_rmsnorm_matches_division_form_and_scales():
    rng = np.random.default_rng(5)
    R, D = 40, 512
    x = W.activations_with_outliers(R, D, 6, 7)
    gamma = W.bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    eps = 1e-5
    y, _, rstd = oracle.rmsnorm(x, gamma, eps)
    xv, gv = f64(x), f64(gamma)
    rms = np.sqrt(np.mean(xv * xv, axis=1) + eps)
    assert np.allclose(rstd, 1 / rms, rtol=1e-14, atol=0)
    assert np.array_equal(y, exact_round(xv / rms[:, None] * gv[None, :]))
    # eps = 0: scaling x by 2^k leaves y unchanged
    y0, _, _ = oracle.rmsnorm(x, gamma, 0.0)
    xs = W.bf16_bits((f64(x) * 2.0 ** -9).astype(np.float32))
    assert np.array_equal(oracle.rmsnorm(xs, gamma, 0.0)[0], y0)


def test_add_rmsnorm_normalizes_the_rounded_sum():
    rng = np.random.default_rng(6)
    R, D = 24, 256
    x = W.normal_bf16((R, D), 1.0, 61)
    r = W.normal_bf16((R, D), 4.0, 62)
    gamma = W.bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    y, h, rstd = oracle.rmsnorm(x, gamma, 1e-6, residual_bits=r)
    # the residual sum is the exact sum rounded once to bf16
    want_h = np.array([[scalar.bf16_round_exact(scalar.bf16_value(int(a)) + scalar.bf16_value(int(b)),
                                                (a & 0x8000) and (b & 0x8000))
                        for a, b in zip(xr, rr)] for xr, rr in zip(x, r)], np.uint16)
    assert np.array_equal(h, want_h)
    # and the norm applies to that rounded sum
    y2, _, rstd2 = oracle.rmsnorm(h, gamma, 1e-6)
    assert np.array_equal(y, y2) and np.array_equal(rstd, rstd2)


@pytest.mark.parametrize("bad", [dict(eps=-1.0), dict(gamma_len=5)])
def test_rmsnorm_rejects(bad):
    x = W.normal_bf16((4, 64), 1.0, 1)
    gamma = np.ones(bad.get("gamma_len", 64), np.uint16)
    with pytest.raises((ValueError, RuntimeError)):
        oracle.rmsnorm(x, gamma, bad.get("eps", 1e-5))
