"""CPU oracle for the MXFP4 block-scaled cast and GEMM.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

What is computed follows the jax-aiter README ("Supported ops" table: the MXFP4
cast turns BF16 into E2M1 elements plus E8M0 block scales, optionally with a
transposed copy; the low-level FP4 GEMM consumes fp4x2 operands with e8m0
block scales) together with the OCP Microscaling conversion rule that fills
in what the page leaves open (block of 32, shared exponent floor(log2 amax)-2,
round-to-nearest-even, saturation).

Two implementations live here:

* ``oracle.scalar`` -- pure Python on exact rationals, one block at a time,
  for hand-sized cases and brute force.
* the C library ``mx_oracle.c`` wrapped below with numpy, for full-size data.

Canonical layouts (all row-major, no padding except where stated):

* row copy of x [R, C]:   q [R, C/2] uint8 (element 2j in the low nibble of
  byte j, 2j+1 in the high nibble), s [R, C/32] uint8 (E8M0 = X + 127)
* column copy of x [R, C]: q [C, Rp/2], s [C, Rp/32], Rp = ceil(R/32)*32; the
  rows past R are +0
* GEMM: ref[m, n] = sum_k dq(a)[m, k] * dq(b)[n, k] in fp64, and
  absref[m, n] = sum_k |dq(a)[m, k] * dq(b)[n, k]|

MXFP8 (E4M3 elements, E8M0 block scales; the FP8 dB variant): ``cast_rows_fp8``
/ ``cast_cols_fp8`` with X = floor(log2 amax) - 8 and nearest-even E4M3
saturating at 448, one code per byte; ``gemm_fp8`` forms exact integer block
sums.

Hadamard-transformed casts (README "Quick start": grad_out is cast with a
Hadamard transform): ``cast_rows_hadamard`` / ``cast_cols_hadamard`` apply
the 32-point Sylvester Walsh-Hadamard matrix to every block in binary32
(butterflies of half-width 1, 2, 4, 8, 16, each (u, w) -> (u + w, u - w)),
divide by 2^shift and quantize by the same rule.  Used on both operands of a
contraction, with shift 5 on one of them (H H = 32 I).

Producers whose BF16 output feeds the cast (README "Supported ops": SiLU-and-Mul
is silu(x[:half]) * x[half:], RMSNorm fuses square, mean, rsqrt and scale, Fused
Add+RMSNorm normalizes x + residual): ``silu_mul``, ``rmsnorm`` -- evaluated in
fp64 from the bf16 inputs and rounded once to bf16 (``bf16_round``); with a
residual the sum is rounded to bf16 first (it is the stored residual) and the
norm applies to that.  A fused producer + cast quantizes exactly these outputs.
"""
import os

import numpy as np

from . import native
from . import scalar  # noqa: F401  (re-exported for tests)


def _threads(nthreads):
    if nthreads is None:
        return len(os.sched_getaffinity(0))
    return int(nthreads)


def _bits(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns as uint16")
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    return x


def cast_rows(x_bits, nthreads=None):
    """Row copy: blocks of 32 along the contiguous dim.  Returns (q, s)."""
    x = _bits(x_bits)
    R, C = x.shape
    if C % 32:
        raise ValueError("the number of columns must be a multiple of 32")
    q = np.empty((R, C // 2), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    rc = native.lib().mxo_cast_rows(x.ctypes.data, R, C, C, q.ctypes.data, s.ctypes.data, _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_cast_rows failed")
    return q, s


def cast_cols(x_bits, nthreads=None):
    """Column copy: blocks of 32 rows in each column, rows padded with +0.  Returns (q, s)."""
    x = _bits(x_bits)
    R, C = x.shape
    Rp = -(-R // 32) * 32
    q = np.empty((C, Rp // 2), np.uint8)
    s = np.empty((C, Rp // 32), np.uint8)
    rc = native.lib().mxo_cast_cols(x.ctypes.data, R, C, C, q.ctypes.data, s.ctypes.data, _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_cast_cols failed")
    return q, s


def cast_rows_hadamard(x_bits, shift=0, nthreads=None):
    """Row copy with each 32-block Walsh-Hadamard transformed (binary32 butterflies) and
    divided by 2^shift before quantization.  Returns (q, s) shaped as cast_rows."""
    x = _bits(x_bits)
    R, C = x.shape
    if C % 32:
        raise ValueError("the number of columns must be a multiple of 32")
    q = np.empty((R, C // 2), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    rc = native.lib().mxo_cast_rows_hadamard(x.ctypes.data, R, C, C, int(shift), q.ctypes.data, s.ctypes.data,
                                             _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_cast_rows_hadamard failed")
    return q, s


def cast_cols_hadamard(x_bits, shift=0, nthreads=None):
    """Column copy (blocks of 32 rows, padded with +0) with the block transform.  Returns (q, s)."""
    x = _bits(x_bits)
    R, C = x.shape
    Rp = -(-R // 32) * 32
    q = np.empty((C, Rp // 2), np.uint8)
    s = np.empty((C, Rp // 32), np.uint8)
    rc = native.lib().mxo_cast_cols_hadamard(x.ctypes.data, R, C, C, int(shift), q.ctypes.data, s.ctypes.data,
                                             _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_cast_cols_hadamard failed")
    return q, s


def fwht32(x_f32):
    """The binary32 32-point Walsh-Hadamard transform of each row of a [n, 32] float32 array."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != 32:
        raise ValueError("expected [n, 32] float32")
    out = np.empty_like(x)
    if native.lib().mxo_fwht32(x.ctypes.data, out.ctypes.data, x.shape[0]):
        raise RuntimeError("mxo_fwht32 failed")
    return out


def cast_rows_fp8(x_bits, nthreads=None):
    """MXFP8 (E4M3, E8M0 block scales) row copy: q [R, C] codes, s [R, C/32]."""
    x = _bits(x_bits)
    R, C = x.shape
    if C % 32:
        raise ValueError("the number of columns must be a multiple of 32")
    q = np.empty((R, C), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    if native.lib().mxo_cast_rows_fp8(x.ctypes.data, R, C, C, q.ctypes.data, s.ctypes.data, _threads(nthreads)):
        raise RuntimeError("mxo_cast_rows_fp8 failed")
    return q, s


def cast_cols_fp8(x_bits, nthreads=None):
    """MXFP8 column copy (blocks of 32 rows, padded with +0): q [C, Rp], s [C, Rp/32]."""
    x = _bits(x_bits)
    R, C = x.shape
    Rp = -(-R // 32) * 32
    q = np.empty((C, Rp), np.uint8)
    s = np.empty((C, Rp // 32), np.uint8)
    if native.lib().mxo_cast_cols_fp8(x.ctypes.data, R, C, C, q.ctypes.data, s.ctypes.data, _threads(nthreads)):
        raise RuntimeError("mxo_cast_cols_fp8 failed")
    return q, s


def dequant_fp8(q, s):
    """Dequantized values (fp64) of an MXFP8 (q [R, K], s [R, K/32]) pair."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    R, K = q.shape
    if s.shape != (R, K // 32):
        raise ValueError("scale shape does not match the codes")
    out = np.empty((R, K), np.float64)
    if native.lib().mxo_dequant_fp8(q.ctypes.data, s.ctypes.data, R, K, out.ctypes.data):
        raise RuntimeError("mxo_dequant_fp8 failed")
    return out


def gemm_fp8(qa, sa, qb, sb, nthreads=None):
    """ref / absref [M, N] for out = A . B^T on MXFP8 operands."""
    qa, sa, qb, sb = (np.ascontiguousarray(t, np.uint8) for t in (qa, sa, qb, sb))
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1]
    if qb.shape[1] != K or sa.shape != (M, K // 32) or sb.shape != (N, K // 32):
        raise ValueError("operand shapes do not agree")
    ref = np.empty((M, N), np.float64)
    absref = np.empty((M, N), np.float64)
    if native.lib().mxo_gemm_fp8(qa.ctypes.data, sa.ctypes.data, qb.ctypes.data, sb.ctypes.data, M, N, K,
                                 ref.ctypes.data, absref.ctypes.data, _threads(nthreads)):
        raise RuntimeError("mxo_gemm_fp8 failed")
    return ref, absref


def dequant(q, s):
    """Dequantized values (fp64) of a canonical (q, s) pair."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    R, K = q.shape[0], q.shape[1] * 2
    if s.shape != (R, K // 32):
        raise ValueError("scale shape does not match the codes")
    out = np.empty((R, K), np.float64)
    if native.lib().mxo_dequant(q.ctypes.data, s.ctypes.data, R, K, out.ctypes.data):
        raise RuntimeError("mxo_dequant failed")
    return out


def _gemm_args(qa, sa, qb, sb):
    qa, sa, qb, sb = (np.ascontiguousarray(t, np.uint8) for t in (qa, sa, qb, sb))
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    if qb.shape[1] * 2 != K or sa.shape != (M, K // 32) or sb.shape != (N, K // 32):
        raise ValueError("operand shapes do not agree")
    return qa, sa, qb, sb, M, N, K


def gemm(qa, sa, qb, sb, nthreads=None):
    """Full ref/absref [M, N] for out = A . B^T on canonical operands."""
    qa, sa, qb, sb, M, N, K = _gemm_args(qa, sa, qb, sb)
    ref = np.empty((M, N), np.float64)
    absref = np.empty((M, N), np.float64)
    rc = native.lib().mxo_gemm(qa.ctypes.data, sa.ctypes.data, qb.ctypes.data, sb.ctypes.data, M, N, K,
                               ref.ctypes.data, absref.ctypes.data, _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_gemm failed")
    return ref, absref


def gemm_pairs(qa, sa, qb, sb, mi, ni, nthreads=None):
    """ref/absref at the sampled outputs (mi[i], ni[i])."""
    qa, sa, qb, sb, M, N, K = _gemm_args(qa, sa, qb, sb)
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    if mi.shape != ni.shape or mi.ndim != 1:
        raise ValueError("mi and ni must be 1-D and of equal length")
    ref = np.empty(mi.shape, np.float64)
    absref = np.empty(mi.shape, np.float64)
    rc = native.lib().mxo_gemm_pairs(qa.ctypes.data, sa.ctypes.data, qb.ctypes.data, sb.ctypes.data, M, N, K,
                                     mi.ctypes.data, ni.ctypes.data, mi.size, ref.ctypes.data, absref.ctypes.data,
                                     _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_gemm_pairs failed")
    return ref, absref


# ---- producers feeding the cast (README "Supported ops": SiLU-and-Mul, RMSNorm,
# Fused Add+RMSNorm); each returns BF16 bit patterns, evaluated in fp64 and rounded once

def bf16_round(values):
    """Nearest-even bf16 bit patterns (uint16) of float64 values, rounded once."""
    v = np.ascontiguousarray(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    if native.lib().mxo_bf16_round(v.ctypes.data, out.ctypes.data, v.size):
        raise RuntimeError("mxo_bf16_round failed")
    return out


def silu_mul(x_bits, nthreads=None):
    """y [R, F] = bf16(silu(gate) * up) for x [R, 2F] = [gate | up]."""
    x = _bits(x_bits)
    R, C = x.shape
    if C % 2:
        raise ValueError("x must have an even number of columns")
    y = np.empty((R, C // 2), np.uint16)
    if native.lib().mxo_silu_mul(x.ctypes.data, R, C // 2, C, y.ctypes.data, _threads(nthreads)):
        raise RuntimeError("mxo_silu_mul failed")
    return y


def rmsnorm(x_bits, gamma_bits, eps, residual_bits=None, nthreads=None):
    """RMSNorm of x [R, D] (of h = bf16(x + residual) with a residual):
    (y = bf16(h * rstd * gamma) [R, D], h [R, D] or None, rstd [R] float64)."""
    x = _bits(x_bits)
    R, D = x.shape
    g = np.ascontiguousarray(gamma_bits, np.uint16).reshape(-1)
    if g.size != D:
        raise ValueError("gamma must have D entries")
    res = None
    if residual_bits is not None:
        res = _bits(residual_bits)
        if res.shape != x.shape:
            raise ValueError("residual must match x")
    y = np.empty((R, D), np.uint16)
    h = np.empty((R, D), np.uint16) if res is not None else None
    rstd = np.empty(R, np.float64)
    rc = native.lib().mxo_rmsnorm(x.ctypes.data, res.ctypes.data if res is not None else None, g.ctypes.data,
                                  float(eps), R, D, y.ctypes.data, h.ctypes.data if h is not None else None,
                                  rstd.ctypes.data, _threads(nthreads))
    if rc:
        raise RuntimeError("mxo_rmsnorm failed")
    return y, h, rstd
