"""Build and load the C oracle (``mx_oracle.c``) with gcc.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "libmxoracle.so")
_lib = None


def build(force=True):
    """Compile the C oracle into oracle/_build/libmxoracle.so."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    """The loaded oracle library (built on first use if absent or stale)."""
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.mxo_cast_rows.argtypes = [p, i64, i64, i64, p, p, i32]
        L.mxo_cast_cols.argtypes = [p, i64, i64, i64, p, p, i32]
        L.mxo_dequant.argtypes = [p, p, i64, i64, p]
        L.mxo_gemm.argtypes = [p, p, p, p, i64, i64, i64, p, p, i32]
        L.mxo_gemm_pairs.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p, p, i32]
        L.mxo_cast_rows_hadamard.argtypes = [p, i64, i64, i64, i32, p, p, i32]
        L.mxo_cast_cols_hadamard.argtypes = [p, i64, i64, i64, i32, p, p, i32]
        L.mxo_fwht32.argtypes = [p, p, i64]
        L.mxo_cast_rows_fp8.argtypes = [p, i64, i64, i64, p, p, i32]
        L.mxo_cast_cols_fp8.argtypes = [p, i64, i64, i64, p, p, i32]
        L.mxo_dequant_fp8.argtypes = [p, p, i64, i64, p]
        L.mxo_gemm_fp8.argtypes = [p, p, p, p, i64, i64, i64, p, p, i32]
        L.mxo_bf16_round.argtypes = [p, p, i64]
        L.mxo_silu_mul.argtypes = [p, i64, i64, i64, p, i32]
        L.mxo_rmsnorm.argtypes = [p, p, p, ctypes.c_double, i64, i64, p, p, p, i32]
        for f in (L.mxo_bf16_round, L.mxo_silu_mul, L.mxo_rmsnorm,
                  L.mxo_cast_rows, L.mxo_cast_cols, L.mxo_dequant, L.mxo_gemm, L.mxo_gemm_pairs,
                  L.mxo_cast_rows_hadamard, L.mxo_cast_cols_hadamard, L.mxo_fwht32, L.mxo_cast_rows_fp8,
                  L.mxo_cast_cols_fp8, L.mxo_dequant_fp8, L.mxo_gemm_fp8):
            f.restype = i32
        _lib = L
    return _lib
