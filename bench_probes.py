"""Build and load the bench's measurement probes (bench_probes.hip) as a library of their own.

Not part of the MXFP4 library: bench.py --ceilings uses them to measure what the chip
sustains on the GEMM's MFMA loop and on 16-byte HBM streams.  The library is compiled
in-tree for gfx950 into _build/libmxfp4_probe.so.
"""
import ctypes
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ROOT, "bench_probes.hip")
LIB = os.path.join(ROOT, "_build", "libmxfp4_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_lib = None

SIGNATURES = [
    ("probe_mfma", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    ("probe_stream", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_void_p]),
]


def build():
    """Always recompiles; returns the library path."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", ROOT, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    os.replace(tmp, LIB)
    return LIB


def lib():
    """The loaded probe library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError("%s is not built; run __graft_entry__.build()" % LIB)
        L = ctypes.CDLL(LIB)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status, where):
    if status != 0:
        raise RuntimeError("%s failed with status %d" % (where, status))
