"""Compile the HIP sources under csrc/ into _lib/libmxfp4.so for gfx950 (in-tree)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libmxfp4.so")
SOURCES = ["cast.hip", "gemm.hip", "gemm_skinny.hip", "api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms stay off (hand-written code never relies on them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    # M0 is written only by the GEMM's own LDS-DMA asm (see gemm.hip)
    "-Wno-inline-asm",
]


def build(verbose=False):
    """Always recompiles; returns the path of the shared library."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errors = [l for l in (r.stdout + r.stderr).splitlines()
              if "warning: unknown" not in l and "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errors) + "\n")
        raise RuntimeError("hipcc failed building %s" % LIB)
    if verbose and errors:
        print("\n".join(errors))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
