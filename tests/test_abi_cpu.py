"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, reports layouts, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from mxfp4_block_scaled_cast_amd import _native as N
from mxfp4_block_scaled_cast_amd import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("mxfp4_cast", "mxfp4_cast_dual", "mxfp4_gemm_nt", "mxfp4_gemm_nn", "gemm_fp4_bf16_fwd",
                 "gemm_fp4_bf16_bwd", "gemm_fp4_bf16_workspace_bytes", "mxfp4_operand_layout_of",
                 "mxfp4_status_string", "gemm_fp4_bf16_workspace_bytes_qw", "gemm_fp4_bf16_fwd_qw",
                 "gemm_fp4_bf16_bwd_qw"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = N.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    bound = {n for n, _, _ in N.SIGNATURES}
    assert bound == set(declared_functions())


def test_library_carries_gfx950_code_for_every_kernel():
    # the shared object must embed a gfx950 code object holding the cast and GEMM kernels
    data = open(N.library_path(), "rb").read()
    assert b"gfx950" in data
    for k in (b"cast_kernel", b"gemm"):
        assert k in data


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = N.status_string(code)
        assert isinstance(s, str) and s
    assert N.status_string(12345) == "unknown status"


@pytest.mark.parametrize("rows,k", [(1, 32), (17, 32), (32, 256), (33, 288), (8192, 4096), (128256, 14336)])
def test_operand_layout(rows, k):
    L = N.operand_layout(rows, k)
    assert L.code_row_tiles == -(-rows // 16) and L.code_k_tiles == -(-k // 128)
    assert L.scale_row_tiles == -(-rows // 128) and L.scale_k_tiles == -(-k // 256)
    assert L.q_bytes == L.code_row_tiles * L.code_k_tiles * 1024 == layout.code_bytes(rows, k)
    assert L.s_bytes == L.scale_row_tiles * L.scale_k_tiles * 1024 == layout.scale_bytes(rows, k)


def test_operand_layout_rejects():
    out = N.OperandLayout()
    assert N.lib().mxfp4_operand_layout_of(4, 33, ctypes.byref(out)) == -1
    assert N.lib().mxfp4_operand_layout_of(-1, 32, ctypes.byref(out)) == -1
    assert N.lib().mxfp4_operand_layout_of(4, 32, None) == -1


FAKE = 1 << 20  # an aligned non-null address; never dereferenced by a rejected call


def test_cast_argument_validation():
    L = N.lib()
    assert L.mxfp4_cast(FAKE, 4, 33, 40, FAKE, FAKE, None) == -1          # cols % 32
    assert L.mxfp4_cast(FAKE, -1, 32, 32, FAKE, FAKE, None) == -1         # negative
    assert L.mxfp4_cast(None, 4, 32, 32, FAKE, FAKE, None) == -1          # null x
    assert L.mxfp4_cast(FAKE, 4, 64, 32, FAKE, FAKE, None) == -1          # ldx < cols
    assert L.mxfp4_cast(FAKE + 2, 4, 32, 32, FAKE, FAKE, None) == -2      # misaligned x
    assert L.mxfp4_cast(FAKE, 4, 32, 36, FAKE, FAKE, None) == -2          # ldx % 8
    assert L.mxfp4_cast(FAKE, 4, 32, 32, FAKE + 8, FAKE, None) == -2      # misaligned q
    assert L.mxfp4_cast(FAKE, 0, 32, 32, None, None, None) == 0           # empty: no-op
    assert L.mxfp4_cast(FAKE, 4, 0, 0, None, None, None) == 0
    assert L.mxfp4_cast(FAKE, 1 << 31, 32, 32, FAKE, FAKE, None) == -5    # range
    assert L.mxfp4_cast_dual(FAKE, 4, 32, 32, FAKE, FAKE, None, FAKE, None) == -1
    assert L.mxfp4_cast_dual(FAKE, 4, 32, 32, FAKE, FAKE, FAKE + 4, FAKE, None) == -2
    pair_ok = [FAKE, 4, 32, 32, FAKE, FAKE, FAKE, FAKE]
    assert L.mxfp4_cast_dual_pair(*pair_ok, FAKE, 4, 33, 40, FAKE, FAKE, FAKE, FAKE, None) == -1  # second: cols % 32
    assert L.mxfp4_cast_dual_pair(FAKE, 4, 32, 32, FAKE, FAKE, None, FAKE, *pair_ok, None) == -1   # first: no q_col
    assert L.mxfp4_cast_dual_pair(*pair_ok, FAKE, 4, 32, 32, FAKE, FAKE, FAKE + 4, FAKE, None) == -2
    assert L.mxfp4_cast_dual_pair(FAKE, 0, 32, 32, None, None, None, None, FAKE, 4, 0, 0, None, None, None, None,
                                  None) == 0                                                          # both empty
    assert L.mxfp4_cast_dual_pair(*pair_ok, *pair_ok, None) == -3                                     # no gfx950 here


def test_gemm_argument_validation():
    L = N.lib()
    for f in (L.mxfp4_gemm_nt, L.mxfp4_gemm_nn):
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 48, FAKE, 4, None) == -1     # K % 32
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 8, 32, FAKE, 4, None) == -1     # ldo < N
        assert f(None, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, None) == -1     # null
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, None, 4, None) == -1
        assert f(FAKE + 4, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, None) == -2
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, FAKE + 1, 4, None) == -2
        assert f(FAKE, FAKE, FAKE, FAKE, 0, 4, 32, None, 4, None) == 0      # empty
        assert f(FAKE, FAKE, FAKE, FAKE, -1, 4, 32, FAKE, 4, None) == -1


def test_step_argument_validation():
    L = N.lib()
    assert L.gemm_fp4_bf16_workspace_bytes(8, 40, 32, 1) == 0               # N % 32 in training
    assert L.gemm_fp4_bf16_workspace_bytes(8, 40, 32, 0) > 0                # fine for inference
    assert L.gemm_fp4_bf16_workspace_bytes(8, 32, 48, 0) == 0
    need = L.gemm_fp4_bf16_workspace_bytes(64, 64, 64, 1)
    assert need > L.gemm_fp4_bf16_workspace_bytes(64, 64, 64, 0)
    assert L.gemm_fp4_bf16_fwd(FAKE, FAKE, 64, 64, 64, FAKE, FAKE, need - 1, 1, None) == -6
    assert L.gemm_fp4_bf16_fwd(FAKE, FAKE, 64, 64, 64, FAKE, FAKE + 16, need, 1, None) == -2
    assert L.gemm_fp4_bf16_fwd(FAKE, FAKE, 64, 64, 48, FAKE, FAKE, need, 1, None) == -1
    assert L.gemm_fp4_bf16_bwd(FAKE, 64, 64, 64, FAKE, need - 1, FAKE, FAKE, None) == -6
    assert L.gemm_fp4_bf16_bwd(FAKE, 64, 64, 64, None, need, FAKE, FAKE, None) == -1


def test_step_with_quantized_weight_argument_validation():
    L = N.lib()
    need = L.gemm_fp4_bf16_workspace_bytes_qw(64, 64, 64, 1)
    assert 0 < need < L.gemm_fp4_bf16_workspace_bytes(64, 64, 64, 1)
    assert L.gemm_fp4_bf16_workspace_bytes_qw(8, 40, 32, 1) == 0            # N % 32 in training
    f = L.gemm_fp4_bf16_fwd_qw
    assert f(FAKE, None, FAKE, 64, 64, 64, FAKE, FAKE, need, 1, None) == -1   # null W codes
    assert f(FAKE, FAKE, None, 64, 64, 64, FAKE, FAKE, need, 1, None) == -1   # null W scales
    assert f(FAKE, FAKE + 4, FAKE, 64, 64, 64, FAKE, FAKE, need, 1, None) == -2
    assert f(FAKE, FAKE, FAKE, 64, 64, 64, FAKE, FAKE, need - 1, 1, None) == -6
    assert f(FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, 0, 1, None) == 0         # empty
    b = L.gemm_fp4_bf16_bwd_qw
    assert b(FAKE, None, FAKE, 64, 64, 64, FAKE, need, FAKE, None, None) == -1  # dA needs W's column copy
    assert b(FAKE, FAKE, FAKE + 8, 64, 64, 64, FAKE, need, FAKE, None, None) == -2
    assert b(FAKE, FAKE, FAKE, 64, 64, 64, FAKE, need - 1, FAKE, FAKE, None) == -6


def test_workspace_size_formula():
    # row copies of A and W, plus (training) column copies of A and W and both copies of dOut
    def op(rows, k):
        return layout.code_bytes(rows, k) + layout.scale_bytes(rows, k)
    M, Nn, K = 17, 96, 64
    Mp = 32
    inf = op(M, K) + op(Nn, K)
    train = inf + op(K, Mp) + op(K, Nn) + op(M, Nn) + op(Nn, Mp)
    assert N.lib().gemm_fp4_bf16_workspace_bytes(M, Nn, K, 0) == inf
    assert N.lib().gemm_fp4_bf16_workspace_bytes(M, Nn, K, 1) == train
    # with a pre-quantized weight the W copies are the caller's
    assert N.lib().gemm_fp4_bf16_workspace_bytes_qw(M, Nn, K, 0) == inf - op(Nn, K)
    assert N.lib().gemm_fp4_bf16_workspace_bytes_qw(M, Nn, K, 1) == train - op(Nn, K) - op(K, Nn)


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device error path; a device is present")
def test_no_device_is_an_error_not_a_fallback():
    L = N.lib()
    assert L.mxfp4_cast(FAKE, 4, 32, 32, FAKE, FAKE, None) == -3
    assert L.mxfp4_gemm_nt(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, None) == -3


def test_layout_offsets_are_a_bijection_into_the_buffer():
    rng = np.random.default_rng(0)
    for rows, k in ((1, 32), (17, 96), (64, 256), (100, 800), (33, 896), (257, 4096)):
        for offs, size in ((layout.code_offsets(rows, k), layout.code_bytes(rows, k)),
                           (layout.scale_offsets(rows, k), layout.scale_bytes(rows, k))):
            off = offs.ravel()
            assert off.min() >= 0 and off.max() < size
            assert np.unique(off).size == off.size
        s = rng.integers(0, 255, (rows, k // 32)).astype(np.uint8)
        assert np.array_equal(layout.scales_to_rowmajor(layout.scales_from_rowmajor(s, rows, k), rows, k), s)
        q = rng.integers(0, 255, (rows, k // 2)).astype(np.uint8)
        assert np.array_equal(layout.codes_to_rowmajor(layout.codes_from_rowmajor(q, rows, k), rows, k), q)


def test_code_tile_is_one_contiguous_kilobyte():
    # a 16-row x 128-element code tile occupies exactly one aligned kilobyte
    off = layout.code_offsets(48, 512)
    for r0 in (0, 16, 32):
        for j0 in (0, 64, 128, 192):
            blk = off[r0:r0 + 16, j0:j0 + 64].ravel()
            assert blk.min() % 1024 == 0 and np.array_equal(np.sort(blk), blk.min() + np.arange(1024))


def test_layout_dword_holds_four_consecutive_k_steps():
    # the dword a 32x32x64 MFMA lane reads (row r, half h) holds blocks h, h+2, h+4, h+6 of a 256-wide K tile,
    # and the four 32-row groups of a 128-row tile are consecutive 256-byte pieces of one kilobyte
    off = layout.scale_offsets(128, 256)
    for r in range(128):
        for h in range(2):
            dword = [off[r, h + 2 * t] for t in range(4)]
            assert dword == [(r // 32) * 256 + (r % 32) * 8 + h * 4 + t for t in range(4)]


@pytest.mark.parametrize("rows,k", [(1, 32), (17, 32), (32, 256), (33, 288), (8192, 4096)])
def test_fp8_operand_layout(rows, k):
    L = N.operand_layout(rows, k, 8)
    assert L.code_row_tiles == -(-rows // 16) and L.code_k_tiles == -(-k // 64)
    assert L.scale_row_tiles == -(-rows // 128) and L.scale_k_tiles == -(-k // 256)
    assert L.q_bytes == L.code_row_tiles * L.code_k_tiles * 1024 == layout.code8_bytes(rows, k)
    assert L.s_bytes == layout.scale_bytes(rows, k)
    out = N.OperandLayout()
    assert N.lib().mxfp8_operand_layout_of(4, 48, ctypes.byref(out)) == -1


def test_fp8_layout_offsets_are_a_bijection_and_tile_kilobytes():
    rng = np.random.default_rng(1)
    for rows, k in ((1, 32), (17, 96), (64, 256), (100, 800), (257, 4096)):
        off = layout.code8_offsets(rows, k).ravel()
        assert off.min() >= 0 and off.max() < layout.code8_bytes(rows, k)
        assert np.unique(off).size == off.size
        q = rng.integers(0, 255, (rows, k)).astype(np.uint8)
        assert np.array_equal(layout.codes8_to_rowmajor(layout.codes8_from_rowmajor(q, rows, k), rows, k), q)
    # a 16-row x 64-element code tile is one aligned kilobyte, rows of 64 consecutive bytes
    off = layout.code8_offsets(32, 256)
    for r0 in (0, 16):
        for k0 in (0, 64, 128, 192):
            blk = off[r0:r0 + 16, k0:k0 + 64]
            assert blk.min() % 1024 == 0 and np.array_equal(blk.ravel(), blk.min() + np.arange(1024))


def test_fp8_argument_validation():
    L = N.lib()
    assert L.mxfp8_cast(FAKE, 4, 33, 40, FAKE, FAKE, None) == -1
    assert L.mxfp8_cast(FAKE + 2, 4, 32, 32, FAKE, FAKE, None) == -2
    assert L.mxfp8_cast(FAKE, 0, 32, 32, None, None, None) == 0
    for f in (L.mxfp8_cast_dual, L.mxfp4_cast_dual_fp8col):
        assert f(FAKE, 4, 32, 32, FAKE, FAKE, None, FAKE, None) == -1
        assert f(FAKE, 4, 32, 32, FAKE, FAKE, FAKE + 4, FAKE, None) == -2
        assert f(FAKE, 4, 48, 48, FAKE, FAKE, FAKE, FAKE, None) == -1
    g = L.mxfp8_gemm_nt
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 48, FAKE, 4, None) == -1
    assert g(FAKE + 4, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, None) == -2
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 4, 32, None, 4, None) == 0


def test_fp8_wgrad_flags_and_workspace():
    L = N.lib()
    T, H, Q, F = N.STEP_TRAINING, N.STEP_HADAMARD_GRAD, N.STEP_QUANTIZED_W, N.STEP_FP8_WGRAD

    def op(rows, k, fmt=4):
        return (layout.code8_bytes(rows, k) if fmt == 8 else layout.code_bytes(rows, k)) + layout.scale_bytes(rows, k)
    M, Nn, K = 17, 96, 64
    Mp = 32
    base = op(M, K) + op(Nn, K) + op(K, Nn) + op(M, Nn)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, T) == base + op(K, Mp) + op(Nn, Mp)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, T | F) == base + op(K, Mp, 8) + op(Nn, Mp, 8)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, T | F | Q) == \
        base + op(K, Mp, 8) + op(Nn, Mp, 8) - op(Nn, K) - op(K, Nn)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, 0) == L.gemm_fp4_bf16_workspace_bytes(M, Nn, K, 0)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, T | H) == L.gemm_fp4_bf16_workspace_bytes(M, Nn, K, 1)
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, T | H | F) == 0      # the transform is MXFP4-only
    assert L.gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, 16) == 0             # unknown flag
    need = L.gemm_fp4_bf16_workspace_bytes_ex(64, 64, 64, T | F)
    fwd, bwd = L.gemm_fp4_bf16_fwd_ex, L.gemm_fp4_bf16_bwd_ex
    assert fwd(FAKE, FAKE, None, None, 64, 64, 64, FAKE, FAKE, need, T | H | F, None) == -1
    assert fwd(FAKE, FAKE, None, None, 64, 64, 64, FAKE, FAKE, need, F, None) == -1   # needs training
    assert fwd(FAKE, FAKE, None, None, 64, 64, 64, FAKE, FAKE, need - 1, T | F, None) == -6
    assert bwd(FAKE, None, None, 64, 64, 64, FAKE, need - 1, FAKE, FAKE, T | F, None) == -6
    assert bwd(FAKE, None, None, 64, 64, 64, FAKE, need, FAKE, FAKE, T | H | F, None) == -1


def test_fused_producer_cast_argument_validation():
    L = N.lib()
    s = L.mxfp4_silu_mul_cast
    assert s(FAKE, 4, 48, 96, FAKE, FAKE, None, None, 4, None, None) == -1        # f % 32
    assert s(FAKE, 4, 32, 48, FAKE, FAKE, None, None, 4, None, None) == -1        # ldx < 2f
    assert s(None, 4, 32, 64, FAKE, FAKE, None, None, 4, None, None) == -1        # null x
    assert s(FAKE, 4, 32, 64, FAKE, FAKE, FAKE, None, 4, None, None) == -1        # half a column copy
    assert s(FAKE, 4, 32, 64, FAKE, FAKE, FAKE, FAKE, 6, None, None) == -1        # column format
    assert s(FAKE + 2, 4, 32, 64, FAKE, FAKE, None, None, 4, None, None) == -2    # misaligned x
    assert s(FAKE, 4, 32, 68, FAKE, FAKE, None, None, 4, None, None) == -2        # ldx % 8
    assert s(FAKE, 4, 32, 64, FAKE, FAKE, None, None, 4, FAKE + 8, None) == -2    # misaligned y_out
    assert s(FAKE, 0, 32, 64, None, None, None, None, 4, None, None) == 0         # empty
    r = L.mxfp4_rmsnorm_cast
    ok = (FAKE, None, FAKE, 1e-5, 4, 64, FAKE, FAKE, None, None, 4, None, FAKE, None, None)

    def call(**kw):
        names = ["x", "res", "gamma", "eps", "rows", "d", "qr", "sr", "qc", "sc", "fmt", "res_out", "rstd", "y", "st"]
        args = dict(zip(names, ok))
        args.update(kw)
        return r(*[args[n] for n in names])
    assert call(d=48) == -1
    assert call(eps=-1.0) == -1
    assert call(eps=float("nan")) == -1
    assert call(gamma=None) == -1
    assert call(rstd=None) == -1
    assert call(res=FAKE) == -1                      # a residual needs residual_out
    assert call(res=FAKE, res_out=FAKE + 4) == -2
    assert call(rstd=FAKE + 4) == -2
    assert call(gamma=FAKE + 2) == -2
    assert call(qc=FAKE, sc=FAKE, fmt=5) == -1
    assert call(rows=0) == 0


def test_bench_probe_argument_validation():
    # the bench's probes are a library of their own (bench_probes.hip), not part of the MXFP4 ABI
    import bench_probes
    if not os.path.exists(bench_probes.LIB):
        bench_probes.build()
    L = bench_probes.lib()
    assert L.probe_mfma(None, 1, 1, FAKE, None) == -1                 # null operands
    assert L.probe_mfma(FAKE, -1, 1, FAKE, None) == -1                # negative iters
    assert L.probe_mfma(FAKE, (1 << 24) + 1, 1, FAKE, None) == -1     # iteration cap
    assert L.probe_mfma(FAKE, 1, 0, FAKE, None) == -1                 # no workgroups
    assert L.probe_mfma(FAKE, 1, 65537, FAKE, None) == -1
    assert L.probe_mfma(FAKE + 8, 1, 1, FAKE, None) == -2             # misaligned operands
    assert L.probe_mfma(FAKE, 1, 1, FAKE + 2, None) == -2             # misaligned out
    assert L.probe_stream(FAKE, 24, None, 0, 1, FAKE, None) == -1     # bytes % 16
    assert L.probe_stream(FAKE, 32, None, 17, 1, FAKE, None) == -1    # writes without dst
    assert L.probe_stream(FAKE, 32, FAKE, 33, 1, FAKE, None) == -1    # writes_per_32 > 32
    assert L.probe_stream(FAKE, 32, FAKE + 4, 17, 1, FAKE, None) == -2
    if _no_gpu():
        # valid arguments: the host has no gfx950, so the call fails on the device check, launching nothing
        assert L.probe_mfma(FAKE, 1, 1, FAKE, None) == -3
        assert L.probe_stream(FAKE, 32, None, 0, 1, FAKE, None) == -3


def test_library_exports_no_measurement_probes():
    assert not any("probe" in n for n in declared_functions())
    L = N.lib()
    for name in ("mxfp4_probe_mfma", "mxfp4_probe_stream", "probe_mfma", "probe_stream"):
        assert not hasattr(L, name), name


@pytest.mark.parametrize("rows,cols", [(1, 32), (17, 96), (8192, 4096), (128256, 14336), (0, 64), (5, 0)])
def test_both_copies_layout(rows, cols):
    L = N.layout(rows, cols)
    rp = -(-rows // 32) * 32
    assert (L.rows, L.cols, L.padded_rows) == (rows, cols, rp)
    assert (L.row.rows, L.row.k) == (rows, cols) and (L.col.rows, L.col.k) == (cols, rp)
    assert L.row.q_bytes == layout.code_bytes(rows, cols) and L.row.s_bytes == layout.scale_bytes(rows, cols)
    assert L.col.q_bytes == layout.code_bytes(cols, rp) and L.col.s_bytes == layout.scale_bytes(cols, rp)


def test_both_copies_layout_rejects():
    out = N.Layout()
    f = N.lib().mxfp4_layout
    assert f(4, 33, ctypes.byref(out)) == -1
    assert f(-1, 32, ctypes.byref(out)) == -1
    assert f(4, 32, None) == -1
    assert f(1 << 31, 32, ctypes.byref(out)) == -5


def test_contraction_limit_of_the_tiled_kernels():
    # lane offsets of the tiled kernels' operand loads are 32-bit: K <= 2^23
    L = N.lib()
    kmax = 1 << 23
    for g in (L.mxfp4_gemm_nt, L.mxfp4_gemm_nn, L.mxfp8_gemm_nt):
        assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, kmax + 32, FAKE, 4, None) == -5
        assert g(FAKE, FAKE, FAKE, FAKE, 0, 4, kmax + 32, None, 4, None) == -5   # checked before the no-op
    if _no_gpu():
        assert L.mxfp4_gemm_nt(FAKE, FAKE, FAKE, FAKE, 4, 4, kmax, FAKE, 4, None) == -3  # in range
    # the step: the forward contracts over K, dA over N, dB over ceil(M/32)*32
    assert L.gemm_fp4_bf16_workspace_bytes(64, 64, kmax + 32, 0) == 0
    assert L.gemm_fp4_bf16_workspace_bytes(64, kmax + 32, 64, 1) == 0
    assert L.gemm_fp4_bf16_workspace_bytes(kmax + 1, 64, 64, 1) == 0
    assert L.gemm_fp4_bf16_workspace_bytes(kmax, 64, 64, 1) > 0
    assert L.gemm_fp4_bf16_workspace_bytes(kmax + 1, 64, 64, 0) > 0          # inference: M is not contracted
    assert L.gemm_fp4_bf16_fwd(FAKE, FAKE, 64, 64, kmax + 32, FAKE, FAKE, 1 << 40, 0, None) == -5
    assert L.gemm_fp4_bf16_bwd(FAKE, kmax + 1, 64, 64, FAKE, 1 << 40, FAKE, FAKE, None) == -5


def test_gemm_scale_pointers_must_be_aligned():
    # the tiled kernels move scale tiles with 16-byte loads
    L = N.lib()
    for g in (L.mxfp4_gemm_nt, L.mxfp8_gemm_nt):
        assert g(FAKE, FAKE + 4, FAKE, FAKE, 4, 4, 32, FAKE, 4, None) == -2
        assert g(FAKE, FAKE, FAKE, FAKE + 8, 4, 4, 32, FAKE, 4, None) == -2


def test_noalloc_forward_rejects_before_any_device_work():
    L = N.lib()
    M, K = 16384, 8192  # A's row copy (71 MB) exceeds the 64 MiB scratch array
    assert L.gemm_fp4_bf16_workspace_bytes_qw(M, 64, K, 0) > N.NOALLOC_SCRATCH_BYTES
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(FAKE, FAKE, FAKE, M, 64, K, FAKE, None) == -5
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(FAKE, FAKE, FAKE, 64, 64, 48, FAKE, None) == -1   # K % 32
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(None, FAKE, FAKE, 0, 64, 64, None, None) == 0    # empty
    if _no_gpu():
        assert L.gemm_fp4_bf16_fwd_qw_noalloc(FAKE, FAKE, FAKE, 64, 64, 64, FAKE, None) == -3


def test_split_workspace_query_and_validation():
    L = N.lib()
    # long contractions behind small outputs split; tiled products and short contractions do not
    assert L.mxfp4_gemm_workspace_bytes(1, 32, 128256) > 0
    assert L.mxfp4_gemm_workspace_bytes(4096, 32, 128256) > 0
    assert L.mxfp4_gemm_workspace_bytes(8192, 28672, 4096) == 0
    assert L.mxfp4_gemm_workspace_bytes(17, 4096, 4096) == 0
    assert L.mxfp4_gemm_workspace_bytes(4, 4, 48) == 0                      # K % 32: invalid
    assert L.mxfp4_gemm_workspace_bytes(4, 4, (1 << 23) + 32) == 0          # past the contraction limit
    f = L.mxfp4_gemm_nt_ws
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 48, FAKE, 4, FAKE, 64, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, FAKE + 4, 64, None) == -2   # misaligned workspace
    assert f(FAKE, FAKE + 4, FAKE, FAKE, 4, 4, 32, FAKE, 4, None, 0, None) == -2   # misaligned scales
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 4, 32, None, 4, None, 0, None) == 0        # empty
    if _no_gpu():
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4, None, 0, None) == -3


def test_panel_split_workspace_sizes():
    # 128 x 128 panel blocks split over the contraction only for 2^20 outputs or more over a contraction
    # of 8192 or more, up to one workgroup per CU of 256; the partials are S copies of the 64 x 64 partial
    # blocks (16 KB of fp32 each)
    L = N.lib()
    blk = 64 * 64 * 4
    assert L.mxfp4_gemm_workspace_bytes(16384, 128, 14336) == 2 * (256 * 2) * blk   # 128 blocks, 2 splits
    assert L.mxfp4_gemm_workspace_bytes(128, 14336, 16384) == 2 * (2 * 224) * blk   # 112 blocks, 2 splits
    assert L.mxfp4_gemm_workspace_bytes(1024, 1024, 14336) == 4 * (16 * 16) * blk   # 64 blocks, 4 splits
    assert L.mxfp4_gemm_workspace_bytes(130, 8150, 8320) == 2 * (3 * 128) * blk     # ragged: 64-row blocks
    # unsplit panel launches (a side of 512 or more, blocks for half the CUs) and shapes that stay on
    # the skinny kernel without a split (its own split needs fewer blocks than CUs)
    assert L.mxfp4_gemm_workspace_bytes(2048, 2048, 4096) == 0
    assert L.mxfp4_gemm_workspace_bytes(1000, 2000, 1024) == 0
    assert L.mxfp4_gemm_workspace_bytes(16384, 128, 4096) == 0


def test_step_workspace_holds_the_split_partials():
    # the step's workspace adds one region for the largest split of its three products
    def op(rows, k):
        return layout.code_bytes(rows, k) + layout.scale_bytes(rows, k)

    def r256(x):
        return -(-x // 256) * 256
    L = N.lib()
    M, Nn, K = 17, 128256, 32          # dA contracts over 128256 behind 17 x 32 outputs
    Mp = 32
    copies = [op(M, K), op(Nn, K), op(K, Mp), op(K, Nn), op(M, Nn), op(Nn, Mp)]
    split = max(L.mxfp4_gemm_workspace_bytes(M, Nn, K), L.mxfp4_gemm_workspace_bytes(M, K, Nn),
                L.mxfp4_gemm_workspace_bytes(Nn, K, Mp))
    assert split == L.mxfp4_gemm_workspace_bytes(M, K, Nn) > 0
    assert L.gemm_fp4_bf16_workspace_bytes(M, Nn, K, 1) == sum(r256(c) for c in copies) + r256(split)


def test_pair_split_query():
    # the training backward's dA [M, K] over N and dB [N, K] over M of the projection configs: one
    # paired launch (4 XCDs each) where a partial last round of two launches goes away (8B QKV, O,
    # MLP down), two launches where both already run in whole rounds (8B gate/up, 70B); uneven and
    # ragged pairs take other splits; a product too small for the tiled kernels, differing trip
    # structures, N % 8 != 0 and invalid sizes: two launches (0)
    L = N.lib()
    f = L.mxfp4_gemm_pair_split
    for M, Nn, K in [(8192, 6144, 4096), (8192, 4096, 4096), (8192, 4096, 14336)]:
        assert f(M, K, Nn, Nn, K, M) == 4, (M, Nn, K)
    for M, Nn, K in [(8192, 28672, 4096), (8192, 10240, 8192), (8192, 57344, 8192), (8192, 8192, 28672)]:
        assert f(M, K, Nn, Nn, K, M) == 0, (M, Nn, K)
    assert f(2100, 4000, 1056, 4000, 2056, 2080) == 3
    assert f(2048, 4000, 640, 2100, 6144, 640) == 2
    assert f(8192, 8192, 640, 2048, 4000, 640) == 7
    # a partial round alone runs faster on its idle CUs' power: kept as two launches
    assert f(4096, 14336, 128256, 128256, 14336, 4096) == 0
    assert f(4096, 4096, 1024, 2048, 4096, 8192) == 0
    assert f(17, 4096, 4096, 4096, 4096, 1024) == 0
    assert f(2048, 4096, 512, 4096, 2048, 1024) == 0
    assert f(2048, 4092, 1024, 2048, 4096, 1024) == 0
    assert f(2048, 4096, 48, 2048, 4096, 1024) == 0
    assert f(-1, 4096, 1024, 2048, 4096, 1024) == 0


def test_pair_gemm_argument_validation():
    # each product validated as mxfp4_gemm_nt_ws, product 0 first, before anything is enqueued
    L = N.lib()
    f = L.mxfp4_gemm_nt_pair_ws
    good = (FAKE, FAKE, FAKE, FAKE, 4, 4, 32, FAKE, 4)
    assert f(*good[:6], 48, *good[7:], *good, None, 0, None) == -1                 # K0 % 32
    assert f(*good, *good[:6], 48, *good[7:], None, 0, None) == -1                 # K1 % 32
    assert f(*good, *good[:5], 8, 32, FAKE, 4, None, 0, None) == -1                # ldo1 < N1
    assert f(*good, FAKE, FAKE + 4, FAKE, FAKE, 4, 4, 32, FAKE, 4, None, 0, None) == -2   # misaligned scales
    assert f(*good[:7], FAKE + 1, 4, *good, None, 0, None) == -2                     # odd output address
    assert f(*good, *good, FAKE + 4, 64, None) == -2                                # misaligned workspace
    assert f(*good[:4], 0, 4, 32, None, 4, *good[:4], 4, 0, 32, None, 4, None, 0, None) == 0   # both empty
    if _no_gpu():
        assert f(*good, *good, None, 0, None) == -3


def test_counter_summary_hash_follows_code_not_comments(tmp_path):
    # the committed HBM counter figure is reported only while the GEMM sources' code is the code it
    # was measured on: comments and blank lines do not count, a changed statement does
    import sys
    sys.path.insert(0, ROOT)
    import bench_rocprof as rs
    src = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    p = tmp_path / "k.hip"
    p.write_text(src)
    h0 = rs.source_hash([str(p)])
    p.write_text("/* a kernel */\n" + src.replace("// one more", "// one more than x") + "\n\n")
    assert rs.source_hash([str(p)]) == h0
    p.write_text(src.replace("x + 1", "x + 2"))
    assert rs.source_hash([str(p)]) != h0
