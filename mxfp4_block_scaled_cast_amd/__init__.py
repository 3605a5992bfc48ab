"""MXFP4 block-scaled cast and GEMM for MI355X (gfx950).

The compute path is the HIP library ``_lib/libmxfp4.so`` (C ABI in
include/mxfp4.h); this package only marshals arguments.  Importing it does not
load the library; the first call does, and fails loudly if it is not built.
"""
from .api import (Mxfp4Tensor, MxOperand, cast, cast_dual, cast_dual_fp8col, cast_dual_pair, cast_fp8, cast_fp8_dual,
                  cast_hadamard, empty_operand, gemm_fp4_bf16, gemm_fp4_bf16_bwd, gemm_fp4_bf16_bwd_qw, gemm_fp4_bf16_fwd,
                  gemm_fp4_bf16_fwd_qw, gemm_fp8_nt, gemm_nn, gemm_nt, gemm_nt_pair, gemm_pair_split, gemm_workspace,
                  gemm_workspace_bytes,
                  rmsnorm_cast, silu_mul_cast, workspace_bytes, workspace_bytes_ex, workspace_bytes_qw)
from .quant import MXFP4Quantizer, WeightWorkspace
from ._native import Mxfp4Error, library_path

__all__ = ["Mxfp4Tensor", "MxOperand", "cast", "cast_dual", "cast_dual_pair", "cast_hadamard", "empty_operand",
           "gemm_fp4_bf16",
           "gemm_fp4_bf16_fwd", "gemm_fp4_bf16_bwd", "gemm_fp4_bf16_fwd_qw", "gemm_fp4_bf16_bwd_qw", "gemm_nn",
           "gemm_nt", "workspace_bytes", "workspace_bytes_qw", "MXFP4Quantizer", "WeightWorkspace", "Mxfp4Error",
           "library_path", "cast_fp8", "cast_fp8_dual", "cast_dual_fp8col", "gemm_fp8_nt", "workspace_bytes_ex",
           "silu_mul_cast", "rmsnorm_cast", "gemm_workspace", "gemm_workspace_bytes", "gemm_nt_pair",
           "gemm_pair_split"]
