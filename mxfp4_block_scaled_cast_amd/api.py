"""PyTorch-facing API over the C ABI (libmxfp4.so).

PyTorch provides device memory and the current stream; every step of the
cast and GEMM runs in the HIP kernels behind include/mxfp4.h.  Names follow
jax-aiter's MXFP4 path (README, "Supported ops" and "Quick start"):
``cast`` / ``cast_dual`` (CastMxfp4JA / CastMxfp4DualJA), ``gemm_nt`` (the
low-level gemm_fp4 on pre-quantized operands), ``gemm_nn`` (the dA form),
and the differentiable ``gemm_fp4_bf16``.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _native as N


@dataclass
class MxOperand:
    """One quantized copy in the tiled MX layout: E2M1 codes q and E8M0 scales s (flat uint8 buffers)."""
    q: torch.Tensor
    s: torch.Tensor
    rows: int
    k: int


@dataclass
class Mxfp4Tensor:
    """Row copy (blocks along the last dim) and optional column copy of a bf16 [R, C] matrix."""
    row: MxOperand
    col: Optional[MxOperand]
    shape: Tuple[int, int]


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check_bf16_matrix(x, name):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("%s must be a 2-D bfloat16 tensor" % name)
    if not x.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if x.stride(1) != 1:
        raise ValueError("%s must have a unit stride along its last dimension" % name)


def empty_operand(rows, k, device):
    L = N.operand_layout(rows, k)
    q = torch.empty((L.q_bytes,), dtype=torch.uint8, device=device)
    s = torch.empty((L.s_bytes,), dtype=torch.uint8, device=device)
    return MxOperand(q, s, rows, k)


def cast(x, out: Optional[MxOperand] = None) -> MxOperand:
    """Row copy of bf16 x [R, C] (C % 32 == 0)."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    op = out if out is not None else empty_operand(R, C, x.device)
    st = N.lib().mxfp4_cast(x.data_ptr(), R, C, x.stride(0), op.q.data_ptr(), op.s.data_ptr(), _stream(x.device))
    N.check(st, "mxfp4_cast")
    return op


def cast_dual(x, row: Optional[MxOperand] = None, col: Optional[MxOperand] = None) -> Mxfp4Tensor:
    """Row and column copies of bf16 x [R, C] from one read of x."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    Rp = -(-R // 32) * 32
    row = row if row is not None else empty_operand(R, C, x.device)
    col = col if col is not None else empty_operand(C, Rp, x.device)
    st = N.lib().mxfp4_cast_dual(x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(),
                                 col.q.data_ptr(), col.s.data_ptr(), _stream(x.device))
    N.check(st, "mxfp4_cast_dual")
    return Mxfp4Tensor(row, col, (R, C))


def _gemm(fn, name, a: MxOperand, b: MxOperand, out):
    if a.k != b.k:
        raise ValueError("contraction lengths differ: %d vs %d" % (a.k, b.k))
    M, Nn, K = a.rows, b.rows, a.k
    if out is None:
        out = torch.empty((M, Nn), dtype=torch.bfloat16, device=a.q.device)
    elif out.dtype != torch.bfloat16 or out.shape != (M, Nn) or out.stride(1) != 1:
        raise ValueError("out must be a bfloat16 [%d, %d] tensor with unit column stride" % (M, Nn))
    st = fn(a.q.data_ptr(), a.s.data_ptr(), b.q.data_ptr(), b.s.data_ptr(), M, Nn, K, out.data_ptr(),
            out.stride(0), _stream(out.device))
    N.check(st, name)
    return out


def gemm_nt(a: MxOperand, b: MxOperand, out=None):
    """out[M, N] = dq(a)[M, K] . dq(b)[N, K]^T in bf16."""
    return _gemm(N.lib().mxfp4_gemm_nt, "mxfp4_gemm_nt", a, b, out)


def gemm_nn(a: MxOperand, bcol: MxOperand, out=None):
    """out[M, N] = dq(a)[M, K] . B[K, N], B given by its column copy (N rows, contraction K)."""
    return _gemm(N.lib().mxfp4_gemm_nn, "mxfp4_gemm_nn", a, bcol, out)


def workspace_bytes(M, Nn, K, training=True):
    return int(N.lib().gemm_fp4_bf16_workspace_bytes(M, Nn, K, 1 if training else 0))


def gemm_fp4_bf16_fwd(a, w, training=True, ws=None, out=None):
    """Forward of gemm_fp4_bf16 on 2-D contiguous bf16 a [M, K], w [N, K] -> (out [M, N], ws)."""
    _check_bf16_matrix(a, "a")
    _check_bf16_matrix(w, "w")
    if not (a.is_contiguous() and w.is_contiguous()):
        raise ValueError("a and w must be contiguous")
    M, K = a.shape
    Nn = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("a and w disagree on K")
    nbytes = workspace_bytes(M, Nn, K, training)
    if ws is None:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=a.device)
    if out is None:
        out = torch.empty((M, Nn), dtype=torch.bfloat16, device=a.device)
    st = N.lib().gemm_fp4_bf16_fwd(a.data_ptr(), w.data_ptr(), M, Nn, K, out.data_ptr(), ws.data_ptr(),
                                   ws.numel(), 1 if training else 0, _stream(a.device))
    N.check(st, "gemm_fp4_bf16_fwd")
    return out, ws


def gemm_fp4_bf16_bwd(dout, M, Nn, K, ws, need_da=True, need_dw=True, da=None, dw=None):
    """Backward of gemm_fp4_bf16 from the workspace of a training forward -> (da, dw)."""
    _check_bf16_matrix(dout, "dout")
    if not dout.is_contiguous():
        dout = dout.contiguous()
    if need_da and da is None:
        da = torch.empty((M, K), dtype=torch.bfloat16, device=dout.device)
    if need_dw and dw is None:
        dw = torch.empty((Nn, K), dtype=torch.bfloat16, device=dout.device)
    st = N.lib().gemm_fp4_bf16_bwd(dout.data_ptr(), M, Nn, K, ws.data_ptr(), ws.numel(),
                                   da.data_ptr() if need_da else None, dw.data_ptr() if need_dw else None,
                                   _stream(dout.device))
    N.check(st, "gemm_fp4_bf16_bwd")
    return (da if need_da else None), (dw if need_dw else None)


def workspace_bytes_qw(M, Nn, K, training=True):
    return int(N.lib().gemm_fp4_bf16_workspace_bytes_qw(M, Nn, K, 1 if training else 0))


def _check_weight_fp4(w_fp4, Nn, K, training):
    if w_fp4.shape != (Nn, K):
        raise ValueError("w_fp4 holds a [%d, %d] weight, expected [%d, %d]" % (w_fp4.shape + (Nn, K)))
    if training and w_fp4.col is None:
        raise ValueError("training needs the weight's column copy: quantize with columnwise=True")


def gemm_fp4_bf16_fwd_qw(a, w_fp4, training=True, ws=None, out=None):
    """Forward with a pre-quantized weight (Mxfp4Tensor of W [N, K]) -> (out [M, N], ws)."""
    _check_bf16_matrix(a, "a")
    if not a.is_contiguous():
        raise ValueError("a must be contiguous")
    M, K = a.shape
    Nn = w_fp4.shape[0]
    _check_weight_fp4(w_fp4, Nn, K, training)
    nbytes = workspace_bytes_qw(M, Nn, K, training)
    if ws is None:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=a.device)
    if out is None:
        out = torch.empty((M, Nn), dtype=torch.bfloat16, device=a.device)
    r = w_fp4.row
    st = N.lib().gemm_fp4_bf16_fwd_qw(a.data_ptr(), r.q.data_ptr(), r.s.data_ptr(), M, Nn, K, out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), 1 if training else 0, _stream(a.device))
    N.check(st, "gemm_fp4_bf16_fwd_qw")
    return out, ws


def gemm_fp4_bf16_bwd_qw(dout, w_fp4, M, Nn, K, ws, need_da=True, need_dw=True, da=None, dw=None):
    """Backward of gemm_fp4_bf16_fwd_qw (W's column copy from w_fp4) -> (da, dw)."""
    _check_bf16_matrix(dout, "dout")
    if not dout.is_contiguous():
        dout = dout.contiguous()
    if need_da and da is None:
        da = torch.empty((M, K), dtype=torch.bfloat16, device=dout.device)
    if need_dw and dw is None:
        dw = torch.empty((Nn, K), dtype=torch.bfloat16, device=dout.device)
    c = w_fp4.col
    st = N.lib().gemm_fp4_bf16_bwd_qw(dout.data_ptr(), c.q.data_ptr() if c is not None else None,
                                      c.s.data_ptr() if c is not None else None, M, Nn, K, ws.data_ptr(), ws.numel(),
                                      da.data_ptr() if need_da else None, dw.data_ptr() if need_dw else None,
                                      _stream(dout.device))
    N.check(st, "gemm_fp4_bf16_bwd_qw")
    return (da if need_da else None), (dw if need_dw else None)


class _GemmFp4Bf16(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, w, w_fp4):
        training = bool(ctx.needs_input_grad[0] or ctx.needs_input_grad[1])
        if w_fp4 is None:
            out, ws = gemm_fp4_bf16_fwd(a, w, training=training)
        else:
            out, ws = gemm_fp4_bf16_fwd_qw(a, w_fp4, training=training)
        ctx.dims = (a.shape[0], w.shape[0], a.shape[1])
        ctx.ws = ws if training else None
        ctx.w_fp4 = w_fp4
        return out

    @staticmethod
    def backward(ctx, dout):
        M, Nn, K = ctx.dims
        if ctx.w_fp4 is None:
            da, dw = gemm_fp4_bf16_bwd(dout, M, Nn, K, ctx.ws, ctx.needs_input_grad[0], ctx.needs_input_grad[1])
        else:
            da, dw = gemm_fp4_bf16_bwd_qw(dout, ctx.w_fp4, M, Nn, K, ctx.ws, ctx.needs_input_grad[0],
                                          ctx.needs_input_grad[1])
        ctx.ws = None
        ctx.w_fp4 = None
        return da, dw, None


def gemm_fp4_bf16(a, w, w_fp4: Optional[Mxfp4Tensor] = None):
    """BF16 in/out MXFP4 GEMM, out = a . w^T, differentiable (FP4 forward, FP4 dA, FP4 dB).

    a: [..., K] bfloat16, w: [N, K] bfloat16 -> [..., N] bfloat16.
    w_fp4: w already quantized (e.g. from WeightWorkspace.get_or_quantize with a weight
    quantizer); its copies replace w's cast in the forward and in dA.  w still receives dW.
    """
    lead = a.shape[:-1]
    a2 = a.reshape(-1, a.shape[-1]).contiguous()
    out = _GemmFp4Bf16.apply(a2, w.contiguous(), w_fp4)
    return out.reshape(*lead, w.shape[0])
