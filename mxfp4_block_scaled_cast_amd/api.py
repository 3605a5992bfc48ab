"""PyTorch-facing API over the C ABI (libmxfp4.so).

PyTorch provides device memory and the current stream; every step of the
cast and GEMM runs in the HIP kernels behind include/mxfp4.h.  Names follow
jax-aiter's MXFP4 path (README, "Supported ops" and "Quick start"):
``cast`` / ``cast_dual`` (CastMxfp4JA / CastMxfp4DualJA), ``gemm_nt`` (the
low-level gemm_fp4 on pre-quantized operands), ``gemm_nn`` (the dA form),
and the differentiable ``gemm_fp4_bf16``.  The MXFP8 functions
(``cast_fp8``, ``cast_fp8_dual``, ``cast_dual_fp8col``, ``gemm_fp8_nt``)
and the ``fp8_wgrad`` step option serve the FP8 dB that the README's
"MXFP4 training architecture" section describes.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _native as N


@dataclass
class MxOperand:
    """One quantized copy in the tiled MX layout: element codes q and E8M0 scales s (flat
    uint8 buffers); fmt 4 = MXFP4 (E2M1, two per byte), 8 = MXFP8 (E4M3, one per byte)."""
    q: torch.Tensor
    s: torch.Tensor
    rows: int
    k: int
    fmt: int = 4


@dataclass
class Mxfp4Tensor:
    """Row copy (blocks along the last dim) and optional column copy of a bf16 [R, C] matrix.
    hadamard_row / hadamard_col mark copies quantized after the block Walsh-Hadamard transform."""
    row: MxOperand
    col: Optional[MxOperand]
    shape: Tuple[int, int]
    hadamard_row: bool = False
    hadamard_col: bool = False


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check_bf16_matrix(x, name):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("%s must be a 2-D bfloat16 tensor" % name)
    if not x.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if x.stride(1) != 1:
        raise ValueError("%s must have a unit stride along its last dimension" % name)


def empty_operand(rows, k, device, fmt=4):
    L = N.operand_layout(rows, k, fmt)
    q = torch.empty((L.q_bytes,), dtype=torch.uint8, device=device)
    s = torch.empty((L.s_bytes,), dtype=torch.uint8, device=device)
    return MxOperand(q, s, rows, k, fmt)


def _check_out_operand(op, rows, k, fmt, name):
    if op.rows != rows or op.k != k or op.fmt != fmt:
        raise ValueError("%s must be an MXFP%d operand of %d rows, k=%d" % (name, fmt, rows, k))


def cast(x, out: Optional[MxOperand] = None) -> MxOperand:
    """Row copy of bf16 x [R, C] (C % 32 == 0)."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    if out is not None:
        _check_out_operand(out, R, C, 4, "out")
    op = out if out is not None else empty_operand(R, C, x.device)
    st = N.lib().mxfp4_cast(x.data_ptr(), R, C, x.stride(0), op.q.data_ptr(), op.s.data_ptr(), _stream(x.device))
    N.check(st, "mxfp4_cast")
    return op


def cast_dual(x, row: Optional[MxOperand] = None, col: Optional[MxOperand] = None) -> Mxfp4Tensor:
    """Row and column copies of bf16 x [R, C] from one read of x."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    Rp = -(-R // 32) * 32
    if row is not None:
        _check_out_operand(row, R, C, 4, "row")
    if col is not None:
        _check_out_operand(col, C, Rp, 4, "col")
    row = row if row is not None else empty_operand(R, C, x.device)
    col = col if col is not None else empty_operand(C, Rp, x.device)
    st = N.lib().mxfp4_cast_dual(x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(),
                                 col.q.data_ptr(), col.s.data_ptr(), _stream(x.device))
    N.check(st, "mxfp4_cast_dual")
    return Mxfp4Tensor(row, col, (R, C))


def cast_dual_pair(x0, x1):
    """Row and column copies of two bf16 matrices in one launch (as the training forward casts its
    A and W); the same results as cast_dual(x0), cast_dual(x1)."""
    outs, args = [], []
    for i, x in enumerate((x0, x1)):
        _check_bf16_matrix(x, "x%d" % i)
        if x.device != x0.device:
            raise ValueError("x0 and x1 must be on the same device")
        R, C = x.shape
        row, col = empty_operand(R, C, x.device), empty_operand(C, -(-R // 32) * 32, x.device)
        outs.append(Mxfp4Tensor(row, col, (R, C)))
        args += [x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(), col.q.data_ptr(),
                 col.s.data_ptr()]
    N.check(N.lib().mxfp4_cast_dual_pair(*args, _stream(x0.device)), "mxfp4_cast_dual_pair")
    return outs[0], outs[1]


def cast_hadamard(x, transform_row=True, transform_col=True, shift=0, columnwise=True) -> Mxfp4Tensor:
    """Row (and, if columnwise, column) copy of bf16 x [R, C] with each 32-block of the chosen
    copies Walsh-Hadamard transformed and divided by 2^shift before quantization (the gradient
    recipe of the README's Quick start; see mxfp4_cast_hadamard)."""
    _check_bf16_matrix(x, "x")
    if transform_col and not columnwise:
        raise ValueError("transform_col needs the column copy")
    R, C = x.shape
    Rp = -(-R // 32) * 32
    row = empty_operand(R, C, x.device)
    col = empty_operand(C, Rp, x.device) if columnwise else None
    st = N.lib().mxfp4_cast_hadamard(x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(),
                                     col.q.data_ptr() if col is not None else None,
                                     col.s.data_ptr() if col is not None else None,
                                     1 if transform_row else 0, 1 if transform_col else 0, int(shift),
                                     _stream(x.device))
    N.check(st, "mxfp4_cast_hadamard")
    return Mxfp4Tensor(row, col, (R, C), bool(transform_row), bool(transform_col and columnwise))


def cast_fp8(x) -> MxOperand:
    """MXFP8 (E4M3) row copy of bf16 x [R, C] (C % 32 == 0)."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    op = empty_operand(R, C, x.device, 8)
    st = N.lib().mxfp8_cast(x.data_ptr(), R, C, x.stride(0), op.q.data_ptr(), op.s.data_ptr(), _stream(x.device))
    N.check(st, "mxfp8_cast")
    return op


def _cast_dual_formats(x, row_fmt, fn, name) -> Mxfp4Tensor:
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    Rp = -(-R // 32) * 32
    row = empty_operand(R, C, x.device, row_fmt)
    col = empty_operand(C, Rp, x.device, 8)
    st = fn(x.data_ptr(), R, C, x.stride(0), row.q.data_ptr(), row.s.data_ptr(), col.q.data_ptr(), col.s.data_ptr(),
            _stream(x.device))
    N.check(st, name)
    return Mxfp4Tensor(row, col, (R, C))


def cast_fp8_dual(x) -> Mxfp4Tensor:
    """MXFP8 row and column copies of bf16 x [R, C] from one read of x."""
    return _cast_dual_formats(x, 8, N.lib().mxfp8_cast_dual, "mxfp8_cast_dual")


def cast_dual_fp8col(x) -> Mxfp4Tensor:
    """MXFP4 row copy and MXFP8 column copy of bf16 x [R, C] from one read of x."""
    return _cast_dual_formats(x, 4, N.lib().mxfp4_cast_dual_fp8col, "mxfp4_cast_dual_fp8col")


def _produced_copies(R, K, device, columnwise, col_fmt):
    if col_fmt not in (4, 8):
        raise ValueError("col_fmt must be 4 (MXFP4) or 8 (MXFP8)")
    Rp = -(-R // 32) * 32
    row = empty_operand(R, K, device)
    col = empty_operand(K, Rp, device, col_fmt) if columnwise else None
    return row, col


def silu_mul_cast(x, columnwise=True, col_fmt=4, return_y=False):
    """Fused SiLU-and-mul + cast (README Supported ops: silu(x[:half]) * x[half:]).

    x: bf16 [R, 2F] = [gate | up] with unit column stride.  Returns the Mxfp4Tensor of
    y = bf16(silu(gate) * up) [R, F] (row copy, and with columnwise the column copy in
    col_fmt 4 = MXFP4 or 8 = MXFP8), and y itself when return_y (else None)."""
    _check_bf16_matrix(x, "x")
    R, C = x.shape
    if C % 64:
        raise ValueError("x must have 2F columns with F a multiple of 32")
    F = C // 2
    row, col = _produced_copies(R, F, x.device, columnwise, col_fmt)
    y = torch.empty((R, F), dtype=torch.bfloat16, device=x.device) if return_y else None
    st = N.lib().mxfp4_silu_mul_cast(x.data_ptr(), R, F, x.stride(0), row.q.data_ptr(), row.s.data_ptr(),
                                     col.q.data_ptr() if col is not None else None,
                                     col.s.data_ptr() if col is not None else None, col_fmt,
                                     y.data_ptr() if y is not None else None, _stream(x.device))
    N.check(st, "mxfp4_silu_mul_cast")
    return Mxfp4Tensor(row, col, (R, F)), y


def rmsnorm_cast(x, gamma, eps=1e-5, residual=None, columnwise=True, col_fmt=4, return_y=False):
    """Fused RMSNorm (or Add+RMSNorm with a residual) + cast (README Supported ops).

    x (and residual): bf16 [R, D] contiguous; gamma: bf16 [D].  h = x, or bf16(x + residual);
    y = bf16(h * rstd * gamma) with rstd = 1 / sqrt(mean(h^2) + eps).  Returns
    (Mxfp4Tensor of y, h when a residual is given else None, rstd float64 [R], y or None)."""
    _check_bf16_matrix(x, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    R, D = x.shape
    if gamma.dtype != torch.bfloat16 or gamma.numel() != D or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bfloat16 tensor of %d elements" % D)
    h = None
    if residual is not None:
        _check_bf16_matrix(residual, "residual")
        if residual.shape != x.shape or not residual.is_contiguous():
            raise ValueError("residual must be contiguous and shaped like x")
        h = torch.empty_like(x)
    row, col = _produced_copies(R, D, x.device, columnwise, col_fmt)
    rstd = torch.empty((R,), dtype=torch.float64, device=x.device)
    y = torch.empty((R, D), dtype=torch.bfloat16, device=x.device) if return_y else None
    st = N.lib().mxfp4_rmsnorm_cast(x.data_ptr(), residual.data_ptr() if residual is not None else None,
                                    gamma.data_ptr(), float(eps), R, D, row.q.data_ptr(), row.s.data_ptr(),
                                    col.q.data_ptr() if col is not None else None,
                                    col.s.data_ptr() if col is not None else None, col_fmt,
                                    h.data_ptr() if h is not None else None, rstd.data_ptr(),
                                    y.data_ptr() if y is not None else None, _stream(x.device))
    N.check(st, "mxfp4_rmsnorm_cast")
    return Mxfp4Tensor(row, col, (R, D)), h, rstd, y


def _gemm(fn, name, a: MxOperand, b: MxOperand, out, ws=None):
    if a.k != b.k:
        raise ValueError("contraction lengths differ: %d vs %d" % (a.k, b.k))
    M, Nn, K = a.rows, b.rows, a.k
    if out is None:
        out = torch.empty((M, Nn), dtype=torch.bfloat16, device=a.q.device)
    elif out.dtype != torch.bfloat16 or out.shape != (M, Nn) or out.stride(1) != 1:
        raise ValueError("out must be a bfloat16 [%d, %d] tensor with unit column stride" % (M, Nn))
    args = (a.q.data_ptr(), a.s.data_ptr(), b.q.data_ptr(), b.s.data_ptr(), M, Nn, K, out.data_ptr(), out.stride(0))
    if ws is not None:
        if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != out.device:
            raise ValueError("ws must be a contiguous uint8 tensor on the output's device")
        st = N.lib().mxfp4_gemm_nt_ws(*args, ws.data_ptr(), ws.numel(), _stream(out.device))
        name = "mxfp4_gemm_nt_ws"
    else:
        st = fn(*args, _stream(out.device))
    N.check(st, name)
    return out


def _out_for(a: MxOperand, b: MxOperand, out):
    if a.k != b.k:
        raise ValueError("contraction lengths differ: %d vs %d" % (a.k, b.k))
    M, Nn = a.rows, b.rows
    if out is None:
        return torch.empty((M, Nn), dtype=torch.bfloat16, device=a.q.device)
    if out.dtype != torch.bfloat16 or out.shape != (M, Nn) or out.stride(1) != 1:
        raise ValueError("out must be a bfloat16 [%d, %d] tensor with unit column stride" % (M, Nn))
    return out


def gemm_nt_pair(a0: MxOperand, b0: MxOperand, a1: MxOperand, b1: MxOperand, out0=None, out1=None, ws=None):
    """(out0, out1) = (dq(a0) . dq(b0)^T, dq(a1) . dq(b1)^T), two independent MXFP4 products in one
    call (mxfp4_gemm_nt_pair_ws): one persistent launch with the chip's XCDs divided between them
    where the cost model favours it (the training backward's dA and dB), else two launches in order
    sharing ws.  Each output is bit-identical to gemm_nt with the same ws."""
    for a, b in ((a0, b0), (a1, b1)):
        _check_formats(a, b, 4)
    out0, out1 = _out_for(a0, b0, out0), _out_for(a1, b1, out1)
    if out0.device != out1.device:
        raise ValueError("both outputs must be on one device")
    wp, wn = 0, 0
    if ws is not None:
        if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != out0.device:
            raise ValueError("ws must be a contiguous uint8 tensor on the outputs' device")
        wp, wn = ws.data_ptr(), ws.numel()
    st = N.lib().mxfp4_gemm_nt_pair_ws(
        a0.q.data_ptr(), a0.s.data_ptr(), b0.q.data_ptr(), b0.s.data_ptr(), a0.rows, b0.rows, a0.k, out0.data_ptr(),
        out0.stride(0), a1.q.data_ptr(), a1.s.data_ptr(), b1.q.data_ptr(), b1.s.data_ptr(), a1.rows, b1.rows, a1.k,
        out1.data_ptr(), out1.stride(0), wp or None, wn, _stream(out0.device))
    N.check(st, "mxfp4_gemm_nt_pair_ws")
    return out0, out1


def gemm_pair_split(M0, N0, K0, M1, N1, K1):
    """XCDs (of 8) the paired launch of gemm_nt_pair gives its first product for these sizes
    (aligned outputs, ldo = N); 0 when the two run as two launches."""
    return int(N.lib().mxfp4_gemm_pair_split(int(M0), int(N0), int(K0), int(M1), int(N1), int(K1)))


def gemm_workspace_bytes(M, Nn, K):
    """Bytes of scratch the split contraction of out[M, N] (contraction K) uses; 0 if it does not split."""
    return int(N.lib().mxfp4_gemm_workspace_bytes(int(M), int(Nn), int(K)))


def gemm_workspace(shapes, device):
    """One scratch tensor for GEMMs run in order on one stream: the largest need among (M, N, K) shapes."""
    nbytes = max([gemm_workspace_bytes(*s) for s in shapes] + [0])
    return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=device)


def _check_formats(a, b, fmt):
    if a.fmt != fmt or b.fmt != fmt:
        raise ValueError("operands are MXFP%d / MXFP%d, this product takes MXFP%d" % (a.fmt, b.fmt, fmt))


def gemm_nt(a: MxOperand, b: MxOperand, out=None, ws=None):
    """out[M, N] = dq(a)[M, K] . dq(b)[N, K]^T in bf16 (two MXFP4 operands).  With ws (a uint8
    scratch tensor, see gemm_workspace) the contraction of an output too small for the tiled
    kernels may be split over several workgroups (mxfp4_gemm_nt_ws)."""
    _check_formats(a, b, 4)
    return _gemm(N.lib().mxfp4_gemm_nt, "mxfp4_gemm_nt", a, b, out, ws)


def gemm_nn(a: MxOperand, bcol: MxOperand, out=None, ws=None):
    """out[M, N] = dq(a)[M, K] . B[K, N], B given by its column copy (N rows, contraction K);
    ws as for gemm_nt (the same kernel on the column copy)."""
    _check_formats(a, bcol, 4)
    return _gemm(N.lib().mxfp4_gemm_nn, "mxfp4_gemm_nn", a, bcol, out, ws)


def gemm_fp8_nt(a: MxOperand, b: MxOperand, out=None):
    """out[M, N] = dq(a)[M, K] . dq(b)[N, K]^T in bf16 (two MXFP8 operands)."""
    _check_formats(a, b, 8)
    return _gemm(N.lib().mxfp8_gemm_nt, "mxfp8_gemm_nt", a, b, out)


def workspace_bytes(M, Nn, K, training=True):
    return int(N.lib().gemm_fp4_bf16_workspace_bytes(M, Nn, K, 1 if training else 0))


def workspace_bytes_qw(M, Nn, K, training=True):
    return int(N.lib().gemm_fp4_bf16_workspace_bytes_qw(M, Nn, K, 1 if training else 0))


def workspace_bytes_ex(M, Nn, K, flags):
    return int(N.lib().gemm_fp4_bf16_workspace_bytes_ex(M, Nn, K, int(flags)))


def _flags(training, hadamard_grad, quantized_w, fp8_wgrad=False):
    if hadamard_grad and not training:
        raise ValueError("the Hadamard gradient recipe only applies to training")
    if fp8_wgrad and not training:
        raise ValueError("the FP8 wgrad only applies to training")
    if fp8_wgrad and hadamard_grad:
        raise ValueError("the Hadamard recipe and the FP8 wgrad do not combine")
    return ((N.STEP_TRAINING if training else 0) | (N.STEP_HADAMARD_GRAD if hadamard_grad else 0) |
            (N.STEP_QUANTIZED_W if quantized_w else 0) | (N.STEP_FP8_WGRAD if fp8_wgrad else 0))


def _check_weight_fp4(w_fp4, Nn, K, training, hadamard_grad):
    if w_fp4.shape != (Nn, K):
        raise ValueError("w_fp4 holds a [%d, %d] weight, expected [%d, %d]" % (w_fp4.shape + (Nn, K)))
    if training and w_fp4.col is None:
        raise ValueError("training needs the weight's column copy: quantize with columnwise=True")
    if training and w_fp4.hadamard_col != bool(hadamard_grad):
        raise ValueError("the weight's column copy %s the Hadamard transform but hadamard_grad is %s" %
                         ("carries" if w_fp4.hadamard_col else "lacks", bool(hadamard_grad)))


def _fwd(a, w, w_fp4, training, ws, out, hadamard_grad, fp8_wgrad=False):
    _check_bf16_matrix(a, "a")
    if not a.is_contiguous():
        raise ValueError("a must be contiguous")
    M, K = a.shape
    if w_fp4 is None:
        _check_bf16_matrix(w, "w")
        if not w.is_contiguous():
            raise ValueError("w must be contiguous")
        if w.shape[1] != K:
            raise ValueError("a and w disagree on K")
        Nn = w.shape[0]
    else:
        Nn = w_fp4.shape[0]
        _check_weight_fp4(w_fp4, Nn, K, training, hadamard_grad)
    flags = _flags(training, hadamard_grad, w_fp4 is not None, fp8_wgrad)
    nbytes = workspace_bytes_ex(M, Nn, K, flags)
    if ws is None:
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=a.device)
    if out is None:
        out = torch.empty((M, Nn), dtype=torch.bfloat16, device=a.device)
    r = w_fp4.row if w_fp4 is not None else None
    st = N.lib().gemm_fp4_bf16_fwd_ex(a.data_ptr(), w.data_ptr() if w_fp4 is None else None,
                                      r.q.data_ptr() if r is not None else None,
                                      r.s.data_ptr() if r is not None else None, M, Nn, K, out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), flags, _stream(a.device))
    N.check(st, "gemm_fp4_bf16_fwd")
    return out, ws


def _bwd(dout, w_fp4, M, Nn, K, ws, need_da, need_dw, da, dw, hadamard_grad, fp8_wgrad=False):
    _check_bf16_matrix(dout, "dout")
    if not dout.is_contiguous():
        dout = dout.contiguous()
    if need_da and da is None:
        da = torch.empty((M, K), dtype=torch.bfloat16, device=dout.device)
    if need_dw and dw is None:
        dw = torch.empty((Nn, K), dtype=torch.bfloat16, device=dout.device)
    c = w_fp4.col if w_fp4 is not None else None
    st = N.lib().gemm_fp4_bf16_bwd_ex(dout.data_ptr(), c.q.data_ptr() if c is not None else None,
                                      c.s.data_ptr() if c is not None else None, M, Nn, K, ws.data_ptr(), ws.numel(),
                                      da.data_ptr() if need_da else None, dw.data_ptr() if need_dw else None,
                                      _flags(True, hadamard_grad, w_fp4 is not None, fp8_wgrad),
                                      _stream(dout.device))
    N.check(st, "gemm_fp4_bf16_bwd")
    return (da if need_da else None), (dw if need_dw else None)


def gemm_fp4_bf16_fwd(a, w, training=True, ws=None, out=None, hadamard_grad=False, fp8_wgrad=False):
    """Forward of gemm_fp4_bf16 on 2-D contiguous bf16 a [M, K], w [N, K] -> (out [M, N], ws)."""
    return _fwd(a, w, None, training, ws, out, hadamard_grad, fp8_wgrad)


def gemm_fp4_bf16_bwd(dout, M, Nn, K, ws, need_da=True, need_dw=True, da=None, dw=None, hadamard_grad=False,
                      fp8_wgrad=False):
    """Backward of gemm_fp4_bf16 from the workspace of a training forward -> (da, dw).
    The options must be the forward's."""
    return _bwd(dout, None, M, Nn, K, ws, need_da, need_dw, da, dw, hadamard_grad, fp8_wgrad)


def gemm_fp4_bf16_fwd_qw(a, w_fp4, training=True, ws=None, out=None, hadamard_grad=False, fp8_wgrad=False):
    """Forward with a pre-quantized weight (Mxfp4Tensor of W [N, K]) -> (out [M, N], ws)."""
    return _fwd(a, None, w_fp4, training, ws, out, hadamard_grad, fp8_wgrad)


def gemm_fp4_bf16_bwd_qw(dout, w_fp4, M, Nn, K, ws, need_da=True, need_dw=True, da=None, dw=None,
                         hadamard_grad=False, fp8_wgrad=False):
    """Backward of gemm_fp4_bf16_fwd_qw (W's column copy from w_fp4) -> (da, dw)."""
    return _bwd(dout, w_fp4, M, Nn, K, ws, need_da, need_dw, da, dw, hadamard_grad, fp8_wgrad)


class _GemmFp4Bf16(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, w, w_fp4, hadamard_grad, fp8_wgrad):
        training = bool(ctx.needs_input_grad[0] or ctx.needs_input_grad[1])
        had = bool(hadamard_grad) and training
        f8 = bool(fp8_wgrad) and training
        out, ws = _fwd(a, w if w_fp4 is None else None, w_fp4, training, None, None, had, f8)
        ctx.dims = (a.shape[0], w.shape[0], a.shape[1])
        ctx.ws = ws if training else None
        ctx.w_fp4 = w_fp4
        ctx.hadamard = had
        ctx.fp8_wgrad = f8
        return out

    @staticmethod
    def backward(ctx, dout):
        M, Nn, K = ctx.dims
        da, dw = _bwd(dout, ctx.w_fp4, M, Nn, K, ctx.ws, ctx.needs_input_grad[0], ctx.needs_input_grad[1], None,
                      None, ctx.hadamard, ctx.fp8_wgrad)
        ctx.ws = None
        ctx.w_fp4 = None
        return da, dw, None, None, None


def gemm_fp4_bf16(a, w, w_fp4: Optional[Mxfp4Tensor] = None, hadamard_grad: bool = False,
                  fp8_wgrad: bool = False):
    """BF16 in/out MXFP4 GEMM, out = a . w^T, differentiable (FP4 forward, FP4 dA, FP4 dB).

    a: [..., K] bfloat16, w: [N, K] bfloat16 -> [..., N] bfloat16.
    w_fp4: w already quantized (e.g. from WeightWorkspace.get_or_quantize with a weight
    quantizer); its copies replace w's cast in the forward and in dA.  w still receives dW.
    hadamard_grad: the README's gradient recipe -- dA and dB contract Walsh-Hadamard
    transformed operands (dOut's copies and the column copies of a and w); a w_fp4 then
    has to come from a weight quantizer with hadamard=True.
    fp8_wgrad: dB as an MXFP8 product (the FP8 dB of the README's training architecture);
    the forward product and dA stay MXFP4.  Does not combine with hadamard_grad.
    """
    lead = a.shape[:-1]
    a2 = a.reshape(-1, a.shape[-1]).contiguous()
    if hadamard_grad and fp8_wgrad:
        raise ValueError("the Hadamard recipe and the FP8 wgrad do not combine")
    out = _GemmFp4Bf16.apply(a2, w.contiguous(), w_fp4, hadamard_grad, fp8_wgrad)
    return out.reshape(*lead, w.shape[0])
