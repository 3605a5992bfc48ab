"""ctypes binding of libmxfp4.so: argument marshalling only.

The shared library is built in-tree by ``build.py`` (``__graft_entry__.build()``).
Every entry point listed in include/mxfp4.h is bound here under its C name.
"""
import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmxfp4.so")
_lib = None

# (name, restype, argtypes) of every symbol include/mxfp4.h declares
_i64, _p, _i32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class OperandLayout(ctypes.Structure):
    _fields_ = [("rows", _i64), ("k", _i64), ("q_bytes", _i64), ("s_bytes", _i64),
                ("code_row_tiles", _i64), ("code_k_tiles", _i64), ("scale_row_tiles", _i64),
                ("scale_k_tiles", _i64)]


class Layout(ctypes.Structure):
    _fields_ = [("rows", _i64), ("cols", _i64), ("padded_rows", _i64), ("row", OperandLayout), ("col", OperandLayout)]


SIGNATURES = [
    ("mxfp4_operand_layout_of", _i32, [_i64, _i64, ctypes.POINTER(OperandLayout)]),
    ("mxfp4_layout", _i32, [_i64, _i64, ctypes.POINTER(Layout)]),
    ("mxfp4_status_string", ctypes.c_char_p, [_i32]),
    ("mxfp4_cast", _i32, [_p, _i64, _i64, _i64, _p, _p, _p]),
    ("mxfp4_cast_dual", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    ("mxfp4_cast_dual_pair", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    ("mxfp4_gemm_nt", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p]),
    ("mxfp4_gemm_nn", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p]),
    ("mxfp4_gemm_workspace_bytes", _sz, [_i64, _i64, _i64]),
    ("mxfp4_gemm_nt_ws", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p, _sz, _p]),
    ("mxfp4_gemm_nt_pair_ws", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64] * 2 + [_p, _sz, _p]),
    ("mxfp4_gemm_pair_split", _i32, [_i64] * 6),
    ("gemm_fp4_bf16_workspace_bytes", _sz, [_i64, _i64, _i64, _i32]),
    ("gemm_fp4_bf16_fwd", _i32, [_p, _p, _i64, _i64, _i64, _p, _p, _sz, _i32, _p]),
    ("gemm_fp4_bf16_bwd", _i32, [_p, _i64, _i64, _i64, _p, _sz, _p, _p, _p]),
    ("gemm_fp4_bf16_workspace_bytes_qw", _sz, [_i64, _i64, _i64, _i32]),
    ("gemm_fp4_bf16_fwd_qw", _i32, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _sz, _i32, _p]),
    ("gemm_fp4_bf16_bwd_qw", _i32, [_p, _p, _p, _i64, _i64, _i64, _p, _sz, _p, _p, _p]),
    ("mxfp4_cast_hadamard", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _p]),
    ("gemm_fp4_bf16_fwd_ex", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _sz, ctypes.c_uint, _p]),
    ("gemm_fp4_bf16_bwd_ex", _i32, [_p, _p, _p, _i64, _i64, _i64, _p, _sz, _p, _p, ctypes.c_uint, _p]),
    ("mxfp8_operand_layout_of", _i32, [_i64, _i64, ctypes.POINTER(OperandLayout)]),
    ("mxfp8_cast", _i32, [_p, _i64, _i64, _i64, _p, _p, _p]),
    ("mxfp8_cast_dual", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    ("mxfp4_cast_dual_fp8col", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    ("mxfp8_gemm_nt", _i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p]),
    ("gemm_fp4_bf16_workspace_bytes_ex", _sz, [_i64, _i64, _i64, ctypes.c_uint]),
    ("mxfp4_silu_mul_cast", _i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p]),
    ("mxfp4_rmsnorm_cast", _i32, [_p, _p, _p, ctypes.c_float, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p, _p, _p]),
    ("gemm_fp4_bf16_fwd_qw_noalloc", _i32, [_p, _p, _p, _i64, _i64, _i64, _p, _p]),
]

STEP_TRAINING, STEP_HADAMARD_GRAD, STEP_QUANTIZED_W, STEP_FP8_WGRAD = 1, 2, 4, 8

NOALLOC_SCRATCH_BYTES = 64 << 20  # MXFP4_NOALLOC_SCRATCH_BYTES

STATUS = {0: "MXFP4_OK", -1: "MXFP4_EINVAL", -2: "MXFP4_EALIGN", -3: "MXFP4_EDEVICE",
          -4: "MXFP4_ELAUNCH", -5: "MXFP4_ERANGE", -6: "MXFP4_ESPACE"}


class Mxfp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS.get(status, status), status_string(status)))


def library_path():
    return _LIB_PATH


def lib():
    """The loaded HIP library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmxfp4.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().mxfp4_status_string(int(status)).decode()


def check(status, where):
    if status != 0:
        raise Mxfp4Error(status, where)


def layout(rows, cols):
    """Sizes of both copies (row copy, column copy) of a cast bf16 matrix [rows, cols]."""
    out = Layout()
    check(lib().mxfp4_layout(int(rows), int(cols), ctypes.byref(out)), "mxfp4_layout")
    return out


def operand_layout(rows, k, fmt=4):
    """Sizes of an MX operand: fmt 4 = MXFP4, 8 = MXFP8."""
    out = OperandLayout()
    name = "mxfp8_operand_layout_of" if fmt == 8 else "mxfp4_operand_layout_of"
    if fmt not in (4, 8):
        raise ValueError("fmt must be 4 or 8")
    check(getattr(lib(), name)(int(rows), int(k), ctypes.byref(out)), name)
    return out
