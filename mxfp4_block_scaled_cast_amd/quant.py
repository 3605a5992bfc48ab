"""Role quantizers and a cache of quantized weights.

jax-aiter's README (Quick start) exposes an object-oriented MXFP4 quantizer,
``MXFP4Quantizer.for_weight()`` whose ``quantize(w)`` returns an
``Mxfp4Tensor`` holding the row copy, the column copy and their scales, and
a ``WeightWorkspace`` whose ``get_or_quantize(w, quantizer, cache_name=...)``
keeps that tensor so later GEMMs skip the weight's cast.  Here the quantizer
runs the library's cast kernels (``mxfp4_cast`` / ``mxfp4_cast_dual``), and
``gemm_fp4_bf16(a, w, w_fp4=...)`` consumes the cached copies through
``gemm_fp4_bf16_fwd_qw`` / ``gemm_fp4_bf16_bwd_qw``.

Roles (which copies a GEMM operand needs in training):
  weight     : row copy (forward B) and column copy (dA's B);
  activation : row copy (forward A) and column copy (dB's B);
  grad       : row copy (dA's A) and column copy (dB's A).
With ``columnwise=False`` only the row copy is made (inference).  With
``hadamard=True`` (the README's gradient recipe) the copies that enter the
backward contractions carry the block Walsh-Hadamard transform
(``cast_hadamard``).
"""
import weakref
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch

from .api import Mxfp4Tensor, cast, cast_dual, cast_hadamard


@dataclass(frozen=True)
class MXFP4Quantizer:
    role: str
    rowwise: bool = True
    columnwise: bool = True
    hadamard: bool = False

    @classmethod
    def for_weight(cls, columnwise=True, hadamard=False):
        return cls("weight", True, columnwise, hadamard)

    @classmethod
    def for_activation(cls, columnwise=True, hadamard=False):
        return cls("activation", True, columnwise, hadamard)

    @classmethod
    def for_grad(cls, columnwise=True, hadamard=False):
        return cls("grad", True, columnwise, hadamard)

    def quantize(self, x: torch.Tensor) -> Mxfp4Tensor:
        """bf16 [R, C] (C % 32 == 0) -> Mxfp4Tensor with the row copy and, if columnwise, the column copy.

        With hadamard (the gradient recipe): a weight or an activation gets its column copy
        Walsh-Hadamard transformed (it is a B operand of dA or dB), a grad both copies, divided
        by 32, so the backward products stay unchanged.
        """
        if not self.rowwise:
            raise ValueError("an MXFP4 operand always carries its row copy")
        if self.hadamard and self.role == "grad":
            return cast_hadamard(x, True, self.columnwise, 5, self.columnwise)
        if self.hadamard and self.columnwise:
            return cast_hadamard(x, False, True, 0, True)
        if self.columnwise:
            return cast_dual(x)
        return Mxfp4Tensor(cast(x), None, tuple(x.shape))


def _key(w: torch.Tensor, q: MXFP4Quantizer) -> Tuple:
    # the storage, the in-place version counter and the view decide whether a cached copy is current
    return (w.device, w.data_ptr(), w._version, tuple(w.shape), tuple(w.stride()), w.dtype, q)


class WeightWorkspace:
    """Quantized weights by name, re-quantized only when the weight changed.

    A cached entry is reused only for the same tensor object (held by a weak
    reference, so a new tensor that the allocator places at a freed weight's
    address never matches) with the same storage, shape, strides and in-place
    version (``Tensor._version`` counts in-place updates such as an optimizer
    step), and the same quantizer.

    Updates that bypass the version counter are not seen: writing through
    ``w.data`` (``w.data.copy_(...)``, ``w.data.add_(...)``) or through another
    tensor that aliases w's memory.  After such an update call
    ``invalidate(cache_name)``.
    """

    def __init__(self):
        self._cache: Dict[str, Tuple[Tuple, "weakref.ref", Mxfp4Tensor]] = {}
        self.hits = 0
        self.misses = 0

    def get_or_quantize(self, w: torch.Tensor, quantizer: MXFP4Quantizer,
                        cache_name: Optional[str] = None) -> Mxfp4Tensor:
        name = cache_name if cache_name is not None else "@%x" % w.data_ptr()
        key = _key(w, quantizer)
        hit = self._cache.get(name)
        if hit is not None and hit[0] == key and hit[1]() is w:
            self.hits += 1
            return hit[2]
        self.misses += 1
        q = quantizer.quantize(w)
        self._cache[name] = (key, weakref.ref(w), q)
        return q

    def invalidate(self, cache_name: Optional[str] = None):
        """Drop one entry (or all)."""
        if cache_name is None:
            self._cache.clear()
        else:
            self._cache.pop(cache_name, None)

    def __len__(self):
        return len(self._cache)

    def __contains__(self, cache_name):
        return cache_name in self._cache
