"""Index maps between the device scale layout and a plain [rows, K/32] array.

The device layout (see include/mxfp4.h) stores the E8M0 scale of
(row r, block b) of an MX operand at
    ((r // 32) * kt + b // 8) * 256 + (r % 32) * 8 + (b % 2) * 4 + (b % 8) // 2
with kt = ceil(K / 256).  The packed codes are already row-major [rows, K/2].
"""
import numpy as np


def scale_offsets(rows, k):
    """int64 [rows, k/32] array of byte offsets of each scale in the device layout."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    kt = -(-k // 256)
    r = np.arange(rows, dtype=np.int64)[:, None]
    b = np.arange(k // 32, dtype=np.int64)[None, :]
    return ((r // 32) * kt + b // 8) * 256 + (r % 32) * 8 + (b % 2) * 4 + (b % 8) // 2


def scale_bytes(rows, k):
    return -(-rows // 32) * (-(-k // 256)) * 256


def scales_to_rowmajor(s_dev, rows, k):
    """Device-layout scale bytes -> uint8 [rows, k/32]."""
    s_dev = np.asarray(s_dev, np.uint8).reshape(-1)
    if s_dev.size < scale_bytes(rows, k):
        raise ValueError("scale buffer too small")
    return s_dev[scale_offsets(rows, k)]


def scales_from_rowmajor(s, rows, k):
    """uint8 [rows, k/32] -> device-layout bytes (padding positions 0)."""
    out = np.zeros(scale_bytes(rows, k), np.uint8)
    out[scale_offsets(rows, k)] = np.asarray(s, np.uint8)
    return out


def padding_mask(rows, k):
    """Boolean mask over the device scale buffer: True where no (row, block) maps."""
    m = np.ones(scale_bytes(rows, k), bool)
    m[scale_offsets(rows, k)] = False
    return m
