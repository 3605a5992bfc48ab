"""Index maps between the tiled MX operand layout and plain row-major arrays.

The layout (include/mxfp4.h) for an operand of `rows` rows and contraction
length `k`:

* codes: 1 KB tiles of 16 rows x 128 elements; byte j of row r (elements 2j,
  2j+1) sits at ((r//16) * KT + j//64) * 1024 + (r%16) * 64 + j%64 with
  KT = ceil(k/128);
* scales: 1 KB tiles of 128 rows x 256 elements; the scale of (r, block b)
  sits at ((r//128) * KT2 + b//8) * 1024 + ((r//32)%4) * 256 + (r%32) * 8
  + (b%2) * 4 + (b%8)//2 with KT2 = ceil(k/256).

MXFP8 operands keep the scales and store one E4M3 code per byte in 1 KB
tiles of 16 rows x 64 elements: element k of row r at ((r//16) * KT8 +
k//64) * 1024 + (r%16) * 64 + k%64 with KT8 = ceil(k/64).
"""
import numpy as np


def _check(k):
    if k % 32:
        raise ValueError("k must be a multiple of 32")


def code_bytes(rows, k):
    return -(-rows // 16) * (-(-k // 128)) * 1024


def scale_bytes(rows, k):
    return -(-rows // 128) * (-(-k // 256)) * 1024


def code_offsets(rows, k):
    """int64 [rows, k/2]: device byte offset of each packed code byte."""
    _check(k)
    kt = -(-k // 128)
    r = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(k // 2, dtype=np.int64)[None, :]
    return ((r // 16) * kt + j // 64) * 1024 + (r % 16) * 64 + j % 64


def scale_offsets(rows, k):
    """int64 [rows, k/32]: device byte offset of each scale."""
    _check(k)
    kt2 = -(-k // 256)
    r = np.arange(rows, dtype=np.int64)[:, None]
    b = np.arange(k // 32, dtype=np.int64)[None, :]
    return ((r // 128) * kt2 + b // 8) * 1024 + ((r // 32) % 4) * 256 + (r % 32) * 8 + (b % 2) * 4 + (b % 8) // 2


def codes_to_rowmajor(q_dev, rows, k):
    """Device code bytes -> uint8 [rows, k/2] (element 2j in the low nibble of byte j)."""
    q_dev = np.asarray(q_dev, np.uint8).reshape(-1)
    if q_dev.size < code_bytes(rows, k):
        raise ValueError("code buffer too small")
    return q_dev[code_offsets(rows, k)]


def scales_to_rowmajor(s_dev, rows, k):
    """Device scale bytes -> uint8 [rows, k/32]."""
    s_dev = np.asarray(s_dev, np.uint8).reshape(-1)
    if s_dev.size < scale_bytes(rows, k):
        raise ValueError("scale buffer too small")
    return s_dev[scale_offsets(rows, k)]


def codes_from_rowmajor(q, rows, k):
    out = np.zeros(code_bytes(rows, k), np.uint8)
    out[code_offsets(rows, k)] = np.asarray(q, np.uint8)
    return out


def scales_from_rowmajor(s, rows, k):
    out = np.zeros(scale_bytes(rows, k), np.uint8)
    out[scale_offsets(rows, k)] = np.asarray(s, np.uint8)
    return out


def code8_bytes(rows, k):
    return -(-rows // 16) * (-(-k // 64)) * 1024


def code8_offsets(rows, k):
    """int64 [rows, k]: device byte offset of each MXFP8 code."""
    _check(k)
    kt = -(-k // 64)
    r = np.arange(rows, dtype=np.int64)[:, None]
    e = np.arange(k, dtype=np.int64)[None, :]
    return ((r // 16) * kt + e // 64) * 1024 + (r % 16) * 64 + e % 64


def codes8_to_rowmajor(q_dev, rows, k):
    """Device MXFP8 code bytes -> uint8 [rows, k]."""
    q_dev = np.asarray(q_dev, np.uint8).reshape(-1)
    if q_dev.size < code8_bytes(rows, k):
        raise ValueError("code buffer too small")
    return q_dev[code8_offsets(rows, k)]


def codes8_from_rowmajor(q, rows, k):
    out = np.zeros(code8_bytes(rows, k), np.uint8)
    out[code8_offsets(rows, k)] = np.asarray(q, np.uint8)
    return out


def code8_padding_mask(rows, k):
    """True at device MXFP8 code bytes that no (row, element) maps to."""
    m = np.ones(code8_bytes(rows, k), bool)
    m[code8_offsets(rows, k)] = False
    return m


def code_padding_mask(rows, k):
    """True at device code bytes that no (row, element) maps to."""
    m = np.ones(code_bytes(rows, k), bool)
    m[code_offsets(rows, k)] = False
    return m


def scale_padding_mask(rows, k):
    """True at device scale bytes that no (row, block) maps to."""
    m = np.ones(scale_bytes(rows, k), bool)
    m[scale_offsets(rows, k)] = False
    return m
