"""Helpers for the GPU parity tests: moving bf16 bit arrays to the device,
reading MX operands back in the oracle's row-major form, and the GEMM bar."""
import sys

import numpy as np
import torch

from mxfp4_block_scaled_cast_amd import layout


def say(msg):
    """Name the case before a GPU step (so a failing run shows what it was doing)."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def to_device(bits):
    """uint16 bf16 bit patterns [R, C] -> bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def operand_rowmajor(op):
    """(q [rows, k/2], s [rows, k/32]) of an MX operand, as the oracle lays them out."""
    q = layout.codes_to_rowmajor(op.q.cpu().numpy(), op.rows, op.k)
    s = layout.scales_to_rowmajor(op.s.cpu().numpy(), op.rows, op.k)
    return q, s


def operand_padding(op):
    """Code and scale bytes at padding positions of the device layout (all must be 0)."""
    q = op.q.cpu().numpy()
    s = op.s.cpu().numpy()
    return np.concatenate([q[layout.code_padding_mask(op.rows, op.k)], s[layout.scale_padding_mask(op.rows, op.k)]])


def gemm_bound(ref, absref):
    """|gpu - ref| allowed per element: 2^-7 |ref| + 1e-5 sum|a b| + 2^-126 (underflow floor)."""
    return 2.0 ** -7 * np.abs(ref) + 1e-5 * absref + 2.0 ** -126


def assert_gemm_close(got, ref, absref, what=""):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = gemm_bound(ref, absref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join("%s: got %r ref %r bound %r" % (tuple(i), got[tuple(i)], ref[tuple(i)], bound[tuple(i)])
                           for i in idx)
        raise AssertionError("%s: %d of %d outputs outside the bound; %s" % (what, bad.sum(), bad.size, detail))


def bf16_rne_of_exact(ref):
    """bf16 (as float64) of values exactly representable in fp32, rounded to nearest even."""
    f = np.asarray(ref, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), ref), "reference is not exact in fp32"
    return torch.from_numpy(f).to(torch.bfloat16).float().numpy().astype(np.float64)
