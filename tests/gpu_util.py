"""Helpers for the GPU parity tests: moving bf16 bit arrays to the device,
reading MX operands back in the oracle's row-major form, and the GEMM bar."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
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
    """(q, s [rows, k/32]) of an MX operand as the oracle lays them out: q [rows, k/2] packed
    E2M1 pairs for MXFP4, q [rows, k] E4M3 bytes for MXFP8."""
    if getattr(op, "fmt", 4) == 8:
        q = layout.codes8_to_rowmajor(op.q.cpu().numpy(), op.rows, op.k)
        return q, layout.scales_to_rowmajor(op.s.cpu().numpy(), op.rows, op.k)
    q = layout.codes_to_rowmajor(op.q.cpu().numpy(), op.rows, op.k)
    s = layout.scales_to_rowmajor(op.s.cpu().numpy(), op.rows, op.k)
    return q, s


def operand_padding(op):
    """Code and scale bytes at padding positions of the device layout (all must be 0)."""
    q = op.q.cpu().numpy()
    s = op.s.cpu().numpy()
    qmask = (layout.code8_padding_mask if getattr(op, "fmt", 4) == 8 else layout.code_padding_mask)(op.rows, op.k)
    return np.concatenate([q[qmask], s[layout.scale_padding_mask(op.rows, op.k)]])


def gemm_bound(ref, absref):
    """|gpu - ref| allowed per element: 2^-7 |ref| + 1e-5 sum|a b| + 2^-126 (underflow floor)."""
    return 2.0 ** -7 * np.abs(ref) + 1e-5 * absref + 2.0 ** -126


def assert_gemm_close(got, ref, absref, what="", extra=0.0):
    """The GEMM bar; `extra` adds a per-output allowance (the FP8 in-group truncation bound)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = gemm_bound(ref, absref) + extra
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


def e4m3_exponents(q, s):
    """int16 [rows, k]: exponent of each MXFP8 element's power-of-two envelope, e + X, where e is
    the E4M3 code's unbiased exponent (exponent field - 7; subnormal and zero codes at -6) and
    X the block's scale exponent.  2^(e + X) >= |value| / 2 for normal codes."""
    field = ((np.asarray(q, np.uint8) >> 3) & 0xF).astype(np.int16)
    e = np.maximum(field, 1) - 7
    X = np.repeat(np.asarray(s, np.int16) - 127, 32, axis=1)
    return e + X


def fp8_truncation_bound(qa, sa, qb, sb, chunk_rows=64):
    """Per-output bound of the error the FP8 scaled MFMA adds inside its product groups.

    Measured arithmetic of V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E4M3 operands (gfx950):
    products are summed in groups of 8 consecutive K elements (inside one 32-element block);
    in a group every product is truncated toward zero to a multiple of 2^(E - 13), E the
    largest exponent sum e_a + e_b (with the scales) in the group; group sums then add
    exactly into the fp32 accumulation.  So a group loses less than 8 * 2^(E - 13), and the
    bound is sum over groups of 2^(E_g - 10), E_g from the exponent envelopes (an upper
    bound of the hardware's own exponents, zero codes included)."""
    import torch
    ea = torch.from_numpy(e4m3_exponents(qa, sa))
    eb = torch.from_numpy(e4m3_exponents(qb, sb))
    M, K = ea.shape
    Nn = eb.shape[0]
    G = K // 8
    ea = ea.reshape(M, G, 8)
    eb = eb.reshape(Nn, G, 8)
    out = np.empty((M, Nn), np.float64)
    for m0 in range(0, M, chunk_rows):
        m1 = min(M, m0 + chunk_rows)
        emax = (ea[m0:m1, None] + eb[None]).amax(-1)                  # [m, N, G] int16
        out[m0:m1] = torch.ldexp(torch.ones((), dtype=torch.float64), (emax - 10).to(torch.float64)).sum(-1).numpy()
    return out


# ---- whole-buffer images of the device layout -------------------------------------------
# The tiled MX layout is a pure tiling of the row-major arrays, so the bytes a device copy must
# hold (padding included) come from the oracle's row-major output by padding and one transpose:
# codes (r//16, k//128, r%16, byte of the 64-byte tile row), scales (r//128, b//8, (r//32)%4,
# r%32, b%2, (b%8)//2).  tests/test_layout_images.py pins these against the index maps.

def codes_image(q_rm, rows, k):
    """Device bytes of an MXFP4 code buffer from row-major q [rows, k/2] (zeros at padding)."""
    kt, r16 = -(-k // 128), -(-rows // 16)
    buf = np.zeros((r16 * 16, kt * 64), np.uint8)
    buf[:rows, :k // 2] = q_rm
    return buf.reshape(r16, 16, kt, 64).transpose(0, 2, 1, 3).ravel()


def codes8_image(q_rm, rows, k):
    """Device bytes of an MXFP8 code buffer from row-major q [rows, k]."""
    kt, r16 = -(-k // 64), -(-rows // 16)
    buf = np.zeros((r16 * 16, kt * 64), np.uint8)
    buf[:rows, :k] = q_rm
    return buf.reshape(r16, 16, kt, 64).transpose(0, 2, 1, 3).ravel()


def scales_image(s_rm, rows, k):
    """Device bytes of a scale buffer from row-major s [rows, k/32]."""
    kt2, r128 = -(-k // 256), -(-rows // 128)
    buf = np.zeros((r128 * 128, kt2 * 8), np.uint8)
    buf[:rows, :k // 32] = s_rm
    return buf.reshape(r128, 4, 32, kt2, 4, 2).transpose(0, 3, 1, 2, 5, 4).ravel()


def assert_operand_equal(op, q_rm, s_rm, what):
    """Every byte of a device MX operand (codes, scales, padding) equals the image of the
    oracle's row-major (q, s)."""
    img = codes8_image if getattr(op, "fmt", 4) == 8 else codes_image
    for part, dev, expect in (("scales", op.s, scales_image(s_rm, op.rows, op.k)),
                              ("codes", op.q, img(q_rm, op.rows, op.k))):
        got = dev.cpu().numpy()
        if got.size != expect.size:
            raise AssertionError("%s %s: device buffer holds %d bytes, layout needs %d"
                                 % (what, part, got.size, expect.size))
        if not np.array_equal(got, expect):
            bad = np.flatnonzero(got != expect)
            raise AssertionError("%s %s: %d of %d bytes differ, first at byte %d (got %#x, expected %#x)"
                                 % (what, part, bad.size, got.size, bad[0], got[bad[0]], expect[bad[0]]))


def dequant_to_device(q, s, device, workers=None, fmt=4):
    """The oracle's dequantized values (fp64, exact) of a canonical (q, s) pair (fmt 4: MXFP4, 8:
    MXFP8), as a float64 tensor on `device`; the oracle runs on row slices in parallel threads."""
    R, K = q.shape[0], q.shape[1] * (2 if fmt == 4 else 1)
    fn = oracle.dequant if fmt == 4 else oracle.dequant_fp8
    out = torch.empty((R, K), dtype=torch.float64, device=device)
    if R == 0:
        return out
    workers = workers or min(16, os.cpu_count() or 1)
    step = max(1, -(-R // (4 * workers)))
    spans = [(r0, min(R, r0 + step)) for r0 in range(0, R, step)]
    with ThreadPoolExecutor(workers) as ex:
        parts = ex.map(lambda sp: fn(q[sp[0]:sp[1]], s[sp[0]:sp[1]]), spans)
        for (r0, r1), part in zip(spans, parts):
            out[r0:r1].copy_(torch.from_numpy(part))
    return out


def fp8_group_envelope(q, s, device):
    """float64 [rows, K/8] on `device`: 2^(E - 5) per group of 8 consecutive K elements, E the largest
    exponent envelope e + X (e4m3_exponents) in the group.  The largest exponent sum of a group of a
    product row pair is at most the sum of the two groups' largest exponents, so
    (envelope_a @ envelope_b^T)[m, n] = sum_g 2^(Ea_g + Eb_g - 10) bounds fp8_truncation_bound from above
    and takes one matrix product."""
    e = torch.from_numpy(e4m3_exponents(q, s))
    R, K = e.shape
    emax = e.reshape(R, K // 8, 8).amax(-1).to(torch.float64)
    return torch.ldexp(torch.ones((), dtype=torch.float64), emax - 5).to(device)


def device_ref_blocks(a, b, device, block_rows=2048, fmt=4):
    """Row blocks (r0, ref, absref, extra) of the exact product of oracle-quantized operands a = (q, s)
    [M, K] and b = (q, s) [N, K]: the oracle dequantizes them (exact in fp64); their products are summed
    by torch.matmul in float64 on the device (a library DGEMM that shares nothing with the kernels under
    test; its rounding, ~1e-16 relative, is far below the GEMM bar), and sum|a b| likewise from the
    magnitudes.  extra: 0 for MXFP4; for MXFP8 the allowance for the FP8 MFMA's in-group truncation from
    fp8_group_envelope (an upper bound of fp8_truncation_bound).  Row blocks bound the device memory."""
    A = dequant_to_device(a[0], a[1], device, fmt=fmt)
    Bt = dequant_to_device(b[0], b[1], device, fmt=fmt).t().contiguous()
    Bt_abs = Bt.abs()
    if fmt == 8:
        Pa = fp8_group_envelope(a[0], a[1], device)
        Pbt = fp8_group_envelope(b[0], b[1], device).t().contiguous()
    for r0 in range(0, A.shape[0], block_rows):
        blk = A[r0:r0 + block_rows]
        extra = Pa[r0:r0 + block_rows] @ Pbt if fmt == 8 else 0.0
        yield r0, blk @ Bt, blk.abs() @ Bt_abs, extra


def assert_gemm_whole(got, a, b, what, block_rows=2048, fmt=4):
    """Every output of got [M, N] (bf16 on the device) against device_ref_blocks(a, b), to the GEMM
    bar 2^-7 |ref| + 1e-5 sum|ab| + 2^-126 (plus, for MXFP8, the in-group truncation envelope)."""
    M, Nn = a[0].shape[0], b[0].shape[0]
    assert tuple(got.shape) == (M, Nn), "output shape %s, operands %d x %d" % (tuple(got.shape), M, Nn)
    bad_total, examples = 0, []
    for r0, ref, absref, extra in device_ref_blocks(a, b, got.device, block_rows, fmt):
        g = got[r0:r0 + ref.shape[0]].double()
        bound = ref.abs() * 2.0 ** -7 + absref * 1e-5 + 2.0 ** -126 + extra
        bad = ~((g - ref).abs() <= bound)
        n = int(bad.sum().item())
        if n and len(examples) < 5:
            for i, j in bad.nonzero()[:5 - len(examples)].tolist():
                examples.append("(%d, %d): got %r ref %r bound %r" % (r0 + i, j, g[i, j].item(), ref[i, j].item(),
                                                                       bound[i, j].item()))
        bad_total += n
        del ref, absref, g, bound, bad, extra
    if bad_total:
        raise AssertionError("%s: %d of %d outputs outside the bound; %s" % (what, bad_total, got.numel(),
                                                                           "; ".join(examples)))
