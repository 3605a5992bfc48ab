"""Seeded synthetic inputs for the MXFP4 cast/GEMM workloads (bf16 bit patterns as uint16).

This module only draws numbers: it holds none of the cast or GEMM arithmetic,
and both the HIP path and the CPU oracle consume what it returns.  The shapes
stand in for the per-GPU projection GEMMs of Llama-3.1-8B and Llama-3-70B
training (jax-aiter README, "Supported ops": the FP4 recipe measured at 8B
and 70B), with activations ~N(0, 1), weights ~N(0, 0.02) (8B) or N(0, 0.01)
(70B), output gradients ~N(0, 1).

Values are drawn in float32 with numpy's PCG64 generator and rounded to bf16
(nearest even).  Seeds: 1000 * config_id + operand (A = 0, W = 1, dOut = 2,
outlier-channel pick = 3); the ragged sweep adds 10 * combo_index.
"""
import numpy as np

A, W, DOUT, OUTLIER = 0, 1, 2, 3


def bf16_bits(f32):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def seed_of(config_id, operand, combo=0):
    return 1000 * config_id + operand + 10 * combo


def normal_f32(shape, std, seed):
    rng = np.random.default_rng(seed)
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal_bf16(shape, std, seed):
    return bf16_bits(normal_f32(shape, std, seed))


def outlier_channels(K, seed, frac=0.01):
    """round(frac * K) distinct channel indices, drawn without replacement."""
    n = int(round(frac * K))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, size=n, replace=False))


def activations_with_outliers(M, K, seed_values, seed_pick, factor=50.0):
    """N(0, 1) activations with 1% of the K channels multiplied by `factor` before rounding."""
    f = normal_f32((M, K), 1.0, seed_values)
    f[:, outlier_channels(K, seed_pick)] *= np.float32(factor)
    return bf16_bits(f)


def ragged_values(shape, seed, lo=-1e3, hi=1e3, zero_frac=0.05, subnormal_frac=0.05):
    """U(lo, hi) with 5% all-zero and 5% subnormal-magnitude aligned 32x32 tiles.

    Subnormal tiles hold random signs, bf16 exponent field 0 and mantissas
    uniform in 1..127.  Tiles are aligned so both the row and the column
    copies see whole zero / subnormal blocks.  Drawn one 32-row strip at a
    time (tile kinds first, then per strip the uniform values, then the
    subnormal tiles of that strip) to bound host memory.
    """
    R, C = shape
    rng = np.random.default_rng(seed)
    tr, tc = -(-R // 32), -(-C // 32)
    kind = rng.random((tr, tc))
    bits = np.empty(shape, np.uint16)
    for ti in range(tr):
        r0, r1 = ti * 32, min(R, ti * 32 + 32)
        strip = bits[r0:r1]
        strip[:] = bf16_bits(rng.uniform(lo, hi, size=(r1 - r0, C)).astype(np.float32))
        for tj in np.nonzero(kind[ti] < zero_frac)[0]:
            strip[:, tj * 32:(tj + 1) * 32] = 0
        for tj in np.nonzero((kind[ti] >= zero_frac) & (kind[ti] < zero_frac + subnormal_frac))[0]:
            c0, c1 = tj * 32, min(C, tj * 32 + 32)
            mant = rng.integers(1, 128, size=(r1 - r0, c1 - c0), dtype=np.uint16)
            sign = rng.integers(0, 2, size=(r1 - r0, c1 - c0), dtype=np.uint16) << 15
            strip[:, c0:c1] = mant | sign
    return bits


def hand_block_matrix():
    """[64, 32] bf16 matrix of 64 hand-built blocks, one block per row.

    Families: all-zero (+0 / -0), a single non-zero element, amax exactly
    6 * 2^e, and elements on the E2M1 midpoints (ties) beside an anchor
    of 4 * 2^e that fixes the block exponent.
    """
    def f2b(v):
        return int(bf16_bits(np.array([v], np.float32))[0])

    rows = []
    rows.append([0] * 32)
    rows.append([0x8000] * 32)
    # single non-zero at varying positions and magnitudes
    for i, v in enumerate([1.0, -3.0, 2.5, 0.75, 1e-3, -7.0, 448.0, 1.25, 1.3, -1e30, 3e-38, 5.0]):
        r = [0] * 32
        r[(5 * i) % 32] = f2b(v)
        rows.append(r)
    # amax exactly 6 * 2^e with a few smaller companions
    for e in (-120, -20, -3, -1, 0, 1, 4, 10, 60, 125):
        r = [0] * 32
        r[e % 32] = f2b(6.0 * 2.0 ** e)
        r[(e + 7) % 32] = f2b(-1.5 * 2.0 ** e)
        r[(e + 13) % 32] = f2b(0.5 * 2.0 ** e)
        rows.append(r)
    # midpoints: anchor 4*2^e, then t*2^e for every E2M1 midpoint t, both signs
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for e in (-127, -126, -60, -8, -2, 0, 2, 9, 30, 100, 125):
        r = [0] * 32
        r[0] = f2b(4.0 * 2.0 ** e)
        for j, t in enumerate(mids):
            r[1 + j] = f2b(t * 2.0 ** e)
            r[8 + j] = f2b(-t * 2.0 ** e)
        rows.append(r)
    # subnormal blocks and the clamp boundary
    for m in (1, 3, 8, 64, 96, 127):
        r = [0] * 32
        r[m % 32] = m
        r[(m + 1) % 32] = 0x8000 | (m // 2 + 1)
        rows.append(r)
    rows.append([0x0100] + [0] * 31)       # amax 2^-125 (no clamp needed)
    rows.append([0x0180, 0x0100] + [0] * 30)
    rows.append([0x7F7F, 0xFF7F] + [0x3F80] * 30)  # +-bf16 max beside ones
    # fill to 64 with dense random-magnitude blocks
    rng = np.random.default_rng(64)
    while len(rows) < 64:
        f = (rng.standard_normal(32) * 2.0 ** rng.integers(-30, 30)).astype(np.float32)
        rows.append([int(b) for b in bf16_bits(f)])
    return np.array(rows[:64], np.uint16)


# ---- workload catalogue ---------------------------------------------------

# (name, M, N, K) projection GEMMs, one GPU's share (M = 8192 tokens = bs1 x seq 8192)
LLAMA8B_ATTN = [("qkv", 8192, 6144, 4096), ("o", 8192, 4096, 4096)]
LLAMA8B_MLP = [("gate_up", 8192, 28672, 4096), ("down", 8192, 4096, 14336)]
LLAMA70B = [("qkv", 8192, 10240, 8192), ("gate_up", 8192, 57344, 8192), ("down", 8192, 8192, 28672)]
RAGGED_M = (1, 17, 4096, 16384)
RAGGED_N = (128, 4096, 128256)
RAGGED_K = (32, 4096, 14336)

CONFIG_IDS = {"tiny": 0, "llama8b_attn": 1, "llama8b_mlp": 2, "llama70b": 3, "ragged": 4}
W_STD = {"tiny": 1.0, "llama8b_attn": 0.02, "llama8b_mlp": 0.02, "llama70b": 0.01}


def ragged_combos():
    """All 36 (M, N, K) combinations of the ragged / edge sweep, in a fixed order."""
    return [(m, n, k) for m in RAGGED_M for n in RAGGED_N for k in RAGGED_K]


def projection_inputs(config, index, M, N, K, with_grad=True):
    """(a, w, dout) bf16 bit arrays for GEMM `index` of a projection config.

    The GEMM index is folded into the seed (combo) so each projection has its own data.
    """
    cid = CONFIG_IDS[config]
    if config == "llama8b_mlp":
        a = activations_with_outliers(M, K, seed_of(cid, A, index), seed_of(cid, OUTLIER, index))
    else:
        a = normal_bf16((M, K), 1.0, seed_of(cid, A, index))
    w = normal_bf16((N, K), W_STD[config], seed_of(cid, W, index))
    dout = normal_bf16((M, N), 1.0, seed_of(cid, DOUT, index)) if with_grad else None
    return a, w, dout


def ragged_inputs(combo_index, with_grad=True):
    M, N, K = ragged_combos()[combo_index]
    cid = CONFIG_IDS["ragged"]
    a = ragged_values((M, K), seed_of(cid, A, combo_index))
    w = ragged_values((N, K), seed_of(cid, W, combo_index))
    dout = ragged_values((M, N), seed_of(cid, DOUT, combo_index)) if with_grad else None
    return a, w, dout


def ragged_values_torch(shape, seed, device, lo=-1e3, hi=1e3, zero_frac=0.05, subnormal_frac=0.05):
    """The ragged recipe drawn on a device with torch's seeded generator (for sizes the host draws too slowly).

    Same distribution as ``ragged_values`` (U(lo, hi), 5% all-zero and 5%
    subnormal aligned 32x32 tiles), different random stream.  Returns an
    int16 tensor of bf16 bit patterns on `device`.
    """
    import torch

    R, C = shape
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    vals = torch.empty((R, C), dtype=torch.float32, device=device).uniform_(lo, hi, generator=g)
    bits = vals.to(torch.bfloat16).view(torch.int16)
    del vals
    tr, tc = -(-R // 32), -(-C // 32)
    kind = torch.rand((tr, tc), generator=g, device=device)
    tile_kind = kind.repeat_interleave(32, 0)[:R].repeat_interleave(32, 1)[:, :C]
    zero = tile_kind < zero_frac
    sub = (tile_kind >= zero_frac) & (tile_kind < zero_frac + subnormal_frac)
    mant = torch.randint(1, 128, (R, C), generator=g, device=device, dtype=torch.int16)
    sign = torch.randint(0, 2, (R, C), generator=g, device=device, dtype=torch.int16) * -32768
    bits = torch.where(zero, torch.zeros_like(bits), bits)
    bits = torch.where(sub, (mant | sign).to(torch.int16), bits)
    return bits
