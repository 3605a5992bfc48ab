"""Exact, one-block-at-a-time MXFP4 reference on Python rationals.

TEST INFRASTRUCTURE (see the package docstring).  Every quantity is a
``fractions.Fraction``, so nothing here is subject to floating-point rounding.

Formats (jax-aiter README, "Supported ops": E2M1 elements, E8M0 block scales,
fp4x2 packing; field layouts from the OCP Microscaling v1.0 specification):

* bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits
* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
  subnormal (0 or 0.5)
* E8M0: byte e means 2^(e - 127); 0xFF is NaN
"""
from fractions import Fraction

BLOCK = 32


def bf16_value(h):
    """Exact value of bf16 bit pattern h, or None for Inf/NaN."""
    sign = (h >> 15) & 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0xFF:
        return None
    if e == 0:
        mag = Fraction(m, 2 ** 133)
    else:
        mag = Fraction(128 + m, 128) * Fraction(2) ** (e - 127)
    return -mag if sign else mag


def e2m1_value(code):
    """Value of the 4-bit E2M1 code, from its bit fields."""
    sign = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)
    else:
        mag = (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if sign else mag


def floor_log2(q):
    """floor(log2(q)) for a rational q > 0, exactly."""
    q = Fraction(q)
    if q <= 0:
        raise ValueError("floor_log2 needs a positive value")
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # now 2^(e-1) < q < 2^(e+1); settle which side of 2^e q is on
    if q >= Fraction(2) ** e:
        return e
    return e - 1


def shared_exponent(values):
    """Block exponent X: floor(log2(max |v|)) - 2 clamped to [-127, 127]; -127 for an all-zero block."""
    amax = max(abs(v) for v in values)
    if amax == 0:
        return -127
    return min(127, max(-127, floor_log2(amax) - 2))


def nearest_e2m1_magnitude(a):
    """Code 0..7 of the E2M1 magnitude nearest to a >= 0; on a tie the even code wins.

    Saturation needs no special case: above 6 the nearest magnitude is 6.
    """
    best = None
    for c in range(8):
        d = abs(a - e2m1_value(c))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def quantize_block(bits):
    """Quantize up to 32 bf16 bit patterns (missing positions are +0).

    Returns (scale_byte, codes[32]).  A block with an Inf or NaN gets scale
    0xFF and codes 0.
    """
    bits = list(bits) + [0] * (BLOCK - len(bits))
    if len(bits) != BLOCK:
        raise ValueError("a block has at most 32 elements")
    vals = [bf16_value(h) for h in bits]
    if any(v is None for v in vals):
        return 0xFF, [0] * BLOCK
    X = shared_exponent(vals)
    codes = []
    for h, v in zip(bits, vals):
        mag = nearest_e2m1_magnitude(abs(v) / Fraction(2) ** X)
        codes.append(mag | (((h >> 15) & 1) << 3))
    return X + 127, codes


def dequant_block(scale_byte, codes):
    """Exact values of a quantized block (None for a NaN scale)."""
    if scale_byte == 0xFF:
        return None
    f = Fraction(2) ** (scale_byte - 127)
    return [e2m1_value(c) * f for c in codes]


def pack(codes):
    """fp4x2 bytes: element 2j in the low nibble of byte j."""
    return [codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(len(codes) // 2)]


def quantize_row(bits):
    """Row of bf16 bit patterns (length a multiple of 32) -> (scale bytes, packed bytes)."""
    if len(bits) % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    scales, packed = [], []
    for b in range(0, len(bits), BLOCK):
        s, c = quantize_block(bits[b:b + BLOCK])
        scales.append(s)
        packed.extend(pack(c))
    return scales, packed


def dot_exact(a_bits_row, b_bits_row):
    """Exact dot product of the dequantized row copies of two bf16 rows, and sum |a_k b_k|."""
    sa, qa = quantize_row(a_bits_row)
    sb, qb = quantize_row(b_bits_row)
    total, atotal = Fraction(0), Fraction(0)
    for b in range(len(sa)):
        ca = [(qa[b * 16 + j // 2] >> (4 * (j % 2))) & 0xF for j in range(BLOCK)]
        cb = [(qb[b * 16 + j // 2] >> (4 * (j % 2))) & 0xF for j in range(BLOCK)]
        va, vb = dequant_block(sa[b], ca), dequant_block(sb[b], cb)
        for x, y in zip(va, vb):
            total += x * y
            atotal += abs(x * y)
    return total, atotal


# ---- Hadamard-transformed blocks (jax-aiter README, "Quick start": grad_out is cast with a
# Hadamard transform; the transform is read as the 32-point Sylvester Walsh-Hadamard matrix
# on each block along the contraction dimension) ----

def hadamard_entry(i, j):
    """Entry (i, j) of the 32-point Sylvester Walsh-Hadamard matrix: (-1)^popcount(i & j)."""
    return -1 if bin(i & j).count("1") % 2 else 1


def hadamard_block(values):
    """Exact H . values for a block of 32 rationals (the matrix product, no butterflies)."""
    if len(values) != BLOCK:
        raise ValueError("a block has 32 elements")
    return [sum(hadamard_entry(i, j) * Fraction(values[j]) for j in range(BLOCK)) for i in range(BLOCK)]


def quantize_rationals(values, negative=None):
    """(scale byte, codes) of 32 rationals by the block rule.  negative[i] is the code's sign
    bit (default: value < 0; a zero has no sign of its own as a rational)."""
    vals = [Fraction(v) for v in values]
    if negative is None:
        negative = [v < 0 for v in vals]
    X = shared_exponent(vals)
    codes = [nearest_e2m1_magnitude(abs(v) / Fraction(2) ** X) | (8 if neg else 0) for v, neg in zip(vals, negative)]
    return X + 127, codes


# ---- E4M3 (MXFP8 elements): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, exponent
# field 0 subnormal, S.1111.111 NaN, no infinities (OCP 8-bit floating point formats) ----

def e4m3_value(code):
    """Value of the 8-bit E4M3 code, from its bit fields (None for NaN)."""
    sign = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None
    if e == 0:
        mag = Fraction(m, 8) * Fraction(2) ** -6
    else:
        mag = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if sign else mag


def nearest_e4m3_magnitude(a):
    """Code 0..0x7E of the E4M3 magnitude nearest to a >= 0 (search over all codes); on a tie
    the even code wins; past the largest magnitude the nearest is the largest."""
    best = None
    for c in range(0x7F):
        d = abs(a - e4m3_value(c))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def quantize_block_fp8(bits):
    """MXFP8 block: (scale byte, 32 codes); X = floor(log2 amax) - 8 clamped to [-127, 127]."""
    bits = list(bits) + [0] * (BLOCK - len(bits))
    vals = [bf16_value(h) for h in bits]
    if any(v is None for v in vals):
        return 0xFF, [0] * BLOCK
    amax = max(abs(v) for v in vals)
    X = -127 if amax == 0 else min(127, max(-127, floor_log2(amax) - 8))
    codes = [nearest_e4m3_magnitude(abs(v) / Fraction(2) ** X) | (((h >> 15) & 1) << 7) for h, v in zip(bits, vals)]
    return X + 127, codes


def bf16_round_exact(q, negative=None):
    """Bit pattern of the bf16 nearest to the rational q (ties to even mantissa), rounded
    once; magnitudes at or past the midpoint above the largest finite bf16 give infinity.
    `negative` gives the sign of a zero q (a rational has none)."""
    q = Fraction(q)
    sign = 0x8000 if (q < 0 or (q == 0 and negative)) else 0
    a = abs(q)
    if a == 0:
        return sign
    e = floor_log2(a)
    qexp = -133 if e < -126 else e - 7
    unit = Fraction(2) ** qexp
    t = a / unit
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * unit
    if val == 0:
        return sign
    e2 = floor_log2(val)
    if e2 > 127:
        return sign | 0x7F80
    if e2 < -126:
        return sign | n
    m = val / Fraction(2) ** (e2 - 7)
    return sign | ((e2 + 127) << 7) | (int(m) - 128)
