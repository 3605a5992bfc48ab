"""Pins for the CPU oracle: each check ties the oracle to something other than itself.

* the 16-entry E2M1 table of the OCP Microscaling v1.0 specification
* hand-worked blocks (tests/golden/hand_blocks.txt), derived from the rule
* closed-form block families (single non-zero, amax = 6*2^e, exact midpoints)
* a threshold formulation of round-to-nearest-even on the E2M1 grid, checked
  on every bf16 bit pattern at several block exponents
* invariants (power-of-two scaling, sign symmetry, idempotence, monotonicity,
  error bound)
* exact rational brute force for small GEMMs
* planted mistakes in the Python oracle, each of which must fail a pin
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import scalar
from golden_io import hand_blocks

# OCP Microscaling v1.0, FP4 E2M1 element table (codes 0..7; 8..15 negate).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32_to_bf16_bits(a):
    """bf16 bit patterns of float32 values that are exactly representable in bf16."""
    a = np.asarray(a, np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(h):
    h = np.asarray(h, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return h.view(np.float32).astype(np.float64)


def threshold_code(v):
    """RNE on the E2M1 grid written as comparisons against the midpoints (|v| >= 0)."""
    v = np.abs(np.asarray(v, np.float64))
    c = np.zeros(v.shape, np.int64)
    c += v > 0.25
    c += v >= 0.75
    c += v > 1.25
    c += v >= 1.75
    c += v > 2.5
    c += v >= 3.5
    c += v > 5.0
    return c


# ---------------------------------------------------------------- code table

def test_e2m1_table_scalar():
    for code in range(16):
        expect = E2M1_TABLE[code & 7] * (-1 if code & 8 else 1)
        assert scalar.e2m1_value(code) == Fraction(expect)
        if code & 8:
            assert math.copysign(1.0, float(-0.0 if code == 8 else scalar.e2m1_value(code))) < 0


def test_e2m1_table_c():
    # every code in one row of 32, scale byte 127 (2^0): dequant must give the table
    codes = list(range(16)) * 2
    q = np.array([[codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(16)]], np.uint8)
    s = np.array([[127]], np.uint8)
    d = oracle.dequant(q, s)[0]
    for i, code in enumerate(codes):
        expect = E2M1_TABLE[code & 7] * (-1 if code & 8 else 1)
        assert d[i] == expect
        if code == 8:
            assert math.copysign(1.0, d[i]) < 0


# ---------------------------------------------------------------- hand blocks

HAND = hand_blocks()


def check_hand_blocks(quantize):
    """Names of the hand blocks that `quantize(bits) -> (scale, codes)` gets wrong."""
    bad = []
    for name, bits, scale, codes in HAND:
        s, c = quantize(bits)
        if s != scale or list(c) != codes:
            bad.append(name)
    return bad


def test_hand_blocks_scalar():
    assert check_hand_blocks(scalar.quantize_block) == []


def _c_quantize(bits):
    q, s = oracle.cast_rows(np.array([bits], np.uint16))
    codes = []
    for byte in q[0]:
        codes += [int(byte) & 0xF, int(byte) >> 4]
    return int(s[0, 0]), codes


def test_hand_blocks_c_rows():
    assert check_hand_blocks(_c_quantize) == []


def test_hand_blocks_c_cols():
    # the same blocks laid out down columns must give the same codes in the column copy
    x = np.array([b for _, b, _, _ in HAND], np.uint16).T.copy()  # [32, nblocks]
    q, s = oracle.cast_cols(x)
    for j, (name, _, scale, codes) in enumerate(HAND):
        got = []
        for byte in q[j]:
            got += [int(byte) & 0xF, int(byte) >> 4]
        assert int(s[j, 0]) == scale and got == codes, name


def test_ties_block_packing():
    # packed bytes of the ties block: element 2j in the low nibble of byte j
    bits = dict((n, b) for n, b, _, _ in HAND)["ties_x0"]
    q, s = oracle.cast_rows(np.array([bits], np.uint16))
    assert list(q[0, :5]) == [0x06, 0x22, 0x44, 0x86, 0x0E]
    assert scalar.pack(scalar.quantize_block(bits)[1])[:5] == [0x06, 0x22, 0x44, 0x86, 0x0E]


def test_one_block_gemm_ties_times_ones():
    # ties block dequantizes to 4,0,1,1,2,2,4,-0,-4 -> dot with all-ones is 10 (the bf16 dot is 9.75)
    ties = dict((n, b) for n, b, _, _ in HAND)["ties_x0"]
    ones = [0x3F80] * 32
    qa, sa = oracle.cast_rows(np.array([ties], np.uint16))
    qb, sb = oracle.cast_rows(np.array([ones], np.uint16))
    ref, absref = oracle.gemm(qa, sa, qb, sb)
    assert ref[0, 0] == 10.0 and absref[0, 0] == 18.0
    exact, aexact = scalar.dot_exact(ties, ones)
    assert exact == 10 and aexact == 18


# ---------------------------------------------------------------- closed-form families

def _all_normal_bf16(lo_exp, hi_exp):
    e = np.arange(lo_exp, hi_exp + 1)
    m = np.arange(128)
    E, Mm = np.meshgrid(e, m, indexing="ij")
    return ((E + 127) << 7 | Mm).astype(np.uint16).ravel()


@pytest.mark.parametrize("neg", [False, True])
def test_single_nonzero_family(neg):
    # x = m*2^e, 1 <= m < 2: X = e-2 (byte e+125), v = 4m -> code 6 if 4m <= 5 else 7
    bits = _all_normal_bf16(-125, 127)
    if neg:
        bits = bits | 0x8000
    x = np.zeros((bits.size, 32), np.uint16)
    pos = np.arange(bits.size) % 32
    x[np.arange(bits.size), pos] = bits
    q, s = oracle.cast_rows(x)
    e = ((bits >> 7) & 0xFF).astype(np.int64) - 127
    m = 1 + (bits & 0x7F) / 128.0
    assert np.array_equal(s[:, 0].astype(np.int64), e + 125)
    byte = q[np.arange(bits.size), pos // 2]
    code = np.where(pos % 2 == 0, byte & 0xF, byte >> 4)
    expect = np.where(4 * m <= 5, 6, 7) | (8 if neg else 0)
    assert np.array_equal(code, expect)


def test_amax_six_times_pow2_family():
    # amax = 6*2^e = 1.5*2^(e+2): X = e exactly, v = 6 -> code 7, no clipping
    rows = []
    for e in range(-127, 126):
        h = int(f32_to_bf16_bits(np.float32(6.0 * 2.0 ** e))[()]) if e >= -126 else 0
        if e < -126:
            continue
        rows.append((e, h))
    x = np.zeros((len(rows), 32), np.uint16)
    for i, (_, h) in enumerate(rows):
        x[i, i % 32] = h
    q, s = oracle.cast_rows(x)
    for i, (e, _) in enumerate(rows):
        assert s[i, 0] == e + 127
        byte = q[i, (i % 32) // 2]
        assert ((byte >> (4 * (i % 2))) & 0xF) == 7


@pytest.mark.parametrize("X", [-127, -100, -3, 0, 7, 120])
def test_midpoint_family(X):
    # anchor 4*2^X fixes the exponent; t*2^X at each E2M1 midpoint rounds to the even neighbour
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 2, 4, 4, 6, 6]
    vals = [4.0] + mids + [-t for t in mids]
    # at X = -127 the anchor 2^-125 is normal and the midpoints below 2^-126 are bf16 subnormals
    f = np.array([v * 2.0 ** X for v in vals], np.float64).astype(np.float32)
    x = np.zeros((1, 32), np.uint16)
    x[0, :len(vals)] = f32_to_bf16_bits(f)
    q, s = oracle.cast_rows(x)
    assert s[0, 0] == X + 127
    codes = [(int(q[0, j // 2]) >> (4 * (j % 2))) & 0xF for j in range(32)]
    assert codes[0] == 6
    assert codes[1:8] == expect
    assert codes[8:15] == [c | 8 for c in expect]


# ---------------------------------------------------------------- threshold formulation, every bf16

@pytest.mark.parametrize("X", [-127, -126, -60, -2, 0, 3, 40, 125])
def test_every_bf16_against_threshold_rule(X):
    # block = [anchor 4*2^X, h]; keep every finite h with |h| < 2^(X+3) so the exponent stays X
    anchor = f32_to_bf16_bits(np.float32(4.0 * 2.0 ** X))
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    val = bf16_bits_to_f64(h)
    keep = np.isfinite(val) & (np.abs(val) < 2.0 ** (X + 3))
    h = h[keep]
    x = np.zeros((h.size, 32), np.uint16)
    x[:, 0] = anchor
    x[:, 1] = h
    q, s = oracle.cast_rows(x)
    assert np.all(s[:, 0] == X + 127)
    code = q[:, 0] >> 4
    v = np.abs(bf16_bits_to_f64(h)) / 2.0 ** X  # exact: power-of-two scaling of a double
    expect = threshold_code(v) | ((h >> 15) << 3)
    assert np.array_equal(code.astype(np.int64), expect.astype(np.int64))


def test_scalar_against_threshold_rule_sample():
    rng = np.random.default_rng(11)
    h = rng.integers(0, 65536, 3000).astype(np.uint16)
    val = bf16_bits_to_f64(h)
    h = h[np.isfinite(val)]
    for X in (-127, -5, 0, 9):
        for hv in h[:600]:
            v = abs(scalar.bf16_value(int(hv))) / Fraction(2) ** X
            if v >= 8:
                continue
            t = threshold_code(float(v))[()]
            assert scalar.nearest_e2m1_magnitude(v) == t


# ---------------------------------------------------------------- invariants

def _randn_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = f.view(np.uint32)
    # round to nearest even into bf16
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(1)
    x = _randn_bf16(rng, (64, 256))
    q0, s0 = oracle.cast_rows(x)
    for j in (-20, -1, 1, 5, 30):
        f = bf16_bits_to_f64(x) * 2.0 ** j
        xj = f32_to_bf16_bits(f.astype(np.float32))
        q1, s1 = oracle.cast_rows(xj)
        assert np.array_equal(q0, q1)
        nz = s0 > 0
        assert np.array_equal(s1[nz].astype(int), s0[nz].astype(int) + j)


def test_sign_symmetry():
    rng = np.random.default_rng(2)
    x = _randn_bf16(rng, (64, 256))
    q0, s0 = oracle.cast_rows(x)
    q1, s1 = oracle.cast_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(s0, s1)
    assert np.array_equal(q1, q0 ^ np.uint8(0x88))


def test_idempotence():
    rng = np.random.default_rng(3)
    x = _randn_bf16(rng, (64, 512), 3.0)
    x[0] = 0x0001  # subnormal row
    x[1, :32] = 0
    q, s = oracle.cast_rows(x)
    d = oracle.dequant(q, s)
    x2 = f32_to_bf16_bits(d.astype(np.float32))
    q2, s2 = oracle.cast_rows(x2)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_unclamped_blocks_reach_top_codes():
    rng = np.random.default_rng(4)
    x = _randn_bf16(rng, (128, 512), 10.0)
    q, s = oracle.cast_rows(x)
    mag = np.stack([q & 7, (q >> 4) & 7], -1).reshape(128, -1, 32)
    assert np.all(np.isin(mag.max(-1)[s > 0], [6, 7]))


def test_monotone_and_error_bound():
    rng = np.random.default_rng(5)
    x = _randn_bf16(rng, (32, 1024))
    q, s = oracle.cast_rows(x)
    d = oracle.dequant(q, s).reshape(32, -1, 32)
    xv = bf16_bits_to_f64(x).reshape(32, -1, 32)
    X = s.astype(np.float64)[..., None] - 127
    v = np.abs(xv) / 2.0 ** X
    err = np.abs(np.abs(d) - np.abs(xv)) / 2.0 ** X
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    assert np.all(err[v <= 6] <= half_step[v <= 6])
    assert np.all(err[v > 6] < 2)
    order = np.argsort(np.abs(xv), axis=-1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(np.abs(d), order, -1), axis=-1) >= 0)
    # signs agree wherever the code is non-zero
    nz = d != 0
    assert np.all(np.sign(d[nz]) == np.sign(xv[nz]))


# ---------------------------------------------------------------- non-finite blocks

def test_nonfinite_block():
    x = np.zeros((3, 64), np.uint16)
    x[0, 3] = 0x7F80   # +Inf
    x[1, 40] = 0x7FC1  # NaN
    x[2, 0] = 0x3F80
    x[:, 33] = 0x4000
    q, s = oracle.cast_rows(x)
    assert s[0, 0] == 0xFF and np.all(q[0, :16] == 0) and s[0, 1] == 0x7E
    assert s[1, 1] == 0xFF and np.all(q[1, 16:] == 0) and s[1, 0] == 0x00
    assert s[2, 0] == 0x7D
    assert scalar.quantize_block([0x7F80])[0] == 0xFF


# ---------------------------------------------------------------- GEMM brute force

@pytest.mark.parametrize("K", [32, 96])
def test_gemm_bruteforce_exact(K):
    rng = np.random.default_rng(K)
    a = _randn_bf16(rng, (8, K), 2.0)
    b = _randn_bf16(rng, (8, K), 0.5)
    a[0, :32] = 0  # a zero block
    b[1, 32 % K:] = 0x0005  # subnormal tail
    qa, sa = oracle.cast_rows(a)
    qb, sb = oracle.cast_rows(b)
    ref, absref = oracle.gemm(qa, sa, qb, sb)
    for m in range(8):
        for n in range(8):
            exact, aexact = scalar.dot_exact([int(v) for v in a[m]], [int(v) for v in b[n]])
            assert Fraction(ref[m, n]) == exact
            assert Fraction(absref[m, n]) == aexact


def test_gemm_one_hot():
    # A = e_k rows: out[m, n] = dequant(B)[n, k_m], exactly
    rng = np.random.default_rng(9)
    K = 128
    b = _randn_bf16(rng, (16, K))
    a = np.zeros((8, K), np.uint16)
    ks = rng.integers(0, K, 8)
    a[np.arange(8), ks] = 0x3F80
    qa, sa = oracle.cast_rows(a)
    qb, sb = oracle.cast_rows(b)
    ref, _ = oracle.gemm(qa, sa, qb, sb)
    db = oracle.dequant(qb, sb)
    for m in range(8):
        assert np.array_equal(ref[m], db[:, ks[m]])


def test_gemm_pairs_matches_full():
    rng = np.random.default_rng(10)
    a = _randn_bf16(rng, (20, 160))
    b = _randn_bf16(rng, (24, 160))
    qa, sa = oracle.cast_rows(a)
    qb, sb = oracle.cast_rows(b)
    ref, absref = oracle.gemm(qa, sa, qb, sb)
    mi = rng.integers(0, 20, 50)
    ni = rng.integers(0, 24, 50)
    r2, a2 = oracle.gemm_pairs(qa, sa, qb, sb, mi, ni)
    assert np.array_equal(r2, ref[mi, ni]) and np.array_equal(a2, absref[mi, ni])


def test_column_copy_is_row_copy_of_transpose():
    # the column copy of x equals the row copy of x^T (with rows padded by +0)
    rng = np.random.default_rng(12)
    x = _randn_bf16(rng, (70, 64))
    qc, sc = oracle.cast_cols(x)
    xt = np.zeros((64, 96), np.uint16)
    xt[:, :70] = x.T
    qr, sr = oracle.cast_rows(xt)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


def test_c_matches_scalar_random():
    rng = np.random.default_rng(13)
    x = _randn_bf16(rng, (6, 128), 30.0)
    x[2, 5] = 0x0003
    x[3] = 0x8000
    q, s = oracle.cast_rows(x)
    for r in range(6):
        ss, qq = scalar.quantize_row([int(v) for v in x[r]])
        assert list(s[r]) == ss and list(q[r]) == qq


# ---------------------------------------------------------------- planted mistakes

def _mutants():
    def ties_away(a):
        best = None
        for c in range(8):
            d = abs(a - scalar.e2m1_value(c))
            if best is None or d < best[0] or (d == best[0] and c > best[1]):
                best = (d, c)
        return best[1]

    def ties_down(a):
        best = None
        for c in range(8):
            d = abs(a - scalar.e2m1_value(c))
            if best is None or d < best[0]:
                best = (d, c)
        return best[1]

    def exp_minus_one(values):
        amax = max(abs(v) for v in values)
        return -127 if amax == 0 else min(127, max(-127, scalar.floor_log2(amax) - 1))

    def no_clamp(values):
        amax = max(abs(v) for v in values)
        return -127 if amax == 0 else scalar.floor_log2(amax) - 2

    def zero_block_max(values):
        amax = max(abs(v) for v in values)
        return 127 if amax == 0 else min(127, max(-127, scalar.floor_log2(amax) - 2))

    return {
        "ties_away": ("nearest_e2m1_magnitude", ties_away),
        "ties_down": ("nearest_e2m1_magnitude", ties_down),
        "exp_minus_one": ("shared_exponent", exp_minus_one),
        "no_clamp": ("shared_exponent", no_clamp),
        "zero_block_max": ("shared_exponent", zero_block_max),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(scalar, attr, fn)
    assert check_hand_blocks(scalar.quantize_block) != []


def test_planted_sign_loss_is_caught(monkeypatch):
    orig = scalar.quantize_block

    def unsigned_zero(bits):
        s, c = orig(bits)
        return s, [0 if (v & 7) == 0 else v for v in c]

    assert check_hand_blocks(unsigned_zero) != []


def test_planted_nibble_swap_is_caught():
    bits = dict((n, b) for n, b, _, _ in HAND)["ties_x0"]
    codes = scalar.quantize_block(bits)[1]
    swapped = [codes[2 * j + 1] | (codes[2 * j] << 4) for j in range(16)]
    assert swapped[:5] != [0x06, 0x22, 0x44, 0x86, 0x0E]


def test_planted_gemm_scale_offset_is_caught():
    # a GEMM that forgets the -2 in 2^(Xa+Xb-2) (i.e. uses 2*e2m1 products) is 4x off
    ties = dict((n, b) for n, b, _, _ in HAND)["ties_x0"]
    exact, _ = scalar.dot_exact(ties, [0x3F80] * 32)
    assert exact * 4 != 10 and exact == 10
