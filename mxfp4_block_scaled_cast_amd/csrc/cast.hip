// BF16 -> MXFP4 cast kernels for gfx950: row copy and row + column copy in one pass.
//
// Operation: jax-aiter README, Supported ops, "MXFP4 Cast" (CastMxfp4JA /
// CastMxfp4DualJA: BF16 to E2M1 elements with E8M0 block scales, with a
// transposed copy).  The per-block rule is the OCP Microscaling conversion:
// X = floor(log2 amax) - 2 clamped to [-127, 127], elements rounded to E2M1
// nearest-even with saturation.
//
// Work decomposition.  A workgroup of 256 threads owns a tile of TILE_R rows
// (64, or 32 for small plain casts: see cast_tile_rows) x 256 columns of x.  Loads are 16 bytes per lane with consecutive lanes on
// consecutive columns (a wave reads 2 rows x 512 contiguous bytes per
// instruction).  Four consecutive lanes hold one 32-element row block; its
// amax is a packed-u16 max in registers followed by two DPP quad exchanges,
// and each lane converts its 8 elements to one dword of codes with the
// hardware scaled conversion (one instruction per element pair).
//
// For the column copy the tile is written to LDS once (row-major, 512 bytes
// per row, conflict-free 16-byte writes) and each thread then walks a
// 32-row x 2-column strip with 4-byte LDS reads (a wave reads 256 contiguous
// bytes per row); v_perm pairs rows 2j and 2j+1 of one column, the pair is
// converted to a byte, and each column's 32 codes leave as one 16-byte store.
//
// Both copies are written in the tiled MX operand layout (16 x 128 code
// tiles, 128 x 256 scale tiles).  The grid is extended to cover the padded
// regions of both copies, so every padding byte is written (codes and scales
// 0: padded positions load as +0).
#include "mx_device.h"

namespace mx {

// Walsh-Hadamard variant (HROW / HCOL: transform the row / column copy).
// jax-aiter README, "Quick start": grad_out is cast with a Hadamard
// transform.  Each 32-element block along the contraction dimension is
// multiplied by the 32-point Sylvester Walsh-Hadamard matrix in binary32,
// by butterflies of half-width 1, 2, 4, 8, 16 in that order, (u, w) ->
// (u + w, u - w); the result divided by 2^hshift is quantized by the usual
// rule (shared exponent from its amax, E2M1 RNE via the fp32 scaled
// conversion).  Row copy: a lane's 8 elements take half-widths 1, 2, 4 in
// registers and 8, 16 across the quad (DPP); column copy: each thread holds
// its two 32-row columns in registers.

// E8M0 byte of a transformed block from the binary32 bits of its amax, with
// the block divided by 2^shift: max(floor(log2 amax) - 2 - shift, -127) + 127;
// 0xFF for Inf/NaN (the byte also covers amax = 0 and binary32 subnormals,
// whose exponent is clamped).
__device__ __forceinline__ unsigned scale_byte_from_f32_amax(unsigned amax_bits, int shift) {
    const int e = (int)(amax_bits >> 23);
    if (e == 255) return 255u;
    if (e == 0) return 0u;
    const int b = e - 2 - shift;
    return b > 0 ? (unsigned)b : 0u;
}

// Two binary32 values -> byte SEL of `old`: RNE(x / scale) to E2M1, saturating, sign kept.
template <int SEL>
__device__ __forceinline__ unsigned cvt_pair_f32(unsigned old, float lo, float hi, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, scale, SEL);
}

__device__ __forceinline__ float bf16_lo(unsigned pair) { return __builtin_bit_cast(float, pair << 16); }
__device__ __forceinline__ float bf16_hi(unsigned pair) { return __builtin_bit_cast(float, pair & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Producers: the values the cast quantizes can be computed in registers from
// the kernel's inputs instead of read from HBM (jax-aiter README, Supported
// ops: SiLU-and-Mul is silu(x[:half]) * x[half:]; RMSNorm fuses square, mean,
// rsqrt and scale; Fused Add+RMSNorm normalizes x + residual).  The produced
// values are the producer's BF16 output -- its exact result rounded once to
// bf16 -- so the fused kernel quantizes exactly what the producer would have
// stored.  PROD_RMS scales rows by a per-row rstd the statistics kernel below
// computed in fp64.
// ---------------------------------------------------------------------------
enum : int { PROD_LOAD = 0, PROD_SILU_MUL = 1, PROD_RMS = 2 };

struct ProdArgs {
    int64_t up_offset;      // SiLU-and-mul: elements from a gate value to its up value
    const uint16_t* gamma;  // RMS: gamma [C]
    const double* rstd;     // RMS: 1 / sqrt(mean(h^2) + eps) per row
    uint16_t* y_out;        // optional: the produced bf16 values [R, C], row stride C
};

// A second tensor converted by the same launch: workgroups from `split` on
// (a multiple of 8, so that workgroup b and its index within its tensor sit on
// the same XCD) take its tiles; the first tensor's grid is padded up to
// `split` with workgroups that return at once.  split = INT_MAX: one tensor.
struct CastSeg {
    const uint16_t* x;
    int64_t R, C, ldx;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int n_rtiles, n_ctiles, split;
};
constexpr CastSeg kOneTensor = {nullptr, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, 0, 0, 0x7FFFFFFF};

// bf16 bits (nearest even) of a double, rounded once: the significand is cut at
// the bf16 grid of the value's binade (2^(e-7), or 2^-133 below 2^-126); past
// the largest finite bf16 the result is infinity; NaN gives the quiet NaN 0x7FC0.
__device__ __forceinline__ unsigned bf16_from_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const unsigned sign = (unsigned)(b >> 48) & 0x8000u;
    const int e = (int)((b >> 52) & 0x7FF);
    const uint64_t mant = b & 0xFFFFFFFFFFFFFull;
    if (e == 0x7FF) return mant ? 0x7FC0u : (sign | 0x7F80u);
    if (e == 0) return sign;  // double subnormals lie far below half the smallest bf16
    const int ue = e - 1023;
    if (ue > 127) return sign | 0x7F80u;
    const uint64_t sig = mant | (1ull << 52);
    const int q = ue >= -126 ? ue - 7 : -133;  // exponent of the bf16 grid spacing
    const int sh = q - ue + 52;                // >= 45
    if (sh > 63) return sign;
    uint64_t n = sig >> sh;
    const uint64_t rem = sig & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (n & 1))) ++n;
    if (ue < -126) return sign | (unsigned)n;  // subnormal (n = 128 is the smallest normal)
    // n in [128, 256]: 256 carries into the exponent field (to infinity from the top binade)
    return sign | ((unsigned)((ue + 127) << 7) + (unsigned)n - 128u);
}

// A binary32 result y known to within a few units of its last place rounds to
// the same bf16 as the exact value unless the low half of its pattern is near
// 0x8000 (a bf16 rounding midpoint within 16 units).  The error bounds below
// hold for normal values far from overflow: 2^-100 <= |y| < 2^101 (exponent
// field 27 .. 227).
__device__ __forceinline__ bool decides(float y) {
    const unsigned b = __builtin_bit_cast(unsigned, y);
    const unsigned ef = (b >> 23) & 0xFFu;
    return ((b & 0xFFFFu) - 0x7FF0u) > 0x20u && (ef - 27u) <= 200u;
}

// bf16(silu(g) * u) in double, rounded once: the rare fallback (out of line,
// so the call sites of a tile do not each carry a copy).
__device__ __attribute__((noinline)) unsigned silu_mul_f64(float g, float u) {
    const double gd = g;
    return bf16_from_f64(gd / (1.0 + exp(-gd)) * (double)u);
}

// Replace half e & 1 of word r[e >> 1] by the bf16 bits b.
__device__ __forceinline__ void put_half(unsigned (&r)[4], int e, unsigned b) {
    r[e >> 1] = (e & 1) ? ((r[e >> 1] & 0xFFFFu) | (b << 16)) : ((r[e >> 1] & 0xFFFF0000u) | b);
}

// bf16(silu(g) * u), rounded once, for 8 gate / 8 up bf16 values, as
// (g * u) / (1 + e^-g).  The product of two bf16 values is exact in binary32
// (and, when the result is normal, not below it).  e^-g = 2^t with t = -g
// log2(e) carried as hi + lo (an fma recovers the product's rounding error),
// e^-g = exp2(hi) (1 + lo ln 2): v_exp_f32 is within an ulp and the
// correction's own error is far below one; v_rcp is within an ulp; with the
// remaining roundings the binary32 result is within 5 units of the exact one.
// It decides unless it is near a midpoint, out of range or g <= -80 (e^-g near
// overflow), and is exact when g * u = 0.  The rest is redone in double.  One
// branch per 8 values keeps the common case straight-line.
__device__ __forceinline__ u32x4 silu_mul8(u32x4 gv, u32x4 uv) {
    const unsigned gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    float g[8], u[8], y[8];
    bool ok[8];
    bool all_ok = true;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        g[e] = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
        u[e] = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
        const float p = g[e] * u[e];
        const float hi = -g[e] * 1.44269502f;  // log2(e) rounded to binary32, and the rest below
        const float lo = __builtin_fmaf(-g[e], 1.92596303e-8f, __builtin_fmaf(-g[e], 1.44269502f, -hi));
        const float e0 = __builtin_amdgcn_exp2f(hi);
        y[e] = p * __builtin_amdgcn_rcpf(1.0f + __builtin_fmaf(e0, lo * 0.693147182f, e0));
        if (p == 0.0f) y[e] = p;  // exact signed zero (the factor may be NaN when e^-g overflows)
        ok[e] = (decides(y[e]) && g[e] > -80.0f) || p == 0.0f;
        all_ok = all_ok && ok[e];
    }
    unsigned r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = f32x2_to_bf16x2_rne(y[2 * k], y[2 * k + 1]);
    if (!all_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!ok[e]) put_half(r, e, silu_mul_f64(g[e], u[e]));
    }
    return u32x4{r[0], r[1], r[2], r[3]};
}

// bf16(h * rstd * gamma), rounded once, for 8 values of a row, as
// (h * gamma) * rstd32: the bf16 product is exact, rstd rounded to binary32
// and one more rounding leave the result within 2 units; it decides unless
// near a midpoint or out of range, and is exact when h * gamma = 0.  The rest
// is redone in double with the double rstd.
__device__ __forceinline__ u32x4 rms8(u32x4 hv, double rs, u32x4 gmv) {
    const float rs32 = (float)rs;
    const unsigned hw[4] = {hv.x, hv.y, hv.z, hv.w}, gw[4] = {gmv.x, gmv.y, gmv.z, gmv.w};
    float h[8], gm[8], y[8];
    bool ok[8];
    bool all_ok = true;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = (e & 1) ? bf16_hi(hw[e >> 1]) : bf16_lo(hw[e >> 1]);
        gm[e] = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
        const float p = h[e] * gm[e];
        y[e] = p * rs32;
        ok[e] = decides(y[e]) || p == 0.0f;
        all_ok = all_ok && ok[e];
    }
    unsigned r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = f32x2_to_bf16x2_rne(y[2 * k], y[2 * k + 1]);
    if (!all_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!ok[e]) put_half(r, e, bf16_from_f64((double)h[e] * rs * (double)gm[e]));
    }
    return u32x4{r[0], r[1], r[2], r[3]};
}

// Half-width H butterflies inside an array of N values (N a multiple of 2H).
template <int H, int N>
__device__ __forceinline__ void butterflies(float (&f)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * H)
#pragma unroll
        for (int j = i; j < i + H; ++j) {
            const float u = f[j], w = f[j + H];
            f[j] = u + w;
            f[j + H] = u - w;
        }
}

// Half-width butterfly across lanes: this lane holds element j (lower) or
// j + H (upper) of every pair; DPP mask MASK reads the partner lane.
template <int MASK>
__device__ __forceinline__ float butterfly_lanes(float own, bool upper) {
    const float other = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, own), MASK,
                                                                               0xF, 0xF, false));
    return upper ? other - own : own + other;
}

// ROWF / COLF: element format of the row / column copy, 4 = MXFP4 (E2M1),
// 8 = MXFP8 (E4M3, one byte per code, X = floor(log2 amax) - 8, saturating
// at 448; the transform is only offered with MXFP4).
// PROD: where the quantized values come from (PROD_LOAD: x itself).
template <int TILE_R, bool DUAL, bool HROW, bool HCOL, int ROWF, int COLF, int PROD = PROD_LOAD>
__global__ __launch_bounds__(256, 4) void cast_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
                                                   uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                   uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                   int n_rtiles, int n_ctiles, int hshift, ProdArgs P,
                                                   CastSeg second) {
    static_assert((ROWF == 4 || ROWF == 8) && (COLF == 4 || COLF == 8), "MXFP4 or MXFP8");
    static_assert(!(HROW && ROWF == 8) && !(HCOL && COLF == 8), "the transform goes with MXFP4 copies");
    static_assert(TILE_R == 32 || TILE_R == 64, "32- or 64-row tiles");
    constexpr int NI = TILE_R / 8;  // 16-byte loads per thread
    const int t = threadIdx.x;
    int bid = blockIdx.x;
    if (bid >= second.split) {  // the second tensor (uniform per workgroup)
        bid -= second.split;
        x = second.x;
        R = second.R;
        C = second.C;
        ldx = second.ldx;
        q_row = second.q_row;
        s_row = second.s_row;
        q_col = second.q_col;
        s_col = second.s_col;
        n_rtiles = second.n_rtiles;
        n_ctiles = second.n_ctiles;
    } else if (bid >= n_rtiles * n_ctiles) {
        return;  // padding between the two tensors' grids
    }
    const int tile = xcd_remap(bid, n_rtiles * n_ctiles);
    const int rt = tile % n_rtiles;
    const int ct = tile / n_rtiles;
    const int64_t r0 = (int64_t)rt * TILE_R;
    const int64_t c0 = (int64_t)ct * 256;

    const int64_t row16 = (R + 15) & ~(int64_t)15;     // code rows of the row copy (padded)
    const int64_t row128 = (R + 127) & ~(int64_t)127;  // scale rows of the row copy (padded)
    const int64_t kt128_row = (C + 127) >> 7;          // 128-wide code tiles of the row copy
    const int64_t kt64_row = (C + 63) >> 6;            // 64-wide (MXFP8) code tiles of the row copy
    const int64_t kt256_row = (C + 255) >> 8;          // 256-wide scale tiles of the row copy
    const int cl = t & 31;                              // 16-byte column chunk within the tile
    const int64_t col = c0 + cl * 8;
    const bool col_ok = col < C;

    // every load is issued before any producer arithmetic or store (the optional
    // y_out stores may alias the inputs as far as the compiler knows); the inputs
    // are read once, with the non-temporal hint (6% faster dual casts in the
    // training step: they no longer displace the operands the GEMMs reuse)
    u32x4 v[NI];
    u32x4 aux[PROD == PROD_SILU_MUL ? NI : 1];  // SiLU-and-mul: the up values
    double rsd[PROD == PROD_RMS ? NI : 1];      // RMS: the rows' rstd
    u32x4 gm = {0u, 0u, 0u, 0u};
    if constexpr (PROD == PROD_RMS)
        if (col_ok) gm = *reinterpret_cast<const u32x4*>(P.gamma + col);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t row = r0 + i * 8 + (t >> 5);
        const bool ok = col_ok && row < R;
        v[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + row * ldx + col))
                  : u32x4{0u, 0u, 0u, 0u};
        if constexpr (PROD == PROD_SILU_MUL)
            aux[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + row * ldx + P.up_offset + col))
                        : u32x4{0u, 0u, 0u, 0u};
        if constexpr (PROD == PROD_RMS) rsd[i] = ok ? P.rstd[row] : 0.0;
    }
    if constexpr (PROD != PROD_LOAD) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t row = r0 + i * 8 + (t >> 5);
            if constexpr (PROD == PROD_SILU_MUL) v[i] = silu_mul8(v[i], aux[i]);
            else v[i] = rms8(v[i], rsd[i], gm);
            // padding rows and columns stay +0 (0 * rstd * gamma could be -0)
            if (!(col_ok && row < R)) v[i] = u32x4{0u, 0u, 0u, 0u};
        }
        if (P.y_out) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int64_t row = r0 + i * 8 + (t >> 5);
                if (col_ok && row < R) *reinterpret_cast<u32x4*>(P.y_out + row * C + col) = v[i];
            }
        }
    }

    // ---- row copy: blocks of 32 along the row
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t row = r0 + i * 8 + (t >> 5);
        if constexpr (ROWF == 8) {
            unsigned m = pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu);
            m = pk_max_u16(m, v[i].z & 0x7FFF7FFFu);
            m = pk_max_u16(m, v[i].w & 0x7FFF7FFFu);
            unsigned amax = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
            amax = quad_max_u32(amax);
            const unsigned sb8 = scale_byte_fp8_from_amax(amax);
            const unsigned lim = e4m3_limit_bf16(sb8);
            uint2 c8 = cvt8_e4m3(v[i], scale_value(sb8), lim | (lim << 16));
            if (sb8 == 255u) c8 = uint2{0u, 0u};
            if (row < row16 && col < kt64_row * 64) {
                *reinterpret_cast<uint2*>(q_row + code8_offset(row, col, kt64_row)) = c8;
            }
            if ((cl & 3) == 0 && row < row128) {
                s_row[scale_offset(row, col >> 5, kt256_row)] = (uint8_t)sb8;
            }
            continue;
        }
        unsigned sb, codes;
        if constexpr (HROW) {
            // this lane holds elements 8q .. 8q+7 of its block, q = lane % 4
            float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                          bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
            butterflies<1>(f);
            butterflies<2>(f);
            butterflies<4>(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = butterfly_lanes<0xB1>(f[e], (t & 1) != 0);  // half-width 8
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = butterfly_lanes<0x4E>(f[e], (t & 2) != 0);  // half-width 16
            unsigned am = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned a = __builtin_bit_cast(unsigned, f[e]) & 0x7FFFFFFFu;
                am = a > am ? a : am;
            }
            sb = scale_byte_from_f32_amax(quad_max_u32(am), hshift);
            const float sc = scale_value(sb + (unsigned)hshift);
            codes = 0u;
            codes = cvt_pair_f32<0>(codes, f[0], f[1], sc);
            codes = cvt_pair_f32<1>(codes, f[2], f[3], sc);
            codes = cvt_pair_f32<2>(codes, f[4], f[5], sc);
            codes = cvt_pair_f32<3>(codes, f[6], f[7], sc);
        } else {
            unsigned m = pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu);
            m = pk_max_u16(m, v[i].z & 0x7FFF7FFFu);
            m = pk_max_u16(m, v[i].w & 0x7FFF7FFFu);
            unsigned amax = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
            amax = quad_max_u32(amax);
            sb = scale_byte_from_amax(amax);
            codes = cvt8(v[i], scale_value(sb));
        }
        if (sb == 255u) codes = 0u;
        if (row < row16 && col < kt128_row * 128) {
            *reinterpret_cast<unsigned*>(q_row + code_offset(row, col, kt128_row)) = codes;
        }
        if ((cl & 3) == 0 && row < row128) {
            s_row[scale_offset(row, col >> 5, kt256_row)] = (uint8_t)sb;
        }
    }

    if constexpr (DUAL) {
        // ---- column copy: blocks of 32 rows down each column
        __shared__ unsigned lds[TILE_R * 128];  // TILE_R rows x 512 bytes
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            *reinterpret_cast<u32x4*>(&lds[(i * 8 + (t >> 5)) * 128 + cl * 4]) = v[i];
        }
        __syncthreads();

        const int64_t Rp = (R + 31) & ~(int64_t)31;  // contraction length of the column copy
        const int64_t kt128_col = (Rp + 127) >> 7;
        const int64_t kt64_col = (Rp + 63) >> 6;
        const int64_t kt256_col = (Rp + 255) >> 8;
        const int64_t col16 = (C + 15) & ~(int64_t)15;
        const int64_t col128 = (C + 127) & ~(int64_t)127;
        constexpr int ITEMS = TILE_R >= 64 ? TILE_R / 64 : 1;  // 32x2 strips per thread
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = it * 256 + t;
            if (TILE_R < 64 && item >= 128) continue;  // a 32-row tile has 128 strips
            const int cp = item & 127;              // column pair within the tile
            const int rb = item >> 7;               // 32-row block within the tile
            const int64_t c = c0 + cp * 2;
            const int64_t rblk = r0 + rb * 32;      // first row of the block
            if (rblk >= kt256_col * 256) continue;  // beyond the padded scale region
            if constexpr (COLF == 8) {
                const unsigned* strip = &lds[rb * 32 * 128 + cp];
                unsigned m = strip[0] & 0x7FFF7FFFu;
#pragma unroll
                for (int r = 1; r < 32; ++r) m = pk_max_u16(m, strip[r * 128] & 0x7FFF7FFFu);
                const unsigned sb0 = scale_byte_fp8_from_amax(m & 0xFFFFu);
                const unsigned sb1 = scale_byte_fp8_from_amax(m >> 16);
                const float f0 = scale_value(sb0), f1 = scale_value(sb1);
                const unsigned l0 = e4m3_limit_bf16(sb0), l1 = e4m3_limit_bf16(sb1);
                const unsigned lim0 = l0 | (l0 << 16), lim1 = l1 | (l1 << 16);
                typedef short s16x2 __attribute__((ext_vector_type(2)));
                unsigned o0[8], o1[8];
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    // rows 4w .. 4w+3: two pairs per column, one dword of four codes
                    const unsigned d0 = strip[(4 * w + 0) * 128], d1 = strip[(4 * w + 1) * 128];
                    const unsigned d2 = strip[(4 * w + 2) * 128], d3 = strip[(4 * w + 3) * 128];
                    s16x2 a0 = {0, 0}, a1 = {0, 0};
                    a0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
                        a0, __builtin_bit_cast(bf16x2, clamp_pair_bf16(__builtin_amdgcn_perm(d1, d0, 0x05040100u), lim0)),
                        f0, false);
                    a0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
                        a0, __builtin_bit_cast(bf16x2, clamp_pair_bf16(__builtin_amdgcn_perm(d3, d2, 0x05040100u), lim0)),
                        f0, true);
                    a1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
                        a1, __builtin_bit_cast(bf16x2, clamp_pair_bf16(__builtin_amdgcn_perm(d1, d0, 0x07060302u), lim1)),
                        f1, false);
                    a1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
                        a1, __builtin_bit_cast(bf16x2, clamp_pair_bf16(__builtin_amdgcn_perm(d3, d2, 0x07060302u), lim1)),
                        f1, true);
                    o0[w] = sb0 == 255u ? 0u : __builtin_bit_cast(unsigned, a0);
                    o1[w] = sb1 == 255u ? 0u : __builtin_bit_cast(unsigned, a1);
                }
                if (c < col16 && rblk < kt64_col * 64) {
                    u32x4* p0 = reinterpret_cast<u32x4*>(q_col + code8_offset(c, rblk, kt64_col));
                    u32x4* p1 = reinterpret_cast<u32x4*>(q_col + code8_offset(c + 1, rblk, kt64_col));
                    p0[0] = u32x4{o0[0], o0[1], o0[2], o0[3]};
                    p0[1] = u32x4{o0[4], o0[5], o0[6], o0[7]};
                    p1[0] = u32x4{o1[0], o1[1], o1[2], o1[3]};
                    p1[1] = u32x4{o1[4], o1[5], o1[6], o1[7]};
                }
                if (c < col128) {
                    s_col[scale_offset(c, rblk >> 5, kt256_col)] = (uint8_t)sb0;
                    s_col[scale_offset(c + 1, rblk >> 5, kt256_col)] = (uint8_t)sb1;
                }
                continue;
            }
            u32x4 o0, o1;
            unsigned sb0, sb1;
            if constexpr (HCOL) {
                // both columns of the strip as 32 binary32 values each, transformed in registers
                float y0[32], y1[32];
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    const unsigned d = lds[(rb * 32 + r) * 128 + cp];
                    y0[r] = bf16_lo(d);
                    y1[r] = bf16_hi(d);
                }
                butterflies<1>(y0), butterflies<1>(y1);
                butterflies<2>(y0), butterflies<2>(y1);
                butterflies<4>(y0), butterflies<4>(y1);
                butterflies<8>(y0), butterflies<8>(y1);
                butterflies<16>(y0), butterflies<16>(y1);
                unsigned m0 = 0u, m1 = 0u;
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    const unsigned a0 = __builtin_bit_cast(unsigned, y0[r]) & 0x7FFFFFFFu;
                    const unsigned a1 = __builtin_bit_cast(unsigned, y1[r]) & 0x7FFFFFFFu;
                    m0 = a0 > m0 ? a0 : m0;
                    m1 = a1 > m1 ? a1 : m1;
                }
                sb0 = scale_byte_from_f32_amax(m0, hshift);
                sb1 = scale_byte_from_f32_amax(m1, hshift);
                const float f0 = scale_value(sb0 + (unsigned)hshift), f1 = scale_value(sb1 + (unsigned)hshift);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    unsigned a0 = 0u, a1 = 0u;
                    a0 = cvt_pair_f32<0>(a0, y0[w * 8 + 0], y0[w * 8 + 1], f0);
                    a0 = cvt_pair_f32<1>(a0, y0[w * 8 + 2], y0[w * 8 + 3], f0);
                    a0 = cvt_pair_f32<2>(a0, y0[w * 8 + 4], y0[w * 8 + 5], f0);
                    a0 = cvt_pair_f32<3>(a0, y0[w * 8 + 6], y0[w * 8 + 7], f0);
                    a1 = cvt_pair_f32<0>(a1, y1[w * 8 + 0], y1[w * 8 + 1], f1);
                    a1 = cvt_pair_f32<1>(a1, y1[w * 8 + 2], y1[w * 8 + 3], f1);
                    a1 = cvt_pair_f32<2>(a1, y1[w * 8 + 4], y1[w * 8 + 5], f1);
                    a1 = cvt_pair_f32<3>(a1, y1[w * 8 + 6], y1[w * 8 + 7], f1);
                    o0[w] = sb0 == 255u ? 0u : a0;
                    o1[w] = sb1 == 255u ? 0u : a1;
                }
            } else {
            unsigned d[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) d[r] = lds[(rb * 32 + r) * 128 + cp];
            unsigned m = d[0] & 0x7FFF7FFFu;
#pragma unroll
            for (int r = 1; r < 32; ++r) m = pk_max_u16(m, d[r] & 0x7FFF7FFFu);
            sb0 = scale_byte_from_amax(m & 0xFFFFu);
            sb1 = scale_byte_from_amax(m >> 16);
            const float f0 = scale_value(sb0), f1 = scale_value(sb1);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                unsigned a0 = 0u, a1 = 0u;
#define MX_COLPAIR(SEL)                                                                  \
    {                                                                                    \
        const unsigned lo = d[w * 8 + 2 * SEL], hi = d[w * 8 + 2 * SEL + 1];            \
        a0 = cvt_pair<SEL>(a0, __builtin_amdgcn_perm(hi, lo, 0x05040100u), f0);         \
        a1 = cvt_pair<SEL>(a1, __builtin_amdgcn_perm(hi, lo, 0x07060302u), f1);         \
    }
                MX_COLPAIR(0) MX_COLPAIR(1) MX_COLPAIR(2) MX_COLPAIR(3)
#undef MX_COLPAIR
                o0[w] = sb0 == 255u ? 0u : a0;
                o1[w] = sb1 == 255u ? 0u : a1;
            }
            }
            if (c < col16 && rblk < kt128_col * 128) {
                *reinterpret_cast<u32x4*>(q_col + code_offset(c, rblk, kt128_col)) = o0;
                *reinterpret_cast<u32x4*>(q_col + code_offset(c + 1, rblk, kt128_col)) = o1;
            }
            if (c < col128) {
                s_col[scale_offset(c, rblk >> 5, kt256_col)] = (uint8_t)sb0;
                s_col[scale_offset(c + 1, rblk >> 5, kt256_col)] = (uint8_t)sb1;
            }
        }
    }
}

}  // namespace mx

namespace mx {

// Rows covered by the grid: the row copy's padded scale rows (a multiple of
// 128), and for the dual cast the column copy's padded contraction (a
// multiple of 256).
static int64_t cast_rows_cover(int64_t R, bool dual) {
    return dual ? ((R + 255) & ~(int64_t)255) : ((R + 127) & ~(int64_t)127);
}

// Tile rows of a plain MXFP4 cast (no transform, no MXFP8 copy) covering
// `tiles64` 64-row tiles in all: a workgroup's tile takes ~9 us of the chip's
// steady stream, and the grid's tail (the last workgroups running with part
// of the chip idle) costs about one tile's time, so casts of few tiles use
// 32-row tiles.  Measured (dual casts, 1 GiB read before each, 64 vs 32 rows,
// us): 2048 x 4096 12.4 -> 11.5, 4096 x 4096 18.2 -> 16.4, 8192 x 4096 28.4 ->
// 27.3, 16384 x 4096 46.4 -> 45.8 (4096 tiles), 4096 x 14336 42.8 -> 42.5;
// larger casts were 0.4-3.7% slower with 32 rows (8192 x 28672 140.9 ->
// 146.1), their column copy then leaving in 16-byte pieces of more lines.
constexpr int64_t kSmallCastTiles = 4096;
static int cast_tile_rows(int64_t tiles64) { return tiles64 <= kSmallCastTiles ? 32 : 64; }

}  // namespace mx

// Launchers (internal, called by the C ABI layer after validation).
// transform_row / transform_col: Walsh-Hadamard on the row / column copy, the
// transformed copies divided by 2^hshift.
extern "C" hipError_t mx_launch_cast_f(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                       void* q_col, void* s_col, bool dual, int row_fmt, int col_fmt, bool transform_row,
                                       bool transform_col, int hshift, hipStream_t stream) {
    const int64_t rows_cover = mx::cast_rows_cover(R, dual);
    const int64_t n_ctiles = (C + 255) / 256;
    const bool plain = row_fmt == 4 && col_fmt == 4 && !transform_row && !transform_col;
    const int tile_r = plain ? mx::cast_tile_rows((rows_cover + 63) / 64 * n_ctiles) : 64;
    const int64_t n_rtiles = (rows_cover + tile_r - 1) / tile_r;
    const int64_t total = n_rtiles * n_ctiles;
    if (total == 0) return hipSuccess;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total), block(256);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t *qr = static_cast<uint8_t*>(q_row), *sr = static_cast<uint8_t*>(s_row);
    uint8_t *qc = static_cast<uint8_t*>(q_col), *scl = static_cast<uint8_t*>(s_col);
    const int nr = (int)n_rtiles, nc = (int)n_ctiles;
    const mx::ProdArgs P{};
#define MX_CAST_T(T, D, HR, HC, RF, CF)                                                                      \
    hipLaunchKernelGGL((mx::cast_kernel<T, D, HR, HC, RF, CF>), grid, block, 0, stream, xb, R, C, ldx, qr, sr,   \
                       D ? qc : nullptr, D ? scl : nullptr, nr, nc, hshift, P, mx::kOneTensor)
#define MX_CAST(D, HR, HC, RF, CF) MX_CAST_T(64, D, HR, HC, RF, CF)
    if (plain && tile_r == 32) {
        if (dual) MX_CAST_T(32, true, false, false, 4, 4);
        else MX_CAST_T(32, false, false, false, 4, 4);
    } else if (row_fmt == 8 || col_fmt == 8) {
        if (transform_row || transform_col) return hipErrorInvalidValue;
        if (!dual) {
            if (row_fmt != 8) return hipErrorInvalidValue;
            MX_CAST(false, false, false, 8, 4);
        } else if (row_fmt == 8) {
            if (col_fmt != 8) return hipErrorInvalidValue;
            MX_CAST(true, false, false, 8, 8);
        } else {
            MX_CAST(true, false, false, 4, 8);
        }
    } else if (!dual) {
        if (transform_row) MX_CAST(false, true, false, 4, 4);
        else MX_CAST(false, false, false, 4, 4);
    } else if (transform_row) {
        if (transform_col) MX_CAST(true, true, true, 4, 4);
        else MX_CAST(true, true, false, 4, 4);
    } else {
        if (transform_col) MX_CAST(true, false, true, 4, 4);
        else MX_CAST(true, false, false, 4, 4);
    }
#undef MX_CAST
#undef MX_CAST_T
    return hipGetLastError();
}

extern "C" hipError_t mx_launch_cast_h(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                       void* q_col, void* s_col, bool dual, bool transform_row, bool transform_col,
                                       int hshift, hipStream_t stream) {
    return mx_launch_cast_f(x, R, C, ldx, q_row, s_row, q_col, s_col, dual, 4, 4, transform_row, transform_col, hshift,
                            stream);
}

extern "C" hipError_t mx_launch_cast(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                     void* q_col, void* s_col, bool dual, hipStream_t stream) {
    return mx_launch_cast_f(x, R, C, ldx, q_row, s_row, q_col, s_col, dual, 4, 4, false, false, 0, stream);
}

namespace mx {

// Row statistics of RMSNorm (and the residual sum of Add+RMSNorm): one wave per
// row, 16-byte loads.  With a residual, h = bf16(x + r): the binary32 sum of two
// bf16 values is exact when their exponents differ by at most 15, and otherwise
// lies too close to the larger one for a bf16 midpoint to fall in between, so
// its nearest-even bf16 is the exactly rounded sum; h is stored (the residual
// output, and the input of the cast pass).  The squares of h (exact in double,
// tiny values included) are accumulated in double, chunk by chunk in column
// order; rstd = 1 / sqrt(ss / D + eps) in double.
//
// h_out may be x or res itself (an in-place residual update), so x, res and
// h_out are not declared __restrict__.  The row is processed in groups of
// kStatChunks 16-byte chunks per lane: all loads of a group are issued before
// any of its stores (several loads in flight per wave), and a store only
// overwrites a chunk that this lane has already read from both inputs.
constexpr int kStatChunks = 8;

__global__ __launch_bounds__(256) void rms_stats_kernel(const uint16_t* x, const uint16_t* res, uint16_t* h_out,
                                                        int64_t R, int64_t D, float eps,
                                                        double* __restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= R) return;
    const uint16_t* xr = x + row * D;
    const uint16_t* rr = res ? res + row * D : nullptr;
    uint16_t* hr = res ? h_out + row * D : nullptr;
    double ss = 0.0;
    for (int64_t c0 = lane * 8; c0 < D; c0 += 512 * kStatChunks) {
        u32x4 h[kStatChunks], r[kStatChunks];
#pragma unroll
        for (int g = 0; g < kStatChunks; ++g) {
            const int64_t c = c0 + g * 512;
            h[g] = c < D ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
            r[g] = (rr && c < D) ? *reinterpret_cast<const u32x4*>(rr + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int g = 0; g < kStatChunks; ++g) {
            const int64_t c = c0 + g * 512;
            if (c >= D) break;
            if (rr) {
#define MX_ADD(F) h[g].F = f32x2_to_bf16x2_rne(bf16_lo(h[g].F) + bf16_lo(r[g].F), bf16_hi(h[g].F) + bf16_hi(r[g].F));
                MX_ADD(x) MX_ADD(y) MX_ADD(z) MX_ADD(w)
#undef MX_ADD
                *reinterpret_cast<u32x4*>(hr + c) = h[g];
            }
#define MX_SQ(F)                                                  \
    {                                                             \
        const double lo = bf16_lo(h[g].F), hi = bf16_hi(h[g].F);  \
        ss = __builtin_fma(lo, lo, ss);                           \
        ss = __builtin_fma(hi, hi, ss);                           \
    }
            MX_SQ(x) MX_SQ(y) MX_SQ(z) MX_SQ(w)
#undef MX_SQ
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) rstd[row] = 1.0 / sqrt(ss / (double)D + (double)eps);
}

// Grid of the cast kernel over x [R, C] (tile_r rows x 256 columns per
// workgroup), covering the padded rows of the copies it writes.
static bool cast_grid(int64_t R, int64_t C, bool dual, int tile_r, int& nr, int& nc) {
    const int64_t rows_cover = cast_rows_cover(R, dual);
    const int64_t n_rtiles = (rows_cover + tile_r - 1) / tile_r, n_ctiles = (C + 255) / 256;
    if (n_rtiles * n_ctiles > 0x7FFFFFFF) return false;
    nr = (int)n_rtiles;
    nc = (int)n_ctiles;
    return true;
}

template <int PROD>
static hipError_t launch_produced_cast(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, void* q_row,
                                       void* s_row, void* q_col, void* s_col, bool dual, int col_fmt,
                                       const ProdArgs& P, hipStream_t stream) {
    int nr = 0, nc = 0;
    if (!cast_grid(R, C, dual, 64, nr, nc)) return hipErrorInvalidValue;
    if ((int64_t)nr * nc == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)nr * nc)), block(256);
    uint8_t *qr = static_cast<uint8_t*>(q_row), *sr = static_cast<uint8_t*>(s_row);
    uint8_t *qc = static_cast<uint8_t*>(q_col), *scl = static_cast<uint8_t*>(s_col);
    if (!dual)
        hipLaunchKernelGGL((cast_kernel<64, false, false, false, 4, 4, PROD>), grid, block, 0, stream, x, R, C, ldx,
                           qr, sr, nullptr, nullptr, nr, nc, 0, P, kOneTensor);
    else if (col_fmt == 8)
        hipLaunchKernelGGL((cast_kernel<64, true, false, false, 4, 8, PROD>), grid, block, 0, stream, x, R, C, ldx, qr,
                           sr, qc, scl, nr, nc, 0, P, kOneTensor);
    else
        hipLaunchKernelGGL((cast_kernel<64, true, false, false, 4, 4, PROD>), grid, block, 0, stream, x, R, C, ldx, qr,
                           sr, qc, scl, nr, nc, 0, P, kOneTensor);
    return hipGetLastError();
}

}  // namespace mx

// SiLU-and-mul + cast: x [R, 2F] (row stride ldx; gate = columns 0..F-1, up =
// F..2F-1) -> MXFP4 row copy (and, dual, the column copy in col_fmt) of
// bf16(silu(gate) * up), optionally also written to y_out [R, F].
extern "C" hipError_t mx_launch_silu_mul_cast(const void* x, int64_t R, int64_t F, int64_t ldx, void* q_row,
                                              void* s_row, void* q_col, void* s_col, bool dual, int col_fmt,
                                              void* y_out, hipStream_t stream) {
    mx::ProdArgs P{};
    P.up_offset = F;
    P.y_out = static_cast<uint16_t*>(y_out);
    return mx::launch_produced_cast<mx::PROD_SILU_MUL>(static_cast<const uint16_t*>(x), R, F, ldx, q_row, s_row,
                                                       q_col, s_col, dual, col_fmt, P, stream);
}

// RMSNorm (+ residual) + cast: the statistics kernel (rstd [R] in double; with a
// residual, h = bf16(x + residual) into h_out), then the cast of
// bf16(h * rstd * gamma) -- h read back from h_out, or x itself without a
// residual -- optionally also written to y_out [R, D].
extern "C" hipError_t mx_launch_rmsnorm_cast(const void* x, const void* residual, const void* gamma, float eps,
                                             int64_t R, int64_t D, void* q_row, void* s_row, void* q_col, void* s_col,
                                             bool dual, int col_fmt, void* h_out, void* rstd, void* y_out,
                                             hipStream_t stream) {
    if (R == 0 || D == 0) return hipSuccess;
    const int64_t blocks = (R + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* rb = static_cast<const uint16_t*>(residual);
    uint16_t* hb = static_cast<uint16_t*>(h_out);
    double* rs = static_cast<double*>(rstd);
    hipLaunchKernelGGL(mx::rms_stats_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, xb, rb, hb, R, D, eps, rs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    mx::ProdArgs P{};
    P.gamma = static_cast<const uint16_t*>(gamma);
    P.rstd = rs;
    P.y_out = static_cast<uint16_t*>(y_out);
    return mx::launch_produced_cast<mx::PROD_RMS>(rb ? hb : xb, R, D, D, q_row, s_row, q_col, s_col, dual, col_fmt, P,
                                                  stream);
}

// Dual casts (MXFP4 row + column copies) of two tensors in one launch: the
// first tensor's workgroups, padded to a multiple of 8, then the second's.
extern "C" hipError_t mx_launch_cast_dual_pair(const void* x0, int64_t R0, int64_t C0, int64_t ldx0, void* q_row0,
                                               void* s_row0, void* q_col0, void* s_col0, const void* x1, int64_t R1,
                                               int64_t C1, int64_t ldx1, void* q_row1, void* s_row1, void* q_col1,
                                               void* s_col1, hipStream_t stream) {
    // one tile size for both tensors, chosen by their 64-row tiles together
    const int64_t tiles64 = (mx::cast_rows_cover(R0, true) + 63) / 64 * ((C0 + 255) / 256) +
                            (mx::cast_rows_cover(R1, true) + 63) / 64 * ((C1 + 255) / 256);
    const int tile_r = mx::cast_tile_rows(tiles64);
    int nr0 = 0, nc0 = 0, nr1 = 0, nc1 = 0;
    if (!mx::cast_grid(R0, C0, true, tile_r, nr0, nc0) || !mx::cast_grid(R1, C1, true, tile_r, nr1, nc1))
        return hipErrorInvalidValue;
    const int64_t t0 = (int64_t)nr0 * nc0, t1 = (int64_t)nr1 * nc1;
    const int64_t split = (t0 + 7) & ~(int64_t)7;
    if (split + t1 > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (t0 + t1 == 0) return hipSuccess;
    const mx::CastSeg second = {static_cast<const uint16_t*>(x1), R1, C1, ldx1,
                                static_cast<uint8_t*>(q_row1), static_cast<uint8_t*>(s_row1),
                                static_cast<uint8_t*>(q_col1), static_cast<uint8_t*>(s_col1), nr1, nc1, (int)split};
    auto kern = tile_r == 32 ? mx::cast_kernel<32, true, false, false, 4, 4> : mx::cast_kernel<64, true, false, false, 4, 4>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(split + t1)), dim3(256), 0, stream, static_cast<const uint16_t*>(x0), R0,
                       C0, ldx0, static_cast<uint8_t*>(q_row0), static_cast<uint8_t*>(s_row0),
                       static_cast<uint8_t*>(q_col0), static_cast<uint8_t*>(s_col0), nr0, nc0, 0, mx::ProdArgs{},
                       second);
    return hipGetLastError();
}
