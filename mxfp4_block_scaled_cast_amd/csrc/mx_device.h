// Internal device helpers shared by the HIP kernels of this library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 32;  // elements per scale block (along the contraction dim)

// MX operand layout (rows R, contraction length K; see include/mxfp4.h).
//
// Codes: 1 KB tiles of 16 rows x 128 elements (64 bytes per row), stored
// tile-row-major: tile (r/16, k/128) at ((r/16) * KT + k/128) * 1024 with
// KT = ceil(K/128); inside a tile, row r%16 owns 64 bytes, element k%128 sits
// in byte (k%128)/2, even elements in the low nibble.  One tile is exactly
// what one 16-byte-per-lane wave load moves, so a GEMM load touches one
// contiguous kilobyte (one page) instead of 16 rows of a row-major matrix.
__device__ __forceinline__ int64_t code_offset(int64_t r, int64_t k, int64_t kt128) {
    return ((r >> 4) * kt128 + (k >> 7)) * 1024 + (r & 15) * 64 + ((k & 127) >> 1);
}

// MXFP8 codes (one byte per element): 1 KB tiles of 16 rows x 64 elements,
// tile (r/16, k/64) at ((r/16) * KT8 + k/64) * 1024 with KT8 = ceil(K/64);
// row r%16 owns 64 bytes, element k%64 is byte k%64.  Same tile geometry in
// bytes as the FP4 codes, so the GEMM moves either with the same loads.
__device__ __forceinline__ int64_t code8_offset(int64_t r, int64_t k, int64_t kt64) {
    return ((r >> 4) * kt64 + (k >> 6)) * 1024 + (r & 15) * 64 + (k & 63);
}

// Scales: 1 KB tiles of 128 rows x 256 elements (8 blocks of 32), tile
// (r/128, b/8) at ((r/128) * KT2 + b/8) * 1024 with KT2 = ceil(K/256); inside
// a tile, 32-row group (r/32)%4 owns 256 bytes, row r%32 owns 8 of them, and
// block b%8 sits at byte (b%2)*4 + (b%8)/2 -- so the dword a 32x32x64 MFMA
// lane reads (row r, half h = b%2) holds blocks h, h+2, h+4, h+6, the scales
// of four consecutive 64-wide K steps.
__device__ __forceinline__ int64_t scale_offset(int64_t r, int64_t b, int64_t kt256) {
    return ((r >> 7) * kt256 + (b >> 3)) * 1024 + ((r >> 5) & 3) * 256 + (r & 31) * 8 + (b & 1) * 4 + ((b & 7) >> 1);
}

// E8M0 scale byte of a block from the bf16 magnitude bits of its amax
// (amax_bits = max over the block of (bits & 0x7fff); integer order of
// non-negative bf16 patterns is value order, with Inf/NaN on top).
// floor(log2 amax) is the unbiased exponent field for normal amax; a
// subnormal or zero amax is below 2^-126, where X = floor(log2) - 2 is
// clamped to -127 anyway.  So the byte is max(E - 2, 0), or 0xFF when the
// block holds Inf/NaN (E = 255).
__device__ __forceinline__ unsigned scale_byte_from_amax(unsigned amax_bits) {
    unsigned e = amax_bits >> 7;
    if (e == 255u) return 255u;
    return e >= 2u ? e - 2u : 0u;
}

// 2^X as an fp32 value for the scaled down-conversion (X = byte - 127);
// byte 0 is 2^-127, an fp32 subnormal.
__device__ __forceinline__ float scale_value(unsigned sbyte) {
    return __builtin_bit_cast(float, sbyte ? (sbyte << 23) : 0x00400000u);
}

// Two bf16 (low half = even element) -> one byte of two E2M1 codes in byte
// `sel` of `old`: round(x / scale) to nearest-even with saturation, sign
// kept (hardware conversion, matches the quantization rule bit for bit).
template <int SEL>
__device__ __forceinline__ unsigned cvt_pair(unsigned old, unsigned pair, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, pair), scale, SEL);
}

// Eight bf16 (4 dwords) -> 8 codes (one dword).
__device__ __forceinline__ unsigned cvt8(u32x4 v, float scale) {
    unsigned r = 0u;
    r = cvt_pair<0>(r, v.x, scale);
    r = cvt_pair<1>(r, v.y, scale);
    r = cvt_pair<2>(r, v.z, scale);
    r = cvt_pair<3>(r, v.w, scale);
    return r;
}

// A 32x32x64 FP4 MFMA operand from the lane's 16 bytes (32 codes): FP4
// operands occupy the low four registers of the 8-register operand; the rest
// is ignored.
__device__ __forceinline__ v8i as_operand(u32x4 v) {
    v8i r;
    r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// A 32x32x64 FP8 MFMA operand (8 registers) from two 16-byte pieces: lane half h
// supplies K elements 16h .. 16h+15 of the step in registers 0-3 (`lo`) and
// 32+16h .. 47+16h in registers 4-7 (`hi`).
__device__ __forceinline__ v8i as_operand8(u32x4 lo, u32x4 hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// Per-half max of two packed u16 pairs.
__device__ __forceinline__ unsigned pk_max_u16(unsigned a, unsigned b) {
    u16x2 x = __builtin_bit_cast(u16x2, a);
    u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(unsigned, __builtin_elementwise_max(x, y));
}

// Per-half min of two packed u16 pairs.
__device__ __forceinline__ unsigned pk_min_u16(unsigned a, unsigned b) {
    u16x2 x = __builtin_bit_cast(u16x2, a);
    u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(unsigned, __builtin_elementwise_min(x, y));
}

// Max over the 4 lanes of a quad (DPP quad permutations).
__device__ __forceinline__ unsigned quad_max_u32(unsigned v) {
    unsigned o = (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    v = v > o ? v : o;
    o = (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    return v > o ? v : o;
}

// MXFP8 (E4M3) scale byte: X = floor(log2 amax) - 8 clamped to [-127, 127],
// i.e. max(E - 8, 0) for the amax's bf16 exponent field E; 0xFF for Inf/NaN.
__device__ __forceinline__ unsigned scale_byte_fp8_from_amax(unsigned amax_bits) {
    unsigned e = amax_bits >> 7;
    if (e == 255u) return 255u;
    return e >= 8u ? e - 8u : 0u;
}

// bf16 bits of 448 * 2^X for scale byte X + 127 (448 = 1.75 * 2^8, E4M3's largest
// magnitude): exponent field byte + 8, mantissa 0.75.
__device__ __forceinline__ unsigned e4m3_limit_bf16(unsigned sbyte) { return ((sbyte + 8u) << 7) | 0x60u; }

// Two bf16 (one dword) with magnitudes clamped to `lim2` (the limit in both
// halves), sign kept: the saturating half of the E4M3 conversion.
__device__ __forceinline__ unsigned clamp_pair_bf16(unsigned pair, unsigned lim2) {
    return pk_min_u16(pair & 0x7FFF7FFFu, lim2) | (pair & 0x80008000u);
}

// Four bf16 pairs -> 8 E4M3 codes (two dwords), each x / scale rounded to the
// nearest E4M3 value after the magnitude clamp (so values past 448 saturate).
__device__ __forceinline__ uint2 cvt8_e4m3(u32x4 v, float scale, unsigned lim2) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    s16x2 lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2, clamp_pair_bf16(v.x, lim2)), scale,
                                                    false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2, clamp_pair_bf16(v.y, lim2)), scale,
                                                    true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2, clamp_pair_bf16(v.z, lim2)), scale,
                                                    false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2, clamp_pair_bf16(v.w, lim2)), scale,
                                                    true);
    return uint2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Map a hardware workgroup id to a logical tile id so that each of the 8
// XCDs (which receive workgroups round-robin) works on one contiguous range
// of logical tiles.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    int xcd = bid & 7;
    int idx = bid >> 3;
    int per = total >> 3;
    int rem = total & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}

// Two fp32 -> two bf16 in one dword (lo in the low half), same rounding, one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned f32x2_to_bf16x2_rne(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

}  // namespace mx
