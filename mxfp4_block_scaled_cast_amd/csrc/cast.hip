// BF16 -> MXFP4 cast kernels for gfx950: row copy and row + column copy in one pass.
//
// Operation: jax-aiter README, Supported ops, "MXFP4 Cast" (CastMxfp4JA /
// CastMxfp4DualJA: BF16 to E2M1 elements with E8M0 block scales, with a
// transposed copy).  The per-block rule is the OCP Microscaling conversion:
// X = floor(log2 amax) - 2 clamped to [-127, 127], elements rounded to E2M1
// nearest-even with saturation.
//
// Work decomposition.  A workgroup of 256 threads owns a tile of TILE_R rows
// x 256 columns of x.  Loads are 16 bytes per lane with consecutive lanes on
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

template <int TILE_R, bool DUAL>
__global__ __launch_bounds__(256, 4) void cast_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
                                                   uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                   uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                   int n_rtiles, int n_ctiles) {
    constexpr int NI = TILE_R / 8;  // 16-byte loads per thread
    const int t = threadIdx.x;
    const int tile = xcd_remap(blockIdx.x, n_rtiles * n_ctiles);
    const int rt = tile % n_rtiles;
    const int ct = tile / n_rtiles;
    const int64_t r0 = (int64_t)rt * TILE_R;
    const int64_t c0 = (int64_t)ct * 256;

    const int64_t row16 = (R + 15) & ~(int64_t)15;     // code rows of the row copy (padded)
    const int64_t row128 = (R + 127) & ~(int64_t)127;  // scale rows of the row copy (padded)
    const int64_t kt128_row = (C + 127) >> 7;          // 128-wide code tiles of the row copy
    const int64_t kt256_row = (C + 255) >> 8;          // 256-wide scale tiles of the row copy
    const int cl = t & 31;                              // 16-byte column chunk within the tile
    const int64_t col = c0 + cl * 8;
    const bool col_ok = col < C;

    u32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t row = r0 + i * 8 + (t >> 5);
        if (col_ok && row < R) {
            v[i] = *reinterpret_cast<const u32x4*>(x + row * ldx + col);
        } else {
            v[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // ---- row copy: blocks of 32 along the row
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int64_t row = r0 + i * 8 + (t >> 5);
        unsigned m = pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu);
        m = pk_max_u16(m, v[i].z & 0x7FFF7FFFu);
        m = pk_max_u16(m, v[i].w & 0x7FFF7FFFu);
        unsigned amax = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
        amax = quad_max_u32(amax);
        const unsigned sb = scale_byte_from_amax(amax);
        unsigned codes = cvt8(v[i], scale_value(sb));
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
        const int64_t kt256_col = (Rp + 255) >> 8;
        const int64_t col16 = (C + 15) & ~(int64_t)15;
        const int64_t col128 = (C + 127) & ~(int64_t)127;
        constexpr int ITEMS = TILE_R / 64;          // 32x2 strips per thread
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = it * 256 + t;
            const int cp = item & 127;              // column pair within the tile
            const int rb = item >> 7;               // 32-row block within the tile
            const int64_t c = c0 + cp * 2;
            const int64_t rblk = r0 + rb * 32;      // first row of the block
            if (rblk >= kt256_col * 256) continue;  // beyond the padded scale region
            unsigned d[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) d[r] = lds[(rb * 32 + r) * 128 + cp];
            unsigned m = d[0] & 0x7FFF7FFFu;
#pragma unroll
            for (int r = 1; r < 32; ++r) m = pk_max_u16(m, d[r] & 0x7FFF7FFFu);
            const unsigned sb0 = scale_byte_from_amax(m & 0xFFFFu);
            const unsigned sb1 = scale_byte_from_amax(m >> 16);
            const float f0 = scale_value(sb0), f1 = scale_value(sb1);
            u32x4 o0, o1;
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

// Launchers (internal, called by the C ABI layer after validation).
extern "C" hipError_t mx_launch_cast(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                     void* q_col, void* s_col, bool dual, hipStream_t stream) {
    constexpr int TILE_R = 64;
    // rows covered: the row copy's padded scale rows (a multiple of 128), and for
    // the dual cast the column copy's padded contraction (a multiple of 256)
    const int64_t rows_cover = dual ? ((R + 255) & ~(int64_t)255) : ((R + 127) & ~(int64_t)127);
    const int64_t n_rtiles = (rows_cover + TILE_R - 1) / TILE_R;
    const int64_t n_ctiles = (C + 255) / 256;
    const int64_t total = n_rtiles * n_ctiles;
    if (total == 0) return hipSuccess;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total), block(256);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (dual) {
        hipLaunchKernelGGL((mx::cast_kernel<TILE_R, true>), grid, block, 0, stream, xb, R, C, ldx,
                           static_cast<uint8_t*>(q_row), static_cast<uint8_t*>(s_row), static_cast<uint8_t*>(q_col),
                           static_cast<uint8_t*>(s_col), (int)n_rtiles, (int)n_ctiles);
    } else {
        hipLaunchKernelGGL((mx::cast_kernel<TILE_R, false>), grid, block, 0, stream, xb, R, C, ldx,
                           static_cast<uint8_t*>(q_row), static_cast<uint8_t*>(s_row), nullptr, nullptr,
                           (int)n_rtiles, (int)n_ctiles);
    }
    return hipGetLastError();
}
