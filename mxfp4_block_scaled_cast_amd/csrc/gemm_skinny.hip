// MXFP4 / MXFP8 GEMMs for gfx950 whose output is too small to fill the chip with 256 x 256
// tiles: out[M, N] = bf16( A[M, K] . B[N, K]^T ) by the skinny kernel (operands straight from
// memory, the contraction split over the waves of a workgroup) or, for MXFP4 outputs with both
// sides of 128 rows or more, the panel kernel (128 x 128 blocks sharing operand panels through
// LDS); both split a long contraction over several workgroups when given a workspace.
//
// Operation: jax-aiter README, Supported ops, "FP4 GEMM (low-level)" in the A[M,K] @ B[N,K]^T
// convention of its GEMM rows; the same products as the tiled kernels of gemm.hip, for the small
// and ragged shapes of the path (an LM head's M = 1 or 17 rows, K = 32, N = 128256).
#include <algorithm>
#include <type_traits>

#include "mx_device.h"
#include "mx_host.h"

namespace mx {

// ---------------------------------------------------------------------------
// Skinny kernel, for outputs too small to fill the chip with 256 x 256 tiles
// (one side below 128, or few tiles) and for long contractions behind a small
// output (e.g. dA of an LM head: 1 x 4096 outputs, contraction 128256).
//
// C[i, j] = sum_k A[i, k] B[j, k], written to out[i * ld_i + j * ld_j]; the
// launcher passes the smaller operand as A (and swaps the output strides when
// that is the GEMM's B).  A wave owns 32*MA rows of A x 32*NB rows of B (MA x
// NB scaled MFMAs per 64-wide K step; each A fragment serves NB of them, each
// B fragment MA) over one slice of the contraction; the W waves of a
// workgroup take consecutive slices of the same output block and add their
// partial sums through LDS.  Operands come straight from global memory in
// 256-wide K chunks: per lane four 16-byte code loads per 32-row group (one
// per K step; 32 rows x 256 K = four whole 1 KB code tiles) and one scale
// dword, whose four bytes are the lane's scales for the four steps (the MFMA
// picks one with opsel).  All of a chunk's loads are issued before its MFMAs;
// the other waves of the CU cover the latency.  Rows past the operands and K
// steps past the padded code tiles are not loaded (zero).
//
// Split contraction: with a workspace, S workgroups per output block take
// consecutive parts of the contraction (S * W slices in all) and write their
// fp32 partial blocks to the workspace; skinny_reduce_kernel then adds the S
// partials of each output in split order and stores the bf16 result.  This
// keeps the whole chip streaming when the output has few blocks (dA of an LM
// head: contraction 128256 behind 32 or 544 outputs).
// ---------------------------------------------------------------------------

// A single 32 x 32 block per wave runs up to 16 waves per workgroup (at most
// 128 VGPRs), wider blocks up to 8.
template <int MA, int NB>
constexpr int skinny_max_waves() { return MA * NB == 1 ? 16 : 8; }

template <int MA, int NB, int FMT>
__global__ __launch_bounds__((64 * skinny_max_waves<MA, NB>())) void gemm_skinny_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bq,
    const uint8_t* __restrict__ bs, int Ma, int Nb, int K, uint16_t* __restrict__ out, int64_t ld_i, int64_t ld_j,
    int tiles_b, int tiles, float* __restrict__ part) {
    extern __shared__ float red[];  // [W][MA][NB][16][64] partial sums (W > 1)
    constexpr int ELEMS = MA * NB * 16 * 64;  // accumulators of a block (per workgroup)
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int W = blockDim.x >> 6;
    const int half = lane >> 5;
    // workgroup = split * tiles + output block; S = 1 without a workspace (part == nullptr)
    const int tile = (int)(blockIdx.x % (unsigned)tiles);
    const int split = (int)(blockIdx.x / (unsigned)tiles);
    const int S = (int)(gridDim.x / (unsigned)tiles);
    const int i0 = (tile / tiles_b) * (32 * MA);
    const int j0 = (tile % tiles_b) * (32 * NB);
    const int64_t kt128 = (K + 127) >> 7, kt64 = (K + 63) >> 6, kt256 = (K + 255) >> 8;
    const int64_t k_pad = FMT == 8 ? kt64 * 64 : kt128 * 128;  // K padded to whole code tiles

    int ia[MA];
    bool a_ok[MA];
#pragma unroll
    for (int ma = 0; ma < MA; ++ma) {
        ia[ma] = i0 + ma * 32 + (lane & 31);
        a_ok[ma] = ia[ma] < Ma;
    }
    int jb[NB];
    bool b_ok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        jb[nb] = j0 + nb * 32 + (lane & 31);
        b_ok[nb] = jb[nb] < Nb;
    }

    // this wave's slice of the 256-wide chunks: slice split * W + (w + tile) % W of S * W.  Every
    // output block reads the small operand's rows; rotating the slices by the block index makes
    // concurrent workgroups read W different parts of them at a time rather than all the same
    // lines at once
    const int chunks = (int)kt256;
    const int64_t slice = (int64_t)split * W + (w + tile) % W, slices = (int64_t)S * W;
    const int c_begin = (int)(chunks * slice / slices), c_end = (int)(chunks * (slice + 1) / slices);

    f32x16 acc[MA][NB];
#pragma unroll
    for (int ma = 0; ma < MA; ++ma)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[ma][nb] = f32x16{};

    // lane fragment of (row, 64-wide step at k0): FP4, the 16 bytes of K k0+32h .. +31 (widened
    // to the MFMA's 8-register operand at use); FP8, K k0+16h .. +15 and k0+32+16h .. +15
    typedef typename std::conditional<FMT == 8, v8i, u32x4>::type Frag;
    auto load = [&](const uint8_t* q, int64_t row, int64_t k0, bool ok) {
        if constexpr (FMT == 8) {
            if (!ok) return v8i{};
            const uint8_t* p = q + code8_offset(row, k0 + half * 16, kt64);
            return as_operand8(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 32));
        } else {
            if (!ok) return u32x4{0u, 0u, 0u, 0u};
            return *reinterpret_cast<const u32x4*>(q + code_offset(row, k0 + half * 32, kt128));
        }
    };
    auto operand = [](const Frag& f) {
        if constexpr (FMT == 8) return f;
        else return as_operand(f);
    };
    constexpr int CODE = FMT == 8 ? 0 : 4;

    // one 256-wide chunk: the lane's fragments of its four K steps and the scale dwords
    struct Chunk {
        Frag av[MA][4], bv[NB][4];
        unsigned sa[MA], sb[NB];
    };
    auto load_chunk = [&](int c, Chunk& X) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int64_t k0 = (int64_t)c * 256 + st * 64;
            const bool k_ok = k0 < k_pad;
#pragma unroll
            for (int ma = 0; ma < MA; ++ma) X.av[ma][st] = load(aq, ia[ma], k0, a_ok[ma] && k_ok);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) X.bv[nb][st] = load(bq, jb[nb], k0, b_ok[nb] && k_ok);
        }
        // scale dword of (row, half): blocks c*8 + half + 2*st, st = 0..3
#pragma unroll
        for (int ma = 0; ma < MA; ++ma)
            X.sa[ma] = a_ok[ma] ? *reinterpret_cast<const unsigned*>(as + scale_offset(ia[ma], (int64_t)c * 8 + half,
                                                                                          kt256))
                                : 0u;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            X.sb[nb] = b_ok[nb] ? *reinterpret_cast<const unsigned*>(bs + scale_offset(jb[nb], (int64_t)c * 8 + half,
                                                                                          kt256))
                                : 0u;
    };
    auto mfma_chunk = [&](const Chunk& X) {
#define MX_SKINNY_STEP(ST)                                                                                            \
    _Pragma("unroll") for (int ma = 0; ma < MA; ++ma) _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)              \
        acc[ma][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(operand(X.av[ma][ST]), operand(X.bv[nb][ST]),   \
                                                                      acc[ma][nb], CODE, CODE, ST, (int)X.sa[ma], ST, \
                                                                      (int)X.sb[nb]);
        MX_SKINNY_STEP(0) MX_SKINNY_STEP(1) MX_SKINNY_STEP(2) MX_SKINNY_STEP(3)
#undef MX_SKINNY_STEP
    };
    if constexpr (MA * NB == 1 && FMT == 4) {
        // a single FP4 block per wave has the registers for two chunks: the next chunk's loads
        // are issued before the current chunk's MFMAs, so each wave keeps two chunks in flight
        Chunk X0, X1;
        if (c_begin < c_end) load_chunk(c_begin, X0);
        for (int c = c_begin; c < c_end; c += 2) {
            if (c + 1 < c_end) load_chunk(c + 1, X1);
            mfma_chunk(X0);
            if (c + 1 >= c_end) break;
            if (c + 2 < c_end) load_chunk(c + 2, X0);
            mfma_chunk(X1);
        }
    } else {
        for (int c = c_begin; c < c_end; ++c) {
            Chunk X;
            load_chunk(c, X);
            mfma_chunk(X);
        }
    }

    // acc[ma][nb][r] is C[i0 + ma*32 + (r/4)*8 + half*4 + r%4, j0 + nb*32 + lane%32]; in a
    // partial block, element ((ma*NB + nb)*16 + r)*64 + lane
    float* pblk = part ? part + ((int64_t)split * tiles + tile) * ELEMS : nullptr;
    if (W == 1 && pblk) {
#pragma unroll
        for (int ma = 0; ma < MA; ++ma)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) pblk[((ma * NB + nb) * 16 + r) * 64 + lane] = acc[ma][nb][r];
        return;
    }
    if (W == 1) {
#pragma unroll
        for (int ma = 0; ma < MA; ++ma)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (!b_ok[nb]) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = i0 + ma * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                    if (i < Ma) out[(int64_t)i * ld_i + (int64_t)jb[nb] * ld_j] = f32_to_bf16_rne(acc[ma][nb][r]);
                }
            }
        return;
    }
#pragma unroll
    for (int ma = 0; ma < MA; ++ma)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(((w * MA + ma) * NB + nb) * 16 + r) * 64 + lane] = acc[ma][nb][r];
    __syncthreads();
    for (int e = threadIdx.x; e < ELEMS; e += blockDim.x) {
        float v = 0.f;
        for (int ww = 0; ww < W; ++ww) v += red[ww * ELEMS + e];
        if (pblk) {
            pblk[e] = v;
            continue;
        }
        const int l = e & 63, r = (e >> 6) & 15, blk = e >> 10;
        const int ma = blk / NB, nb = blk % NB;
        const int i = i0 + ma * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        const int j = j0 + nb * 32 + (l & 31);
        if (i < Ma && j < Nb) out[(int64_t)i * ld_i + (int64_t)j * ld_j] = f32_to_bf16_rne(v);
    }
}

// Sum of the S partial blocks of each output (split order), rounded to bf16:
// one thread per accumulator of every block.
template <int MA, int NB>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ part, int tiles, int S,
                                                            int tiles_b, int Ma, int Nb, uint16_t* __restrict__ out,
                                                            int64_t ld_i, int64_t ld_j) {
    constexpr int ELEMS = MA * NB * 16 * 64;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)tiles * ELEMS) return;
    const int tile = (int)(idx / ELEMS), e = (int)(idx % ELEMS);
    // eight partials loaded at a time, added in split order
    const float* p = part + (int64_t)tile * ELEMS + e;
    const int64_t stride = (int64_t)tiles * ELEMS;
    float v = 0.f;
    int sp = 0;
    for (; sp + 8 <= S; sp += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = p[(sp + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += t[u];
    }
    for (; sp < S; ++sp) v += p[sp * stride];
    const int l = e & 63, r = (e >> 6) & 15, blk = e >> 10;
    const int ma = blk / NB, nb = blk % NB;
    const int i = (tile / tiles_b) * (32 * MA) + ma * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
    const int j = (tile % tiles_b) * (32 * NB) + nb * 32 + (l & 31);
    if (i < Ma && j < Nb) out[(int64_t)i * ld_i + (int64_t)j * ld_j] = f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// Panel kernel, for skinny-regime outputs whose smaller side has 128 rows or
// more (e.g. 16384 x 128 outputs over a contraction of 14336, or 2048 x 2048):
// a workgroup owns a 128 x 128 output block and its 4 waves (2 x 2, each 64 x
// 64 = 2 x 2 MFMA tiles) share the block's operand panels through LDS, so an
// operand byte crosses L2 -> CU once per workgroup rather than once per wave
// as in the skinny kernel.  Per 256-wide chunk of the contraction the
// workgroup moves 34 KB: 16 code tiles of A and 16 of B (one 1 KB tile per
// wave load instruction, lane l taking its bytes 16l .. 16l+15) and the A and
// B scale tiles that cover the chunk.  Chunks are staged in registers two
// ahead (the loads of chunk c+2 are in flight while chunk c's MFMAs run) and
// double-buffered in LDS, one barrier per chunk.  An LDS row holds a row's
// 256 codes (128 bytes) as eight 16-byte pieces, piece p at slot p ^ f(r)
// with f(r) = 4 (r % 2) + (r / 2) % 4: the fragment reads (8 consecutive
// rows at one piece per lane group) and the tile stores (2 rows x 4 pieces)
// each hit 8 distinct slots.  With a workspace, S workgroups split each
// block's contraction as in the skinny kernel; each wave writes its 64 x 64
// partial block in the 2 x 2 skinny layout (virtual block (2 ta + wa) of
// vt_a x (2 tb + wb) of vt_b) and skinny_reduce_kernel<2, 2> adds them.
// ---------------------------------------------------------------------------
constexpr unsigned kRsrcFlags = 0x00020000u;             // gfx9 raw buffer: dword format, no swizzle
constexpr int kPanelRows = 128;                            // rows of A and of B per block
constexpr int kPanelCodes = kPanelRows * 128;              // 16 KB of codes per operand and chunk
constexpr int kPanelStage = 2 * kPanelCodes + 2 * 1024;    // + the two scale tiles: 34 KB

__device__ __forceinline__ int panel_slot(int row) { return ((row & 1) << 2) | ((row >> 1) & 3); }

__global__ __launch_bounds__(256, 2) void gemm_panel_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bq,
    const uint8_t* __restrict__ bs, int Ma, int Nb, int K, uint16_t* __restrict__ out, int64_t ld_i, int64_t ld_j,
    int tiles_b, int tiles, float* __restrict__ part, int vt_a, int vt_b) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kPanelStage];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (descriptors in SGPRs)
    const int half = lane >> 5;
    const int wa = w >> 1, wb = w & 1;
    // workgroup = split * tiles + block; S = 1 without a workspace (part == nullptr)
    const int tile = (int)(blockIdx.x % (unsigned)tiles);
    const int split = (int)(blockIdx.x / (unsigned)tiles);
    const int S = (int)(gridDim.x / (unsigned)tiles);
    const int ta = tile / tiles_b, tb = tile % tiles_b;
    const int64_t kt128 = (K + 127) >> 7, kt256 = (K + 255) >> 8;
    const int chunks = (int)kt256;
    const int c_begin = (int)((int64_t)chunks * split / S), c_end = (int)((int64_t)chunks * (split + 1) / S);

    // load u (0..7) of wave w moves code tile 8w + u of the chunk: operand w / 2 (A, B), 16-row
    // group 4 (w % 2) + u / 2 of the block, K tile u % 2 of the chunk; load 8 moves half w % 2 of
    // the operand's scale tile (rows of the block x the chunk's 256 elements; lanes 0-31).  Raw
    // buffer loads through descriptors that span the wave's four 16-row groups and the block's scale
    // row: groups past the operand, K tiles past the codes and chunks past the split read as zero,
    // and every load is issued unconditionally (static wait counts).
    const int op = w >> 1;
    const int64_t groups = op == 0 ? ((int64_t)Ma + 15) >> 4 : ((int64_t)Nb + 15) >> 4;
    const int64_t g0 = (int64_t)(op == 0 ? ta : tb) * 8 + 4 * (w & 1);
    const int64_t left = groups - g0 < 0 ? 0 : (groups - g0 < 4 ? groups - g0 : 4);
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>((op == 0 ? aq : bq) + (left > 0 ? g0 * kt128 * 1024 : 0)), (short)0,
        (int)(left * kt128 * 1024), (int)kRsrcFlags);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>((op == 0 ? as : bs) + (int64_t)(op == 0 ? ta : tb) * kt256 * 1024), (short)0,
        (int)(kt256 * 1024), (int)kRsrcFlags);
    typedef u32x4 Stage[9];
    auto load_chunk = [&](int c, Stage& R, bool valid) {
        // offsets are pushed past the descriptor by setting bit 31 (arithmetic, not a select: a
        // select on the uniform flag becomes branches around the loads, and the wait counts
        // then no longer see which loads are in flight)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int kt = c * 2 + (u & 1);
            const unsigned out_bit = (unsigned)(!(valid && kt < kt128)) << 31;
            const unsigned off = (unsigned)(((u >> 1) * (int)kt128 + kt) * 1024 + lane * 16) | out_bit;
            R[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)off, 0, 0);
        }
        const unsigned s_out = ((unsigned)!valid | (unsigned)(lane >> 5)) << 31;
        R[8] = __builtin_amdgcn_raw_buffer_load_b128(srs, (int)((unsigned)(c * 1024 + (w & 1) * 512 + lane * 16) | s_out),
                                                     0, 0);
    };
    // LDS place of load u: row 16 (4 (w % 2) + u / 2) + lane / 4 of operand w / 2, piece 4 (u % 2) + lane % 4
    const int lrow = lane >> 2;
    auto store_chunk = [&](const Stage& R, int buf) {
        uint8_t* L = lds + buf * kPanelStage;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int row = 16 * (4 * (w & 1) + (u >> 1)) + lrow;
            const int piece = 4 * (u & 1) + (lane & 3);
            *reinterpret_cast<u32x4*>(L + op * kPanelCodes + row * 128 + ((piece ^ panel_slot(row)) << 4)) = R[u];
        }
        if (lane < 32) *reinterpret_cast<u32x4*>(L + 2 * kPanelCodes + op * 1024 + (w & 1) * 512 + lane * 16) = R[8];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[ma][nb] = f32x16{};

    // the MFMAs of one chunk from LDS buffer buf: the lane's fragments of rows lane % 32 of each
    // 32-row group at piece 2 st + half (K step st), its scale dwords (the skinny layout's
    // (row, half) dword; byte st scales step st)
    const int frow = lane & 31;
    const int fslot = panel_slot(frow);
    auto mfma_chunk = [&](int buf) {
        const uint8_t* L = lds + buf * kPanelStage;
        int sa[2], sb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            sa[m] = *reinterpret_cast<const int*>(L + 2 * kPanelCodes + (wa * 2 + m) * 256 + frow * 8 + half * 4);
            sb[m] = *reinterpret_cast<const int*>(L + 2 * kPanelCodes + 1024 + (wb * 2 + m) * 256 + frow * 8 +
                                                  half * 4);
        }
#define MX_PANEL_STEP(ST)                                                                                            \
    {                                                                                                                \
        u32x4 af[2], bf[2];                                                                                          \
        _Pragma("unroll") for (int m = 0; m < 2; ++m) {                                                              \
            af[m] = *reinterpret_cast<const u32x4*>(L + (wa * 64 + m * 32 + frow) * 128 +                            \
                                                    (((2 * ST + half) ^ fslot) << 4));                               \
            bf[m] = *reinterpret_cast<const u32x4*>(L + kPanelCodes + (wb * 64 + m * 32 + frow) * 128 +              \
                                                    (((2 * ST + half) ^ fslot) << 4));                               \
        }                                                                                                            \
        _Pragma("unroll") for (int ma = 0; ma < 2; ++ma) _Pragma("unroll") for (int nb = 0; nb < 2; ++nb)           \
            acc[ma][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(af[ma]), as_operand(bf[nb]),    \
                                                                          acc[ma][nb], 4, 4, ST, sa[ma], ST, sb[nb]); \
    }
        MX_PANEL_STEP(0) MX_PANEL_STEP(1) MX_PANEL_STEP(2) MX_PANEL_STEP(3)
#undef MX_PANEL_STEP
    };

    // chunk c in LDS buffer (c - c_begin) % 2; registers X and Y alternate as the staging of the
    // chunk two ahead.  Every thread's reads of a buffer are done before the barrier that precedes
    // the next store into it.  Past the split's last chunk the loads read zeros and the odd
    // chunk's MFMAs are skipped (a uniform branch; no exit from the middle of the body, so the
    // accumulators keep their registers).
    Stage X, Y;
    load_chunk(c_begin, X, c_begin < c_end);
    load_chunk(c_begin + 1, Y, c_begin + 1 < c_end);
    store_chunk(X, 0);
    __syncthreads();
    for (int c = c_begin; c < c_end; c += 2) {
        load_chunk(c + 2, X, c + 2 < c_end);
        mfma_chunk(0);
        store_chunk(Y, 1);
        __syncthreads();
        load_chunk(c + 3, Y, c + 3 < c_end);
        if (c + 1 < c_end) mfma_chunk(1);
        store_chunk(X, 0);
        __syncthreads();
    }

    // acc[ma][nb][r] is C[i0 + ma*32 + (r/4)*8 + half*4 + r%4, j0 + nb*32 + lane%32] of the wave's
    // 64 x 64 block (i0, j0)
    const int va = 2 * ta + wa, vb = 2 * tb + wb;
    if (part) {
        if (va >= vt_a || vb >= vt_b) return;
        float* pblk = part + ((int64_t)split * vt_a * vt_b + (int64_t)va * vt_b + vb) * 4096;
#pragma unroll
        for (int ma = 0; ma < 2; ++ma)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) pblk[((ma * 2 + nb) * 16 + r) * 64 + lane] = acc[ma][nb][r];
        return;
    }
    const int i0 = va * 64, j0 = vb * 64;
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int j = j0 + nb * 32 + frow;
            if (j >= Nb) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + ma * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (i < Ma) out[(int64_t)i * ld_i + (int64_t)j * ld_j] = f32_to_bf16_rne(acc[ma][nb][r]);
            }
        }
}

// Launch plan of the skinny kernel for out[M, N] = a . b^T: the smaller side is A
// (32*MA-row groups), the larger one B (32*NB-row groups).
//
// Wave block MA x NB MFMA tiles: fragments loaded per MFMA fall from 1 + 1/NB (MA = 1) to
// 1 (2 x 2).  The contraction is split over W waves (LDS: W * MA * NB * 4 KB <= 64 KB), W
// doubling until the launch has 16 waves per CU (or a limit); the first candidate whose launch
// then has at least `qualify` waves is taken, else the last one (a single 32 x 32 block: the
// most waves).  The 2 x 2 block (179 VGPRs, 2 waves per SIMD) pays from 6 waves per CU, 1 x 2
// from 8; 1 x 4 needs 16.  FP8 fragments are twice as wide: only 1 x 1 and 1 x 2.
//
// Split contraction: when the launch has fewer workgroups than CUs (and fewer than 16 waves per
// CU) and each wave would run through at least kSplitMinChunks 256-wide chunks one after another,
// S workgroups share each output block (S up to the factor that gives every CU a workgroup, at
// most kMaxSplits, at least one chunk per wave), as far as the workspace holds their S * blocks
// fp32 partial blocks.  Launches that already cover the CUs gain nothing from the partials' extra
// traffic and second kernel (measured: 16384 x 128 x 14336, 512 workgroups, 15% slower split).
struct SkinnyPlan {
    bool swap;
    int64_t Ma, Nb;
    bool panel;          // the panel kernel (128 x 128 blocks, operands shared through LDS)
    int ma, nb, W;
    int64_t tiles_a, tiles_b, chunks;
    int64_t vt_a, vt_b;  // panel kernel: 64 x 64 partial blocks along A and B
    int64_t S;
    int64_t part_bytes;  // workspace the S partial blocks take (0 for S = 1)
};

constexpr int64_t kMaxSplits = 64;
constexpr int64_t kSplitMinChunks = 4;
constexpr int64_t kPanelMinChunks = 4;  // 256-wide chunks per split of the panel kernel, at least

template <int FMT>
static SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t cus, int64_t ws_bytes) {
    SkinnyPlan P{};
    P.swap = M > N;
    P.Ma = P.swap ? N : M;
    P.Nb = P.swap ? M : N;
    P.chunks = (K + 255) / 256;
    if (FMT == 4 && P.Ma >= kPanelRows) {
        // Both sides hold at least one 128-row panel.  The panel kernel is taken where it measured
        // faster than the skinny kernel in the step's order (the GEMM right after the casts that
        // wrote its operands, which then sit in the MALL):
        //  (a) a smaller side of 512 rows or more with blocks for half the CUs, unsplit -- there
        //      the skinny kernel re-reads both operands once per 64-row group of the other side
        //      (2048 x 2048 x 4096: 38.7 -> 24.1 us; 1000 x 2000 x 1024: 14.2 -> 12.6 us);
        //  (b) at least 2^20 outputs over a contraction of 8192 or more, split up to one workgroup
        //      per CU (16384 x 128 x 14336: 56.5 -> 46.0 us; 128 x 14336 x 16384: 60.6 -> 44.2;
        //      1024 x 1024 x 14336: 33.0 -> 28.3), when the split launch covers 3/4 of the CUs.
        // Elsewhere the skinny kernel stays faster: its waves split the contraction inside the
        // workgroup at no traffic, while the panel split writes and reads back S fp32 copies of
        // the output and adds a launch (4096 x 128 x 14336: 20.5 us against 24.0 at best;
        // 16384 x 128 x 4096: 26.4 against 27.5; 16384 x 128 x 32: 10.0 against 14.4).
        const int64_t ta = (P.Ma + kPanelRows - 1) / kPanelRows, tb = (P.Nb + kPanelRows - 1) / kPanelRows;
        const int64_t vt_a = (P.Ma + 63) / 64, vt_b = (P.Nb + 63) / 64;
        const int64_t tiles = ta * tb;
        const int64_t part1 = vt_a * vt_b * 4096 * (int64_t)sizeof(float);  // one split's partials
        const bool wide = P.Ma >= 512 && tiles * 2 >= cus;
        const bool deep = P.Ma * P.Nb >= ((int64_t)1 << 20) && K >= 8192;
        int64_t S = 1;
        if (deep && tiles < cus) {
            S = std::min(std::min(cus / tiles, P.chunks / kPanelMinChunks), kMaxSplits);
            S = std::min(S, ws_bytes / part1);
            if (S < 2) S = 1;
        }
        if (wide || (deep && tiles * S * 4 >= cus * 3)) {
            P.panel = true;
            P.ma = P.nb = 2;
            P.W = 4;
            P.tiles_a = ta;
            P.tiles_b = tb;
            P.vt_a = vt_a;
            P.vt_b = vt_b;
            P.S = S;
            P.part_bytes = S > 1 ? S * part1 : 0;
            return P;
        }
    }
    const int64_t grow = cus * 16;
    struct Cand { int ma, nb; int64_t qualify; };
    const Cand cands4[] = {{2, 2, cus * 6}, {1, 4, cus * 16}, {1, 2, cus * 8}, {1, 1, 0}};
    const Cand cands8[] = {{1, 2, cus * 16}, {1, 1, 0}};
    const Cand* cands = FMT == 8 ? cands8 : cands4;
    const int ncand = FMT == 8 ? 2 : 4;
    P.ma = P.nb = P.W = 1;
    for (int ci = 0; ci < ncand; ++ci) {
        const Cand& cd = cands[ci];
        if ((cd.ma > 1 && P.Ma < 32 * cd.ma) || (cd.nb > 1 && P.Nb < 32 * cd.nb)) continue;
        const int wmax = cd.ma * cd.nb == 1 ? 16 : 8;
        const int64_t ta = (P.Ma + 32 * cd.ma - 1) / (32 * cd.ma), tb = (P.Nb + 32 * cd.nb - 1) / (32 * cd.nb);
        int w = 1;
        while (w * 2 <= wmax && w * 2 * cd.ma * cd.nb <= 16 && w * 2 <= P.chunks && ta * tb * w < grow) w *= 2;
        P.ma = cd.ma;
        P.nb = cd.nb;
        P.W = w;
        P.tiles_a = ta;
        P.tiles_b = tb;
        if (ta * tb * w >= cd.qualify) break;
    }
    const int64_t tiles = P.tiles_a * P.tiles_b;
    const int64_t waves = tiles * P.W;
    const int64_t block_bytes = (int64_t)P.ma * P.nb * 1024 * (int64_t)sizeof(float);
    P.S = 1;
    if (tiles > 0 && tiles < cus && waves < grow && P.chunks >= kSplitMinChunks * P.W) {
        int64_t S = std::min(std::min((cus + tiles - 1) / tiles, P.chunks / P.W), kMaxSplits);
        S = std::min(S, ws_bytes / (tiles * block_bytes));
        P.S = S >= 2 ? S : 1;
    }
    P.part_bytes = P.S > 1 ? P.S * tiles * block_bytes : 0;
    return P;
}

template <int FMT>
static hipError_t launch_skinny(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t M,
                                int64_t N, int64_t K, uint16_t* out, int64_t ldo, void* ws, int64_t ws_bytes,
                                hipStream_t stream) {
    const SkinnyPlan P = plan_skinny<FMT>(M, N, K, mx::num_cus(), ws ? ws_bytes : 0);
    const int64_t ld_i = P.swap ? 1 : ldo, ld_j = P.swap ? ldo : 1;
    const int64_t tiles = P.tiles_a * P.tiles_b;
    if (tiles * P.S > 0x7FFFFFFF || P.Ma > 0x7FFFFFFF || P.Nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = P.W > 1 ? (size_t)P.W * P.ma * P.nb * 16 * 64 * sizeof(float) : 0;
    const dim3 grid((unsigned)(tiles * P.S)), block((unsigned)(64 * P.W));
    const uint8_t *pa = P.swap ? bq : aq, *psa = P.swap ? bs : as, *pb = P.swap ? aq : bq, *psb = P.swap ? as : bs;
    float* part = P.S > 1 ? static_cast<float*>(ws) : nullptr;
    if (P.panel) {
        const int64_t vtiles = P.vt_a * P.vt_b;
        if (vtiles * 4096 > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(mx::gemm_panel_kernel, dim3((unsigned)(tiles * P.S)), dim3(256), 0, stream, pa, psa, pb,
                           psb, (int)P.Ma, (int)P.Nb, (int)K, out, ld_i, ld_j, (int)P.tiles_b, (int)tiles, part,
                           (int)P.vt_a, (int)P.vt_b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || P.S == 1) return e;
        auto red22 = mx::skinny_reduce_kernel<2, 2>;
        hipLaunchKernelGGL(red22, dim3((unsigned)((vtiles * 4096 + 255) / 256)), dim3(256), 0,
                           stream, part, (int)vtiles, (int)P.S, (int)P.vt_b, (int)P.Ma, (int)P.Nb, out, ld_i, ld_j);
        return hipGetLastError();
    }
    auto kern = P.nb == 2 ? mx::gemm_skinny_kernel<1, 2, FMT> : mx::gemm_skinny_kernel<1, 1, FMT>;
    auto red = P.nb == 2 ? mx::skinny_reduce_kernel<1, 2> : mx::skinny_reduce_kernel<1, 1>;
    if constexpr (FMT == 4) {
        if (P.nb == 4) kern = mx::gemm_skinny_kernel<1, 4, FMT>, red = mx::skinny_reduce_kernel<1, 4>;
        if (P.ma == 2) kern = mx::gemm_skinny_kernel<2, 2, FMT>, red = mx::skinny_reduce_kernel<2, 2>;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, stream, pa, psa, pb, psb, (int)P.Ma, (int)P.Nb, (int)K, out, ld_i,
                       ld_j, (int)P.tiles_b, (int)tiles, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || P.S == 1) return e;
    const int64_t outputs = tiles * P.ma * P.nb * 1024;
    hipLaunchKernelGGL(red, dim3((unsigned)((outputs + 255) / 256)), dim3(256), 0, stream, part, (int)tiles, (int)P.S,
                       (int)P.tiles_b, (int)P.Ma, (int)P.Nb, out, ld_i, ld_j);
    return hipGetLastError();
}

}  // namespace mx

extern "C" hipError_t mx_launch_skinny(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                                       int64_t M, int64_t N, int64_t K, uint16_t* out, int64_t ldo, int fmt, void* ws,
                                       int64_t ws_bytes, hipStream_t stream) {
    if (fmt == 8) return mx::launch_skinny<8>(aq, as, bq, bs, M, N, K, out, ldo, ws, ws_bytes, stream);
    if (fmt == 4) return mx::launch_skinny<4>(aq, as, bq, bs, M, N, K, out, ldo, ws, ws_bytes, stream);
    return hipErrorInvalidValue;
}

extern "C" int64_t mx_skinny_split_bytes(int64_t M, int64_t N, int64_t K, int fmt, int64_t cus) {
    const int64_t unlimited = (int64_t)1 << 62;
    return fmt == 8 ? mx::plan_skinny<8>(M, N, K, cus, unlimited).part_bytes
                    : mx::plan_skinny<4>(M, N, K, cus, unlimited).part_bytes;
}
