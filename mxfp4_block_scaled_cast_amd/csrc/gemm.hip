// Block-scaled MXFP4 GEMM for gfx950: out[M, N] = bf16( A[M, K] . B[N, K]^T ).
//
// Operation: jax-aiter README, Supported ops, "FP4 GEMM (low-level)"
// (gemm_fp4 on pre-quantized fp4x2 operands with e8m0 block scales, BF16
// out) in the A[M,K] @ B[N,K]^T convention of its GEMM rows; used for the
// forward, dA and dB products of gemm_fp4_bf16 ("MXFP4 training
// architecture").
//
// Every product runs on V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both operands
// in FP4 (format code 4).  Lane l of a wave supplies, for operand rows
// l%32, the 32 FP4 values of K block (l/32) of the current 64-wide K step
// (16 bytes, low nibble first) and the E8M0 scale of that block as byte
// `opsel` of a dword; the MX operand scale layout packs the four blocks a
// lane needs over a 256-wide K range into one dword.  Accumulation is fp32;
// the epilogue rounds to bf16 (nearest even).
#include <stdlib.h>

#include "mx_device.h"

// MXFP4_GEMM_DIRECT=1 forces the untiled kernel (testing aid).
static int getenv_direct() {
    static const int v = [] {
        const char* e = getenv("MXFP4_GEMM_DIRECT");
        return e && e[0] == '1' ? 1 : 0;
    }();
    return v;
}

namespace mx {

// Reference-shaped kernel: each wave computes a 32x32 output tile reading its
// operands straight from global memory (no LDS).  Used for small problems and
// as the correctness baseline for the tiled kernel.
__global__ __launch_bounds__(256) void gemm_direct_kernel(const uint8_t* __restrict__ aq,
                                                          const uint8_t* __restrict__ as,
                                                          const uint8_t* __restrict__ bq,
                                                          const uint8_t* __restrict__ bs, int M, int N, int K,
                                                          uint16_t* __restrict__ out, int64_t ldo) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int m0 = blockIdx.y * 64 + (w >> 1) * 32;
    const int n0 = blockIdx.x * 64 + (w & 1) * 32;
    const int ra = m0 + (lane & 31);
    const int rb = n0 + (lane & 31);
    const int half = lane >> 5;
    const int64_t kt = (K + 255) >> 8;
    const int64_t ldq = K >> 1;

    f32x16 acc = {};
    for (int k0 = 0; k0 < K; k0 += 64) {
        const int kk = k0 + half * 32;
        v8i a = {}, b = {};
        int sa = 0, sb = 0;
        if (kk < K) {
            if (ra < M) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(aq + (int64_t)ra * ldq + (kk >> 1));
                a[0] = (int)v.x; a[1] = (int)v.y; a[2] = (int)v.z; a[3] = (int)v.w;
                sa = as[scale_offset(ra, kk >> 5, kt)];
            }
            if (rb < N) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(bq + (int64_t)rb * ldq + (kk >> 1));
                b[0] = (int)v.x; b[1] = (int)v.y; b[2] = (int)v.z; b[3] = (int)v.w;
                sb = bs[scale_offset(rb, kk >> 5, kt)];
            }
        }
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, 0, sa, 0, sb);
    }
    const int n = n0 + (lane & 31);
    if (n < N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + (i >> 2) * 8 + half * 4 + (i & 3);
            if (m < M) out[(int64_t)m * ldo + n] = f32_to_bf16_rne(acc[i]);
        }
    }
}


// ---------------------------------------------------------------------------
// Tiled kernel.  Workgroup tile BM x BN = 256 x 256, K tile 256 (128 bytes of
// FP4 per row), 4 waves in a 2 x 2 grid, each wave 128 x 128 = 4 x 4 MFMA
// tiles (256 fp32 accumulators per lane).
//
// Global -> LDS: direct DMA (buffer_load_dwordx4 ... lds), 16 bytes per lane,
// eight lanes per 128-byte row, so one wave instruction fills 8 rows (1 KB)
// of a tile.  Each row's eight 16-byte chunks are stored XOR-swizzled, chunk
// c of tile row r at position c ^ f(r) with f(r) = (r & 7) ^ ((r >> 3) & 1):
// the MFMA fragment reads (lanes 0..31 = 32 consecutive rows at one chunk)
// then hit distinct banks in every group of 8 (and 16) lanes.
// Buffer resources are rebased per workgroup and bounded by the operand's
// size, so rows past M / N read as zero without any predicate.
//
// Scales: the dword a lane needs for one K tile (four 64-wide K steps, byte
// s for step s) is read straight into a VGPR with a bounded buffer load.
// A K tail (K not a multiple of 256) needs no special case: the codes past K
// in a row are finite FP4 values (from the next row, or zero past the end)
// and the scale bytes past K/32 are the zero padding of the MX layout, so
// their products are at most 6*6*2^-254 per term and vanish in fp32.
//
// Pipeline: two LDS stages.  Iteration kt waits for its own DMA (vmcnt 0),
// meets the other waves at one barrier (tile kt is then complete and
// everyone has finished reading stage (kt+1)%2), issues the DMA of tile
// kt+1 into the other stage and runs the MFMAs of tile kt meanwhile.
// ---------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TBM = 256, TBN = 256, TBK = 256;  // tile sizes (elements)
constexpr int TROWB = TBK / 2;                  // bytes per tile row (128)
constexpr unsigned kRsrcWord3 = 0x00020000u;    // gfx9 raw buffer: 32-bit dwords, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t cap = 0xFFFFFFFFll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes < cap ? bytes : cap),
                                             (int)kRsrcWord3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The same descriptor as four dwords (base lo, base hi | stride 0, num_records, word3) for inline asm.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, int64_t bytes) {
    const int64_t cap = 0xFFFFFFFFll;
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = (int)(uint32_t)a;
    r.y = (int)(uint32_t)(a >> 32) & 0xFFFF;
    r.z = (int)(uint32_t)(bytes < cap ? bytes : cap);
    r.w = (int)kRsrcWord3;
    return r;
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding: expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void wait_vmcnt0() {
    __builtin_amdgcn_sched_barrier(0);
    // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) through the builtin, so the
    // compiler's wait tracking knows every earlier load has completed
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// DMA one K tile of a 256-row operand tile into LDS (8 instructions per wave).
// Instruction i of wave w fills tile rows (8w + i)*8 .. +7; lane l serves row
// (8w + i)*8 + l/8 and physical chunk l%8, i.e. logical chunk
// (l%8) ^ swz(row) = (l%8) ^ (l/8) ^ (i & 1).  voff[p] is the lane's byte
// offset for instructions of parity p at K tile 0.
//
// The DMA is issued as inline assembly: the compiler's own wait insertion
// treats every LDS read as possibly aliasing every outstanding LDS DMA and
// would drain the prefetch (vmcnt(0)) before the current tile's fragment
// reads.  The kernel instead waits for its DMA explicitly (wait_vmcnt0 before
// the per-tile barrier); M0 (the DMA's LDS base) is written by the same asm
// statement and nothing else in these kernels uses M0.
__device__ __forceinline__ void dma_tile(const i32x4& rs, int row_step, int kbyte, const int (&voff)[2],
                                         unsigned lds_base, int wave) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const unsigned m0v = lds_base + (unsigned)((wave * 8 + i) * 1024);
        const int vo = voff[i & 1] + i * row_step + kbyte;
        asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(vo), "s"(rs), "s"(m0v)
                     : "memory", "m0");
    }
}

__device__ __forceinline__ v8i as_operand(u32x4 v) {
    v8i r;
    r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;  // FP4 operands occupy four registers; the rest is ignored
    return r;
}

typedef const __attribute__((address_space(3))) char* lds_cptr;

// Fragments of one 64-wide K step: 4 A (rows i*32 + lane%32 of the wave's
// 128) and 4 B, 16 bytes each.
struct Frags {
    u32x4 a[4], b[4];
};

__device__ __forceinline__ void read_frags(Frags& f, lds_cptr la, lds_cptr lb, int a_base, int b_base, int choff) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(la + a_base + i * 32 * TROWB + choff);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        f.b[j] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lb + b_base + j * 32 * TROWB + choff);
}

template <int S>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[4][4], const Frags& f, const int (&sa)[4],
                                          const int (&sb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(f.a[i]), as_operand(f.b[j]),
                                                                        acc[i][j], 4, 4, S, sa[i], S, sb[j]);
}

// Keeps each K step's LDS reads and MFMAs in program order: a compiler memory
// fence (IR level) plus a scheduling barrier (machine scheduler).
__device__ __forceinline__ void mem_fence_compiler() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One K tile: the reads of step s+1 are in flight while the MFMAs of step s run.
__device__ __forceinline__ void compute_tile(f32x16 (&acc)[4][4], lds_cptr la, lds_cptr lb, int a_base, int b_base,
                                             const int (&choff)[4], const int (&sa)[4], const int (&sb)[4]) {
    Frags f0, f1;
    read_frags(f0, la, lb, a_base, b_base, choff[0]);
    mem_fence_compiler();
    read_frags(f1, la, lb, a_base, b_base, choff[1]);
    mem_fence_compiler();
    mfma_step<0>(acc, f0, sa, sb);
    read_frags(f0, la, lb, a_base, b_base, choff[2]);
    mem_fence_compiler();
    mfma_step<1>(acc, f1, sa, sb);
    read_frags(f1, la, lb, a_base, b_base, choff[3]);
    mem_fence_compiler();
    mfma_step<2>(acc, f0, sa, sb);
    mem_fence_compiler();
    mfma_step<3>(acc, f1, sa, sb);
    mem_fence_compiler();
}

__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(const uint8_t* __restrict__ aq,
                                                            const uint8_t* __restrict__ as,
                                                            const uint8_t* __restrict__ bq,
                                                            const uint8_t* __restrict__ bs, int M, int N, int K,
                                                            uint16_t* __restrict__ out, int64_t ldo, int tiles_m,
                                                            int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(1024))) char lds_a0[TBM * TROWB];
    __shared__ __attribute__((aligned(1024))) char lds_b0[TBN * TROWB];
    __shared__ __attribute__((aligned(1024))) char lds_a1[TBM * TROWB];
    __shared__ __attribute__((aligned(1024))) char lds_b1[TBN * TROWB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // tile order: XCD-contiguous ranges, grouped by `group_m` tile rows for L2 reuse
    const int total = tiles_m * tiles_n;
    const int t = xcd_remap(blockIdx.x, total);
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int local = t - g * per_group;
    const int tm = first_m + local % gsize;
    const int tn = local / gsize;
    const int64_t m0 = (int64_t)tm * TBM, n0 = (int64_t)tn * TBN;

    const int ldq = K >> 1;
    const int nkt = (K + TBK - 1) / TBK;
    const int64_t kt_total = nkt;  // scale tiles per 32-row group

    const i32x4 ra = make_rsrc_words(aq + m0 * ldq, (M - m0) * (int64_t)ldq);
    const i32x4 rb = make_rsrc_words(bq + n0 * ldq, (N - n0) * (int64_t)ldq);
    const unsigned la0 = (unsigned)(uintptr_t)(lds_cptr)lds_a0, lb0 = (unsigned)(uintptr_t)(lds_cptr)lds_b0;
    const unsigned la1 = (unsigned)(uintptr_t)(lds_cptr)lds_a1, lb1 = (unsigned)(uintptr_t)(lds_cptr)lds_b1;
    const int64_t a_rows32 = (M + 31) >> 5, b_rows32 = (N + 31) >> 5;
    const rsrc_t rsa = make_rsrc(as + (m0 >> 5) * kt_total * 256, (a_rows32 - (m0 >> 5)) * kt_total * 256);
    const rsrc_t rsb = make_rsrc(bs + (n0 >> 5) * kt_total * 256, (b_rows32 - (n0 >> 5)) * kt_total * 256);

    // DMA lane offsets (see dma_tile) and the per-instruction row step (8 rows)
    int voff[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
        voff[p] = (wave * 64 + (lane >> 3)) * ldq + (((lane & 7) ^ (lane >> 3) ^ p) * 16);
    const int row_step = 8 * ldq;

    // per-lane scale offset inside a 256-byte scale tile
    const int s_lane = (lane & 31) * 8 + (lane >> 5) * 4;
    // per-lane LDS fragment offsets: row (lane & 31) of a 32-row group, chunk (2s + lane/32) swizzled
    const int frow = lane & 31;
    const int a_base = (wm * 128 + frow) * TROWB;
    const int b_base = (wn * 128 + frow) * TROWB;
    int choff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) choff[s] = ((2 * s + (lane >> 5)) ^ swz(frow)) * 16;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    int sa[4], sb[4], sa_n[4], sb_n[4];
    auto load_scales = [&](int kt, int (&da)[4], int (&db)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ga = (wm * 4 + i) * (int)kt_total + kt;   // 32-row group of the fragment, K tile kt
            const int gb = (wn * 4 + i) * (int)kt_total + kt;
            da[i] = __builtin_amdgcn_raw_buffer_load_b32(rsa, ga * 256 + s_lane, 0, 0);
            db[i] = __builtin_amdgcn_raw_buffer_load_b32(rsb, gb * 256 + s_lane, 0, 0);
        }
    };

    dma_tile(ra, row_step, 0, voff, la0, wave);
    dma_tile(rb, row_step, 0, voff, lb0, wave);
    load_scales(0, sa, sb);

    // Main loop, two K tiles per iteration and no branches inside (a branch
    // lets the compiler sink the MFMAs past the next barrier).  The prefetch
    // of a tile past the end goes through an empty descriptor, so it moves
    // no data.
    i32x4 ra_none = ra, rb_none = rb;
    ra_none.z = 0;
    rb_none.z = 0;
    const int iters = nkt >> 1;
    for (int it = 0; it < iters; ++it) {
        const int kt = 2 * it;
        // ---- tile kt from stage 0; prefetch tile kt+1 into stage 1
        wait_vmcnt0();
        __syncthreads();
        dma_tile(ra, row_step, (kt + 1) * TROWB, voff, la1, wave);
        dma_tile(rb, row_step, (kt + 1) * TROWB, voff, lb1, wave);
        load_scales(kt + 1, sa_n, sb_n);
        compute_tile(acc, (lds_cptr)lds_a0, (lds_cptr)lds_b0, a_base, b_base, choff, sa, sb);
        // ---- tile kt+1 from stage 1; prefetch tile kt+2 (if any) into stage 0
        wait_vmcnt0();
        __syncthreads();
        const bool more = kt + 2 < nkt;
        dma_tile(more ? ra : ra_none, row_step, (kt + 2) * TROWB, voff, la0, wave);
        dma_tile(more ? rb : rb_none, row_step, (kt + 2) * TROWB, voff, lb0, wave);
        load_scales(kt + 2, sa, sb);
        compute_tile(acc, (lds_cptr)lds_a1, (lds_cptr)lds_b1, a_base, b_base, choff, sa_n, sb_n);
    }
    if (nkt & 1) {
        // ---- odd tail: the last tile sits in stage 0
        wait_vmcnt0();
        __syncthreads();
        compute_tile(acc, (lds_cptr)lds_a0, (lds_cptr)lds_b0, a_base, b_base, choff, sa, sb);
    }

    // ---- epilogue: fp32 -> bf16 (nearest even), predicated stores
    const int half = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
                if (m < M) out[m * ldo + n] = f32_to_bf16_rne(acc[i][j][e]);
            }
        }
    }
}

}  // namespace mx

extern "C" hipError_t mx_launch_gemm(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                     int64_t N, int64_t K, void* out, int64_t ldo, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const bool tiled = K > 0 && M >= 128 && N >= 128 && getenv_direct() == 0;
    if (tiled) {
        const int64_t tiles_m = (M + mx::TBM - 1) / mx::TBM, tiles_n = (N + mx::TBN - 1) / mx::TBN;
        if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
        const int group_m = 8;
        hipLaunchKernelGGL(mx::gemm_tiled_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream,
                           static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                           static_cast<const uint8_t*>(bq), static_cast<const uint8_t*>(bs), (int)M, (int)N, (int)K,
                           static_cast<uint16_t*>(out), ldo, (int)tiles_m, (int)tiles_n, group_m);
        return hipGetLastError();
    }
    if ((M + 63) / 64 > 65535 || (N + 63) / 64 > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64)), block(256);
    hipLaunchKernelGGL(mx::gemm_direct_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(aq),
                       static_cast<const uint8_t*>(as), static_cast<const uint8_t*>(bq),
                       static_cast<const uint8_t*>(bs), (int)M, (int)N, (int)K, static_cast<uint16_t*>(out), ldo);
    return hipGetLastError();
}
