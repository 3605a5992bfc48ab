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
//
// The training backward's two products (dA on dOut's row copy and W's column
// copy, dB on the column copies of dOut and A) can share one persistent launch,
// the chip's XCDs divided between them (mx_launch_gemm_pair_ws).
//
// The same kernels also run the MXFP8 product of the FP8 dB variant (format
// code 0, E4M3 on both sides): an FP8 code tile has the FP4 tile's geometry
// in bytes (64 bytes per row = one 64-wide K step), so loads, LDS stages and
// swizzle are shared; lane half h supplies K elements 16h .. 16h+15 and
// 32+16h .. 47+16h of the step (two 16-byte pieces), while the scale of K
// block b still comes from lane half b % 2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "mx_device.h"
#include "mx_host.h"

// The skinny kernel and its split contraction (gemm_skinny.hip): out[M, N] for outputs
// too small for 256 x 256 tiles; fmt 4 or 8; ws / ws_bytes the optional split workspace.
extern "C" hipError_t mx_launch_skinny(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                                       int64_t M, int64_t N, int64_t K, uint16_t* out, int64_t ldo, int fmt, void* ws,
                                       int64_t ws_bytes, hipStream_t stream);
// Workspace bytes of the skinny launch's split contraction on a chip of `cus` CUs (0: no split).
extern "C" int64_t mx_skinny_split_bytes(int64_t M, int64_t N, int64_t K, int fmt, int64_t cus);

namespace mx {

// ---------------------------------------------------------------------------
// Pipelined kernel.  Workgroup tile 256 x 256, K tile 128 (64 bytes of FP4 per
// row), 4 waves in a 2 x 2 grid, each wave 128 x 128 = 4 x 4 MFMA tiles
// (256 fp32 accumulators per lane, in AGPRs).
//
// LDS holds NST = 4 stages of 36 KB: A codes [256 rows][64 B], B codes
// [256][64 B], then the A and B scale tiles of the 256-wide K range the tile
// belongs to (2 x 1 KB each, straight copies of the MX scale layout).  All
// global data arrives by direct DMA (buffer_load_dwordx4 ... lds), 16 bytes
// per lane: a wave instruction moves one 1 KB code tile of the MX layout
// (16 rows x 64 B, contiguous in memory, so one instruction touches one page;
// row-major codes made every instruction span 16 rows and stalled the L1
// address translation) or one 1 KB scale tile.  Row r keeps its four
// 16-byte chunks XOR-swizzled, chunk c at position c ^ swz(r) with
// swz(r) = ((r >> 1) & 3) ^ (3 * ((r >> 3) & 1)): for the fragment reads (32
// consecutive rows at one chunk) every aligned group of 8 rows then covers 8
// distinct 16-byte slots of a 128-byte bank window and every aligned group of
// 16 rows 16 distinct slots of a 256-byte window.  Descriptors are rebased per workgroup and
// bounded by the operand size: rows past the padded M / N, and whole tiles
// past K (an empty descriptor), read as zero.  A K tail inside a tile needs
// no special case: the layout pads codes to a multiple of 128 elements with
// zero codes and the scales with zero bytes.
//
// Schedule of iteration kt (register set p = kt % 2 holds tile kt, read
// from stage kt%4 during the previous iteration):
//   MFMAs of K step 0 of tile kt
//   wait for the DMA of tile kt+1 and for this wave's LDS reads, barrier
//     (after it no wave reads stage kt%4 any more)
//   MFMAs of K step 1 of tile kt, with the LDS reads of tile kt+1 (set 1-p)
//     and the DMA instructions of tile kt+4 into stage kt%4 spread
//     between them (8 for the codes, plus the scale tile for the first K
//     tile of each 256-wide scale tile; the other K tiles take the scale
//     dwords of the previous one from registers -- one dword holds them all)
// Memory instructions are spread one or two per MFMA: a wave that issues a
// burst of them stalls on the address unit's queue and lets the MFMA pipe
// drain.  With the register double buffer, 4 stages give a tile's DMA about
// three tiles of MFMA work to land; LDS read latency hides behind half a
// tile.  The loop is unrolled by 4 (static stage and register set) and runs
// a multiple of 4 tiles; tiles past K are empty (zero codes, zero scales)
// and add nothing.
// ---------------------------------------------------------------------------

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(3))) char* lds_cptr;

constexpr int PBM = 256, PBN = 256, PBK = 128;   // tile sizes (elements)
constexpr int PROWB = PBK / 2;                    // bytes per tile row (64)
constexpr int NST = 4;                            // LDS stages
constexpr int ST_A = 0, ST_B = PBM * PROWB;       // code regions in a stage
constexpr int ST_SA = ST_B + PBN * PROWB;         // 32768: A scale tiles
constexpr int ST_SB = ST_SA + (PBM / 32) * 256;   // 34816: B scale tiles
constexpr int STAGE = ST_SB + (PBN / 32) * 256;   // 36864 bytes
constexpr unsigned kRsrcWord3 = 0x00020000u;      // gfx9 raw buffer: dword format, no swizzle
// DMA instructions per wave per K tile: 8 for the codes, plus 1 for the scale
// tile when the K tile is the first one its scale tile covers (a scale tile
// spans 256 elements: 2 FP4 K tiles or 4 FP8 ones, and one scale dword holds
// the scales of all of them, so the other K tiles reuse the dwords already in
// registers).  t4 = K tile index mod 4 (the stage).
template <int FMT>
constexpr bool tile_loads_scales(int t4) { return FMT == 8 ? t4 == 0 : (t4 & 1) == 0; }
template <int FMT>
constexpr int dma_count(int t4) { return tile_loads_scales<FMT>(t4) ? 9 : 8; }

// Chunk swizzle of a 64-byte tile row (depends on the row's low 4 bits only).
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) & 3) ^ (3 * ((r >> 3) & 1)); }

// Raw buffer descriptor as four dwords: base, stride 0, num_records (bytes, capped at 4 GiB - 1), word3.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, int64_t bytes) {
    const int64_t cap = 0xFFFFFFFFll;
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    r.z = (int)(uint32_t)(bytes <= 0 ? 0 : (bytes < cap ? bytes : cap));
    r.w = (int)kRsrcWord3;
    return r;
}

__device__ __forceinline__ i32x4 uniform(i32x4 v) {
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(v.x);
    r.y = __builtin_amdgcn_readfirstlane(v.y);
    r.z = __builtin_amdgcn_readfirstlane(v.z);
    r.w = __builtin_amdgcn_readfirstlane(v.w);
    return r;
}

// One LDS DMA instruction: 64 lanes x 16 bytes from rs + voff into LDS at
// m0v + 16 * lane.  Issued as inline assembly: the compiler's own wait
// insertion treats every LDS read as aliasing every outstanding LDS DMA and
// would drain the prefetch before each fragment read.  The kernel counts its
// DMA instructions and waits for them explicitly (vmcnt); M0 is written here
// and used by nothing else in these kernels.
__device__ __forceinline__ void dma16(const i32x4& rs, int voff, unsigned m0v) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(m0v)
                 : "memory", "m0");
}

// Same, with the LDS address given as a wave-uniform base plus a compile-time
// offset (keeps one SGPR live instead of one per destination), and the
// K-tile part of the source offset in the scalar offset `soff`.  `soff` must
// stay below the size of one 16-row tile, so that the in-bounds test on the
// lane offset alone decides whether the whole address is in bounds.
template <int IMM>
__device__ __forceinline__ void dma16_at(const i32x4& rs, int voff, int soff, unsigned base) {
    // s_add_u32 writes SCC: declared, so no compare result is kept in SCC across this
    asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff),
                 "s"(base), "i"(IMM)
                 : "memory", "m0", "scc");
}

// s_waitcnt vmcnt(N) (expcnt/lgkmcnt left alone) through the builtin, so the
// compiler's own wait tracking sees it.
// With LDS0, also lgkmcnt(0): every LDS read this wave issued has returned.
template <int N, bool LDS0 = false>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | ((LDS0 ? 0x0 : 0xF) << 8));
}

// s_waitcnt lgkmcnt(0): every LDS access this wave issued has completed.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 and expcnt 7 (no wait), lgkmcnt 0
}

// Keeps LDS reads and MFMAs in program order (IR-level memory fence plus a
// machine-scheduler barrier).
__device__ __forceinline__ void order_point() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Component-wise select of two uniform descriptors, kept in SGPRs.
__device__ __forceinline__ i32x4 pick(bool c, const i32x4& a, const i32x4& b) {
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(c ? a.x : b.x);
    r.y = __builtin_amdgcn_readfirstlane(c ? a.y : b.y);
    r.z = __builtin_amdgcn_readfirstlane(c ? a.z : b.z);
    r.w = __builtin_amdgcn_readfirstlane(c ? a.w : b.w);
    return r;
}

// Descriptors of one output tile's operands: A codes, B codes, and this
// wave's scale source (A scales for waves 0, 1, B scales for waves 2, 3).
struct TileSrc {
    i32x4 ra, rb, rs;
};

struct DmaPlan {
    int va, vb;          // lane byte offsets of instruction 0 of the A / B code DMA at K tile 0
    int tstep;           // bytes between consecutive 16-row code tiles (KT * 1 KB)
    int vs;              // lane byte offset of this wave's scale DMA at K-tile pair 0
    int scale_region;    // LDS offset of this wave's scale copy inside a stage
    unsigned lds0;       // LDS address of stage 0
    unsigned code_base;  // lds0 + 4 KB * wave: this wave's code rows in stage 0 (uniform)
    unsigned scale_base; // lds0 + scale_region (uniform)
    int wave;
};

// Instruction Q (0..8) of the DMA of K tile kt of source S into stage ST:
// 0-3 A codes, 4-7 B codes, 8 scales.  P.code_base / P.scale_base are this
// wave's LDS bases (wave-uniform SGPRs); the rest of the address is constant.
// FMT 4: K tile = 128 FP4 elements, the scale tile (256 elements) spans 2 K
// tiles; FMT 8: K tile = 64 FP8 elements (the same 64 bytes per row), the
// scale tile spans 4 K tiles.
template <int ST, int Q, int FMT = 4>
__device__ __forceinline__ void dma_one(const DmaPlan& P, const TileSrc& S, int kt, bool valid) {
    // a tile past K goes through a descriptor with num_records 0: every lane reads zero
    if constexpr (Q < 4) {
        i32x4 r = S.ra;
        r.z = __builtin_amdgcn_readfirstlane(valid ? r.z : 0);
        dma16_at<ST * STAGE + ST_A + Q * 1024>(r, P.va + Q * P.tstep, kt * 1024, P.code_base);
    } else if constexpr (Q < 8) {
        i32x4 r = S.rb;
        r.z = __builtin_amdgcn_readfirstlane(valid ? r.z : 0);
        dma16_at<ST * STAGE + ST_B + (Q - 4) * 1024>(r, P.vb + (Q - 4) * P.tstep, kt * 1024, P.code_base);
    } else {
        i32x4 r = S.rs;
        r.z = __builtin_amdgcn_readfirstlane(valid ? r.z : 0);
        dma16_at<ST * STAGE>(r, P.vs, (kt >> (FMT == 8 ? 2 : 1)) * 1024, P.scale_base);
    }
}

// All DMA instructions of K tile kt (kt % 4 == ST) into stage ST.
template <int ST, int FMT = 4>
__device__ __forceinline__ void dma_tile_all(const DmaPlan& P, const TileSrc& S, int kt, bool valid) {
    dma_one<ST, 0, FMT>(P, S, kt, valid);
    dma_one<ST, 1, FMT>(P, S, kt, valid);
    dma_one<ST, 2, FMT>(P, S, kt, valid);
    dma_one<ST, 3, FMT>(P, S, kt, valid);
    dma_one<ST, 4, FMT>(P, S, kt, valid);
    dma_one<ST, 5, FMT>(P, S, kt, valid);
    dma_one<ST, 6, FMT>(P, S, kt, valid);
    dma_one<ST, 7, FMT>(P, S, kt, valid);
    if constexpr (tile_loads_scales<FMT>(ST)) dma_one<ST, 8, FMT>(P, S, kt, valid);
}

// DMA instructions of K tiles 1, 2, 3: in flight while the prologue waits for K tile 0.
template <int FMT>
constexpr int prologue_wait() { return dma_count<FMT>(1) + dma_count<FMT>(2) + dma_count<FMT>(3); }

// Operand descriptors of the output tile at (m0, n0), rebased at the tile and
// bounded by the operand sizes (tiles past M / N read zero).
__device__ __forceinline__ TileSrc tile_src(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                                            const uint8_t* bs, int M, int N, int nkt, int kt2, int64_t m0, int64_t n0,
                                            int wave) {
    const int64_t a_t16 = (M + 15) >> 4, b_t16 = (N + 15) >> 4;
    const int64_t a_t128 = (M + 127) >> 7, b_t128 = (N + 127) >> 7;
    TileSrc S;
    S.ra = uniform(make_rsrc_words(aq + (m0 >> 4) * nkt * 1024, (a_t16 - (m0 >> 4)) * nkt * 1024));
    S.rb = uniform(make_rsrc_words(bq + (n0 >> 4) * nkt * 1024, (b_t16 - (n0 >> 4)) * nkt * 1024));
    const i32x4 rsa = make_rsrc_words(as + (m0 >> 7) * kt2 * 1024, (a_t128 - (m0 >> 7)) * kt2 * 1024);
    const i32x4 rsb = make_rsrc_words(bs + (n0 >> 7) * kt2 * 1024, (b_t128 - (n0 >> 7)) * kt2 * 1024);
    S.rs = pick(wave >= 2, rsb, rsa);
    return S;
}

// Grouped tile order: `group_m` tile rows at a time, tile rows fastest.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int local = t - g * per_group;
    tm = first_m + local % gsize;
    tn = local / gsize;
}

// Registers holding one tile: fragments of its two 64-wide K steps and the scale dwords.
struct TileRegs {
    u32x4 a0[4], b0[4], a1[4], b1[4];
    int sa[4], sb[4];
};

struct ReadPlan {
    int a_off[2], b_off[2];  // per lane: fragment row + swizzled chunk c (c = 2*step + lane/32), A and B
    int sa_off, sb_off;      // per lane: scale dword of the wave's first 32-row group
};

__device__ __forceinline__ u32x4 lds128(lds_cptr p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
__device__ __forceinline__ int lds32(lds_cptr p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) int*>(p);
}

// K tiles of the operands: 128 FP4 or 64 FP8 elements, 64 bytes per row either way.
template <int FMT>
__device__ __forceinline__ int k_tiles(int K) { return FMT == 8 ? (K + 63) >> 6 : (K + 127) >> 7; }

// DMA addressing of a wave.  Code DMA: instruction q of wave w moves 16-row
// tile 4w + q; lane l takes row l/4 of it, physical chunk l%4, i.e. logical
// chunk (l%4) ^ swz64(l/4).  Waves 0, 1 copy the A scale tiles (rows 0-127,
// 128-255 of the output tile), waves 2, 3 the B ones.
__device__ __forceinline__ DmaPlan dma_plan(int lane, int wave, int nkt, int kt2, lds_cptr lds) {
    DmaPlan P;
    P.wave = wave;
    P.scale_region = (wave >= 2 ? ST_SB : ST_SA) + (wave & 1) * 1024;
    const int chunk = (lane & 3) ^ swz64(lane >> 2);
    P.tstep = nkt * 1024;
    P.va = wave * 4 * P.tstep + (lane >> 2) * 64 + chunk * 16;
    P.vb = P.va;
    P.vs = (wave & 1) * kt2 * 1024 + lane * 16;
    P.lds0 = (unsigned)(uintptr_t)lds;
    P.code_base = __builtin_amdgcn_readfirstlane(P.lds0 + (unsigned)(wave * 4 * 1024));
    P.scale_base = __builtin_amdgcn_readfirstlane(P.lds0 + (unsigned)P.scale_region);
    return P;
}

// LDS read addressing of a lane: fragment row lane%32 of the wave's 128-row
// blocks, at the 16-byte chunks c = 2*st + h (h = lane/32, st = 0, 1) of its
// 64-byte tile row.  FP4: chunk c holds K elements 32c .. 32c+31 of the
// tile, the lane's whole operand for K step st.  FP8: the tile is one K
// step and the 32x32x64 FP8 operand of lane half h is K elements 16h ..
// 16h+15 (registers 0-3) and 32+16h .. 47+16h (registers 4-7), i.e. chunks h
// and 2 + h -- the same two chunks.  Scales: the dword of (row, half); the
// scale of K block b (32 elements) comes from the lanes of half b % 2.
__device__ __forceinline__ ReadPlan read_plan(int lane, int wm, int wn) {
    ReadPlan R;
    const int frow = lane & 31;
    const int sw = swz64(frow);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int c = 2 * st + (lane >> 5);
        R.a_off[st] = (wm * 128 + frow) * PROWB + ((c ^ sw) << 4);
        R.b_off[st] = (wn * 128 + frow) * PROWB + ((c ^ sw) << 4);
    }
    const int s_lane = frow * 8 + (lane >> 5) * 4;
    R.sa_off = wm * 4 * 256 + s_lane;
    R.sb_off = wn * 4 * 256 + s_lane;
    return R;
}

// Order of the FP8 fragment reads (slots 8..23 of read_one): an MFMA needs
// both halves of its A and B fragments, so they come in the order the MFMAs
// (i-major) first use them.
__device__ __forceinline__ constexpr int read8_slot(int q) {
    constexpr int order[24] = {0,  1,  2,  3,  4,  5,  6,  7,  8,  16, 12, 20,
                               13, 21, 14, 22, 15, 23, 9,  17, 10, 18, 11, 19};
    return order[q];
}

// LDS read q (0..23) of a tile: scales first, then (FP4) the step-0
// fragments, then step 1; FP8 reads the same slots in read8_slot order.
template <int FMT = 4>
__device__ __forceinline__ void read_one(TileRegs& T, const ReadPlan& R, lds_cptr stage, int q0) {
    const int q = FMT == 8 ? read8_slot(q0) : q0;
    if (q < 4) T.sa[q] = lds32(stage + ST_SA + R.sa_off + q * 256);
    else if (q < 8) T.sb[q - 4] = lds32(stage + ST_SB + R.sb_off + (q - 4) * 256);
    else if (q < 12) T.a0[q - 8] = lds128(stage + ST_A + R.a_off[0] + (q - 8) * 32 * PROWB);
    else if (q < 16) T.b0[q - 12] = lds128(stage + ST_B + R.b_off[0] + (q - 12) * 32 * PROWB);
    else if (q < 20) T.a1[q - 16] = lds128(stage + ST_A + R.a_off[1] + (q - 16) * 32 * PROWB);
    else T.b1[q - 20] = lds128(stage + ST_B + R.b_off[1] + (q - 20) * 32 * PROWB);
}

// MFMA q (0..15) of one K step, (i, j) = (q / 4, q % 4).  B fragments enter the
// first operand, so the accumulator row is the output column: each lane ends
// up with 4 consecutive output columns of one output row.  OPSEL picks the
// scale byte of the step.
template <int OPSEL>
__device__ __forceinline__ void mfma_one(f32x16 (&acc)[4][4], const u32x4 (&a)[4], const u32x4 (&b)[4],
                                         const int (&sa)[4], const int (&sb)[4], int q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(b[j]), as_operand(a[i]), acc[i][j], 4, 4,
                                                                OPSEL, sb[j], OPSEL, sa[i]);
}

// FP8 MFMA q (0..15) of a K tile: (i, j) = (q / 4, q % 4), operands from the
// two 16-byte chunks the lane read (see read_plan), format code 0 (E4M3) on
// both sides.
template <int OPSEL>
__device__ __forceinline__ void mfma8_one(f32x16 (&acc)[4][4], const TileRegs& T, int q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand8(T.b0[j], T.b1[j]),
                                                                as_operand8(T.a0[i], T.a1[i]), acc[i][j], 0, 0,
                                                                OPSEL, T.sb[j], OPSEL, T.sa[i]);
}

constexpr int kEpiStores = 32;  // 16-byte output stores per wave per tile (persistent kernel)

// Iteration kt = 4t + U of the main loop (see the schedule above).  The DMA
// it issues is for K tile kt+4 of the current output tile, or with LAST (the
// final trip of a tile) for K tile U of the next output tile; both land in
// stage U.  With POST (first trip after an epilogue) the waits of the first
// three iterations also let the epilogue's stores, issued after the DMA of K
// tile 3, be outstanding.  MFMA_LIVE: K tile kt holds contraction data (off
// for the K tiles that one-trip launches run wholly past K: their MFMAs would
// add zeros); READ_LIVE: the K tile read into registers here (kt+1, or the next
// output tile's K tile 0) does.  The DMA and the waits are the same either way.
template <int U, bool POST = false, bool LAST = false, int FMT = 4, bool MFMA_LIVE = true, bool READ_LIVE = true>
__device__ __forceinline__ void pipe_iter(f32x16 (&acc)[4][4], TileRegs& cur, TileRegs& nxt, const DmaPlan& P,
                                          const TileSrc& Scur, const TileSrc& Snext, bool next_ok,
                                          const ReadPlan& R, lds_cptr lds, int kt, int nkt) {
    constexpr int DST = U;
    // the DMA of K tiles kt+2 and kt+3 may still be in flight
    constexpr int WAIT = dma_count<FMT>((U + 2) & 3) + dma_count<FMT>((U + 3) & 3) + ((POST && U < 3) ? kEpiStores : 0);
    // K tile kt+1 reads its scale dwords from LDS, or takes tile kt's (same scale tile)
    constexpr bool NXT_SCALES = tile_loads_scales<FMT>((U + 1) & 3);
    // the K tile DMA'd here (kt+4, or K tile U of the next output tile) is congruent to U
    constexpr bool DMA_SCALES = tile_loads_scales<FMT>(U);
    constexpr int R0 = NXT_SCALES ? 0 : 8;  // first LDS read slot (0..7 are the scales)
    if constexpr (!NXT_SCALES) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            nxt.sa[i] = cur.sa[i];
            nxt.sb[i] = cur.sb[i];
        }
    }
    const TileSrc& S = LAST ? Snext : Scur;
    const int dkt = LAST ? U : kt + NST;
    const bool valid = LAST ? (next_ok && U < nkt) : (kt + NST < nkt);
    lds_cptr next = lds + ((U + 1) % NST) * STAGE;
    if constexpr (FMT == 4) {
        constexpr int OP = (U & 1) * 2;  // tile kt uses bytes 2*(kt%2) and 2*(kt%2)+1 of its scale dwords
        if constexpr (MFMA_LIVE) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                mfma_one<OP>(acc, cur.a0, cur.b0, cur.sa, cur.sb, q);
                order_point();
            }
        }
        // tile kt+1 has landed (tiles kt+2 and kt+3 may be in flight), this wave's
        // LDS reads are done, and after the barrier nobody reads stage U any more
        wait_vmcnt<WAIT, true>();
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            // the scales and step-0 data of tile kt+1 (reads 0..15; the scales only for
            // the first K tile of a scale tile) go first: they are needed first
            const int r0 = (q * 3) / 2, r1 = ((q + 1) * 3) / 2;
            if constexpr (READ_LIVE) {
#pragma unroll
                for (int r = r0; r < r1; ++r)
                    if (r >= R0) read_one<FMT>(nxt, R, next, r);
            }
            // DMA instructions 0..7 before the odd MFMAs, 8 (scales, even K tiles) before MFMA 14
            if (q == 1) dma_one<DST, 0, FMT>(P, S, dkt, valid);
            if (q == 3) dma_one<DST, 1, FMT>(P, S, dkt, valid);
            if (q == 5) dma_one<DST, 2, FMT>(P, S, dkt, valid);
            if (q == 7) dma_one<DST, 3, FMT>(P, S, dkt, valid);
            if (q == 9) dma_one<DST, 4, FMT>(P, S, dkt, valid);
            if (q == 11) dma_one<DST, 5, FMT>(P, S, dkt, valid);
            if (q == 13) dma_one<DST, 6, FMT>(P, S, dkt, valid);
            if constexpr (DMA_SCALES)
                if (q == 14) dma_one<DST, 8, FMT>(P, S, dkt, valid);
            if (q == 15) dma_one<DST, 7, FMT>(P, S, dkt, valid);
            if constexpr (MFMA_LIVE) mfma_one<OP + 1>(acc, cur.a1, cur.b1, cur.sa, cur.sb, q);
            order_point();
        }
    } else {
        // FP8: one 64-wide K step per tile, each MFMA twice as long; a0/a1 (b0/b1) are registers
        // 0-3 / 4-7 of a lane's 32-byte operand; tile kt uses byte kt%4 of its scale dwords
        constexpr int OP = U;
        if constexpr (MFMA_LIVE) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                mfma8_one<OP>(acc, cur, q);
                order_point();
            }
        }
        wait_vmcnt<WAIT, true>();
        __syncthreads();
#pragma unroll
        for (int q = 8; q < 16; ++q) {
            // the reads of tile kt+1 (24, or 16 without the scales; every MFMA of the next
            // tile needs both halves)
            if constexpr (READ_LIVE) {
#pragma unroll
                for (int r = (q - 8) * 3; r < (q - 7) * 3; ++r)
                    if (r >= R0) read_one<FMT>(nxt, R, next, r);
            }
            if (q == 8) dma_one<DST, 0, FMT>(P, S, dkt, valid);
            if (q == 9) dma_one<DST, 1, FMT>(P, S, dkt, valid);
            if (q == 10) dma_one<DST, 2, FMT>(P, S, dkt, valid);
            if (q == 11) dma_one<DST, 3, FMT>(P, S, dkt, valid);
            if (q == 12) dma_one<DST, 4, FMT>(P, S, dkt, valid);
            if (q == 13) dma_one<DST, 5, FMT>(P, S, dkt, valid);
            if (q == 14) dma_one<DST, 6, FMT>(P, S, dkt, valid);
            if (q == 15) {
                dma_one<DST, 7, FMT>(P, S, dkt, valid);
                if constexpr (DMA_SCALES) dma_one<DST, 8, FMT>(P, S, dkt, valid);
            }
            if constexpr (MFMA_LIVE) mfma8_one<OP>(acc, cur, q);
            order_point();
        }
    }
}

// Four iterations kt0 .. kt0+3 (kt0 a multiple of 4).  LIVE < 4 only for the one
// trip of a tile whose contraction has LIVE K tiles (K tiles LIVE..3 past K): their
// MFMAs and register reads are left out, the last iteration's read (the next output
// tile's K tile 0) stays.
template <bool POST, bool LAST, int FMT = 4, int LIVE = NST>
__device__ __forceinline__ void pipe_trip(f32x16 (&acc)[4][4], TileRegs& r0, TileRegs& r1, const DmaPlan& P,
                                          const TileSrc& Scur, const TileSrc& Snext, bool next_ok,
                                          const ReadPlan& R, lds_cptr lds, int kt0, int nkt) {
    static_assert(LIVE >= 1 && LIVE <= NST && (LIVE == NST || LAST), "dead K tiles only in a tile's one trip");
    pipe_iter<0, POST, LAST, FMT, (0 < LIVE), (1 < LIVE)>(acc, r0, r1, P, Scur, Snext, next_ok, R, lds, kt0 + 0, nkt);
    pipe_iter<1, POST, LAST, FMT, (1 < LIVE), (2 < LIVE)>(acc, r1, r0, P, Scur, Snext, next_ok, R, lds, kt0 + 1, nkt);
    pipe_iter<2, POST, LAST, FMT, (2 < LIVE), (3 < LIVE)>(acc, r0, r1, P, Scur, Snext, next_ok, R, lds, kt0 + 2, nkt);
    pipe_iter<3, POST, LAST, FMT, (3 < LIVE), true>(acc, r1, r0, P, Scur, Snext, next_ok, R, lds, kt0 + 3, nkt);
}

template <bool VEC_STORE, int FMT>
__global__ __launch_bounds__(256, 1) void gemm_pipe_kernel(const uint8_t* __restrict__ aq,
                                                           const uint8_t* __restrict__ as,
                                                           const uint8_t* __restrict__ bq,
                                                           const uint8_t* __restrict__ bs, int M, int N, int K,
                                                           uint16_t* __restrict__ out, int64_t ldo, int tiles_m,
                                                           int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(1024))) char lds_raw[NST * STAGE];
    lds_cptr lds = (lds_cptr)lds_raw;

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
    const int64_t m0 = (int64_t)tm * PBM, n0 = (int64_t)tn * PBN;

    const int nkt = k_tiles<FMT>(K);   // K tiles (= code tiles per 16-row group)
    const int kt2 = (K + 255) >> 8;     // 256-wide scale tiles per 128-row group
    const DmaPlan P = dma_plan(lane, wave, nkt, kt2, lds);
    const ReadPlan R = read_plan(lane, wm, wn);
    const TileSrc S = tile_src(aq, as, bq, bs, M, N, nkt, kt2, m0, n0, wave);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // prologue: tiles 0..3 in flight, then tile 0 into registers
    dma_tile_all<0, FMT>(P, S, 0, 0 < nkt);
    dma_tile_all<1, FMT>(P, S, 1, 1 < nkt);
    dma_tile_all<2, FMT>(P, S, 2, 2 < nkt);
    dma_tile_all<3, FMT>(P, S, 3, 3 < nkt);
    wait_vmcnt<prologue_wait<FMT>(), true>();
    __syncthreads();
    TileRegs r0, r1;
#pragma unroll
    for (int q = 0; q < 24; ++q) read_one<FMT>(r0, R, lds, q);
    order_point();

    const int trips = (nkt + NST - 1) / NST;
    for (int tr = 0; tr < trips; ++tr) pipe_trip<false, false, FMT>(acc, r0, r1, P, S, S, false, R, lds, tr * NST, nkt);
    // drain the DMA of the (empty) tiles past the end before the workgroup can exit
    wait_vmcnt<0>();

    // ---- epilogue: fp32 -> bf16 (nearest even).  acc[i][j][g*4 + e] is output row
    // m0 + wm*128 + i*32 + lane%32, column n0 + wn*128 + j*32 + g*8 + (lane/32)*4 + e.
    const int64_t mrow = m0 + wm * 128 + (lane & 31);
    const int64_t ncol = n0 + wn * 128 + (lane >> 5) * 4;
    const bool full = (m0 + wm * 128 + 128 <= M) && (n0 + wn * 128 + 128 <= N);
    if (VEC_STORE && full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t* orow = out + (mrow + i * 32) * ldo + ncol;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x16& c = acc[i][j];
                    uint2 v;
                    v.x = f32x2_to_bf16x2_rne(c[gq * 4 + 0], c[gq * 4 + 1]);
                    v.y = f32x2_to_bf16x2_rne(c[gq * 4 + 2], c[gq * 4 + 3]);
                    *reinterpret_cast<uint2*>(orow + j * 32 + gq * 8) = v;
                }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mrow + i * 32;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t n = ncol + j * 32 + gq * 8 + e;
                        if (n < N) out[m * ldo + n] = f32_to_bf16_rne(acc[i][j][gq * 4 + e]);
                    }
        }
    }
}



// ---------------------------------------------------------------------------
// Persistent kernel: one workgroup per CU walks its output tiles (logical tile
// slot, slot + G, ... with G the grid size).  The K loop runs on across tiles:
// the last trip of a tile issues the DMA of K tiles 0..3 of the next tile
// (every tile runs a multiple of 4 K tiles, those past K reading as zero, so
// K tile k of every tile lives in stage k % 4) and
// its last iteration reads the next tile's K tile 0 into registers.  Between
// the two the finished tile is written through LDS stage 0 (free at that
// point): exactly 32 16-byte buffer stores per wave, bounded by a per-tile
// descriptor so rows and columns outside the output are dropped; they drain
// while the next tile's MFMAs run, and the first three waits of the next tile
// allow for them.  Needs N % 8 == 0 (16-byte output chunks).
// ---------------------------------------------------------------------------

// fp32 x4 -> 4 bf16 (nearest even) in two dwords.
__device__ __forceinline__ void pack4(const f32x16& c, int g, unsigned& lo, unsigned& hi) {
    lo = f32x2_to_bf16x2_rne(c[g * 4 + 0], c[g * 4 + 1]);
    hi = f32x2_to_bf16x2_rne(c[g * 4 + 2], c[g * 4 + 3]);
}

// Epilogue of one tile, staged through LDS so that every store writes whole
// 128-byte lines.  Each wave owns a 9 KB slice of the stage that is free at a
// tile boundary and goes through its 128 x 128 outputs in four passes of 32
// rows: lanes l and l+32 hold columns 0-3 and 4-7 of each 8-column group of
// row l % 32; a permlane32 swap gives each lane 8 consecutive columns (16
// bytes), written to the slice row-major; read back, 16 lanes cover one
// 256-byte row of the wave's block, so a store moves 4 rows x 256 contiguous
// bytes.  Stores carry the non-temporal hint (the output is not read again
// here; operand panels keep the L2).  Chunks outside the output get an offset
// past the descriptor's end and are dropped.  Needs N % 8 == 0.
constexpr int kEpiPitch = 272;          // bytes per staged row: 256 + 16 (conflict-free 16-byte writes)
constexpr int kEpiSlice = STAGE / 4;    // per-wave slice, 32 * 272 <= 9216
constexpr int kStoreNT = 2;             // buffer store cache policy: non-temporal
static_assert(32 * kEpiPitch <= kEpiSlice, "a pass of 32 staged rows fits the wave's slice");

__device__ __forceinline__ void persist_epilogue(const f32x16 (&acc)[4][4], uint16_t* out, int64_t ldo, int M, int N,
                                                 int64_t m0, int64_t n0, int wm, int wn, lds_cptr slice_c) {
    typedef __attribute__((address_space(3))) char* lds_ptr;
    typedef __attribute__((address_space(3))) u32x4* lds_v4;
    lds_ptr slice = (lds_ptr)slice_c;
    // 32-bit tile-local arithmetic: the launcher guarantees 256 * ldo * 2 < 2^31
    const int rows_left = (int)min((int64_t)M - m0, (int64_t)PBM);  // >= 1
    const int cols_left = (int)min((int64_t)N - n0, (int64_t)PBN);
    const int row_bytes = (int)(ldo * 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        out + m0 * ldo + n0, (short)0, rows_left * row_bytes, (int)kRsrcWord3);
    // the lane id is recomputed here (volatile, so it is neither hoisted nor
    // merged with an earlier copy): the per-lane offsets below are then formed
    // once per tile instead of living in registers across the main loop
    int lane_v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_v));
    const int h = lane_v >> 5;
    const int lr = lane_v & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                unsigned x0, x1, y0, y1;
                pack4(acc[i][j], 2 * p, x0, x1);      // columns 16p + 4h .. +3
                pack4(acc[i][j], 2 * p + 1, y0, y1);  // columns 16p + 8 + 4h .. +3
                const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                // lower lanes: own x then partner's x; upper lanes: partner's y then own y
                const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
                const int c = j * 32 + p * 16 + h * 8;  // column within the wave's block
                *reinterpret_cast<lds_v4>(slice + lr * kEpiPitch + c * 2) = v;
            }
        }
        wait_lgkm0();  // this wave's slice is written (the slice is private: no barrier)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int rr = k * 4 + (lane_v >> 4);  // row within the pass
            const int ch = lane_v & 15;            // 16-byte chunk of the wave's 256-byte row
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                slice + rr * kEpiPitch + ch * 16);
            const int r = wm * 128 + i * 32 + rr;  // tile-local row and column
            const int c = wn * 128 + ch * 8;
            const int off = (r < rows_left && c < cols_left) ? r * row_bytes + c * 2 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, kStoreNT);
        }
        wait_lgkm0();  // read back before the next pass overwrites the slice
    }
}

// One product of a persistent launch: out[M, N] (row stride ldo) = A . B^T over
// K, in tiles_m x tiles_n output tiles, run by G workgroups.
struct PersistProblem {
    const uint8_t* aq;
    const uint8_t* as;
    const uint8_t* bq;
    const uint8_t* bs;
    uint16_t* out;
    int64_t ldo;
    int M, N, K, tiles_m, tiles_n, G;
};

// XCD-aware slot of workgroup `bid` among G workgroups spread over nx XCDs
// (bid % nx is the XCD): each XCD takes a contiguous range of slots per round.
__device__ __forceinline__ int xcd_remap_n(int bid, int G, int nx) {
    const int x = bid % nx, idx = bid / nx;
    return x * (G / nx) + min(x, G % nx) + idx;
}

// PAIR: two independent products of the same K-tile parity (SINGLE) in one
// grid of 8 x 32 workgroups: the workgroups of XCDs 0 .. split_xcds-1 run p0,
// the others p1 (each XCD's L2 then holds the panels of one product); the
// workgroups beyond a product's G leave at once.  Without PAIR, p0 runs on the
// whole grid (G = gridDim.x).
// LIVE (one trip per tile only): the K tiles that hold contraction data, the
// larger of the two products' counts when PAIR.
template <bool SINGLE, int FMT, bool PAIR, int LIVE = NST>
__global__ __launch_bounds__(256, 1) void gemm_persist_kernel(PersistProblem p0, PersistProblem p1, int split_xcds,
                                                              int group_m) {
    static_assert(SINGLE || LIVE == NST, "dead K tiles only with one trip per tile");
    __shared__ __attribute__((aligned(1024))) char lds_raw[NST * STAGE];
    lds_cptr lds = (lds_cptr)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    int slot, G;
    PersistProblem Q = p0;
    if constexpr (PAIR) {
        const int xcd = blockIdx.x & 7;
        const bool second = xcd >= split_xcds;
        if (second) Q = p1;
        const int nx = second ? 8 - split_xcds : split_xcds;
        const int lb = (blockIdx.x >> 3) * nx + (xcd - (second ? split_xcds : 0));
        G = Q.G;
        if (lb >= G) return;
        slot = xcd_remap_n(lb, G, nx);
    } else {
        G = gridDim.x;
        slot = xcd_remap(blockIdx.x, G);  // each XCD takes a contiguous range of slots per round
    }
    const uint8_t* __restrict__ aq = Q.aq;
    const uint8_t* __restrict__ as = Q.as;
    const uint8_t* __restrict__ bq = Q.bq;
    const uint8_t* __restrict__ bs = Q.bs;
    uint16_t* __restrict__ out = Q.out;
    const int64_t ldo = Q.ldo;
    const int M = Q.M, N = Q.N, K = Q.K, tiles_m = Q.tiles_m, tiles_n = Q.tiles_n;
    const int total = tiles_m * tiles_n;

    const int nkt = k_tiles<FMT>(K);
    const int trips = (nkt + NST - 1) / NST;  // 1 with SINGLE, else >= 2; K tiles past nkt read as zero
    const int kt2 = (K + 255) >> 8;
    const DmaPlan P = dma_plan(lane, wave, nkt, kt2, lds);
    const ReadPlan R = read_plan(lane, wm, wn);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    int tm = 0, tn = 0;
    tile_coords(slot, tiles_m, tiles_n, group_m, tm, tn);
    int64_t m0 = (int64_t)tm * PBM, n0 = (int64_t)tn * PBN;
    TileSrc S = tile_src(aq, as, bq, bs, M, N, nkt, kt2, m0, n0, wave);

    // first tile: K tiles 0..3 in flight, K tile 0 into registers, then its first trip
    dma_tile_all<0, FMT>(P, S, 0, 0 < nkt);
    dma_tile_all<1, FMT>(P, S, 1, 1 < nkt);
    dma_tile_all<2, FMT>(P, S, 2, 2 < nkt);
    dma_tile_all<3, FMT>(P, S, 3, 3 < nkt);
    wait_vmcnt<prologue_wait<FMT>(), true>();
    __syncthreads();
    TileRegs r0, r1;
#pragma unroll
    for (int q = 0; q < 24; ++q) read_one<FMT>(r0, R, lds, q);
    order_point();

    // one tile's last trip, then its epilogue; returns false after the last tile
    auto finish_tile = [&](int t, auto post_tag, int kt0) {
        constexpr bool POST = decltype(post_tag)::value;
        // the last trip streams K tiles 0..3 of the next tile into stages 0..3
        // (every tile runs a multiple of 4 K tiles, so K tile k of every tile
        // lives in stage k % 4) and ends with the next tile's K tile 0 in r0
        const int64_t em0 = m0, en0 = n0;
        const int tnext = t + G;
        const bool more = tnext < total;
        if (more) tile_coords(tnext, tiles_m, tiles_n, group_m, tm, tn);
        m0 = (int64_t)tm * PBM;
        n0 = (int64_t)tn * PBN;
        const TileSrc Sn = tile_src(aq, as, bq, bs, M, N, nkt, kt2, m0, n0, wave);
        pipe_trip<POST, true, FMT, LIVE>(acc, r0, r1, P, S, Sn, more, R, lds, kt0, nkt);
        S = Sn;

        // stage 0 (the next tile's K tile 0, now in r0) is free until the next
        // DMA into it, after the first barrier of the next trip; every wave's
        // reads of it must be done before the epilogue writes its slice
        wait_lgkm0();
        __syncthreads();
        persist_epilogue(acc, out, ldo, M, N, em0, en0, wm, wn, lds + wave * kEpiSlice);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
        order_point();
        return more;
    };

    if constexpr (SINGLE) {
        // one trip per tile (K <= 512): the first tile's trip is not POST, the others are
        if (finish_tile(slot, std::false_type{}, 0)) {
            for (int t = slot + G;; t += G)
                if (!finish_tile(t, std::true_type{}, 0)) break;
        }
    } else {
        pipe_trip<false, false, FMT>(acc, r0, r1, P, S, S, false, R, lds, 0, nkt);
        for (int t = slot;;) {
            // trip 0 of tile t is done; K tiles 4..7 are in flight or landed
            for (int tr = 1; tr < trips - 1; ++tr)
                pipe_trip<false, false, FMT>(acc, r0, r1, P, S, S, false, R, lds, tr * NST, nkt);
            if (!finish_tile(t, std::false_type{}, (trips - 1) * NST)) break;
            t += G;
            // trip 0 of the next tile; its first three waits allow for the 32 stores
            pipe_trip<true, false, FMT>(acc, r0, r1, P, S, S, false, R, lds, 0, nkt);
        }
    }
    // drain the last (empty) prefetch and the last stores
    wait_vmcnt<0>();
}

}  // namespace mx

namespace mx {

// Tiles are ordered in groups of 4 tile rows: an XCD's 32 concurrent tiles then span 4 A panels
// and 8 B panels (0.3-2% faster per GEMM than groups of 8 rows, 0.8% on the MLP, 8B attention
// and 70B steps; groups of 16 were slower).
constexpr int kGroupM = 4;

// Workgroups of a persistent launch of `tiles` tiles on `slots` CUs: as many rounds as the tiles
// need, every workgroup the same number of tiles.
static int64_t balanced_grid(int64_t tiles, int64_t slots) {
    const int64_t rounds = (tiles + slots - 1) / slots;
    return (tiles + rounds - 1) / rounds;
}

// 256 x 256 tiles need both sides >= 128 and enough tiles to fill half the CUs.
static bool uses_tiles(int64_t M, int64_t N, int64_t K, int64_t cus) {
    const int64_t tiles_m = (M + PBM - 1) / PBM, tiles_n = (N + PBN - 1) / PBN;
    return K > 0 && M >= 128 && N >= 128 && tiles_m * tiles_n * 2 >= cus;
}

// The persistent kernel needs 16-byte aligned output rows, N % 8 == 0, and a tile's output
// bytes (256 rows) addressable by a 31-bit buffer offset.
static bool persist_ok(const uint16_t* o16, int64_t ldo, int64_t N) {
    return (reinterpret_cast<uintptr_t>(o16) & 15u) == 0 && (ldo & 7) == 0 && (N & 7) == 0 &&
           (int64_t)PBM * ldo * 2 < 0x7FFFFFF0ll;
}

// Two independent products in one persistent launch (XCDs split between them) or one after the
// other, by a cost model in K tiles per workgroup: a tile costs its K tiles (a multiple of 4)
// plus kEpiKTiles (its epilogue), and a second launch kLaunchKTiles more.  A launch whose
// balanced grid leaves CUs idle runs each round faster (the others clock higher under the power
// limit): measured 0.904x per round on 224 of 256 CUs and 0.816x on 192, i.e. about
// (grid / CUs)^0.7, which the model applies to each of the two launches, no lower than the
// 0.8x measured (the clock has a ceiling; smaller grids were not measured).  The pair is taken only
// when it comes out at least 1% cheaper: what it gains is the tail of a partial last round (8B
// QKV's dB, 384 tiles: -6.5% on dA + dB; the MLP down projection's dB, 896 tiles: -1.9%), while
// two large products in one launch share the caches between them (70B down, 3584 + 3584 tiles in
// even rounds either way: +1.3% paired; 4096 x 14336 over 128256 beside 128256 x 14336 over 4096:
// +7% paired).
constexpr int64_t kEpiKTiles = 1;
constexpr int64_t kLaunchKTiles = 3;
constexpr double kIdleCuExponent = 0.7;
constexpr double kIdleCuFloor = 0.8;

struct PairPlan {
    bool pair;
    int split_xcds;  // XCDs of the first product
    int64_t g0, g1;  // workgroups of each
};

static PairPlan plan_pair(int64_t tiles0, int64_t kt0, int64_t tiles1, int64_t kt1, int64_t cus) {
    PairPlan P{false, 0, 0, 0};
    constexpr int64_t kXcds = 8, kPerXcd = 32;
    if (cus != kXcds * kPerXcd) return P;
    const int64_t c0 = kt0 + kEpiKTiles, c1 = kt1 + kEpiKTiles;
    const auto rounds = [](int64_t t, int64_t g) { return (t + g - 1) / g; };
    // one launch alone: its rounds, each shortened when its balanced grid leaves CUs idle
    const auto alone = [&](int64_t t, int64_t c) {
        const double busy = (double)balanced_grid(t, cus) / (double)cus;
        return (double)(rounds(t, cus) * c) * std::max(std::pow(busy, kIdleCuExponent), kIdleCuFloor);
    };
    // one after the other: both launches and one more launch cost than the pair
    const double seq = alone(tiles0, c0) + alone(tiles1, c1) + (double)kLaunchKTiles;
    double best = seq;
    for (int s = 1; s < kXcds; ++s) {
        const int64_t w0 = s * kPerXcd, w1 = (kXcds - s) * kPerXcd;
        const double t = (double)std::max(rounds(tiles0, w0) * c0, rounds(tiles1, w1) * c1);
        if (t < best && t <= 0.99 * seq) {
            best = t;
            P = PairPlan{true, s, balanced_grid(tiles0, w0), balanced_grid(tiles1, w1)};
        }
    }
    return P;
}

// The paired launch of two MXFP4 products (outputs assumed to meet persist_ok): both on the
// tiled kernel, with the same trip structure (one trip per tile or several), and cheaper than
// two launches by the model.
static PairPlan plan_pair_for(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1, int64_t cus) {
    if (M0 <= 0 || N0 <= 0 || M1 <= 0 || N1 <= 0 || !uses_tiles(M0, N0, K0, cus) || !uses_tiles(M1, N1, K1, cus))
        return PairPlan{false, 0, 0, 0};
    const int64_t nkt0 = (K0 + PBK - 1) / PBK, nkt1 = (K1 + PBK - 1) / PBK;
    const int64_t tiles0 = ((M0 + PBM - 1) / PBM) * ((N0 + PBN - 1) / PBN);
    const int64_t tiles1 = ((M1 + PBM - 1) / PBM) * ((N1 + PBN - 1) / PBN);
    if ((nkt0 <= NST) != (nkt1 <= NST) || tiles0 > 0x7FFFFFFF || tiles1 > 0x7FFFFFFF) return PairPlan{false, 0, 0, 0};
    const auto kt4 = [](int64_t n) { return (n + NST - 1) / NST * NST; };  // K tiles a tile runs
    return plan_pair(tiles0, kt4(nkt0), tiles1, kt4(nkt1), cus);
}

// The persistent kernel for nkt K tiles per tile (the larger count of a pair): one trip per
// tile up to NST K tiles, with the MFMAs of the K tiles past K left out.
using PersistKernel = void (*)(PersistProblem, PersistProblem, int, int);
template <int FMT, bool PAIR>
static PersistKernel persist_kernel(int64_t nkt) {
    switch (nkt) {
    case 1: return gemm_persist_kernel<true, FMT, PAIR, 1>;
    case 2: return gemm_persist_kernel<true, FMT, PAIR, 2>;
    case 3: return gemm_persist_kernel<true, FMT, PAIR, 3>;
    case NST: return gemm_persist_kernel<true, FMT, PAIR, NST>;
    default: return gemm_persist_kernel<false, FMT, PAIR>;
    }
}

template <int FMT>
static hipError_t launch_gemm(const uint8_t* a8, const uint8_t* as8, const uint8_t* b8, const uint8_t* bs8, int64_t M,
                              int64_t N, int64_t K, uint16_t* o16, int64_t ldo, void* ws, int64_t ws_bytes,
                              hipStream_t stream) {
    const int64_t tiles_m = (M + PBM - 1) / PBM, tiles_n = (N + PBN - 1) / PBN;
    if (!uses_tiles(M, N, K, num_cus())) return mx_launch_skinny(a8, as8, b8, bs8, M, N, K, o16, ldo, FMT, ws, ws_bytes,
                                                                 stream);
    if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int group_m = kGroupM;
    const int64_t nkt = FMT == 8 ? (K + 63) / 64 : (K + 127) / 128;
    if (persist_ok(o16, ldo, N)) {
        // as many rounds as the tiles need on all CUs, spread evenly: every workgroup
        // gets the same number of tiles (896 tiles run as 224 x 4, not 256 x 3.5)
        const int64_t tiles_all = tiles_m * tiles_n;
        const int64_t grid = balanced_grid(tiles_all, num_cus());
        const PersistProblem p{a8, as8, b8, bs8, o16, ldo, (int)M, (int)N, (int)K, (int)tiles_m, (int)tiles_n,
                               (int)grid};
        auto kern = persist_kernel<FMT, false>(nkt);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream, p, p, 8, kGroupM);
        return hipGetLastError();
    }
    // 8-byte output stores need an 8-byte aligned start for every row
    const bool vec = (reinterpret_cast<uintptr_t>(o16) & 7u) == 0 && (ldo & 3) == 0;
    auto kern = vec ? gemm_pipe_kernel<true, FMT> : gemm_pipe_kernel<false, FMT>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream, a8, as8, b8, bs8, (int)M,
                       (int)N, (int)K, o16, ldo, (int)tiles_m, (int)tiles_n, group_m);
    return hipGetLastError();
}

}  // namespace mx

// fmt 4: both operands MXFP4; fmt 8: both MXFP8 (E4M3).  ws / ws_bytes: optional scratch
// for the split contraction of the skinny kernel (nullptr: no split).
extern "C" hipError_t mx_launch_gemm_ws(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                        int64_t N, int64_t K, void* out, int64_t ldo, int fmt, void* ws,
                                        int64_t ws_bytes, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const uint8_t *a8 = static_cast<const uint8_t*>(aq), *as8 = static_cast<const uint8_t*>(as);
    const uint8_t *b8 = static_cast<const uint8_t*>(bq), *bs8 = static_cast<const uint8_t*>(bs);
    uint16_t* o16 = static_cast<uint16_t*>(out);
    if (fmt == 8) return mx::launch_gemm<8>(a8, as8, b8, bs8, M, N, K, o16, ldo, ws, ws_bytes, stream);
    if (fmt == 4) return mx::launch_gemm<4>(a8, as8, b8, bs8, M, N, K, o16, ldo, ws, ws_bytes, stream);
    return hipErrorInvalidValue;
}

extern "C" hipError_t mx_launch_gemm_f(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                       int64_t N, int64_t K, void* out, int64_t ldo, int fmt, hipStream_t stream) {
    return mx_launch_gemm_ws(aq, as, bq, bs, M, N, K, out, ldo, fmt, nullptr, 0, stream);
}

extern "C" hipError_t mx_launch_gemm(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                     int64_t N, int64_t K, void* out, int64_t ldo, hipStream_t stream) {
    return mx_launch_gemm_f(aq, as, bq, bs, M, N, K, out, ldo, 4, stream);
}

// out0 = A0 . B0^T and out1 = A1 . B1^T (independent products, both MXFP4 or both MXFP8):
// one persistent launch when both use the tiled kernel with the same trip structure and the
// cost model favours it, else the two launches of mx_launch_gemm_ws in order (ws shared).
extern "C" hipError_t mx_launch_gemm_pair_ws(const void* aq0, const void* as0, const void* bq0, const void* bs0,
                                             int64_t M0, int64_t N0, int64_t K0, void* out0, int64_t ldo0,
                                             const void* aq1, const void* as1, const void* bq1, const void* bs1,
                                             int64_t M1, int64_t N1, int64_t K1, void* out1, int64_t ldo1, int fmt,
                                             void* ws, int64_t ws_bytes, hipStream_t stream) {
    using namespace mx;
    uint16_t *o0 = static_cast<uint16_t*>(out0), *o1 = static_cast<uint16_t*>(out1);
    const int64_t cus = num_cus();
    if (fmt == 4 && persist_ok(o0, ldo0, N0) && persist_ok(o1, ldo1, N1)) {
        const PairPlan P = plan_pair_for(M0, N0, K0, M1, N1, K1, cus);
        if (P.pair) {
            const PersistProblem p0{static_cast<const uint8_t*>(aq0), static_cast<const uint8_t*>(as0),
                                    static_cast<const uint8_t*>(bq0), static_cast<const uint8_t*>(bs0),
                                    o0, ldo0, (int)M0, (int)N0, (int)K0, (int)((M0 + PBM - 1) / PBM),
                                    (int)((N0 + PBN - 1) / PBN), (int)P.g0};
            const PersistProblem p1{static_cast<const uint8_t*>(aq1), static_cast<const uint8_t*>(as1),
                                    static_cast<const uint8_t*>(bq1), static_cast<const uint8_t*>(bs1),
                                    o1, ldo1, (int)M1, (int)N1, (int)K1, (int)((M1 + PBM - 1) / PBM),
                                    (int)((N1 + PBN - 1) / PBN), (int)P.g1};
            // both products have the same trip structure; one trip per tile runs the larger K-tile count
            auto kern = persist_kernel<4, true>(std::max((K0 + PBK - 1) / PBK, (K1 + PBK - 1) / PBK));
            hipLaunchKernelGGL(kern, dim3((unsigned)cus), dim3(256), 0, stream, p0, p1, P.split_xcds, kGroupM);
            return hipGetLastError();
        }
    }
    hipError_t e = mx_launch_gemm_ws(aq0, as0, bq0, bs0, M0, N0, K0, out0, ldo0, fmt, ws, ws_bytes, stream);
    if (e != hipSuccess) return e;
    return mx_launch_gemm_ws(aq1, as1, bq1, bs1, M1, N1, K1, out1, ldo1, fmt, ws, ws_bytes, stream);
}

// XCDs the paired launch of two MXFP4 products gives the first (16-byte aligned outputs, ldo =
// N), on a chip of 256 CUs (MI355X); 0 when they run as two launches.  Host only.
extern "C" int mx_gemm_pair_split(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1) {
    if (N0 % 8 != 0 || N1 % 8 != 0 || (int64_t)mx::PBM * N0 * 2 >= 0x7FFFFFF0ll ||
        (int64_t)mx::PBM * N1 * 2 >= 0x7FFFFFF0ll)
        return 0;
    const mx::PairPlan P = mx::plan_pair_for(M0, N0, K0, M1, N1, K1, 256);
    return P.pair ? P.split_xcds : 0;
}

// Workspace the split contraction of out[M, N] (contraction K) can use, sized for a chip of
// 256 CUs (MI355X); 0 when the launch would not split.  Host only.
extern "C" int64_t mx_gemm_split_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
    constexpr int64_t kCus = 256;
    if (M <= 0 || N <= 0 || K <= 0 || mx::uses_tiles(M, N, K, kCus)) return 0;
    return mx_skinny_split_bytes(M, N, K, fmt, kCus);
}
