/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 cast + block-scaled GEMM library.
 *
 * The operations are the ones the jax-aiter README lists for its MXFP4 path:
 *   - "MXFP4 Cast" (Supported ops table): BF16 to E2M1 elements with E8M0
 *     block scales, as a row copy (CastMxfp4JA) or as row plus transposed
 *     copies (CastMxfp4DualJA);
 *   - "FP4 GEMM (low-level)" (Supported ops table): a GEMM on pre-quantized
 *     fp4x2 operands with e8m0 block scales, BF16 out;
 *   - "FP4 GEMM (training)", gemm_fp4_bf16 (Supported ops table and the
 *     "MXFP4 training architecture" section): BF16 in/out, forward = cast
 *     activations, cast weights, GEMM; backward = cast the output gradient,
 *     then the dA and dB (NT wgrad) GEMMs on the same FP4 kernels.
 *
 * Quantization rule (block of 32 along the contraction dimension; the OCP
 * Microscaling conversion the README relies on):
 *   X = floor(log2(max |x| over the block)) - 2, clamped to [-127, 127];
 *   an all-zero block has X = -127; the scale byte is X + 127 (E8M0);
 *   each element is x / 2^X rounded to the nearest E2M1 value (ties to the
 *   even code, saturating at +-6), sign bit copied from x (so -0 and small
 *   negatives give code 0x8).  A block holding Inf/NaN gets scale 0xFF and
 *   codes 0; every GEMM output whose dot product takes in such a block is NaN.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE memory owned by the caller; the library
 *     never allocates, frees, synchronizes or copies between host and device.
 *   - Work is enqueued on `stream` (0 = the null stream) of the current device.
 *   - Return value: MXFP4_OK or a negative mxfp4_status.  Arguments are
 *     validated before anything is enqueued; on an error nothing is enqueued
 *     and no output is touched.
 *   - Calls are thread-safe; calls on different streams may run concurrently
 *     as long as their output buffers do not overlap.
 *
 * Quantized operand format ("MX operand", R rows, contraction length K,
 * K a multiple of 32).  Both parts are tiled so that the GEMM moves one
 * contiguous kilobyte per wave load:
 *   q : codes in 1 KB tiles of 16 rows x 128 elements.  With KT = ceil(K/128),
 *       element (r, k) sits in byte
 *         ((r/16) * KT + k/128) * 1024 + (r%16) * 64 + (k%128)/2
 *       low nibble for even k, high nibble for odd k.  Rows past R and
 *       elements past K hold code 0.  Size: ceil(R/16) * KT * 1024 bytes.
 *   s : E8M0 scales in 1 KB tiles of 128 rows x 256 elements.  With
 *       KT2 = ceil(K/256), the scale of (row r, block b = k/32) sits in byte
 *         ((r/128) * KT2 + b/8) * 1024 + ((r/32)%4) * 256 + (r%32) * 8
 *           + (b%2) * 4 + (b%8)/2
 *       so that one dword holds the scales a 32x32x64 scaled-MFMA lane needs
 *       for four consecutive 64-wide K steps.  Positions past R rows or K/32
 *       blocks hold 0.  Size: ceil(R/128) * KT2 * 1024 bytes.
 *   The row copy of x[R, C] is the MX operand (R rows, K = C).  The column
 *   copy is the MX operand (C rows, K = Rp) with Rp = ceil(R/32)*32: row c of
 *   it quantizes column c of x in blocks of 32 rows, rows R..Rp-1 taken as +0.
 *
 * MXFP8 operand (the FP8 dB variant, see MXFP4_STEP_FP8_WGRAD): the same
 * block scales (X = floor(log2 amax) - 8, byte X + 127, same scale tiles and
 * byte positions as above), E4M3 elements x / 2^X rounded to nearest even
 * and saturating at +-448, one code per byte.  Codes in 1 KB tiles of 16
 * rows x 64 elements: with KT8 = ceil(K/64), element (r, k) is byte
 *         ((r/16) * KT8 + k/64) * 1024 + (r%16) * 64 + k%64.
 *   Size: ceil(R/16) * KT8 * 1024 bytes.  A block holding Inf/NaN gets scale
 *   0xFF and codes 0, as for MXFP4.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXFP4_OK = 0,
    MXFP4_EINVAL = -1,   /* null pointer, negative size, size not a multiple of 32, ld too small */
    MXFP4_EALIGN = -2,   /* pointer not 16-byte aligned, or bf16 leading dimension not a multiple of 8 */
    MXFP4_EDEVICE = -3,  /* no device, or the current device is not gfx950 */
    MXFP4_ELAUNCH = -4,  /* the HIP runtime reported an error at launch */
    MXFP4_ERANGE = -5,   /* a size exceeds the supported range (see each entry point) */
    MXFP4_ESPACE = -6    /* the workspace is smaller than gemm_fp4_bf16_workspace_bytes() */
} mxfp4_status;

/* Sizes of one MX operand.  Host only; touches no device. */
typedef struct {
    int64_t rows;             /* R */
    int64_t k;                /* contraction length, a multiple of 32 */
    int64_t q_bytes;          /* ceil(R/16) * ceil(K/128) * 1024 */
    int64_t s_bytes;          /* ceil(R/128) * ceil(K/256) * 1024 */
    int64_t code_row_tiles;   /* ceil(R/16) */
    int64_t code_k_tiles;     /* ceil(K/128) */
    int64_t scale_row_tiles;  /* ceil(R/128) */
    int64_t scale_k_tiles;    /* ceil(K/256) */
} mxfp4_operand_layout;

/* Fill *out for an operand of `rows` rows and contraction length `k`.
 * Returns MXFP4_EINVAL for a null `out`, negative sizes or k % 32 != 0. */
int mxfp4_operand_layout_of(int64_t rows, int64_t k, mxfp4_operand_layout* out);

/* Sizes of both copies of a cast bf16 matrix x [rows, cols] (jax-aiter README,
 * "Quick start": quantize(w) returns an Mxfp4Tensor of row + column copies and
 * their scales).  Host only; touches no device. */
typedef struct {
    int64_t rows, cols;          /* x [rows, cols] */
    int64_t padded_rows;         /* ceil(rows/32) * 32: the column copy's contraction length */
    mxfp4_operand_layout row;    /* the row copy: operand (rows, K = cols) */
    mxfp4_operand_layout col;    /* the column copy: operand (cols, K = padded_rows) */
} mxfp4_layout_t;

/* Fill *out for x [rows, cols].  MXFP4_EINVAL for a null `out`, negative sizes
 * or cols % 32 != 0; MXFP4_ERANGE for rows or cols >= 2^31. */
int mxfp4_layout(int64_t rows, int64_t cols, mxfp4_layout_t* out);

/* Static description of a status code (never NULL). */
const char* mxfp4_status_string(int status);

/*
 * A1 -- row cast (jax-aiter README, Supported ops: "MXFP4 Cast", CastMxfp4JA).
 * x    : bf16 [rows, cols], row stride ldx elements (ldx >= cols, ldx % 8 == 0,
 *        x 16-byte aligned); cols % 32 == 0.
 * q, s : the MX operand (rows, K = cols), sizes from mxfp4_operand_layout_of;
 *        16-byte aligned.
 * rows == 0 or cols == 0 is a successful no-op.
 */
int mxfp4_cast(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, void* s, hipStream_t stream);

/*
 * A2 -- dual cast (jax-aiter README, Supported ops: "MXFP4 Cast",
 * CastMxfp4DualJA, BF16 to MXFP4 "with transpose"; the row + col copies of an
 * Mxfp4Tensor in the Quick start).  One read of x produces
 *   q_row, s_row : the row copy, MX operand (rows, K = cols)
 *   q_col, s_col : the column copy, MX operand (cols, K = ceil(rows/32)*32)
 * Requirements as for mxfp4_cast.
 */
int mxfp4_cast_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row, void* q_col,
                    void* s_col, hipStream_t stream);

/*
 * A2 for two tensors in one launch -- e.g. a product's A and W before the
 * forward GEMM (the training step's forward casts both).  Results are those
 * of mxfp4_cast_dual on (x0, ...) and on (x1, ...); each tensor's arguments
 * have the requirements of mxfp4_cast_dual, and a tensor with rows == 0 or
 * cols == 0 is skipped.  The two tensors' buffers must not overlap.
 */
int mxfp4_cast_dual_pair(const void* x0, int64_t rows0, int64_t cols0, int64_t ldx0, void* q_row0, void* s_row0,
                         void* q_col0, void* s_col0, const void* x1, int64_t rows1, int64_t cols1, int64_t ldx1,
                         void* q_row1, void* s_row1, void* q_col1, void* s_col1, hipStream_t stream);

/*
 * F2 -- Hadamard-transformed cast (jax-aiter README, "Quick start": in the
 * training recipe grad_out is cast with a Hadamard transform).  As
 * mxfp4_cast_dual when q_col / s_col are given, as mxfp4_cast when both are
 * NULL, except that every 32-element block of the row copy (transform_row !=
 * 0) and / or of the column copy (transform_col != 0, needs q_col, s_col) is
 * first multiplied by the 32-point Sylvester Walsh-Hadamard matrix H
 * (H[i][j] = (-1)^popcount(i & j), H H = 32 I) and divided by 2^shift:
 *   - the transform is evaluated in IEEE binary32 from the bf16 values by
 *     butterflies of half-width 1, 2, 4, 8, 16 in that order, each (u, w) ->
 *     (u + w, u - w); a column copy's padding rows enter as +0;
 *   - the result / 2^shift is quantized by the rule above (shared exponent
 *     from its amax, E2M1 nearest-even, sign kept); a block that becomes
 *     non-finite (bf16 Inf/NaN, binary32 overflow) gets scale 0xFF, codes 0.
 * Both operands of a GEMM contraction must carry the transform; shift = 5 on
 * one of them keeps their product.  0 <= shift <= 64; other requirements and
 * errors as mxfp4_cast_dual.
 */
int mxfp4_cast_hadamard(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row,
                        void* q_col, void* s_col, int transform_row, int transform_col, int shift,
                        hipStream_t stream);

/*
 * A3/A4 -- block-scaled GEMM, NT (jax-aiter README, Supported ops: "FP4 GEMM
 * (low-level)", gemm_fp4(a, b, a_scale, b_scale), and the A[M,K] @ B[N,K]^T
 * convention of its GEMM rows):
 *   out[m, n] = bf16_rne( sum_k dq(a)[m, k] * dq(b)[n, k] ),  fp32 accumulation
 * a_q, a_s : MX operand (M rows, K);   b_q, b_s : MX operand (N rows, K);
 *            all four 16-byte aligned (MXFP4_EALIGN otherwise)
 * out      : bf16 [M, N], row stride ldo >= N elements (2-byte aligned).
 * K % 32 == 0.  M or N == 0: no-op.  K == 0: out is filled with +0.
 * Limits: M, N < 2^31; K <= 2^23 = 8388608 (the tiled kernels address a
 * wave's operand loads with 32-bit offsets); MXFP4_ERANGE beyond.
 */
int mxfp4_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N, int64_t K,
                  void* out, int64_t ldo, hipStream_t stream);

/*
 * A5 -- NN form (jax-aiter README, "MXFP4 training architecture": the dA
 * GEMM, GemmFp4FwdJA(dA), on the same FP4 kernel):
 *   out[m, n] = sum_k dq(a)[m, k] * dq(b)[k, n]
 * with b given by its column copy (MX operand: N rows, contraction K), e.g.
 * dA[M,K] = dOut[M,N] . W[N,K] takes a = row copy of dOut and b = column copy
 * of W.  Same kernel and requirements as mxfp4_gemm_nt.
 */
int mxfp4_gemm_nn(const void* a_q, const void* a_s, const void* bcol_q, const void* bcol_s, int64_t M, int64_t N,
                  int64_t K, void* out, int64_t ldo, hipStream_t stream);

/*
 * A3 with a workspace -- the same product as mxfp4_gemm_nt (and, on a column
 * copy, mxfp4_gemm_nn), for outputs too small to fill the chip behind a long
 * contraction (A8: e.g. the dA of an LM head, 1..17 x 4096 or 4096 x 32
 * outputs over a contraction of 128256; 16384 x 128 outputs over 14336):
 * several workgroups then share each output block, write fp32 partial sums
 * to ws, and a second kernel adds them in a fixed order and rounds to bf16.
 * The result does not depend on the workspace beyond the tolerance of the
 * product (the split count changes only the fp32 summation order).
 * mxfp4_gemm_workspace_bytes: the bytes that split needs for these sizes (0
 *   when the launch does not split, or for invalid sizes).  Host only.
 * mxfp4_gemm_nt_ws: arguments and errors as mxfp4_gemm_nt; ws is device
 *   memory of ws_bytes, 16-byte aligned (MXFP4_EALIGN otherwise), or NULL.
 *   With fewer bytes than mxfp4_gemm_workspace_bytes (or NULL) the
 *   contraction is split only as far as ws holds the partials.  The
 *   workspace needs no initialization; calls sharing one ws must be ordered
 *   (e.g. on one stream).
 */
size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

int mxfp4_gemm_nt_ws(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N,
                     int64_t K, void* out, int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * A5 + A6 in one call -- two independent MXFP4 products, as the training
 * backward's dA = dOut . W and dB = dOut^T . A, which read the copies of one
 * dOut cast (jax-aiter README, "MXFP4 training architecture"):
 *   out0[M0, N0] = A0 . B0^T over K0,   out1[M1, N1] = A1 . B1^T over K1.
 * Each product's arguments, alignment, limits and errors as for
 * mxfp4_gemm_nt_ws (products 0, then 1, validated before anything is
 * enqueued); out0 and out1 must not overlap each other or any operand.
 * When both outputs take the tiled kernel (16-byte aligned rows, N % 8 == 0)
 * with the same trip structure and a cost model favours it, both run in one
 * persistent launch with the chip's 8 XCDs divided between them: what a
 * launch costs beyond its tile rounds (the pipeline's first fill, the last
 * round's output written back) is paid once and the rounds of the two
 * balance.  Otherwise the two products run as two mxfp4_gemm_nt_ws calls in
 * order, sharing ws.  Either way each output is bit-identical to its own
 * mxfp4_gemm_nt_ws call.
 * mxfp4_gemm_pair_split: the XCDs (of 8) the paired launch gives product 0
 * for these sizes (16-byte aligned outputs, ldo = N, a chip of 256 CUs); 0
 * when the products run as two launches, and for invalid sizes.  Host only.
 */
int mxfp4_gemm_nt_pair_ws(const void* a0_q, const void* a0_s, const void* b0_q, const void* b0_s, int64_t M0,
                          int64_t N0, int64_t K0, void* out0, int64_t ldo0, const void* a1_q, const void* a1_s,
                          const void* b1_q, const void* b1_s, int64_t M1, int64_t N1, int64_t K1, void* out1,
                          int64_t ldo1, void* ws, size_t ws_bytes, hipStream_t stream);

int mxfp4_gemm_pair_split(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1);

/*
 * F3 -- MXFP8 (E4M3) operands for the FP8 dB of the jax-aiter README,
 * "MXFP4 training architecture" (its backward runs dB as an FP8 dot while
 * the forward pass and dA stay FP4).  Argument rules, alignment and errors
 * as for the MXFP4 counterparts above; operands in the MXFP8 format above.
 *
 * mxfp8_operand_layout_of : sizes of an MXFP8 operand (code_k_tiles =
 *   ceil(k/64)); host only.
 * mxfp8_cast              : row copy of x as MXFP8.
 * mxfp8_cast_dual         : row and column copies, both MXFP8.
 * mxfp4_cast_dual_fp8col  : MXFP4 row copy and MXFP8 column copy in one pass
 *   (the activation / dOut cast of the FP8-dB step: the row copy feeds an
 *   FP4 product, the column copy the FP8 dB).
 * mxfp8_gemm_nt           : out[M, N] = bf16( A[M, K] . B[N, K]^T ) on two
 *   MXFP8 operands (fp32 accumulation, nearest-even bf16 output).
 */
int mxfp8_operand_layout_of(int64_t rows, int64_t k, mxfp4_operand_layout* out);

int mxfp8_cast(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, void* s, hipStream_t stream);

int mxfp8_cast_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row, void* q_col,
                    void* s_col, hipStream_t stream);

int mxfp4_cast_dual_fp8col(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row,
                           void* q_col, void* s_col, hipStream_t stream);

int mxfp8_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N, int64_t K,
                  void* out, int64_t ldo, hipStream_t stream);

/*
 * F4 -- fused producer + cast (jax-aiter README, Supported ops: SiLU-and-Mul
 * computes silu(x[:half]) * x[half:]; RMSNorm fuses square, mean, rsqrt and
 * scale; Fused Add+RMSNorm normalizes x + residual in one kernel).  These are
 * the steps that produce the A operand of the MLP GEMMs; here the cast reads
 * the producer's inputs and computes its BF16 output in registers, so that
 * output need never be stored and read back.  The quantized values are
 * exactly the producer's BF16 output (its exact result rounded once to bf16,
 * nearest even), so the copies equal mxfp4_cast / mxfp4_cast_dual of that
 * output bit for bit.
 *
 * Output copies (both entry points): q_row / s_row, the MXFP4 row copy,
 * operand (rows, K) with K the output width; with q_col / s_col (both or
 * neither) also the column copy, operand (K, ceil(rows/32)*32), in col_fmt 4
 * (MXFP4) or 8 (MXFP8, the FP8 dB variant); col_fmt is ignored without a
 * column copy.  y_out: optional bf16 [rows, K] contiguous, 16-byte aligned --
 * the producer's output itself, for callers that also need it.  Copies are
 * 16-byte aligned.  Errors as for mxfp4_cast; rows == 0 or K == 0 is a
 * successful no-op.
 *
 * mxfp4_silu_mul_cast: x bf16 [rows, 2f], row stride ldx (>= 2f, % 8 == 0),
 *   16-byte aligned; gate = columns 0..f-1, up = f..2f-1; f % 32 == 0.
 *   Output y = bf16(silu(gate) * up) [rows, f], silu(g) = g / (1 + e^-g).
 * mxfp4_rmsnorm_cast: x bf16 [rows, d] contiguous, d % 32 == 0; gamma bf16
 *   [d]; 0 <= eps (finite).  Without a residual h = x; with residual (bf16
 *   [rows, d] contiguous) h = bf16(x + residual), written to residual_out
 *   (required then; it may be the residual or x buffer itself, updated in
 *   place).  With eps = 0 an all-zero row gives rstd = inf and y = NaN, as
 *   the formula does.  rstd: double [rows], 8-byte aligned, required: gets
 *   1 / sqrt(mean(h^2) + eps) (the norm's saved statistic; the cast pass
 *   reads it).  Output y = bf16(h * rstd * gamma) [rows, d].  Two kernels:
 *   the row statistics (and residual sum), then the producing cast.
 */
int mxfp4_silu_mul_cast(const void* x, int64_t rows, int64_t f, int64_t ldx, void* q_row, void* s_row, void* q_col,
                        void* s_col, int col_fmt, void* y_out, hipStream_t stream);

int mxfp4_rmsnorm_cast(const void* x, const void* residual, const void* gamma, float eps, int64_t rows, int64_t d,
                       void* q_row, void* s_row, void* q_col, void* s_col, int col_fmt, void* residual_out,
                       void* rstd, void* y_out, hipStream_t stream);

/*
 * A7 -- workspace for gemm_fp4_bf16_fwd/bwd with activations [M, K] and
 * weights [N, K].  training != 0 sizes for fwd + bwd: it holds the row copies
 * of A and W, the saved column copies of A and W that the backward pass reads,
 * and the row and column copies of dOut.  training == 0 sizes for an
 * inference forward (row copies only).  Both also hold the partial sums of
 * the step's GEMMs where they split their contraction (the largest
 * mxfp4_gemm_workspace_bytes of the step's products).  Returns 0 for invalid
 * sizes.
 */
size_t gemm_fp4_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, int training);

/*
 * A7 -- forward of gemm_fp4_bf16 (jax-aiter README, Supported ops "FP4 GEMM
 * (training)" and "MXFP4 training architecture"):
 *   out[M, N] = bf16( cast(a)[M, K] . cast(w)[N, K]^T )
 * a : bf16 [M, K] contiguous;  w : bf16 [N, K] contiguous;  out : bf16 [M, N]
 * contiguous.  K % 32 == 0; with training != 0 also N % 32 == 0 (the backward
 * pass contracts over N).  Each product's contraction is at most 2^23 (K; in
 * training also N and ceil(M/32)*32), MXFP4_ERANGE beyond.  ws : device
 * workspace of ws_bytes >=
 * gemm_fp4_bf16_workspace_bytes(M, N, K, training) bytes, 256-byte aligned.
 * training != 0: a and w are dual-cast and their column copies stay in ws for
 * gemm_fp4_bf16_bwd; otherwise they are row-cast only.
 */
int gemm_fp4_bf16_fwd(const void* a, const void* w, int64_t M, int64_t N, int64_t K, void* out, void* ws,
                      size_t ws_bytes, int training, hipStream_t stream);

/*
 * A7 -- backward of gemm_fp4_bf16: dout bf16 [M, N] contiguous ->
 *   da[M, K] = bf16( cast(dout) . W )      (FP4 dA, NN on W's column copy)
 *   dw[N, K] = bf16( cast(dout)^T . A )    (FP4 dB, NT wgrad on column copies)
 * ws must be the workspace a training-mode gemm_fp4_bf16_fwd with the same
 * M, N, K filled (it reads the saved column copies and overwrites the dOut
 * copies).  Either of da / dw may be NULL to skip that product.
 */
int gemm_fp4_bf16_bwd(const void* dout, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* da,
                      void* dw, hipStream_t stream);

/*
 * Cached weight quantization (jax-aiter README, Quick start: a weight
 * quantizer, MXFP4Quantizer.for_weight(), turns W into an Mxfp4Tensor with
 * row and column copies, and WeightWorkspace.get_or_quantize(...) keeps it
 * for later GEMMs).  These are gemm_fp4_bf16_fwd / _bwd with W's cast
 * skipped: the caller passes W's copies, made once by mxfp4_cast_dual(w, N,
 * K, ...) and reused while W is unchanged (inference, gradient-accumulation
 * micro-batches).
 *
 * Workspace without W's slots: A's row (and, training, column) copy and
 * dOut's copies.  Returns 0 for invalid sizes.
 */
size_t gemm_fp4_bf16_workspace_bytes_qw(int64_t M, int64_t N, int64_t K, int training);

/*
 * Forward with a pre-quantized weight:
 *   out[M, N] = bf16( cast(a)[M, K] . W_row^T )
 * w_row_q, w_row_s : W's row copy, MX operand (N rows, K), 16-byte aligned,
 *                    read only.  Other arguments, requirements and errors as
 *                    gemm_fp4_bf16_fwd, with ws_bytes >=
 *                    gemm_fp4_bf16_workspace_bytes_qw(M, N, K, training).
 */
int gemm_fp4_bf16_fwd_qw(const void* a, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N, int64_t K,
                         void* out, void* ws, size_t ws_bytes, int training, hipStream_t stream);

/*
 * Backward with a pre-quantized weight (ws from a training
 * gemm_fp4_bf16_fwd_qw with the same M, N, K):
 *   da[M, K] = bf16( cast(dout) . W )  on W's column copy
 *   dw[N, K] = bf16( cast(dout)^T . A )
 * w_col_q, w_col_s : W's column copy, MX operand (K rows, ceil(N/32)*32),
 *                    needed only when da != NULL.  Otherwise as
 *                    gemm_fp4_bf16_bwd.
 */
int gemm_fp4_bf16_bwd_qw(const void* dout, const void* w_col_q, const void* w_col_s, int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, void* da, void* dw, hipStream_t stream);

/*
 * The gemm_fp4_bf16 step with options, as flags:
 *   MXFP4_STEP_TRAINING      : forward keeps the column copies for the backward pass;
 *   MXFP4_STEP_HADAMARD_GRAD : F2 recipe (needs TRAINING in the forward): the
 *     column copies of A and W carry the transform of mxfp4_cast_hadamard
 *     (shift 0) and both copies of dOut carry it with shift 5, so dA and dB
 *     contract transformed operands (same products, smaller quantization error
 *     for blocks with outliers);
 *   MXFP4_STEP_QUANTIZED_W   : W is given quantized (w == NULL, w_row_q /
 *     w_row_s in the forward, w_col_q / w_col_s in the backward, made by
 *     mxfp4_cast_dual, or by mxfp4_cast_hadamard with transform_col = 1,
 *     shift 0 under HADAMARD_GRAD); the workspace is
 *     gemm_fp4_bf16_workspace_bytes_qw's, else gemm_fp4_bf16_workspace_bytes';
 *   MXFP4_STEP_FP8_WGRAD     : F3, dB in MXFP8 (README "MXFP4 training
 *     architecture": the backward's dB is an FP8 dot).  Needs TRAINING in the
 *     forward; the column copies of A and dOut are MXFP8 (made in the same
 *     passes as the MXFP4 row copies) and dB is mxfp8_gemm_nt on them; the
 *     forward product and dA are unchanged.  Not combinable with
 *     HADAMARD_GRAD (MXFP4_EINVAL).
 * gemm_fp4_bf16_workspace_bytes_ex sizes the workspace for any flag set
 * (0 for invalid sizes or flags).
 * The backward pass takes the forward's flags.  Unknown flags: MXFP4_EINVAL.
 * gemm_fp4_bf16_fwd / _bwd / _fwd_qw / _bwd_qw are these with HADAMARD_GRAD
 * clear.
 */
#define MXFP4_STEP_TRAINING 1u
#define MXFP4_STEP_HADAMARD_GRAD 2u
#define MXFP4_STEP_QUANTIZED_W 4u
#define MXFP4_STEP_FP8_WGRAD 8u

size_t gemm_fp4_bf16_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, unsigned flags);

int gemm_fp4_bf16_fwd_ex(const void* a, const void* w, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N,
                         int64_t K, void* out, void* ws, size_t ws_bytes, unsigned flags, hipStream_t stream);

int gemm_fp4_bf16_bwd_ex(const void* dout, const void* w_col_q, const void* w_col_s, int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, void* da, void* dw, unsigned flags, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * inference forward of gemm_fp4_bf16_fwd_qw (training = 0) with no workspace
 * argument.  The forward's scratch -- A's row copy, and the partial sums where
 * the GEMM splits its contraction over workgroups -- goes into a device array
 * of MXFP4_NOALLOC_SCRATCH_BYTES that the library itself holds on each GPU it
 * runs on until the process ends; nothing is allocated per call.
 *   out[M, N] = bf16( cast(a)[M, K] . W_row^T )
 * Arguments, requirements and errors as gemm_fp4_bf16_fwd_qw, plus
 * MXFP4_ERANGE when that scratch (gemm_fp4_bf16_workspace_bytes_qw(M, N, K, 0)
 * bytes, about 0.53 * M * K plus any split) exceeds
 * MXFP4_NOALLOC_SCRATCH_BYTES, and
 * MXFP4_ELAUNCH if the runtime cannot give the array's device address.
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int gemm_fp4_bf16_fwd_qw_noalloc(const void* a, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N,
                                 int64_t K, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
