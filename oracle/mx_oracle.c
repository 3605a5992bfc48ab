/*
 * CPU oracle for the MXFP4 block-scaled cast and the block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (jax-aiter README, "Supported ops" table, rows "MXFP4
 * Cast" and "FP4 GEMM (low-level)": BF16 is cast to E2M1 elements with one
 * E8M0 block scale, two E2M1 codes per byte; the GEMM consumes those packed
 * operands with their e8m0 scales and returns BF16):
 *
 *   block   : 32 consecutive elements along the contraction dimension
 *   scale   : X = floor(log2(max |x| over the block)) - 2, clamped to
 *             [-127, 127]; an all-zero block gets X = -127; the stored E8M0
 *             byte is X + 127 (OCP Microscaling v1.0 conversion rule)
 *   element : x / 2^X rounded to the nearest E2M1 value, ties to the code
 *             whose mantissa bit is 0, magnitudes past 6 go to 6; the sign
 *             bit is the sign bit of x (so -0 and small negatives give 0x8)
 *   packing : byte j of a row holds element 2j in bits 0..3 and element 2j+1
 *             in bits 4..7
 *   GEMM    : out[m,n] = sum over blocks b of 2^(Xa+Xb) * sum_{k in b}
 *             e2m1(a[m,k]) * e2m1(b[n,k]); the inner sums are formed exactly
 *             as integers (2*e2m1 is an integer) and the blocks are added in
 *             fp64 in increasing b.
 *
 * A block that holds an Inf or NaN gets scale byte 0xFF (the E8M0 NaN) and
 * element codes 0; a GEMM output that touches a 0xFF scale is NaN.
 *
 * Plain C99 + pthreads.  Row-parallel; no blocking or reordering of the sums
 * beyond the definition above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MXO_BLOCK 32

/* ---- bf16 decoding (IEEE-754 binary32 with the low 16 bits dropped) ---- */

static int bf16_is_finite(uint16_t h) { return ((h >> 7) & 0xFF) != 0xFF; }

/* Exact value of a finite bf16 as a double. */
static double bf16_value(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 7) & 0xFF;
    int m = h & 0x7F;
    double mag;
    if (e == 0) mag = ldexp((double)m, -133);          /* subnormal: m * 2^-126 * 2^-7 */
    else mag = ldexp((double)(128 + m), e - 127 - 7);  /* normal: (1 + m/128) * 2^(e-127) */
    return sign ? -mag : mag;
}

/* ---- E2M1 (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit) ---- */

/* Magnitude of E2M1 code c (0..7) as a double, from the bit fields. */
static double e2m1_magnitude(int c) {
    int e = (c >> 1) & 3;
    int m = c & 1;
    if (e == 0) return 0.5 * m;                       /* subnormal: 2^(1-1) * m/2 */
    return ldexp(1.0 + 0.5 * m, e - 1);
}

/* Nearest E2M1 magnitude code for a = |v|; ties go to the even code. */
static int e2m1_round(double a) {
    if (a > 6.0) return 7;   /* saturation: anything past the largest E2M1 magnitude maps to it */
    int best = 0;
    double bestd = fabs(a - e2m1_magnitude(0));
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - e2m1_magnitude(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* floor(log2(a)) for a finite a > 0, exactly (frexp returns a = f * 2^e, f in [0.5, 1)). */
static int floor_log2(double a) {
    int e;
    frexp(a, &e);
    return e - 1;
}

/* Quantize one block of n (<= 32) bf16 values read with stride `stride`;
 * positions n..31 are +0 (padding).  Writes 32 codes and returns the scale byte. */
static uint8_t quantize_block(const uint16_t* x, int64_t stride, int n, uint8_t codes[MXO_BLOCK]) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        uint16_t h = x[i * stride];
        if (!bf16_is_finite(h)) {
            memset(codes, 0, MXO_BLOCK);
            return 0xFF;
        }
        double a = fabs(bf16_value(h));
        if (a > amax) amax = a;
    }
    int X;
    if (amax == 0.0) {
        X = -127;
    } else {
        X = floor_log2(amax) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    for (int i = 0; i < MXO_BLOCK; ++i) {
        if (i >= n) { codes[i] = 0; continue; }
        uint16_t h = x[i * stride];
        double v = ldexp(fabs(bf16_value(h)), -X);   /* exact: power-of-two scaling */
        codes[i] = (uint8_t)(e2m1_round(v) | ((h >> 15) << 3));
    }
    return (uint8_t)(X + 127);
}

/* ---- thread fan-out ---- */

typedef void (*mxo_range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { mxo_range_fn fn; void* ctx; int64_t lo, hi; } mxo_job;

static void* mxo_run(void* p) {
    mxo_job* j = (mxo_job*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, mxo_range_fn fn, void* ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    mxo_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn; jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads; jobs[t].hi = n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, mxo_run, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ---- row copy: blocks along the contiguous dimension ---- */

typedef struct { const uint16_t* x; int64_t R, C, ldx; uint8_t *q, *s; } cast_ctx;

static void cast_rows_range(void* p, int64_t lo, int64_t hi) {
    cast_ctx* c = (cast_ctx*)p;
    uint8_t codes[MXO_BLOCK];
    int64_t nb = c->C / MXO_BLOCK;
    for (int64_t r = lo; r < hi; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            c->s[r * nb + b] = quantize_block(c->x + r * c->ldx + b * MXO_BLOCK, 1, MXO_BLOCK, codes);
            uint8_t* qrow = c->q + r * (c->C / 2) + b * (MXO_BLOCK / 2);
            for (int i = 0; i < MXO_BLOCK / 2; ++i) qrow[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

/* x: bf16 bits [R, C] with row stride ldx (elements); C % 32 == 0.
 * q: [R, C/2] packed codes; s: [R, C/32] scale bytes.  Returns 0 or -1. */
int mxo_cast_rows(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, uint8_t* s, int nthreads) {
    if (R < 0 || C < 0 || C % MXO_BLOCK != 0 || ldx < C) return -1;
    cast_ctx c = {x, R, C, ldx, q, s};
    parallel_for(R, nthreads, cast_rows_range, &c);
    return 0;
}

/* ---- column copy: blocks of 32 rows within each column, rows padded with +0 ---- */

static void cast_cols_range(void* p, int64_t lo, int64_t hi) {
    cast_ctx* c = (cast_ctx*)p;
    uint8_t codes[MXO_BLOCK];
    int64_t nb = (c->R + MXO_BLOCK - 1) / MXO_BLOCK;
    int64_t Rp = nb * MXO_BLOCK;
    for (int64_t col = lo; col < hi; ++col) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = b * MXO_BLOCK;
            int n = (int)((c->R - r0) < MXO_BLOCK ? (c->R - r0) : MXO_BLOCK);
            c->s[col * nb + b] = quantize_block(c->x + r0 * c->ldx + col, c->ldx, n, codes);
            uint8_t* qrow = c->q + col * (Rp / 2) + r0 / 2;
            for (int i = 0; i < MXO_BLOCK / 2; ++i) qrow[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

/* Column copy of x [R, C]: q [C, Rp/2], s [C, Rp/32] with Rp = ceil(R/32)*32. */
int mxo_cast_cols(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, uint8_t* s, int nthreads) {
    if (R < 0 || C < 0 || ldx < C) return -1;
    cast_ctx c = {x, R, C, ldx, q, s};
    parallel_for(C, nthreads, cast_cols_range, &c);
    return 0;
}

/* ---- Hadamard-transformed casts ----
 *
 * jax-aiter README, "Quick start" comment on gemm_fp4_bf16: in the training
 * recipe grad_out is cast with a Hadamard transform.  Nothing else is stated;
 * the reading implemented here:
 *   - the transform is the 32-point Sylvester Walsh-Hadamard matrix H
 *     (H[i][j] = (-1)^popcount(i & j), entries +-1, H H = 32 I), applied to
 *     each 32-element block along the contraction dimension (a column copy's
 *     padding rows enter as +0);
 *   - it is evaluated in IEEE binary32 from the exact binary32 values of the
 *     bf16 inputs, by the butterfly with half-widths 1, 2, 4, 8, 16 in that
 *     order, each butterfly replacing (u, w) by (u + w, u - w);
 *   - the transformed block divided by 2^shift (exactly, in double) is
 *     quantized by the rule above, the sign bit of each value giving the
 *     code's sign; a non-finite value (bf16 Inf/NaN, or binary32 overflow)
 *     makes the block scale 0xFF with codes 0.
 * Both operands of a contraction carry the transform; with shift 5 on one of
 * them (H^T H = 32 I) their product is that of the untransformed operands up
 * to quantization.
 */

/* In-place 32-point Walsh-Hadamard transform of v in binary32. */
static void fwht32_f32(float v[MXO_BLOCK]) {
    for (int h = 1; h < MXO_BLOCK; h <<= 1)
        for (int i = 0; i < MXO_BLOCK; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                const float u = v[j], w = v[j + h];
                v[j] = u + w;
                v[j + h] = u - w;
            }
}

/* bf16 bits -> binary32 (exact: bf16 is binary32 with the low 16 bits dropped). */
static float bf16_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* Quantize 32 real values (doubles) by the block rule; returns the scale byte. */
static uint8_t quantize_values(const double v[MXO_BLOCK], uint8_t codes[MXO_BLOCK]) {
    double amax = 0.0;
    for (int i = 0; i < MXO_BLOCK; ++i) {
        if (!isfinite(v[i])) {
            memset(codes, 0, MXO_BLOCK);
            return 0xFF;
        }
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    }
    int X;
    if (amax == 0.0) {
        X = -127;
    } else {
        X = floor_log2(amax) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    for (int i = 0; i < MXO_BLOCK; ++i)
        codes[i] = (uint8_t)(e2m1_round(ldexp(fabs(v[i]), -X)) | (signbit(v[i]) ? 8 : 0));
    return (uint8_t)(X + 127);
}

/* Transform and quantize one block of n (<= 32) bf16 values read with `stride`. */
static uint8_t quantize_block_hadamard(const uint16_t* x, int64_t stride, int n, int shift,
                                       uint8_t codes[MXO_BLOCK]) {
    float y[MXO_BLOCK];
    for (int i = 0; i < MXO_BLOCK; ++i) y[i] = i < n ? bf16_to_f32(x[i * stride]) : 0.0f;
    fwht32_f32(y);
    double v[MXO_BLOCK];
    for (int i = 0; i < MXO_BLOCK; ++i) v[i] = ldexp((double)y[i], -shift);
    return quantize_values(v, codes);
}

typedef struct { const uint16_t* x; int64_t R, C, ldx; int shift; uint8_t *q, *s; } hcast_ctx;

static void hcast_rows_range(void* p, int64_t lo, int64_t hi) {
    hcast_ctx* c = (hcast_ctx*)p;
    uint8_t codes[MXO_BLOCK];
    int64_t nb = c->C / MXO_BLOCK;
    for (int64_t r = lo; r < hi; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            c->s[r * nb + b] = quantize_block_hadamard(c->x + r * c->ldx + b * MXO_BLOCK, 1, MXO_BLOCK, c->shift, codes);
            uint8_t* qrow = c->q + r * (c->C / 2) + b * (MXO_BLOCK / 2);
            for (int i = 0; i < MXO_BLOCK / 2; ++i) qrow[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

static void hcast_cols_range(void* p, int64_t lo, int64_t hi) {
    hcast_ctx* c = (hcast_ctx*)p;
    uint8_t codes[MXO_BLOCK];
    int64_t nb = (c->R + MXO_BLOCK - 1) / MXO_BLOCK;
    int64_t Rp = nb * MXO_BLOCK;
    for (int64_t col = lo; col < hi; ++col) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = b * MXO_BLOCK;
            int n = (int)((c->R - r0) < MXO_BLOCK ? (c->R - r0) : MXO_BLOCK);
            c->s[col * nb + b] = quantize_block_hadamard(c->x + r0 * c->ldx + col, c->ldx, n, c->shift, codes);
            uint8_t* qrow = c->q + col * (Rp / 2) + r0 / 2;
            for (int i = 0; i < MXO_BLOCK / 2; ++i) qrow[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

/* Row copy of x [R, C] with every 32-block transformed, divided by 2^shift, quantized.
 * Same output shapes as mxo_cast_rows.  0 <= shift <= 64. */
int mxo_cast_rows_hadamard(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int shift, uint8_t* q, uint8_t* s,
                           int nthreads) {
    if (R < 0 || C < 0 || C % MXO_BLOCK != 0 || ldx < C || shift < 0 || shift > 64) return -1;
    hcast_ctx c = {x, R, C, ldx, shift, q, s};
    parallel_for(R, nthreads, hcast_rows_range, &c);
    return 0;
}

/* Column copy of x [R, C] (blocks of 32 rows, rows padded with +0) with the transform. */
int mxo_cast_cols_hadamard(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int shift, uint8_t* q, uint8_t* s,
                           int nthreads) {
    if (R < 0 || C < 0 || ldx < C || shift < 0 || shift > 64) return -1;
    hcast_ctx c = {x, R, C, ldx, shift, q, s};
    parallel_for(C, nthreads, hcast_cols_range, &c);
    return 0;
}

/* The binary32 transform alone, on n blocks of 32 floats (for the tests). */
int mxo_fwht32(const float* in, float* out, int64_t nblocks) {
    if (nblocks < 0) return -1;
    for (int64_t b = 0; b < nblocks; ++b) {
        float v[MXO_BLOCK];
        memcpy(v, in + b * MXO_BLOCK, sizeof v);
        fwht32_f32(v);
        memcpy(out + b * MXO_BLOCK, v, sizeof v);
    }
    return 0;
}

/* ---- MXFP8: E4M3 elements with E8M0 block scales ----
 *
 * The pages run dB in FP8 (README "MXFP4 training architecture": hipBLASLt
 * FP8 dB; the 8B recipe note: FP8 current scaling).  This oracle implements
 * the block-scaled FP8 form (OCP Microscaling v1.0, MXFP8 with E4M3), the FP8
 * format the MI355X scaled MFMA takes; a per-tensor scale is the case of
 * equal block scales:
 *   E4M3    : 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *             field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no
 *             infinities; largest magnitude 448 (code 0x7E)
 *   scale   : X = floor(log2 amax) - 8 (8 = exponent of 448), clamped to
 *             [-127, 127], -127 for an all-zero block; byte X + 127
 *   element : x / 2^X rounded to the nearest E4M3 value, ties to the even
 *             mantissa, magnitudes past 448 saturating to 448, sign bit of x
 *   codes   : one byte per element; a block with Inf/NaN gets scale 0xFF,
 *             codes 0
 *   GEMM    : every E4M3 value is an integer times 2^-9, so block sums are
 *             exact 64-bit integers, scaled by 2^(Xa + Xb - 18).
 */
#define MXO_E4M3_MAX_CODE 0x7E

/* Magnitude of E4M3 code c (0..0x7E) from its bit fields. */
static double e4m3_magnitude(int c) {
    int e = (c >> 3) & 0xF, m = c & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp((double)(8 + m), e - 10);
}

/* The same magnitude as an integer number of 2^-9 units. */
static int64_t e4m3_units(int c) {
    int e = (c >> 3) & 0xF, m = c & 7;
    if (e == 0) return m;
    return (int64_t)(8 + m) << (e - 1);
}

/* Nearest E4M3 magnitude code for a >= 0 (finite): the quantum of the binade
 * of a (2^-9 below 2^-6) divides a exactly; the quotient rounds to the nearest
 * integer, ties to even (= even mantissa); past 448 the code saturates. */
static int e4m3_round(double a) {
    if (a >= 448.0) return MXO_E4M3_MAX_CODE;
    int e = a > 0.0 ? floor_log2(a) : -6;
    if (e < -6) e = -6;
    double q = nearbyint(ldexp(a, 3 - e));      /* a / 2^(e-3), exact; default mode rounds ties to even */
    int code = (e + 7) * 8 + (int)q - 8;        /* q = 16 carries into the next binade */
    return code > MXO_E4M3_MAX_CODE ? MXO_E4M3_MAX_CODE : code;
}

static uint8_t quantize_block_fp8(const uint16_t* x, int64_t stride, int n, uint8_t codes[MXO_BLOCK]) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        uint16_t h = x[i * stride];
        if (!bf16_is_finite(h)) {
            memset(codes, 0, MXO_BLOCK);
            return 0xFF;
        }
        double a = fabs(bf16_value(h));
        if (a > amax) amax = a;
    }
    int X;
    if (amax == 0.0) {
        X = -127;
    } else {
        X = floor_log2(amax) - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    for (int i = 0; i < MXO_BLOCK; ++i) {
        if (i >= n) { codes[i] = 0; continue; }
        uint16_t h = x[i * stride];
        codes[i] = (uint8_t)(e4m3_round(ldexp(fabs(bf16_value(h)), -X)) | ((h >> 15) << 7));
    }
    return (uint8_t)(X + 127);
}

static void cast_rows_fp8_range(void* p, int64_t lo, int64_t hi) {
    cast_ctx* c = (cast_ctx*)p;
    int64_t nb = c->C / MXO_BLOCK;
    for (int64_t r = lo; r < hi; ++r)
        for (int64_t b = 0; b < nb; ++b)
            c->s[r * nb + b] = quantize_block_fp8(c->x + r * c->ldx + b * MXO_BLOCK, 1, MXO_BLOCK,
                                                  c->q + r * c->C + b * MXO_BLOCK);
}

/* MXFP8 row copy of x [R, C] (C % 32 == 0): q [R, C] codes, s [R, C/32]. */
int mxo_cast_rows_fp8(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, uint8_t* s, int nthreads) {
    if (R < 0 || C < 0 || C % MXO_BLOCK != 0 || ldx < C) return -1;
    cast_ctx c = {x, R, C, ldx, q, s};
    parallel_for(R, nthreads, cast_rows_fp8_range, &c);
    return 0;
}

static void cast_cols_fp8_range(void* p, int64_t lo, int64_t hi) {
    cast_ctx* c = (cast_ctx*)p;
    int64_t nb = (c->R + MXO_BLOCK - 1) / MXO_BLOCK;
    int64_t Rp = nb * MXO_BLOCK;
    for (int64_t col = lo; col < hi; ++col)
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = b * MXO_BLOCK;
            int n = (int)((c->R - r0) < MXO_BLOCK ? (c->R - r0) : MXO_BLOCK);
            c->s[col * nb + b] = quantize_block_fp8(c->x + r0 * c->ldx + col, c->ldx, n, c->q + col * Rp + r0);
        }
}

/* MXFP8 column copy of x [R, C]: q [C, Rp], s [C, Rp/32], Rp = ceil(R/32)*32, rows past R +0. */
int mxo_cast_cols_fp8(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, uint8_t* s, int nthreads) {
    if (R < 0 || C < 0 || ldx < C) return -1;
    cast_ctx c = {x, R, C, ldx, q, s};
    parallel_for(C, nthreads, cast_cols_fp8_range, &c);
    return 0;
}

/* out[r, k] = e4m3(q[r, k]) * 2^(s[r, k/32] - 127); NaN for scale 0xFF or a NaN code. */
int mxo_dequant_fp8(const uint8_t* q, const uint8_t* s, int64_t R, int64_t K, double* out) {
    if (R < 0 || K < 0 || K % MXO_BLOCK != 0) return -1;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) {
            int code = q[r * K + k];
            uint8_t sc = s[r * (K / MXO_BLOCK) + k / MXO_BLOCK];
            if (sc == 0xFF || (code & 0x7F) == 0x7F) { out[r * K + k] = NAN; continue; }
            double mag = e4m3_magnitude(code & 0x7F);
            out[r * K + k] = ldexp((code & 0x80) ? -mag : mag, (int)sc - 127);
        }
    return 0;
}

typedef struct {
    const uint8_t *qa, *sa, *qb, *sb;
    int64_t M, N, K;
    double *ref, *absref;
    int32_t* ub;   /* B as signed 2^-9 units, [N, K] */
} gemm8_ctx;

static int32_t e4m3_signed_units(uint8_t c) {
    int32_t v = (int32_t)e4m3_units(c & 0x7F);
    return (c & 0x80) ? -v : v;
}

static void unpack8_b_range(void* p, int64_t lo, int64_t hi) {
    gemm8_ctx* g = (gemm8_ctx*)p;
    for (int64_t n = lo; n < hi; ++n)
        for (int64_t k = 0; k < g->K; ++k) g->ub[n * g->K + k] = e4m3_signed_units(g->qb[n * g->K + k]);
}

static void gemm8_rows_range(void* p, int64_t lo, int64_t hi) {
    gemm8_ctx* g = (gemm8_ctx*)p;
    int64_t nb = g->K / MXO_BLOCK;
    int32_t* ua = (int32_t*)malloc((size_t)(g->K > 0 ? g->K : 1) * sizeof(int32_t));
    if (!ua) return;
    for (int64_t m = lo; m < hi; ++m) {
        for (int64_t k = 0; k < g->K; ++k) ua[k] = e4m3_signed_units(g->qa[m * g->K + k]);
        for (int64_t n = 0; n < g->N; ++n) {
            double acc = 0.0, aacc = 0.0;
            const int32_t* ub = g->ub + n * g->K;
            for (int64_t b = 0; b < nb; ++b) {
                uint8_t xa = g->sa[m * nb + b], xb = g->sb[n * nb + b];
                if (xa == 0xFF || xb == 0xFF) { acc = NAN; aacc = NAN; continue; }
                int64_t dot = 0, adot = 0;
                for (int i = 0; i < MXO_BLOCK; ++i) {
                    int64_t prod = (int64_t)ua[b * MXO_BLOCK + i] * (int64_t)ub[b * MXO_BLOCK + i];
                    dot += prod;
                    adot += prod < 0 ? -prod : prod;
                }
                int e = (int)xa + (int)xb - 254 - 18;
                acc += ldexp((double)dot, e);
                aacc += ldexp((double)adot, e);
            }
            g->ref[m * g->N + n] = acc;
            g->absref[m * g->N + n] = aacc;
        }
    }
    free(ua);
}

/* ref / absref [M, N] of out = A . B^T on MXFP8 operands (canonical row-major codes). */
int mxo_gemm_fp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t M, int64_t N,
                 int64_t K, double* ref, double* absref, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K % MXO_BLOCK != 0) return -1;
    gemm8_ctx g = {qa, sa, qb, sb, M, N, K, ref, absref, NULL};
    g.ub = (int32_t*)malloc((size_t)(N > 0 ? N : 1) * (size_t)(K > 0 ? K : 1) * sizeof(int32_t));
    if (!g.ub) return -1;
    parallel_for(N, nthreads, unpack8_b_range, &g);
    parallel_for(M, nthreads, gemm8_rows_range, &g);
    free(g.ub);
    return 0;
}

/* ---- dequantization ---- */

/* out[r, k] = e2m1(q[r,k]) * 2^(s[r, k/32] - 127), NaN for scale 0xFF.  K % 32 == 0. */
int mxo_dequant(const uint8_t* q, const uint8_t* s, int64_t R, int64_t K, double* out) {
    if (R < 0 || K < 0 || K % MXO_BLOCK != 0) return -1;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            int code = (q[r * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
            uint8_t sc = s[r * (K / MXO_BLOCK) + k / MXO_BLOCK];
            double mag = e2m1_magnitude(code & 7);
            double v = (code & 8) ? -mag : mag;
            out[r * K + k] = sc == 0xFF ? NAN : ldexp(v, (int)sc - 127);
        }
    }
    return 0;
}

/* ---- GEMM ---- */

/* 2 * e2m1 value of each code, an integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}. */
static int twice_e2m1(int code) {
    int v = (int)(2.0 * e2m1_magnitude(code & 7));
    return (code & 8) ? -v : v;
}

typedef struct {
    const uint8_t *qa, *sa, *qb, *sb;
    int64_t M, N, K;
    const int64_t *mi, *ni;   /* pair mode when non-null */
    double *ref, *absref;
    int8_t* ub;               /* B unpacked to 2*e2m1 values, [N, K] (full mode) */
} gemm_ctx;

/* One output: sum over blocks of 2^(Xa+Xb-2) * (exact integer dot of 2*a and 2*b). */
static void gemm_one(const gemm_ctx* g, const int8_t* ua, const int8_t* ub, int64_t m, int64_t n, double* ref, double* absref) {
    int64_t nb = g->K / MXO_BLOCK;
    double acc = 0.0, aacc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        uint8_t xa = g->sa[m * nb + b], xb = g->sb[n * nb + b];
        if (xa == 0xFF || xb == 0xFF) { acc = NAN; aacc = NAN; continue; }
        int32_t dot = 0, adot = 0;
        const int8_t* pa = ua + b * MXO_BLOCK;
        const int8_t* pb = ub + b * MXO_BLOCK;
        for (int i = 0; i < MXO_BLOCK; ++i) {
            int32_t p = (int32_t)pa[i] * (int32_t)pb[i];
            dot += p;
            adot += p < 0 ? -p : p;
        }
        int e = (int)xa + (int)xb - 254 - 2;
        acc += ldexp((double)dot, e);
        aacc += ldexp((double)adot, e);
    }
    *ref = acc;
    *absref = aacc;
}

static void unpack_row(const uint8_t* q, int64_t K, int8_t* u) {
    for (int64_t k = 0; k < K; ++k) u[k] = (int8_t)twice_e2m1((q[k / 2] >> (4 * (k & 1))) & 0xF);
}

static void unpack_b_range(void* p, int64_t lo, int64_t hi) {
    gemm_ctx* g = (gemm_ctx*)p;
    for (int64_t n = lo; n < hi; ++n) unpack_row(g->qb + n * (g->K / 2), g->K, g->ub + n * g->K);
}

static void gemm_rows_range(void* p, int64_t lo, int64_t hi) {
    gemm_ctx* g = (gemm_ctx*)p;
    int8_t* ua = (int8_t*)malloc((size_t)(g->K > 0 ? g->K : 1));
    for (int64_t m = lo; m < hi; ++m) {
        unpack_row(g->qa + m * (g->K / 2), g->K, ua);
        for (int64_t n = 0; n < g->N; ++n)
            gemm_one(g, ua, g->ub + n * g->K, m, n, &g->ref[m * g->N + n], &g->absref[m * g->N + n]);
    }
    free(ua);
}

/* ref[m,n], absref[m,n] (= sum_k |a_k b_k| of the dequantized operands) for
 * a: q [M, K/2], s [M, K/32]; b: q [N, K/2], s [N, K/32].  K % 32 == 0. */
int mxo_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t M, int64_t N,
             int64_t K, double* ref, double* absref, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K % MXO_BLOCK != 0) return -1;
    gemm_ctx g = {qa, sa, qb, sb, M, N, K, NULL, NULL, ref, absref, NULL};
    /* B is unpacked once, shared by all workers; each worker unpacks its A rows */
    g.ub = (int8_t*)malloc((size_t)(N > 0 ? N : 1) * (size_t)(K > 0 ? K : 1));
    if (!g.ub) return -1;
    parallel_for(N, nthreads, unpack_b_range, &g);
    parallel_for(M, nthreads, gemm_rows_range, &g);
    free(g.ub);
    return 0;
}

static void gemm_pairs_range(void* p, int64_t lo, int64_t hi) {
    gemm_ctx* g = (gemm_ctx*)p;
    int8_t* ua = (int8_t*)malloc((size_t)(g->K > 0 ? g->K : 1));
    int8_t* ub = (int8_t*)malloc((size_t)(g->K > 0 ? g->K : 1));
    for (int64_t i = lo; i < hi; ++i) {
        int64_t m = g->mi[i], n = g->ni[i];
        unpack_row(g->qa + m * (g->K / 2), g->K, ua);
        unpack_row(g->qb + n * (g->K / 2), g->K, ub);
        gemm_one(g, ua, ub, m, n, &g->ref[i], &g->absref[i]);
    }
    free(ua);
    free(ub);
}

/* Sampled outputs: ref[i] = out[mi[i], ni[i]] (indices must be in range). */
int mxo_gemm_pairs(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t M, int64_t N,
                   int64_t K, const int64_t* mi, const int64_t* ni, int64_t npairs, double* ref, double* absref,
                   int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K % MXO_BLOCK != 0 || npairs < 0) return -1;
    for (int64_t i = 0; i < npairs; ++i)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return -1;
    gemm_ctx g = {qa, sa, qb, sb, M, N, K, mi, ni, ref, absref, NULL};
    parallel_for(npairs, nthreads, gemm_pairs_range, &g);
    return 0;
}

/* ==== Producers that feed the cast (jax-aiter README, "Supported ops": SiLU-and-Mul,
 * RMSNorm, Fused Add+RMSNorm).  Each returns its BF16 output; quantizing that output
 * with the casts above is what a fused producer + cast computes. ==== */

/* Nearest-even bf16 of a double, rounded once (no intermediate binary32):
 * the grid of the value's binade (2^(e-7), or 2^-133 below 2^-126), RNE by rint,
 * magnitudes that round past the largest finite bf16 become infinity. */
static uint16_t bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e = floor_log2(a);
    int qexp = e < -126 ? -133 : e - 7;          /* exponent of the grid spacing */
    double r = rint(ldexp(a, -qexp));            /* integer multiple of the spacing, ties to even */
    double val = ldexp(r, qexp);
    if (val == 0.0) return sign;
    int e2 = floor_log2(val);
    if (e2 > 127) return sign | 0x7F80;
    if (e2 < -126) return sign | (uint16_t)r;    /* subnormal: r < 128 */
    double m = ldexp(val, 7 - e2);               /* in [128, 256) */
    return sign | (uint16_t)((e2 + 127) << 7) | (uint16_t)((int)m - 128);
}

int mxo_bf16_round(const double* v, uint16_t* out, int64_t n) {
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
    return 0;
}

typedef struct {
    const uint16_t* x;
    int64_t F, ldx;
    uint16_t* y;
} silu_ctx;

static void silu_mul_range(void* p, int64_t lo, int64_t hi) {
    silu_ctx* c = (silu_ctx*)p;
    for (int64_t r = lo; r < hi; ++r)
        for (int64_t j = 0; j < c->F; ++j) {
            double g = bf16_value(c->x[r * c->ldx + j]);
            double u = bf16_value(c->x[r * c->ldx + c->F + j]);
            double silu = g / (1.0 + exp(-g));   /* SiLU(g) = g * sigmoid(g) */
            c->y[r * c->F + j] = bf16_round(silu * u);
        }
}

/* SiLU-and-Mul of x [R, 2F] (finite bf16; gate = columns 0..F-1, up = F..2F-1):
 * y [R, F] = bf16(silu(gate) * up), evaluated in double. */
int mxo_silu_mul(const uint16_t* x, int64_t R, int64_t F, int64_t ldx, uint16_t* y, int nthreads) {
    if (R < 0 || F < 0 || ldx < 2 * F) return -1;
    silu_ctx c = {x, F, ldx, y};
    parallel_for(R, nthreads, silu_mul_range, &c);
    return 0;
}

typedef struct {
    const uint16_t *x, *res, *gamma;
    int64_t D;
    double eps;
    uint16_t *y, *h;
    double* rstd;
} rms_ctx;

static void rmsnorm_range(void* p, int64_t lo, int64_t hi) {
    rms_ctx* c = (rms_ctx*)p;
    int64_t D = c->D;
    double* hv = (double*)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
    for (int64_t r = lo; r < hi; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < D; ++j) {
            double v = bf16_value(c->x[r * D + j]);
            if (c->res) {
                /* the residual sum is rounded to bf16 (it is also the stored residual) */
                uint16_t hb = bf16_round(v + bf16_value(c->res[r * D + j]));
                if (c->h) c->h[r * D + j] = hb;
                v = bf16_value(hb);
            }
            hv[j] = v;
            ss += v * v;
        }
        double rs = 1.0 / sqrt(ss / (double)D + c->eps);
        if (c->rstd) c->rstd[r] = rs;
        for (int64_t j = 0; j < D; ++j) c->y[r * D + j] = bf16_round(hv[j] * rs * bf16_value(c->gamma[j]));
    }
    free(hv);
}

/* RMSNorm of x [R, D] (or, with res != NULL, of h = bf16(x + res), written to h
 * when h != NULL): y = bf16(h * rstd * gamma) with rstd = 1 / sqrt(mean(h^2) + eps),
 * all in double; rstd [R] written when non-NULL. */
int mxo_rmsnorm(const uint16_t* x, const uint16_t* res, const uint16_t* gamma, double eps, int64_t R, int64_t D,
                uint16_t* y, uint16_t* h, double* rstd, int nthreads) {
    if (R < 0 || D <= 0 || !(eps >= 0.0)) return -1;
    rms_ctx c = {x, res, gamma, D, eps, y, h, rstd};
    parallel_for(R, nthreads, rmsnorm_range, &c);
    return 0;
}
