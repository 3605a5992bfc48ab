// C ABI of the MXFP4 library: argument validation, device check, dispatch,
// and the gemm_fp4_bf16 forward/backward composition over the kernels.
//
// Composition (jax-aiter README, "MXFP4 training architecture", and the
// Quick start note that the training recipe runs FP4 forward, FP4 dA and FP4
// dB NT wgrad):
//   forward : cast A and W, out = A . W^T
//   backward: cast dOut, dA = dOut . W (NN on W's column copy),
//             dB = dOut^T . A (NT on the column copies of dOut and A)
// With the Hadamard-gradient recipe (README "Quick start": grad_out is cast
// with a Hadamard transform) every operand of dA and dB carries the block
// transform along its contraction dimension: the column copies of A and W
// (forward casts, divisor 1) and both copies of dOut (divisor 32 = 2^5, so
// the products are unchanged: H H = 32 I).
// With the FP8 wgrad option (the dB of the "MXFP4 training architecture"
// section runs as an FP8 product) the column copies of A and dOut are MXFP8
// and dB is the MXFP8 GEMM; the forward pass and dA stay MXFP4.
#include <algorithm>
#include <mutex>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/mxfp4.h"

extern "C" hipError_t mx_launch_cast(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                     void* q_col, void* s_col, bool dual, hipStream_t stream);
extern "C" hipError_t mx_launch_cast_h(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                       void* q_col, void* s_col, bool dual, bool transform_row, bool transform_col,
                                       int hshift, hipStream_t stream);
extern "C" hipError_t mx_launch_gemm(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                     int64_t N, int64_t K, void* out, int64_t ldo, hipStream_t stream);
extern "C" hipError_t mx_launch_cast_f(const void* x, int64_t R, int64_t C, int64_t ldx, void* q_row, void* s_row,
                                       void* q_col, void* s_col, bool dual, int row_fmt, int col_fmt,
                                       bool transform_row, bool transform_col, int hshift, hipStream_t stream);
extern "C" hipError_t mx_launch_silu_mul_cast(const void* x, int64_t R, int64_t F, int64_t ldx, void* q_row,
                                              void* s_row, void* q_col, void* s_col, bool dual, int col_fmt,
                                              void* y_out, hipStream_t stream);
extern "C" hipError_t mx_launch_rmsnorm_cast(const void* x, const void* residual, const void* gamma, float eps,
                                             int64_t R, int64_t D, void* q_row, void* s_row, void* q_col, void* s_col,
                                             bool dual, int col_fmt, void* h_out, void* rstd, void* y_out,
                                             hipStream_t stream);
extern "C" hipError_t mx_launch_gemm_f(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                       int64_t N, int64_t K, void* out, int64_t ldo, int fmt, hipStream_t stream);
extern "C" hipError_t mx_launch_gemm_ws(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                        int64_t N, int64_t K, void* out, int64_t ldo, int fmt, void* ws,
                                        int64_t ws_bytes, hipStream_t stream);
extern "C" int64_t mx_gemm_split_bytes(int64_t M, int64_t N, int64_t K, int fmt);
extern "C" hipError_t mx_launch_gemm_pair_ws(const void* aq0, const void* as0, const void* bq0, const void* bs0,
                                             int64_t M0, int64_t N0, int64_t K0, void* out0, int64_t ldo0,
                                             const void* aq1, const void* as1, const void* bq1, const void* bs1,
                                             int64_t M1, int64_t N1, int64_t K1, void* out1, int64_t ldo1, int fmt,
                                             void* ws, int64_t ws_bytes, hipStream_t stream);
extern "C" int mx_gemm_pair_split(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1);
extern "C" hipError_t mx_launch_cast_dual_pair(const void* x0, int64_t R0, int64_t C0, int64_t ldx0, void* q_row0,
                                               void* s_row0, void* q_col0, void* s_col0, const void* x1, int64_t R1,
                                               int64_t C1, int64_t ldx1, void* q_row1, void* s_row1, void* q_col1,
                                               void* s_col1, hipStream_t stream);

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
int g_arch_ok[kMaxDevices];

// The current device must be a gfx950; the answer is cached per device.
int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXFP4_EDEVICE;
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                         strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    });
    return g_arch_ok[dev] ? MXFP4_OK : MXFP4_EDEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Largest element count / byte count the kernels index with 64-bit offsets
// but 32-bit tile counts and row indices.
constexpr int64_t kMaxDim = 0x7FFFFFFF;

// Longest contraction of a GEMM: the tiled kernels address a wave's operand
// loads with 32-bit lane offsets of up to 15 code-tile rows of K/2 bytes
// (MXFP4) or K bytes (MXFP8) each, which stay below 2^31 for K <= 2^23.
constexpr int64_t kMaxK = (int64_t)1 << 23;

struct OperandSizes {
    int64_t q, s;
};

// Tiled MX operand layout: codes in 1 KB tiles of 16 rows x 128 elements,
// scales in 1 KB tiles of 128 rows x 256 elements (include/mxfp4.h).
OperandSizes operand_sizes(int64_t rows, int64_t k) {
    return {((rows + 15) / 16) * ((k + 127) / 128) * 1024, ((rows + 127) / 128) * ((k + 255) / 256) * 1024};
}

// MXFP8 operand: code tiles of 16 rows x 64 elements (one byte each), same scale tiles.
OperandSizes operand_sizes8(int64_t rows, int64_t k) {
    return {((rows + 15) / 16) * ((k + 63) / 64) * 1024, ((rows + 127) / 128) * ((k + 255) / 256) * 1024};
}

int validate_cast(const void* x, int64_t rows, int64_t cols, int64_t ldx, const void* q, const void* s) {
    if (rows < 0 || cols < 0) return MXFP4_EINVAL;
    if (cols % 32 != 0) return MXFP4_EINVAL;
    if (rows > kMaxDim || cols > kMaxDim) return MXFP4_ERANGE;
    if (rows == 0 || cols == 0) return MXFP4_OK;
    if (!x || !q || !s) return MXFP4_EINVAL;
    if (ldx < cols) return MXFP4_EINVAL;
    if (!aligned16(x) || ldx % 8 != 0 || !aligned16(q) || !aligned16(s)) return MXFP4_EALIGN;
    return MXFP4_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ELAUNCH; }

// The checks of mxfp4_cast_dual for one tensor; `empty` tells whether it has no elements.
int validate_cast_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, const void* q_row, const void* s_row,
                       const void* q_col, const void* s_col, bool& empty) {
    int st = validate_cast(x, rows, cols, ldx, q_row, s_row);
    empty = rows == 0 || cols == 0;
    if (st != MXFP4_OK || empty) return st;
    if (!q_col || !s_col) return MXFP4_EINVAL;
    if (!aligned16(q_col) || !aligned16(s_col)) return MXFP4_EALIGN;
    return MXFP4_OK;
}

int validate_gemm(const void* aq, const void* as, const void* bq, const void* bs, int64_t M, int64_t N, int64_t K,
                  const void* out, int64_t ldo) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MXFP4_EINVAL;
    if (M > kMaxDim || N > kMaxDim || K > kMaxK) return MXFP4_ERANGE;
    if (M == 0 || N == 0) return MXFP4_OK;
    if (!out || ldo < N) return MXFP4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(out) & 1u) != 0) return MXFP4_EALIGN;
    if (K == 0) return MXFP4_OK;
    if (!aq || !as || !bq || !bs) return MXFP4_EINVAL;
    if (!aligned16(aq) || !aligned16(bq) || !aligned16(as) || !aligned16(bs)) return MXFP4_EALIGN;
    return MXFP4_OK;
}

// Workspace carve-up for gemm_fp4_bf16 (each region 256-byte aligned).
struct Workspace {
    int64_t a_row_q, a_row_s, w_row_q, w_row_s;  // forward operands
    int64_t a_col_q, a_col_s, w_col_q, w_col_s;  // saved for the backward pass
    int64_t g_row_q, g_row_s, g_col_q, g_col_s;  // backward operands
    int64_t split, split_bytes;                  // partial sums of a split contraction (shared by the GEMMs)
    int64_t total;
};

// with_w == false: W's copies come from the caller (pre-quantized weight), no W slots.
// fp8_wgrad: the column copies of A and dOut (dB's operands) are MXFP8.
Workspace workspace_layout(int64_t M, int64_t N, int64_t K, bool training, bool with_w = true,
                           bool fp8_wgrad = false) {
    Workspace w{};
    int64_t off = 0;
    auto take = [&off](int64_t bytes) {
        const int64_t at = off;
        off += round_up(bytes, 256);
        return at;
    };
    const OperandSizes a_row = operand_sizes(M, K), w_row = operand_sizes(N, K);
    w.a_row_q = take(a_row.q);
    w.a_row_s = take(a_row.s);
    w.w_row_q = take(with_w ? w_row.q : 0);
    w.w_row_s = take(with_w ? w_row.s : 0);
    if (training) {
        const int64_t Mp = round_up(M, 32), Np = round_up(N, 32);
        const OperandSizes a_col = fp8_wgrad ? operand_sizes8(K, Mp) : operand_sizes(K, Mp);
        const OperandSizes w_col = operand_sizes(K, Np);
        const OperandSizes g_row = operand_sizes(M, N);
        const OperandSizes g_col = fp8_wgrad ? operand_sizes8(N, Mp) : operand_sizes(N, Mp);
        w.a_col_q = take(a_col.q);
        w.a_col_s = take(a_col.s);
        w.w_col_q = take(with_w ? w_col.q : 0);
        w.w_col_s = take(with_w ? w_col.s : 0);
        w.g_row_q = take(g_row.q);
        w.g_row_s = take(g_row.s);
        w.g_col_q = take(g_col.q);
        w.g_col_s = take(g_col.s);
    }
    // the step's GEMMs run one after another on one stream, so they share one region
    int64_t split = mx_gemm_split_bytes(M, N, K, 4);
    if (training) {
        const int64_t Mp = round_up(M, 32);
        split = std::max(split, mx_gemm_split_bytes(M, K, N, 4));
        split = std::max(split, mx_gemm_split_bytes(N, K, Mp, fp8_wgrad ? 8 : 4));
    }
    w.split_bytes = split;
    w.split = take(split);
    w.total = off;
    return w;
}

// 2^5 = 32: H H = 32 I for the 32-point Walsh-Hadamard matrix.
constexpr int kHadamardShift = 5;

constexpr unsigned kStepFlags =
    MXFP4_STEP_TRAINING | MXFP4_STEP_HADAMARD_GRAD | MXFP4_STEP_QUANTIZED_W | MXFP4_STEP_FP8_WGRAD;

// Flags valid for a step: known bits; the transform goes with MXFP4 copies only.
bool step_flags_ok(unsigned flags) {
    if (flags & ~kStepFlags) return false;
    return !((flags & MXFP4_STEP_HADAMARD_GRAD) && (flags & MXFP4_STEP_FP8_WGRAD));
}

// The forward contracts over K; in training dA contracts over N and dB over
// ceil(M/32)*32, so those are bounded by the GEMM's contraction limit too.
int validate_step_sizes(int64_t M, int64_t N, int64_t K, bool training) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MXFP4_EINVAL;
    if (training && N % 32 != 0) return MXFP4_EINVAL;
    if (M > kMaxDim || N > kMaxDim || K > kMaxK) return MXFP4_ERANGE;
    if (training && (N > kMaxK || round_up(M, 32) > kMaxK)) return MXFP4_ERANGE;
    return MXFP4_OK;
}

}  // namespace

extern "C" {

const char* mxfp4_status_string(int status) {
    switch (status) {
        case MXFP4_OK: return "ok";
        case MXFP4_EINVAL: return "invalid argument (null pointer, negative size, size not a multiple of 32, or leading dimension too small)";
        case MXFP4_EALIGN: return "misaligned pointer or leading dimension";
        case MXFP4_EDEVICE: return "no usable device: the current device is not a gfx950 (MI355X)";
        case MXFP4_ELAUNCH: return "kernel launch failed";
        case MXFP4_ERANGE: return "size exceeds the supported range";
        case MXFP4_ESPACE: return "workspace too small";
        default: return "unknown status";
    }
}

int mxfp4_operand_layout_of(int64_t rows, int64_t k, mxfp4_operand_layout* out) {
    if (!out || rows < 0 || k < 0 || k % 32 != 0) return MXFP4_EINVAL;
    const OperandSizes sz = operand_sizes(rows, k);
    out->rows = rows;
    out->k = k;
    out->q_bytes = sz.q;
    out->s_bytes = sz.s;
    out->code_row_tiles = (rows + 15) / 16;
    out->code_k_tiles = (k + 127) / 128;
    out->scale_row_tiles = (rows + 127) / 128;
    out->scale_k_tiles = (k + 255) / 256;
    return MXFP4_OK;
}

int mxfp4_layout(int64_t rows, int64_t cols, mxfp4_layout_t* out) {
    if (!out || rows < 0 || cols < 0 || cols % 32 != 0) return MXFP4_EINVAL;
    if (rows > kMaxDim || cols > kMaxDim) return MXFP4_ERANGE;
    out->rows = rows;
    out->cols = cols;
    out->padded_rows = round_up(rows, 32);
    int st = mxfp4_operand_layout_of(rows, cols, &out->row);
    if (st == MXFP4_OK) st = mxfp4_operand_layout_of(cols, out->padded_rows, &out->col);
    return st;
}

int mxfp4_cast(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, void* s, hipStream_t stream) {
    int st = validate_cast(x, rows, cols, ldx, q, s);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_cast(x, rows, cols, ldx, q, s, nullptr, nullptr, false, stream));
}

int mxfp4_cast_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row, void* q_col,
                    void* s_col, hipStream_t stream) {
    int st = validate_cast(x, rows, cols, ldx, q_row, s_row);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if (!q_col || !s_col) return MXFP4_EINVAL;
    if (!aligned16(q_col) || !aligned16(s_col)) return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_cast(x, rows, cols, ldx, q_row, s_row, q_col, s_col, true, stream));
}

int mxfp4_cast_dual_pair(const void* x0, int64_t rows0, int64_t cols0, int64_t ldx0, void* q_row0, void* s_row0,
                         void* q_col0, void* s_col0, const void* x1, int64_t rows1, int64_t cols1, int64_t ldx1,
                         void* q_row1, void* s_row1, void* q_col1, void* s_col1, hipStream_t stream) {
    bool empty0 = true, empty1 = true;
    int st = validate_cast_dual(x0, rows0, cols0, ldx0, q_row0, s_row0, q_col0, s_col0, empty0);
    if (st != MXFP4_OK) return st;
    if ((st = validate_cast_dual(x1, rows1, cols1, ldx1, q_row1, s_row1, q_col1, s_col1, empty1)) != MXFP4_OK)
        return st;
    if (empty0 && empty1) return MXFP4_OK;
    if ((st = check_device()) != MXFP4_OK) return st;
    // an empty tensor contributes no workgroups (its grid is 0 x 0 tiles)
    return status_of(mx_launch_cast_dual_pair(x0, empty0 ? 0 : rows0, empty0 ? 0 : cols0, ldx0, q_row0, s_row0,
                                              q_col0, s_col0, x1, empty1 ? 0 : rows1, empty1 ? 0 : cols1, ldx1,
                                              q_row1, s_row1, q_col1, s_col1, stream));
}

int mxfp4_cast_hadamard(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row,
                        void* q_col, void* s_col, int transform_row, int transform_col, int shift,
                        hipStream_t stream) {
    if (shift < 0 || shift > 64) return MXFP4_EINVAL;
    const bool dual = q_col != nullptr || s_col != nullptr;
    if (transform_col && !dual) return MXFP4_EINVAL;
    int st = validate_cast(x, rows, cols, ldx, q_row, s_row);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if (dual) {
        if (!q_col || !s_col) return MXFP4_EINVAL;
        if (!aligned16(q_col) || !aligned16(s_col)) return MXFP4_EALIGN;
    }
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_cast_h(x, rows, cols, ldx, q_row, s_row, q_col, s_col, dual, transform_row != 0,
                                      transform_col != 0, shift, stream));
}

int mxfp4_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N, int64_t K,
                  void* out, int64_t ldo, hipStream_t stream) {
    int st = validate_gemm(a_q, a_s, b_q, b_s, M, N, K, out, ldo);
    if (st != MXFP4_OK || M == 0 || N == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_gemm(a_q, a_s, b_q, b_s, M, N, K, out, ldo, stream));
}

int mxfp4_gemm_nn(const void* a_q, const void* a_s, const void* bcol_q, const void* bcol_s, int64_t M, int64_t N,
                  int64_t K, void* out, int64_t ldo, hipStream_t stream) {
    // B[K, N] enters through its column copy, which is the MX operand (N rows, K):
    // the NN product is the NT kernel on that operand.
    return mxfp4_gemm_nt(a_q, a_s, bcol_q, bcol_s, M, N, K, out, ldo, stream);
}

size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxK) return 0;
    return (size_t)mx_gemm_split_bytes(M, N, K, 4);
}

int mxfp4_gemm_nt_ws(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N,
                     int64_t K, void* out, int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = validate_gemm(a_q, a_s, b_q, b_s, M, N, K, out, ldo);
    if (st != MXFP4_OK || M == 0 || N == 0) return st;
    if (ws && !aligned16(ws)) return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    const int64_t bytes = ws ? (int64_t)std::min(ws_bytes, (size_t)INT64_MAX) : 0;
    return status_of(mx_launch_gemm_ws(a_q, a_s, b_q, b_s, M, N, K, out, ldo, 4, ws, bytes, stream));
}

int mxfp4_gemm_nt_pair_ws(const void* a0_q, const void* a0_s, const void* b0_q, const void* b0_s, int64_t M0,
                          int64_t N0, int64_t K0, void* out0, int64_t ldo0, const void* a1_q, const void* a1_s,
                          const void* b1_q, const void* b1_s, int64_t M1, int64_t N1, int64_t K1, void* out1,
                          int64_t ldo1, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = validate_gemm(a0_q, a0_s, b0_q, b0_s, M0, N0, K0, out0, ldo0);
    if (st != MXFP4_OK) return st;
    if ((st = validate_gemm(a1_q, a1_s, b1_q, b1_s, M1, N1, K1, out1, ldo1)) != MXFP4_OK) return st;
    if ((M0 == 0 || N0 == 0) && (M1 == 0 || N1 == 0)) return MXFP4_OK;
    if (ws && !aligned16(ws)) return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    const int64_t bytes = ws ? (int64_t)std::min(ws_bytes, (size_t)INT64_MAX) : 0;
    return status_of(mx_launch_gemm_pair_ws(a0_q, a0_s, b0_q, b0_s, M0, N0, K0, out0, ldo0, a1_q, a1_s, b1_q, b1_s,
                                            M1, N1, K1, out1, ldo1, 4, ws, bytes, stream));
}

int mxfp4_gemm_pair_split(int64_t M0, int64_t N0, int64_t K0, int64_t M1, int64_t N1, int64_t K1) {
    if (M0 < 0 || N0 < 0 || K0 < 0 || M1 < 0 || N1 < 0 || K1 < 0 || K0 % 32 != 0 || K1 % 32 != 0 ||
        M0 > kMaxDim || N0 > kMaxDim || M1 > kMaxDim || N1 > kMaxDim || K0 > kMaxK || K1 > kMaxK)
        return 0;
    return mx_gemm_pair_split(M0, N0, K0, M1, N1, K1);
}

int mxfp8_operand_layout_of(int64_t rows, int64_t k, mxfp4_operand_layout* out) {
    if (!out || rows < 0 || k < 0 || k % 32 != 0) return MXFP4_EINVAL;
    const OperandSizes sz = operand_sizes8(rows, k);
    out->rows = rows;
    out->k = k;
    out->q_bytes = sz.q;
    out->s_bytes = sz.s;
    out->code_row_tiles = (rows + 15) / 16;
    out->code_k_tiles = (k + 63) / 64;
    out->scale_row_tiles = (rows + 127) / 128;
    out->scale_k_tiles = (k + 255) / 256;
    return MXFP4_OK;
}

int mxfp8_cast(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q, void* s, hipStream_t stream) {
    int st = validate_cast(x, rows, cols, ldx, q, s);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_cast_f(x, rows, cols, ldx, q, s, nullptr, nullptr, false, 8, 8, false, false, 0, stream));
}

namespace {
int cast_dual_formats(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row, void* q_col,
                      void* s_col, int row_fmt, int col_fmt, hipStream_t stream) {
    int st = validate_cast(x, rows, cols, ldx, q_row, s_row);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if (!q_col || !s_col) return MXFP4_EINVAL;
    if (!aligned16(q_col) || !aligned16(s_col)) return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(
        mx_launch_cast_f(x, rows, cols, ldx, q_row, s_row, q_col, s_col, true, row_fmt, col_fmt, false, false, 0, stream));
}
}  // namespace

int mxfp8_cast_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row, void* q_col,
                    void* s_col, hipStream_t stream) {
    return cast_dual_formats(x, rows, cols, ldx, q_row, s_row, q_col, s_col, 8, 8, stream);
}

int mxfp4_cast_dual_fp8col(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* q_row, void* s_row,
                           void* q_col, void* s_col, hipStream_t stream) {
    return cast_dual_formats(x, rows, cols, ldx, q_row, s_row, q_col, s_col, 4, 8, stream);
}

int mxfp8_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s, int64_t M, int64_t N, int64_t K,
                  void* out, int64_t ldo, hipStream_t stream) {
    int st = validate_gemm(a_q, a_s, b_q, b_s, M, N, K, out, ldo);
    if (st != MXFP4_OK || M == 0 || N == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_gemm_f(a_q, a_s, b_q, b_s, M, N, K, out, ldo, 8, stream));
}

namespace {
// Output copies of a fused producer + cast: the MXFP4 row copy, and the column
// copy (both pointers or neither) in col_fmt 4 or 8.
int validate_copies(const void* q_row, const void* s_row, const void* q_col, const void* s_col, int col_fmt,
                    bool& dual) {
    if (!q_row || !s_row) return MXFP4_EINVAL;
    if ((q_col == nullptr) != (s_col == nullptr)) return MXFP4_EINVAL;
    dual = q_col != nullptr;
    if (dual && col_fmt != 4 && col_fmt != 8) return MXFP4_EINVAL;
    if (!aligned16(q_row) || !aligned16(s_row) || (dual && (!aligned16(q_col) || !aligned16(s_col))))
        return MXFP4_EALIGN;
    return MXFP4_OK;
}
}  // namespace

int mxfp4_silu_mul_cast(const void* x, int64_t rows, int64_t f, int64_t ldx, void* q_row, void* s_row, void* q_col,
                        void* s_col, int col_fmt, void* y_out, hipStream_t stream) {
    if (rows < 0 || f < 0 || f % 32 != 0) return MXFP4_EINVAL;
    if (rows > kMaxDim || 2 * f > kMaxDim) return MXFP4_ERANGE;
    if (rows == 0 || f == 0) return MXFP4_OK;
    if (!x || ldx < 2 * f) return MXFP4_EINVAL;
    bool dual = false;
    int st = validate_copies(q_row, s_row, q_col, s_col, col_fmt, dual);
    if (st != MXFP4_OK) return st;
    if (!aligned16(x) || ldx % 8 != 0 || (y_out && !aligned16(y_out))) return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_silu_mul_cast(x, rows, f, ldx, q_row, s_row, q_col, s_col, dual, col_fmt, y_out,
                                             stream));
}

int mxfp4_rmsnorm_cast(const void* x, const void* residual, const void* gamma, float eps, int64_t rows, int64_t d,
                       void* q_row, void* s_row, void* q_col, void* s_col, int col_fmt, void* residual_out,
                       void* rstd, void* y_out, hipStream_t stream) {
    if (rows < 0 || d < 0 || d % 32 != 0 || !(eps >= 0.0f) || eps > 3.0e38f) return MXFP4_EINVAL;
    if (rows > kMaxDim || d > kMaxDim) return MXFP4_ERANGE;
    if (rows == 0 || d == 0) return MXFP4_OK;
    if (!x || !gamma || !rstd || (residual && !residual_out)) return MXFP4_EINVAL;
    bool dual = false;
    int st = validate_copies(q_row, s_row, q_col, s_col, col_fmt, dual);
    if (st != MXFP4_OK) return st;
    if (!aligned16(x) || !aligned16(gamma) || (reinterpret_cast<uintptr_t>(rstd) & 7u) != 0 ||
        (residual && (!aligned16(residual) || !aligned16(residual_out))) || (y_out && !aligned16(y_out)))
        return MXFP4_EALIGN;
    if ((st = check_device()) != MXFP4_OK) return st;
    return status_of(mx_launch_rmsnorm_cast(x, residual, gamma, eps, rows, d, q_row, s_row, q_col, s_col, dual,
                                            col_fmt, residual ? residual_out : nullptr, rstd, y_out, stream));
}

size_t gemm_fp4_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, int training) {
    if (validate_step_sizes(M, N, K, training != 0) != MXFP4_OK) return 0;
    return (size_t)workspace_layout(M, N, K, training != 0).total;
}

size_t gemm_fp4_bf16_workspace_bytes_qw(int64_t M, int64_t N, int64_t K, int training) {
    if (validate_step_sizes(M, N, K, training != 0) != MXFP4_OK) return 0;
    return (size_t)workspace_layout(M, N, K, training != 0, false).total;
}

size_t gemm_fp4_bf16_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, unsigned flags) {
    const bool train = (flags & MXFP4_STEP_TRAINING) != 0;
    if (!step_flags_ok(flags) || validate_step_sizes(M, N, K, train) != MXFP4_OK) return 0;
    return (size_t)workspace_layout(M, N, K, train, (flags & MXFP4_STEP_QUANTIZED_W) == 0,
                                    (flags & MXFP4_STEP_FP8_WGRAD) != 0)
        .total;
}

}  // extern "C"

namespace {

// Forward: cast A (dual when training, its column copy kept in ws), then the
// GEMM with W's row copy -- cast here from bf16 w (own_w), or given.
int step_fwd(const void* a, bool own_w, const void* w, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N,
             int64_t K, void* out, void* ws, size_t ws_bytes, bool train, bool hadamard, bool fp8_wgrad,
             hipStream_t stream) {
    // the transform and the FP8 wgrad only concern the backward operands
    if ((hadamard || fp8_wgrad) && !train) return MXFP4_EINVAL;
    int st = validate_step_sizes(M, N, K, train);
    if (st != MXFP4_OK) return st;
    if (M == 0 || N == 0) return MXFP4_OK;
    if (!out) return MXFP4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(out) & 1u) != 0) return MXFP4_EALIGN;
    const Workspace L = workspace_layout(M, N, K, train, own_w, fp8_wgrad);
    char* base = static_cast<char*>(ws);
    const void* wq = own_w ? base + L.w_row_q : w_row_q;
    const void* wsc = own_w ? base + L.w_row_s : w_row_s;
    if (K > 0) {
        if (!a || !ws || (own_w ? !w : (!w_row_q || !w_row_s))) return MXFP4_EINVAL;
        if (!aligned16(a) || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MXFP4_EALIGN;
        if (own_w ? !aligned16(w) : (!aligned16(w_row_q) || !aligned16(w_row_s))) return MXFP4_EALIGN;
        if ((int64_t)ws_bytes < L.total) return MXFP4_ESPACE;
    }
    if ((st = check_device()) != MXFP4_OK) return st;
    hipError_t e = hipSuccess;
    if (K > 0) {
        // with the Hadamard recipe the column copies (dB's and dA's B operands) carry the transform
        // with the FP8 wgrad A's column copy (dB's B operand) is MXFP8
        if (train && own_w && !hadamard && !fp8_wgrad) {
            // both dual casts in one launch
            e = mx_launch_cast_dual_pair(a, M, K, K, base + L.a_row_q, base + L.a_row_s, base + L.a_col_q,
                                         base + L.a_col_s, w, N, K, K, base + L.w_row_q, base + L.w_row_s,
                                         base + L.w_col_q, base + L.w_col_s, stream);
        } else {
            e = mx_launch_cast_f(a, M, K, K, base + L.a_row_q, base + L.a_row_s, train ? base + L.a_col_q : nullptr,
                                 train ? base + L.a_col_s : nullptr, train, 4, fp8_wgrad ? 8 : 4, false, hadamard, 0,
                                 stream);
            if (e == hipSuccess && own_w)
                e = mx_launch_cast_h(w, N, K, K, base + L.w_row_q, base + L.w_row_s,
                                     train ? base + L.w_col_q : nullptr, train ? base + L.w_col_s : nullptr, train,
                                     false, hadamard, 0, stream);
        }
    }
    if (e == hipSuccess)
        e = mx_launch_gemm_ws(base + L.a_row_q, base + L.a_row_s, wq, wsc, M, N, K, out, N, 4, base + L.split,
                              L.split_bytes, stream);
    return status_of(e);
}

// Backward: cast dOut (dual), dA = dOut . W on W's column copy (from ws, or
// given), dW = dOut^T . A on the column copies of dOut and A.
int step_bwd(const void* dout, bool own_w, const void* w_col_q, const void* w_col_s, int64_t M, int64_t N, int64_t K,
             void* ws, size_t ws_bytes, void* da, void* dw, bool hadamard, bool fp8_wgrad, hipStream_t stream) {
    int st = validate_step_sizes(M, N, K, true);
    if (st != MXFP4_OK) return st;
    if (!ws || (!da && !dw)) return ws ? MXFP4_OK : MXFP4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MXFP4_EALIGN;
    if ((da && (reinterpret_cast<uintptr_t>(da) & 1u)) || (dw && (reinterpret_cast<uintptr_t>(dw) & 1u)))
        return MXFP4_EALIGN;
    const Workspace L = workspace_layout(M, N, K, true, own_w, fp8_wgrad);
    if ((int64_t)ws_bytes < L.total) return MXFP4_ESPACE;
    if (K == 0) return MXFP4_OK;  // dA [M, 0] and dW [N, 0] have no elements
    if (M == 0 || N == 0) {
        // sums over an empty contraction: the GEMM with contraction length 0 writes +0
        if ((st = check_device()) != MXFP4_OK) return st;
        hipError_t e = hipSuccess;
        if (M == 0 && dw) e = mx_launch_gemm(nullptr, nullptr, nullptr, nullptr, N, K, 0, dw, K, stream);
        if (e == hipSuccess && N == 0 && da) e = mx_launch_gemm(nullptr, nullptr, nullptr, nullptr, M, K, 0, da, K, stream);
        return status_of(e);
    }
    if (!dout) return MXFP4_EINVAL;
    if (!aligned16(dout)) return MXFP4_EALIGN;
    if (!own_w && da) {
        if (!w_col_q || !w_col_s) return MXFP4_EINVAL;
        if (!aligned16(w_col_q) || !aligned16(w_col_s)) return MXFP4_EALIGN;
    }
    if ((st = check_device()) != MXFP4_OK) return st;
    char* base = static_cast<char*>(ws);
    const int64_t Mp = round_up(M, 32);
    const void* wq = own_w ? base + L.w_col_q : w_col_q;
    const void* wsc = own_w ? base + L.w_col_s : w_col_s;
    // Hadamard recipe: both copies of dOut transformed and divided by 32 (kHadamardShift)
    // FP8 wgrad: dOut's column copy (dB's A operand) is MXFP8, and dB the MXFP8 GEMM
    const int wfmt = fp8_wgrad ? 8 : 4;
    hipError_t e = mx_launch_cast_f(dout, M, N, N, base + L.g_row_q, base + L.g_row_s, base + L.g_col_q,
                                    base + L.g_col_s, true, 4, wfmt, hadamard, hadamard,
                                    hadamard ? kHadamardShift : 0, stream);
    if (e == hipSuccess && da && dw && wfmt == 4) {
        // both products read the dOut copies just made: one launch where it pays
        e = mx_launch_gemm_pair_ws(base + L.g_row_q, base + L.g_row_s, wq, wsc, M, K, N, da, K, base + L.g_col_q,
                                   base + L.g_col_s, base + L.a_col_q, base + L.a_col_s, N, K, Mp, dw, K, 4,
                                   base + L.split, L.split_bytes, stream);
        return status_of(e);
    }
    if (e == hipSuccess && da)
        e = mx_launch_gemm_ws(base + L.g_row_q, base + L.g_row_s, wq, wsc, M, K, N, da, K, 4, base + L.split,
                              L.split_bytes, stream);
    if (e == hipSuccess && dw)
        e = mx_launch_gemm_ws(base + L.g_col_q, base + L.g_col_s, base + L.a_col_q, base + L.a_col_s, N, K, Mp, dw, K,
                              wfmt, base + L.split, L.split_bytes, stream);
    return status_of(e);
}

}  // namespace

extern "C" {

int gemm_fp4_bf16_fwd(const void* a, const void* w, int64_t M, int64_t N, int64_t K, void* out, void* ws,
                      size_t ws_bytes, int training, hipStream_t stream) {
    return step_fwd(a, true, w, nullptr, nullptr, M, N, K, out, ws, ws_bytes, training != 0, false, false, stream);
}

int gemm_fp4_bf16_bwd(const void* dout, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* da,
                      void* dw, hipStream_t stream) {
    return step_bwd(dout, true, nullptr, nullptr, M, N, K, ws, ws_bytes, da, dw, false, false, stream);
}

int gemm_fp4_bf16_fwd_qw(const void* a, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N, int64_t K,
                         void* out, void* ws, size_t ws_bytes, int training, hipStream_t stream) {
    return step_fwd(a, false, nullptr, w_row_q, w_row_s, M, N, K, out, ws, ws_bytes, training != 0, false, false, stream);
}

int gemm_fp4_bf16_bwd_qw(const void* dout, const void* w_col_q, const void* w_col_s, int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, void* da, void* dw, hipStream_t stream) {
    return step_bwd(dout, false, w_col_q, w_col_s, M, N, K, ws, ws_bytes, da, dw, false, false, stream);
}

int gemm_fp4_bf16_fwd_ex(const void* a, const void* w, const void* w_row_q, const void* w_row_s, int64_t M, int64_t N,
                         int64_t K, void* out, void* ws, size_t ws_bytes, unsigned flags, hipStream_t stream) {
    if (!step_flags_ok(flags)) return MXFP4_EINVAL;
    const bool qw = (flags & MXFP4_STEP_QUANTIZED_W) != 0;
    if (qw ? w != nullptr : (w_row_q != nullptr || w_row_s != nullptr)) return MXFP4_EINVAL;
    return step_fwd(a, !qw, w, w_row_q, w_row_s, M, N, K, out, ws, ws_bytes, (flags & MXFP4_STEP_TRAINING) != 0,
                    (flags & MXFP4_STEP_HADAMARD_GRAD) != 0, (flags & MXFP4_STEP_FP8_WGRAD) != 0, stream);
}

int gemm_fp4_bf16_bwd_ex(const void* dout, const void* w_col_q, const void* w_col_s, int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, void* da, void* dw, unsigned flags, hipStream_t stream) {
    if (!step_flags_ok(flags)) return MXFP4_EINVAL;
    const bool qw = (flags & MXFP4_STEP_QUANTIZED_W) != 0;
    if (!qw && (w_col_q || w_col_s)) return MXFP4_EINVAL;
    return step_bwd(dout, !qw, w_col_q, w_col_s, M, N, K, ws, ws_bytes, da, dw,
                    (flags & MXFP4_STEP_HADAMARD_GRAD) != 0, (flags & MXFP4_STEP_FP8_WGRAD) != 0, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free inference forward with a pre-quantized weight, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  It is
// gemm_fp4_bf16_fwd_qw(training = 0) with the workspace -- A's row copy, the
// only scratch that forward needs -- taken from a library-owned device array
// instead of a caller buffer.
//
// `scratch` is a file-scope device array; each GPU holds its own copy until
// the process ends.  Host code never uses its name as an address: the device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept in g_scratch_ptr.  Every call on a device shares the
// array (calls that overlap on one device race).  Nothing in it must start at
// zero: the cast writes every byte of the row copy it uses, padding included.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = MXFP4_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array, or nullptr if the runtime could not provide it.
void* scratch_ptr(int dev) {
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
        g_scratch_ptr[dev] = p;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int gemm_fp4_bf16_fwd_qw_noalloc(const void* a, const void* w_row_q, const void* w_row_s, int64_t M,
                                            int64_t N, int64_t K, void* out, hipStream_t stream) {
    int st = validate_step_sizes(M, N, K, false);
    if (st != MXFP4_OK) return st;
    if (M == 0 || N == 0) return MXFP4_OK;
    // A's row copy must fit the scratch array
    if (workspace_layout(M, N, K, false, false).total > (int64_t)kScratchBytes) return MXFP4_ERANGE;
    if ((st = check_device()) != MXFP4_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXFP4_EDEVICE;
    void* ws = scratch_ptr(dev);
    if (!ws) return MXFP4_ELAUNCH;
    return step_fwd(a, false, nullptr, w_row_q, w_row_s, M, N, K, out, ws, kScratchBytes, false, false, false, stream);
}
