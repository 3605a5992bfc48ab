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
#include "mx_device.h"

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

}  // namespace mx

extern "C" hipError_t mx_launch_gemm(const void* aq, const void* as, const void* bq, const void* bs, int64_t M,
                                     int64_t N, int64_t K, void* out, int64_t ldo, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if ((M + 63) / 64 > 65535 || (N + 63) / 64 > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64)), block(256);
    hipLaunchKernelGGL(mx::gemm_direct_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(aq),
                       static_cast<const uint8_t*>(as), static_cast<const uint8_t*>(bq),
                       static_cast<const uint8_t*>(bs), (int)M, (int)N, (int)K, static_cast<uint16_t*>(out), ldo);
    return hipGetLastError();
}
