// Measurement probes for bench.py --ceilings (not part of the MXFP4 library):
// what the chip sustains on the two resources the cast and the GEMM are bound
// by, measured with the same instruction and access shapes as the kernels.
// Built into a library of their own (bench_probes.py), loaded by the bench.
//
// * mfma: the GEMM's inner loop with nothing else -- one workgroup of four
//   waves per CU, each wave a 4 x 4 block of 32x32x64 FP4 scaled MFMAs over
//   register-resident operands (no memory traffic).  Run once on random
//   codes and once on constant codes, it separates the MFMA rate the power
//   limit allows on random data from the one on quiet data.
// * stream: grid-stride 16-byte accesses -- read only, read + write of the
//   same size, or the dual cast's 2 : 1.0625 mix of reads and writes.
#include <string.h>

#include "mxfp4_block_scaled_cast_amd/csrc/mx_device.h"

namespace mx {

__global__ __launch_bounds__(256, 1) void probe_mfma_kernel(const u32x4* __restrict__ ops, int64_t iters,
                                                            float* __restrict__ out) {
    const u32x4* p = ops + ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = p[i];
        b[i] = p[4 + i];
    }
    constexpr int kScale = 0x7F7F7F7F;  // E8M0 127: every block scaled by 1
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = q >> 2, j = q & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(b[j]), as_operand(a[i]), acc[i][j],
                                                                        4, 4, 0, kScale, 0, kScale);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Read every 16-byte chunk of src once (grid-stride, 4 chunks in flight per
// lane) and, of every 32 consecutive chunks, write the first w to dst: chunk
// i goes to dst chunk (i / 32) * w + i % 32 when i % 32 < w.  w = 0 reads
// only, w = 32 is a plain copy, w = 17 is the dual cast's byte mix (2 read :
// 1.0625 written per element = 32 : 17).  What is not written is XORed into
// out so the loads stay.
__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                           u32x4* __restrict__ dst, int w,
                                                           unsigned* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    unsigned x = 0u;
    auto one = [&](int64_t i, const u32x4& v) {
        const int r = (int)(i & 31);
        if (r < w) dst[(i >> 5) * w + r] = v;
        else x ^= v.x ^ v.y ^ v.z ^ v.w;
    };
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i), v1 = __builtin_nontemporal_load(src + i + stride);
        const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
        one(i, v0), one(i + stride, v1), one(i + 2 * stride, v2), one(i + 3 * stride, v3);
    }
    for (; i < chunks; i += stride) one(i, __builtin_nontemporal_load(src + i));
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace mx

// C entry points.  Return 0, -1 for an argument out of range (null pointer,
// size, count), -2 for a misaligned pointer, -3 when the current device is not
// a gfx950, -4 when the launch failed.  All pointers are device memory.

static int probe_device_ok() {
    int dev = -1;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// At most 2^24 passes per wave (a few seconds at the MFMA rate of the chip).
constexpr int64_t kMaxProbeIters = (int64_t)1 << 24;

// `workgroups` (1..65536) workgroups of 4 waves; every wave runs `iters`
// (0..2^24) passes of 16 FP4 32x32x64 scaled MFMAs (a 4 x 4 block of
// accumulators, every scale 1) over operands held in registers.  operands: at
// least workgroups * 32768 bytes, 16-byte aligned (lane t of workgroup g reads
// the 128 bytes at (g * 256 + t) * 128); out: float[workgroups * 256], each
// lane's sum of its accumulators.  FLOPs: workgroups * 4 * iters * 16 * 2 * 32 * 32 * 64.
extern "C" int probe_mfma(const void* operands, int64_t iters, int64_t workgroups, float* out, hipStream_t stream) {
    if (!operands || !out || iters < 0 || iters > kMaxProbeIters || workgroups < 1 || workgroups > 65536) return -1;
    if (!aligned(operands, 16) || !aligned(out, 4)) return -2;
    if (!probe_device_ok()) return -3;
    hipLaunchKernelGGL(mx::probe_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const mx::u32x4*>(operands), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads src_bytes (a multiple of 16) of src once, 16 bytes per lane access,
// grid-stride over `workgroups` (1..65536) workgroups of 256 lanes; of every
// 32 consecutive 16-byte chunks the first writes_per_32 (0..32) are written to
// dst, packed: dst holds ceil(src_bytes / 512) * writes_per_32 * 16 bytes (NULL
// allowed when writes_per_32 == 0).  out: unsigned[workgroups * 256].
extern "C" int probe_stream(const void* src, int64_t src_bytes, void* dst, int writes_per_32, int64_t workgroups,
                            unsigned* out, hipStream_t stream) {
    if (!src || !out || src_bytes < 0 || src_bytes % 16 != 0 || writes_per_32 < 0 || writes_per_32 > 32 ||
        workgroups < 1 || workgroups > 65536 || (writes_per_32 > 0 && !dst))
        return -1;
    if (!aligned(src, 16) || (dst && !aligned(dst, 16)) || !aligned(out, 4)) return -2;
    if (!probe_device_ok()) return -3;
    hipLaunchKernelGGL(mx::probe_stream_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const mx::u32x4*>(src), src_bytes / 16, static_cast<mx::u32x4*>(dst), writes_per_32,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
