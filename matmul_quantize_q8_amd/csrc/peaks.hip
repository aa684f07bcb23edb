// Attainable-peak probes, the measured ceilings that the product kernels are
// compared with beside the published ones: a streaming read of a device
// buffer (HBM, the bound of every decode kernel) and a back-to-back int8 MFMA
// loop (the matrix cores, the bound of the prefill).  Neither computes
// anything of the product path.
#include "qmm_device.h"

namespace qmm {

// One pass with a full grid: workgroup b reads bytes [8192 b, 8192 b + 8192)
// of the buffer, two 16-byte loads per lane, and stores the XOR of their
// 32-bit words to sink[b].  No grid-stride loop (a grid sized to the buffer
// keeps more loads in flight early in the pass) and no atomics (thousands
// of atomic updates would serialise at the L2 and be timed instead of the
// reads); the host can check every chunk.
constexpr int kPeakChunk = 8192;   // bytes per workgroup

__global__ __launch_bounds__(256) void k_peak_read(const uint4 *__restrict__ p, int64_t n16, uint32_t *sink) {
    __shared__ uint32_t red[4];
    const int64_t i = (int64_t)blockIdx.x * (kPeakChunk / 16) + threadIdx.x;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (i < n16) a = p[i];
    if (i + 256 < n16) b = p[i + 256];
    uint32_t acc = (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Four independent accumulator chains of v_mfma_i32_32x32x32_i8 per wave, the
// operands held in registers.  With every operand byte 1 each MFMA adds 32 to
// each of its 16 results per lane, so lane t ends with 4 * 16 * 32 * iters.
__global__ __launch_bounds__(256) void k_peak_mfma_i8(int32_t *__restrict__ out, int iters, int a, int b) {
    const v4i va = {a, a, a, a}, vb = {b, b, b, b};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_peak_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (bytes + kPeakChunk - 1) / kPeakChunk;
    hipLaunchKernelGGL(k_peak_read, dim3((unsigned)grid), dim3(256), 0, st, static_cast<const uint4 *>(buf), n16,
                       sink);
    return hipGetLastError();
}

hipError_t launch_peak_mfma_i8(int32_t *out, int64_t workgroups, int iters, hipStream_t st) {
    hipLaunchKernelGGL(k_peak_mfma_i8, dim3((unsigned)workgroups), dim3(256), 0, st, out, iters, 0x01010101,
                       0x01010101);
    return hipGetLastError();
}

}  // namespace qmm
