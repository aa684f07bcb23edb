// Device-side helpers shared by the qmm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

constexpr int kWave = 64;                 // CDNA wavefront width

constexpr int kQ80Bytes = 34;             // f16 d + int8[32]
constexpr int kQ40Bytes = 18;             // f16 d + uint8[16]
constexpr int kQ2KBytes = 84;             // scales[16] + qs[64] + f16 d + f16 dmin
constexpr int kQ8KBytes = 292;            // f32 d + int8[256] + int16[16]

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// binary32 -> binary16 bits: v_cvt_f16_f32 rounds to nearest even under the
// default MODE and keeps f16 denormals.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// binary16 bits (low 16 bits of h) -> binary32, exact.
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// Bytes [s, s+4) of the little-endian 8-byte value hi:lo (s in 0..3).
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Signed 4-way int8 dot product accumulated into c (v_dot4c_i32_i8).
__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// 16 bytes per lane from global straight into LDS (gfx950 LDS DMA).  `dst` must
// be the same for every lane of the wave: lane i's bytes land at dst + 16*i.
// The LDS write completes with the vector-memory counter, so a reader must
// wait_global_loads() first.
__device__ __forceinline__ void global_to_lds16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)dst, 16, 0, 0);
}

// Wait for every outstanding vector-memory load of this wave (including LDS DMA).
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every outstanding LDS access of this wave.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

}  // namespace qmm
