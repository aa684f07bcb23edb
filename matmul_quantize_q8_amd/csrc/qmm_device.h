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

// Launch helper: kernels that use more than 64 KB of dynamic LDS raise their
// limit once (gfx950 has 160 KB per workgroup).
inline hipError_t allow_dynamic_lds(const void *kernel, size_t bytes, int &done) {
    if (bytes <= 65536 || __atomic_load_n(&done, __ATOMIC_ACQUIRE)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) __atomic_store_n(&done, 1, __ATOMIC_RELEASE);
    return e;
}

// Wave-uniform helpers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

#define QMM_VMCNT_CASE(n) \
    case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
// Wait until at most n vector-memory loads of this wave are outstanding
// (n wave-uniform; above 30 it waits for all of them, which is only stricter).
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (uniform(n)) {
        QMM_VMCNT_CASE(0) QMM_VMCNT_CASE(1) QMM_VMCNT_CASE(2) QMM_VMCNT_CASE(3) QMM_VMCNT_CASE(4)
        QMM_VMCNT_CASE(5) QMM_VMCNT_CASE(6) QMM_VMCNT_CASE(7) QMM_VMCNT_CASE(8) QMM_VMCNT_CASE(9)
        QMM_VMCNT_CASE(10) QMM_VMCNT_CASE(11) QMM_VMCNT_CASE(12) QMM_VMCNT_CASE(13) QMM_VMCNT_CASE(14)
        QMM_VMCNT_CASE(15) QMM_VMCNT_CASE(16) QMM_VMCNT_CASE(17) QMM_VMCNT_CASE(18) QMM_VMCNT_CASE(19)
        QMM_VMCNT_CASE(20) QMM_VMCNT_CASE(21) QMM_VMCNT_CASE(22) QMM_VMCNT_CASE(23) QMM_VMCNT_CASE(24)
        QMM_VMCNT_CASE(25) QMM_VMCNT_CASE(26) QMM_VMCNT_CASE(27) QMM_VMCNT_CASE(28) QMM_VMCNT_CASE(29)
        QMM_VMCNT_CASE(30)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}
#undef QMM_VMCNT_CASE

template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

}  // namespace qmm
