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
constexpr int kQ41Bytes = 20;             // f16 d + f16 m + uint8[16]
constexpr int kQ50Bytes = 22;             // f16 d + qh[4] + uint8[16]
constexpr int kQ51Bytes = 24;             // f16 d + f16 m + qh[4] + uint8[16]
constexpr int kQ4KBytes = 144;            // f16 d + f16 dmin + 12 B scales/mins + qs[128]
constexpr int kQ6KBytes = 210;            // ql[128] + qh[64] + int8 scales[16] + f16 d

// Weight formats.  K-quant weights (256-value super-blocks) pair with Q8_K
// activations, the 32-value formats with Q8_0 (minfer "Two activation
// formats, one pairing rule").
enum Fmt { F_Q4_0 = 0, F_Q8_0 = 1, F_Q2_K = 2, F_Q4_K = 3, F_Q6_K = 4, F_Q4_1 = 5, F_Q5_0 = 6, F_Q5_1 = 7 };

// Token counts up to small_tokens(format) run the products on the decode
// kernel with several tokens per weight pass; larger counts run the MFMA
// prefill kernels.  The decode kernel's cost is flat within each group of
// tokens that share a weight pass (up to 2, 4 or 8) and steps up at the next
// group; the MFMA kernels cost about the same for any M up to their 32-token
// tile.  The switch is where the two meet at N = 12288, K = 4096 (us,
// decode kernel / MFMA): Q4_0 M = 8 13.1 / 14.5, M = 10 22.1 / 15.3; Q4_1
// M = 4 12.1 / 17.9, M = 6 19.2 / 17.4; Q4_K M = 4 9.1 / 11.2, M = 8 13.7 /
// 11.3; Q2_K M = 2 7.2 / 10.2, M = 4 10.7 / 10.1.
constexpr int small_tokens(int fmt) {
    return fmt == F_Q2_K ? 2 : fmt == F_Q4_0 ? 8 : 4;
}
hipError_t launch_matvec_tokens(int fmt, const void *w, const void *xq, float *y, int M, int N, int nb,
                                hipStream_t st);
template <int F> constexpr bool kIsK = F == F_Q2_K || F == F_Q4_K || F == F_Q6_K;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

// Cache-policy bits of a gfx950 vector-memory instruction: NT = non-temporal.
constexpr int kCpolNT = 2;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// 16 bytes per lane from global straight into LDS (gfx950 LDS DMA).  `dst` must
// be the same for every lane of the wave: lane i's bytes land at dst + 16*i.
// The LDS write completes with the vector-memory counter, so a reader must
// wait_global_loads() first.  STREAM marks data read once per launch (the
// decode weights): the load carries the non-temporal cache policy, so the
// stream does not displace reused lines (a 28 MB read runs ~4 % faster).
template <bool STREAM = false>
__device__ __forceinline__ void global_to_lds16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)dst, 16, 0, STREAM ? kCpolNT : 0);
}

// 16 bytes per lane from global memory into registers, issued as inline
// assembly so that the compiler neither tracks nor waits for it: the caller
// waits with wait_vmcnt() and then passes the value through pin_after_wait()
// before any use.  Loads and LDS-DMA copies complete in issue order, so a load
// issued before a run of LDS-DMA copies can be waited for alone.
__device__ __forceinline__ v4f global_load16_async(const void *base, uint32_t off) {
    v4f v;
    asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(v) : "v"(off), "s"(base));
    return v;
}

// Orders every use of v after the preceding (volatile) wait.
__device__ __forceinline__ void pin_after_wait(v4f &v) { asm volatile("" : "+v"(v)); }

// Wait for every outstanding vector-memory load of this wave (including LDS DMA).
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every outstanding LDS access of this wave.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Launch helper for kernels with only dynamic LDS: a launch that asks for
// more than 64 KB first raises the kernel's limit, once per device, to the
// whole 160 KB a gfx950 workgroup may use (the attribute is a permission,
// not an allocation, so later launches of any size up to that need nothing
// more).  `done` is the call site's per-device flag array.
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int kLdsDevices = 64;
inline hipError_t allow_dynamic_lds(const void *kernel, size_t bytes, int (&done)[kLdsDevices]) {
    if (bytes <= 65536) return hipSuccess;
    if (bytes > (size_t)kMaxLdsBytes) return hipErrorInvalidValue;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kLdsDevices) return hipErrorInvalidDevice;
    if (__atomic_load_n(&done[dev], __ATOMIC_ACQUIRE)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
    if (e == hipSuccess) __atomic_store_n(&done[dev], 1, __ATOMIC_RELEASE);
    return e;
}

constexpr int64_t kCUs = 256;   // compute units of the chip
// Prefill launches of at most this many output tiles (one workgroup per CU
// or fewer) split K in two, the parts adding into an output zeroed first.
constexpr int64_t kSplitTiles = kCUs;
// Zero n floats at y (16-byte aligned) on stream st.
hipError_t launch_zero_f32(float *y, int64_t n, hipStream_t st);

// Wave-uniform helpers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

#define QMM_VMCNT_CASE(n) \
    case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
// Wait until at most n vector-memory loads of this wave are outstanding
// (n wave-uniform; above 30 it waits for all of them, which is only stricter).
// s_waitcnt takes its count as an immediate, so a count known only at run
// time selects one of 31 instructions.  The counts a decode wave meets (below
// 8) go through one short compare chain in which each count jumps straight to
// its own wait and then past the rest; the compiler lowers a switch to a
// binary tree of about five compares and taken branches per wait, which with
// three such waits per wave cost the Q2_K 12288 x 4096 decode 0.4 us (6.2
// against 5.8 us per launch) and the Q4_0 one 0.1 us.
__device__ __forceinline__ void wait_vmcnt_small(int n) {
    asm volatile(
        "s_cmp_eq_u32 %0, 0\n\t"
        "s_cbranch_scc1 10f\n\t"
        "s_cmp_eq_u32 %0, 1\n\t"
        "s_cbranch_scc1 11f\n\t"
        "s_cmp_eq_u32 %0, 2\n\t"
        "s_cbranch_scc1 12f\n\t"
        "s_cmp_eq_u32 %0, 3\n\t"
        "s_cbranch_scc1 13f\n\t"
        "s_cmp_eq_u32 %0, 4\n\t"
        "s_cbranch_scc1 14f\n\t"
        "s_cmp_eq_u32 %0, 5\n\t"
        "s_cbranch_scc1 15f\n\t"
        "s_cmp_eq_u32 %0, 6\n\t"
        "s_cbranch_scc1 16f\n\t"
        "s_waitcnt vmcnt(7)\n\t"
        "s_branch 19f\n"
        "10:\n\ts_waitcnt vmcnt(0)\n\ts_branch 19f\n"
        "11:\n\ts_waitcnt vmcnt(1)\n\ts_branch 19f\n"
        "12:\n\ts_waitcnt vmcnt(2)\n\ts_branch 19f\n"
        "13:\n\ts_waitcnt vmcnt(3)\n\ts_branch 19f\n"
        "14:\n\ts_waitcnt vmcnt(4)\n\ts_branch 19f\n"
        "15:\n\ts_waitcnt vmcnt(5)\n\ts_branch 19f\n"
        "16:\n\ts_waitcnt vmcnt(6)\n"
        "19:"
        :: "s"(n) : "memory", "scc");
}
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (__builtin_constant_p(n) && n == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    n = uniform(n);
    if ((unsigned)n < 8u) {
        wait_vmcnt_small(n);
        return;
    }
    switch (n) {
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

// Q8_0 quantization of one 32-value block held by 8 consecutive lanes (lane
// part p = lane & 7 holds values 4p..4p+3): amax over the block by three lane
// exchanges, d = amax/127, id = amax ? 127/amax : 0, q = rne(x*id).  Returns
// the lane's four codes packed little-endian and sets d (f32, not yet rounded
// to f16).  Every step is one correctly rounded f32 operation (division is
// correctly rounded, no contraction, denormals kept), so any kernel using it
// yields the same codes.  All 64 lanes must call it together.
// Lane l reads lane (l & ~7) + 7 - (l & 7) of v, or v's lane l ^ 1 / l ^ 2 within its
// quad (DPP row_half_mirror / quad_perm: a VALU operand modifier, no LDS trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfRowMirror = 0x141;  // row_half_mirror: lane i of 8 reads lane 7 - i
constexpr int kDppRowRor8 = 0x128;        // row_ror:8: lane i of 16 reads lane i ^ 8

// Maximum over each aligned group of 8 lanes (every lane of the group gets
// it): the quad maxima, then the other quad's through the half-row mirror.
__device__ __forceinline__ float max8_lanes(float a) {
    a = fmaxf(a, dpp_f32<kDppQuadXor1>(a));
    a = fmaxf(a, dpp_f32<kDppQuadXor2>(a));
    return fmaxf(a, dpp_f32<kDppHalfRowMirror>(a));
}

// Maximum over the whole wave (every lane gets it): each 16-lane row's by
// DPP (the 8-lane maxima, then the other half row's by a rotation of 8),
// then the four rows' read into scalar registers.  No LDS trip, so it does
// not queue behind DMA traffic into LDS.  Exact in any order.
__device__ __forceinline__ float max64_lanes(float a) {
    a = max8_lanes(a);
    a = fmaxf(a, dpp_f32<kDppRowRor8>(a));
    const int b = __builtin_bit_cast(int, a);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over each aligned quad of lanes (every lane of the quad gets it).
__device__ __forceinline__ int sum4_lanes(int s) {
    s += __builtin_amdgcn_update_dpp(0, s, kDppQuadXor1, 0xF, 0xF, false);
    return s + __builtin_amdgcn_update_dpp(0, s, kDppQuadXor2, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t q8_0_part(float4 v, float &d) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = max8_lanes(a);
    d = a / 127.0f;
    const float id = (a != 0.0f) ? 127.0f / a : 0.0f;
    const int q0 = (int)rintf(v.x * id);
    const int q1 = (int)rintf(v.y * id);
    const int q2 = (int)rintf(v.z * id);
    const int q3 = (int)rintf(v.w * id);
    return (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
           ((uint32_t)(q3 & 0xff) << 24);
}

// Four bits b (b < 16) to bit 0 of four bytes: byte k gets bit k of b.  The
// shifted copies b, b << 7, b << 14, b << 21 do not overlap, so the product
// is their OR.
__device__ __forceinline__ uint32_t bits_to_bytes(uint32_t b) { return (b * 0x00204081u) & 0x01010101u; }

// Store one lane's part of a Q8_0 block at `blk` (a 2-byte aligned 34-byte
// block): its four codes at byte 2 + 4*part, and the f16 scale from part 0.
__device__ __forceinline__ void store_q8_0_part(uint8_t *blk, int part, uint32_t packed, float d) {
    uint16_t *o16 = reinterpret_cast<uint16_t *>(blk + 2 + 4 * part);
    o16[0] = (uint16_t)(packed & 0xffffu);
    o16[1] = (uint16_t)(packed >> 16);
    if (part == 0) *reinterpret_cast<uint16_t *>(blk) = (uint16_t)f32_to_f16_bits(d);
}

// Q8_K quantization (minfer quantize_row_q8_k_buf) of one 256-value
// super-block held by a whole wave, lane L with values 4L..4L+3 (group L/4
// of 16 values): amax over the wave (max64_lanes), d = amax/127 (kept f32), id = amax ?
// 127/amax : 0, q = saturate(rne(x*id)) to [-128, 127].  Returns the lane's
// four codes packed little-endian and sets gsum to its group's code sum (the
// same in the group's four lanes) and d.  The same single correctly rounded
// f32 steps as q8_0_part, so every kernel using it yields the same bytes.
// All 64 lanes must call it together.
__device__ __forceinline__ uint32_t q8_k_wave(float4 v, int &gsum, float &d) {
    const float a = max64_lanes(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    d = a / 127.0f;
    const float id = (a != 0.0f) ? 127.0f / a : 0.0f;
    int q[4];
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float r = rintf(vv[k] * id);
        r = fminf(fmaxf(r, -128.0f), 127.0f);
        q[k] = (int)r;
    }
    gsum = sum4_lanes(q[0] + q[1] + q[2] + q[3]);
    return (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) | ((uint32_t)(q[2] & 0xff) << 16) |
           ((uint32_t)(q[3] & 0xff) << 24);
}

// Store one lane's share of a Q8_K block at `blk` (4-byte aligned, 292
// bytes: f32 d, 256 codes, 16 int16 group sums): its four codes, its group's
// sum from the group's first lane and d from lane 0.
__device__ __forceinline__ void store_q8_k_lane(uint8_t *blk, int lane, uint32_t packed, int gsum, float d) {
    *reinterpret_cast<uint32_t *>(blk + 4 + 4 * lane) = packed;
    if ((lane & 3) == 0) *reinterpret_cast<int16_t *>(blk + 260 + 2 * (lane >> 2)) = (int16_t)gsum;
    if (lane == 0) *reinterpret_cast<float *>(blk) = d;
}

}  // namespace qmm
