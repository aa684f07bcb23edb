// Attainable-peak probes (libqmm_probe.so, declared in include/qmm_probe.h):
// the measured ceilings that the product kernels are compared with beside the
// published ones -- a streaming read of a device buffer (HBM, the bound of
// every decode kernel), a back-to-back int8 MFMA loop (the matrix cores) and
// an issue-rate loop of f32 FMAs, int8 MFMAs or both interleaved (what bounds
// a prefill whose per-block scale fold runs on the vector ALU).  None computes
// anything of the product path, and the product library neither contains nor
// calls them.
#include <atomic>
#include <cstring>

#include "qmm_device.h"
#include "qmm_probe.h"

namespace qmm {

// One pass over `bytes` with a full grid.  Workgroup b of NW waves covers the
// span [S b, S b + S), S = NW * LPL * 1024; wave w of it the 1 KB chunks
// (b NW + w) LPL .. + LPL - 1, lane l bytes [16 l, 16 l + 16) of each, all LPL
// loads issued before any is used (LPL loads in flight per lane).  NT: the
// loads carry the non-temporal cache policy.  sink[b] = XOR of the span's
// 32-bit words (words past the end count as 0).  No grid-stride loop and no
// atomics: one store per workgroup.
template <int LPL, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void k_probe_read(const uint4 *__restrict__ p, int64_t n16,
                                                        uint32_t *__restrict__ sink) {
    __shared__ uint32_t red[NW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * NW + wave) * LPL * 64 + lane;   // first 16-byte granule
    uint4 v[LPL];
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
        const int64_t c = c0 + 64 * k;
        if (c < n16) {
            if constexpr (NT) {
                typedef unsigned int u4v __attribute__((ext_vector_type(4)));
                const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p + c));
                v[k] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
                v[k] = p[c];
            }
        } else {
            v[k] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < LPL; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) s ^= red[w];
        sink[blockIdx.x] = s;
    }
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

// Issue-rate loop, WPS waves per SIMD (workgroups of 4 * WPS waves, one per
// CU).  Per iteration and wave: MODE 0 issues 128 v_fma_f32 whose operands
// are all vector registers (16 independent chains c = c * b + a), MODE 1 four
// v_mfma_i32_32x32x32_i8 (four independent accumulators), MODE 2 both, 32
// FMAs after each MFMA, MODE 3 the FMAs of MODE 0 with b read from a scalar
// register (the form a kernel argument takes).  The prefill folds use the
// vector-register form; the scalar-operand form issues at about half its rate
// with two waves per SIMD (it is not issued two at a time).  With every MFMA
// operand byte 1, outi = 2048 * iters for MODES 1 and 2 (0 otherwise); out
// holds the FMA chains' sum (finite for a in (0, 2), b in (0, 1)).
template <int MODE, int WPS>
__global__ __launch_bounds__(256 * WPS) void k_probe_issue(float *__restrict__ out, int32_t *__restrict__ outi,
                                                           int iters, float a, float b, int ones) {
    const v4i va = {ones, ones, ones, ones};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    // per-lane copies of a and b: vector registers, the fold's operand form
    float av = a + 0.0f * (float)threadIdx.x, bv = b + 0.0f * (float)threadIdx.x;
    asm volatile("" : "+v"(av), "+v"(bv));
    float c[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = av + (float)r;
    auto fmas = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[r] = fmaf(c[r], MODE == 3 ? b : bv, av);
    };
    for (int i = 0; i < iters; ++i) {
        if constexpr (MODE == 1 || MODE == 2) c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, va, c0, 0, 0, 0);
        if constexpr (MODE != 1) fmas();
        if constexpr (MODE == 1 || MODE == 2) c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, va, c1, 0, 0, 0);
        if constexpr (MODE != 1) fmas();
        if constexpr (MODE == 1 || MODE == 2) c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, va, c2, 0, 0, 0);
        if constexpr (MODE != 1) fmas();
        if constexpr (MODE == 1 || MODE == 2) c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, va, c3, 0, 0, 0);
        if constexpr (MODE != 1) fmas();
    }
    int si = 0;
    float sf = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        si += c0[r] + c1[r] + c2[r] + c3[r];
        sf += c[r];
    }
    const int64_t t = (int64_t)blockIdx.x * (256 * WPS) + threadIdx.x;
    out[t] = sf;
    outi[t] = si;
}

template <int MODE, int WPS>
static hipError_t launch_issue(float *out, int32_t *outi, int iters, hipStream_t st) {
    hipLaunchKernelGGL((k_probe_issue<MODE, WPS>), dim3(256), dim3(256 * WPS), 0, st, out, outi, iters, 1.0001f,
                       0.9999f, 0x01010101);
    return hipGetLastError();
}

template <int WPS>
static hipError_t launch_issue_mode(int mode, float *out, int32_t *outi, int iters, hipStream_t st) {
    switch (mode) {
        case 0: return launch_issue<0, WPS>(out, outi, iters, st);
        case 1: return launch_issue<1, WPS>(out, outi, iters, st);
        case 2: return launch_issue<2, WPS>(out, outi, iters, st);
        case 3: return launch_issue<3, WPS>(out, outi, iters, st);
    }
    return hipErrorInvalidValue;
}

template <int LPL, int NW, bool NT>
static hipError_t launch_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t st) {
    const int64_t span = (int64_t)NW * LPL * 1024;
    const int64_t grid = (bytes + span - 1) / span;
    hipLaunchKernelGGL((k_probe_read<LPL, NW, NT>), dim3((unsigned)grid), dim3(64 * NW), 0, st,
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

template <int LPL, bool NT>
static hipError_t launch_read_nw(int nw, const void *buf, int64_t bytes, uint32_t *sink, hipStream_t st) {
    switch (nw) {
        case 4: return launch_read<LPL, 4, NT>(buf, bytes, sink, st);
        case 8: return launch_read<LPL, 8, NT>(buf, bytes, sink, st);
        case 16: return launch_read<LPL, 16, NT>(buf, bytes, sink, st);
    }
    return hipErrorInvalidValue;
}

template <bool NT>
static hipError_t launch_read_lpl(int lpl, int nw, const void *buf, int64_t bytes, uint32_t *sink, hipStream_t st) {
    switch (lpl) {
        case 1: return launch_read_nw<1, NT>(nw, buf, bytes, sink, st);
        case 2: return launch_read_nw<2, NT>(nw, buf, bytes, sink, st);
        case 4: return launch_read_nw<4, NT>(nw, buf, bytes, sink, st);
        case 8: return launch_read_nw<8, NT>(nw, buf, bytes, sink, st);
        case 16: return launch_read_nw<16, NT>(nw, buf, bytes, sink, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qmm

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMM_PROBE_E_DEVICE;
    int s = g_device_state[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return QMM_PROBE_E_DEVICE;
        s = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_state[dev].store(s, std::memory_order_release);
    }
    return s == 1 ? QMM_PROBE_OK : QMM_PROBE_E_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? QMM_PROBE_OK : QMM_PROBE_E_LAUNCH; }

}  // namespace

extern "C" {

int64_t qmm_probe_read_span(int loads_per_lane, int waves_per_wg) {
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 &&
        loads_per_lane != 16)
        return 0;
    if (waves_per_wg != 4 && waves_per_wg != 8 && waves_per_wg != 16) return 0;
    return (int64_t)loads_per_lane * waves_per_wg * 1024;
}

int qmm_peak_read(const void *buf, int64_t bytes, uint32_t *sink, int loads_per_lane, int waves_per_wg,
                  int nontemporal, void *stream) {
    const int64_t span = qmm_probe_read_span(loads_per_lane, waves_per_wg);
    if (span == 0 || bytes <= 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 40) ||
        (bytes + span - 1) / span > 0x7fffffff)
        return QMM_PROBE_E_SHAPE;
    if (!buf || !sink) return QMM_PROBE_E_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return QMM_PROBE_E_ALIGN;
    int s = check_device();
    if (s != QMM_PROBE_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return launched(nontemporal ? qmm::launch_read_lpl<true>(loads_per_lane, waves_per_wg, buf, bytes, sink, st)
                                : qmm::launch_read_lpl<false>(loads_per_lane, waves_per_wg, buf, bytes, sink, st));
}

int qmm_probe_issue(int mode, int waves_per_simd, int64_t iters, float *out, int32_t *outi, void *stream) {
    if (mode < 0 || mode > 3 || (waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || iters > 1000000)
        return QMM_PROBE_E_SHAPE;
    if (!out || !outi) return QMM_PROBE_E_NULL;
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0 || (reinterpret_cast<uintptr_t>(outi) & 3u) != 0)
        return QMM_PROBE_E_ALIGN;
    int s = check_device();
    if (s != QMM_PROBE_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return launched(waves_per_simd == 1 ? qmm::launch_issue_mode<1>(mode, out, outi, (int)iters, st)
                                        : qmm::launch_issue_mode<2>(mode, out, outi, (int)iters, st));
}

int qmm_peak_mfma_i8(int32_t *out, int64_t workgroups, int64_t iters, void *stream) {
    if (workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1 || iters > 1000000) return QMM_PROBE_E_SHAPE;
    if (!out) return QMM_PROBE_E_NULL;
    if ((reinterpret_cast<uintptr_t>(out) & 15u) != 0) return QMM_PROBE_E_ALIGN;
    int s = check_device();
    if (s != QMM_PROBE_OK) return s;
    hipLaunchKernelGGL(qmm::k_peak_mfma_i8, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       out, (int)iters, 0x01010101, 0x01010101);
    return launched(hipGetLastError());
}

}  // extern "C"
