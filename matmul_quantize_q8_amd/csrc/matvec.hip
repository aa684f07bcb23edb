// Decode matvec, one token: y[n] = sum_b d_w[n,b] d_x[b] I_b[n].
//
// Decode is weight streaming: every weight byte is read once per token
// (minfer section 2.1, "the decode physics"), so the kernel is bound by HBM
// and is built around moving the weight bytes at full rate:
//   * a wave owns G consecutive rows (whole rows: every output is reduced
//     inside one wave, in a fixed order, and written once -- minfer's row
//     ownership);
//   * the rows' bytes form one contiguous span; the wave copies it into its
//     own LDS slice with coalesced 16-byte loads (Q4_0 / Q8_0 blocks are only
//     2-byte aligned, so blocks are re-sliced from LDS instead of global);
//   * each lane owns fixed block columns of the row, keeps the matching
//     activation blocks in registers for the whole kernel, and runs packed
//     int8 dot instructions (v_dot4c_i32_i8) on them;
//   * the per-block scale product d_w*d_x is exact in f32 (two binary16
//     values), so each block adds one correctly rounded term;
//   * the lane partial sums of a row are combined with a shuffle tree.
// For rows longer than one LDS slice (very large K) the wave walks the row in
// segments and keeps its partial sums across them.
#include "qmm_device.h"

namespace qmm {

enum Fmt { F_Q4_0 = 0, F_Q8_0 = 1, F_Q2_K = 2 };

template <int F> struct MvTraits;
template <> struct MvTraits<F_Q4_0> { static constexpr int BB = kQ40Bytes, XB = kQ80Bytes, UPB = 1, MAXU = 8; };
template <> struct MvTraits<F_Q8_0> { static constexpr int BB = kQ80Bytes, XB = kQ80Bytes, UPB = 1, MAXU = 4; };
template <> struct MvTraits<F_Q2_K> { static constexpr int BB = kQ2KBytes, XB = kQ8KBytes, UPB = 4, MAXU = 4; };

// Activation registers for one unit a lane owns.
template <int F> struct XUnit;
template <> struct XUnit<F_Q4_0> { int q[8]; int sx8; float d; };
template <> struct XUnit<F_Q8_0> { int q[8]; float d; };
template <> struct XUnit<F_Q2_K> { int q[16]; int bs[4]; float d; };

// --- activation loads (global, once per segment) ----------------------------
// Q8_0 block c: f16 d at byte 34c, codes at 34c+2 (2-byte aligned).  Nine
// aligned dwords cover the codes; the ninth is read only when needed and then
// lies in the same aligned dword as the block's last byte.
__device__ __forceinline__ void load_x_q8_0(const uint8_t *xq, int c, int *q, float &d) {
    const uint32_t o = 34u * (uint32_t)c;
    const uint32_t qd = (o + 2) >> 2, qsh = (o + 2) & 3;
    const uint32_t *p = reinterpret_cast<const uint32_t *>(xq) + qd;
    uint32_t v[9];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[k];
    v[8] = qsh ? p[8] : 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = (int)align_bytes(v[k + 1], v[k], qsh);
    d = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(xq + o));
}

template <int F>
__device__ __forceinline__ void load_x(const uint8_t *xq, int u, XUnit<F> &x);

template <>
__device__ __forceinline__ void load_x<F_Q4_0>(const uint8_t *xq, int u, XUnit<F_Q4_0> &x) {
    load_x_q8_0(xq, u, x.q, x.d);
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = dot4(x.q[k], 0x01010101, s);
    x.sx8 = 8 * s;                 // sum_j (n_j - 8) q_j = sum_j n_j q_j - 8 sum_j q_j
}

template <>
__device__ __forceinline__ void load_x<F_Q8_0>(const uint8_t *xq, int u, XUnit<F_Q8_0> &x) {
    load_x_q8_0(xq, u, x.q, x.d);
}

// Q8_K unit (c, p): part p of super-block c covers qs bytes [16p, 16p+16) of
// the weight block, i.e. values 128h + 32s + 16(p&1) + [0,16) for s < 4, h = p/2,
// which are groups g = 8h + 2s + (p&1).
template <>
__device__ __forceinline__ void load_x<F_Q2_K>(const uint8_t *xq, int u, XUnit<F_Q2_K> &x) {
    const int c = u >> 2, p = u & 3, h = p >> 1, odd = p & 1;
    const uint8_t *b = xq + (int64_t)c * kQ8KBytes;
    const uint32_t *q32 = reinterpret_cast<const uint32_t *>(b + 4 + 128 * h + 16 * odd);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) x.q[4 * s + k] = (int)q32[8 * s + k];
    const int16_t *bs = reinterpret_cast<const int16_t *>(b + 260 + 16 * h + 2 * odd);
#pragma unroll
    for (int s = 0; s < 4; ++s) x.bs[s] = bs[2 * s];
    x.d = *reinterpret_cast<const float *>(b);
}

// --- one unit's contribution, weights read from the LDS slice ---------------
template <int F>
__device__ __forceinline__ float unit_dot(const uint8_t *lds8, uint32_t bo, int p, const XUnit<F> &x, float acc);

// Q4_0 block at LDS byte bo (even): f16 d, then 16 nibble bytes.  Low nibbles
// are elements 0..15, high nibbles 16..31 (minfer scalar kernel; ggml sec. 2).
template <>
__device__ __forceinline__ float unit_dot<F_Q4_0>(const uint8_t *lds8, uint32_t bo, int, const XUnit<F_Q4_0> &x,
                                                  float acc) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(lds8);
    const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
    uint32_t v[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) v[k] = l32[qd + k];
    const float dw = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(lds8 + bo));
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t q = align_bytes(v[k + 1], v[k], qsh);
        s = dot4((int)(q & 0x0f0f0f0fu), x.q[k], s);
        s = dot4((int)((q >> 4) & 0x0f0f0f0fu), x.q[k + 4], s);
    }
    return fmaf(dw * x.d, (float)(s - x.sx8), acc);
}

template <>
__device__ __forceinline__ float unit_dot<F_Q8_0>(const uint8_t *lds8, uint32_t bo, int, const XUnit<F_Q8_0> &x,
                                                  float acc) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(lds8);
    const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
    uint32_t v[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) v[k] = l32[qd + k];
    const float dw = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(lds8 + bo));
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = dot4((int)align_bytes(v[k + 1], v[k], qsh), x.q[k], s);
    return fmaf(dw * x.d, (float)s, acc);
}

// Q2_K part p of the block at LDS byte bo (4-byte aligned):
//   V = sum_s sc_s * sum q x,  Mn = sum_s m_s * bsum_s,
//   t = d d8 V - dmin d8 Mn   (minfer "a K-quant dot kernel, walked").
template <>
__device__ __forceinline__ float unit_dot<F_Q2_K>(const uint8_t *lds8, uint32_t bo, int p, const XUnit<F_Q2_K> &x,
                                                  float acc) {
    const uint32_t *b32 = reinterpret_cast<const uint32_t *>(lds8 + bo);
    const int h = p >> 1, odd = p & 1;
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = b32[4 + 4 * p + k];
    const uint32_t sc01 = b32[2 * h], sc23 = b32[2 * h + 1];
    const uint32_t dd = b32[20];
    int V = 0, Mn = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t sw = (s < 2) ? sc01 : sc23;
        const uint32_t scm = (sw >> (8 * (2 * (s & 1) + odd))) & 0xffu;
        int g = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) g = dot4((int)((q[k] >> (2 * s)) & 0x03030303u), x.q[4 * s + k], g);
        V += (int)(scm & 0x0f) * g;
        Mn += (int)(scm >> 4) * x.bs[s];
    }
    const float d = f16_bits_to_f32(dd), dmin = f16_bits_to_f32(dd >> 16);
    acc = fmaf(d * x.d, (float)V, acc);
    return fmaf(-(dmin * x.d), (float)Mn, acc);
}

// --- the kernel ---------------------------------------------------------------
// gridDim.y tokens: token t reads activation row t (xrow bytes apart) and
// writes output row t; the weight rows are re-read for every token.
template <int F, int LPR>
__global__ __launch_bounds__(256) void k_matvec(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                                float *__restrict__ y, int N, int nb, int64_t xrow) {
    using T = MvTraits<F>;
    xq += (int64_t)blockIdx.y * xrow;
    y += (int64_t)blockIdx.y * N;
    constexpr int G = kWave / LPR;                       // rows per wave
    constexpr int SEGU = LPR * T::MAXU;                  // units per segment
    constexpr int SEGB = SEGU / T::UPB;                  // blocks per segment
    constexpr int LDSW = ((G * SEGB * T::BB + 31) / 16 + 1) * 16;   // bytes per wave slice
    constexpr int CH = (LDSW / 16 + kWave - 1) / kWave;  // 16-byte chunks per lane
    __shared__ uint4 lds_all[4 * (LDSW / 16)];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * G;
    if (row0 >= N) return;                               // whole wave
    const int nrows = (int)min((int64_t)G, (int64_t)N - row0);
    const int lg = lane / LPR, li = lane % LPR;
    const int64_t RB = (int64_t)nb * T::BB;
    uint4 *lds = lds_all + wave * (LDSW / 16);
    const uint8_t *lds8 = reinterpret_cast<const uint8_t *>(lds);

    float acc = 0.0f;
    for (int seg0 = 0; seg0 < nb; seg0 += SEGB) {
        const int seg1 = min(nb, seg0 + SEGB);
        const int64_t lo = row0 * RB + (int64_t)seg0 * T::BB;
        const int64_t hi = (row0 + nrows - 1) * RB + (int64_t)seg1 * T::BB;
        const int64_t A = lo & ~(int64_t)15;
        const int nch = (int)((((hi + 15) & ~(int64_t)15) - A) >> 4);   // <= LDSW/16

        // weights of the span -> this wave's LDS slice, straight from global
        // (global_load_lds_dwordx4: lane i of a load fills bytes [16i, 16i+16)
        // of the 1 KB at the wave-uniform LDS address; no VGPRs involved).
        const uint8_t *src = w + A;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int c = k * kWave + lane;
            if (c < nch) global_to_lds16(src + 16 * (int64_t)c, lds + k * kWave);
        }
        // this lane's activation units for the segment (L2-resident); a lane
        // past the row end loads a valid unit and ignores it
        XUnit<F> xu[T::MAXU];
        const int ulast = seg1 * T::UPB - 1;
#pragma unroll
        for (int i = 0; i < T::MAXU; ++i) load_x<F>(xq, min(seg0 * T::UPB + li + i * LPR, ulast), xu[i]);
        wait_global_loads();
        __builtin_amdgcn_wave_barrier();

        if (lg < nrows) {
            const uint32_t rbase = (uint32_t)((row0 + lg) * RB + (int64_t)seg0 * T::BB - A);
#pragma unroll
            for (int i = 0; i < T::MAXU; ++i) {
                const int u = seg0 * T::UPB + li + i * LPR;
                if (u < seg1 * T::UPB) {
                    const int c = u / T::UPB - seg0;
                    acc = unit_dot<F>(lds8, rbase + (uint32_t)c * T::BB, u % T::UPB, xu[i], acc);
                }
            }
        }
        if (seg1 < nb) {      // the slice is rewritten by the next segment
            wait_lds_reads();
            __builtin_amdgcn_wave_barrier();
        }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += xor_shfl(acc, m);
    if (li == 0 && lg < nrows) y[row0 + lg] = acc;
}

template <int F, int LPR>
static hipError_t launch_mv(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    constexpr int G = kWave / LPR;
    const int64_t waves = ((int64_t)N + G - 1) / G;
    const int64_t grid = (waves + 3) / 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    int64_t xrow = (int64_t)nb * MvTraits<F>::XB;
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&N, (void *)&nb, (void *)&xrow};
    return hipLaunchKernel((const void *)k_matvec<F, LPR>, dim3((unsigned)grid, (unsigned)M), dim3(256), args, 0,
                           st);
}

// Lanes per row: the smallest of 16 / 32 / 64 whose lanes cover a whole row
// in one segment (so several rows share a wave and its loads), else 64.
template <int F>
static hipError_t dispatch_mv(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    using T = MvTraits<F>;
    const int64_t units = (int64_t)nb * T::UPB;
    if (units <= 16 * T::MAXU) return launch_mv<F, 16>(w, xq, y, M, N, nb, st);
    if (units <= 32 * T::MAXU) return launch_mv<F, 32>(w, xq, y, M, N, nb, st);
    return launch_mv<F, 64>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matvec_q4_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q4_0>(w, xq, y, 1, N, nb, st);
}
hipError_t launch_matvec_q8_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q8_0>(w, xq, y, 1, N, nb, st);
}
hipError_t launch_matvec_q2_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st) {
    return dispatch_mv<F_Q2_K>(w, xq, y, 1, N, ns, st);
}
// Q2_K prefill: the matvec kernel with one grid row per token (the weights are
// re-read from cache for each token; correct for any M, not tuned).
hipError_t launch_matmul_q2_k(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    constexpr int kMaxY = 65535;
    for (int m0 = 0; m0 < M; m0 += kMaxY) {
        const int mc = min(kMaxY, M - m0);
        const uint8_t *xp = static_cast<const uint8_t *>(xq) + (int64_t)m0 * ns * kQ8KBytes;
        const hipError_t e = dispatch_mv<F_Q2_K>(w, xp, y + (int64_t)m0 * N, mc, N, ns, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmm
