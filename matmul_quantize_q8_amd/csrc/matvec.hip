// Decode launchers: the rows per wave, the fused quantize + matvec step and the
// entry points of every format (kernel and its design: matvec_kernel.h).
#include "matvec_kernel.h"

namespace qmm {

hipError_t launch_quantize_q8_0(const float *x, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q8_k(const float *x, void *out, int64_t nblocks, hipStream_t st);

// Rows per wave: a slice of about 5 KB.  Measured on MI355X over 28-96 MB
// of weights, slices of 3-5 KB per wave (Q4_0 K=4096: 2 rows, Q8_0: 1 row,
// Q2_K: 2 rows) beat larger ones: the work after the last byte lands is
// smaller and all waves of the launch stay resident.  A row longer than
// that is walked by one wave in segments of 64 units (4.4 KB of Q8_0), so
// that the slices stay small and every workgroup fits in LDS at once (Q8_0
// 4096 x 11008: 11.3 us against 12.4 us with whole-row slices of 11.7 KB,
// which left room for two workgroups per CU and ran in two rounds).  A
// launch also keeps at least 2048 waves (8 per CU) where the matrix has the
// rows: fewer, longer-working waves leave the CUs idle and put several rows'
// arithmetic behind the last byte (Q4_0 512 x 1024, fused step: 8 rows per
// wave 4.89 us, 1 row 2.80 us; 2048 x 4096: 2 rows 3.98 us, 1 row 3.76 us;
// 8192 x 1024: 8 rows 5.61 us, 4 rows 4.34 us).
template <int F, bool PAIRED, bool XF32>
static hipError_t pick_mv(const void *w, const void *xin, uint8_t *xq_out, float *y, int M, int N, int nb,
                          hipStream_t st) {
    using FB = FmtBytes<F>;
    using UT = Unit<F, PAIRED>;
    // The fused kernel runs eight waves per workgroup when a row fits one
    // segment: every workgroup quantizes the whole activation row, so fewer,
    // larger workgroups do less of that redundant work (measured on MI355X,
    // Q4_0 12288x4096: 7.5 us with eight waves against 8.4 us with four; the
    // LDS of eight slices still fits three workgroups per CU).
    constexpr int NW1 = XF32 ? 8 : 4;
    const int nu = (nb / UT::BPU) * UT::UPB;
    const int64_t rb = (int64_t)nb * FB::BB;
    const int64_t g = min(5000 / rb, max((int64_t)1, (int64_t)N / kMinDecodeWaves));
    if (nu > kWave && g == 0) return launch_mv<F, PAIRED, 1, 1, XF32>(w, xin, xq_out, y, M, N, nb, st);
    if (nu <= kWave) {
        if (g >= 8) return launch_mv<F, PAIRED, 8, 1, XF32, NW1>(w, xin, xq_out, y, M, N, nb, st);
        if (g >= 4) return launch_mv<F, PAIRED, 4, 1, XF32, NW1>(w, xin, xq_out, y, M, N, nb, st);
        if (g >= 2) return launch_mv<F, PAIRED, 2, 1, XF32, NW1>(w, xin, xq_out, y, M, N, nb, st);
        return launch_mv<F, PAIRED, 1, 1, XF32, NW1>(w, xin, xq_out, y, M, N, nb, st);
    }
    if (g >= 4) return launch_mv<F, PAIRED, 4, 4, XF32>(w, xin, xq_out, y, M, N, nb, st);
    if (g >= 2) return launch_mv<F, PAIRED, 2, 4, XF32>(w, xin, xq_out, y, M, N, nb, st);
    return launch_mv<F, PAIRED, 1, 4, XF32>(w, xin, xq_out, y, M, N, nb, st);
}

template <int F, bool XF32 = false>
static hipError_t dispatch_mv(const void *w, const void *xin, uint8_t *xq_out, float *y, int M, int N, int nb,
                              hipStream_t st) {
    if constexpr (!kIsK<F>) {
        if (nb % 2 == 0) return pick_mv<F, true, XF32>(w, xin, xq_out, y, M, N, nb, st);
    }
    return pick_mv<F, false, XF32>(w, xin, xq_out, y, M, N, nb, st);
}


hipError_t launch_matvec_q4_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q4_0>(w, xq, nullptr, y, 1, N, nb, st);
}
hipError_t launch_matvec_q8_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q8_0>(w, xq, nullptr, y, 1, N, nb, st);
}
hipError_t launch_matvec_q2_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st) {
    return dispatch_mv<F_Q2_K>(w, xq, nullptr, y, 1, N, ns, st);
}
// Fused decode step.  A row of more than one segment (more than 64 units)
// makes every workgroup quantize a long activation row, as many bytes as its
// weights (Q8_0 4096 x 11008 on MI355X: 16.0 us fused against 13.9 us for two
// launches); there, when the caller supplies the Q8_0 output row, the
// activation is quantized into it once and the plain matvec reads it.  The
// result is the same either way: the same codes, the same per-row order.
template <int F>
static hipError_t quantize_matvec(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                  hipStream_t st) {
    const bool paired = !kIsK<F> && nb % 2 == 0;
    const int nu = kIsK<F> ? 4 * nb : paired ? nb / 2 : nb;   // units per row (a K-quant super-block: 4)
    if (xq != nullptr && nu > kWave) {
        const hipError_t e = kIsK<F> ? launch_quantize_q8_k(x, xq, nb, st) : launch_quantize_q8_0(x, xq, nb, st);
        if (e != hipSuccess) return e;
        return dispatch_mv<F>(w, xq, nullptr, y, 1, N, nb, st);
    }
    return dispatch_mv<F, true>(w, x, static_cast<uint8_t *>(xq), y, 1, N, nb, st);
}

hipError_t launch_quantize_matvec_q4_0(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st) {
    return quantize_matvec<F_Q4_0>(w, x, xq, y, N, nb, st);
}
hipError_t launch_quantize_matvec_q8_0(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st) {
    return quantize_matvec<F_Q8_0>(w, x, xq, y, N, nb, st);
}
// K-quant weights: Q8_K activations, nb = super-blocks per row
hipError_t launch_quantize_matvec_q2_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st) {
    return quantize_matvec<F_Q2_K>(w, x, xq, y, N, nb, st);
}
hipError_t launch_quantize_matvec_q4_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st) {
    return quantize_matvec<F_Q4_K>(w, x, xq, y, N, nb, st);
}
hipError_t launch_quantize_matvec_q6_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st) {
    return quantize_matvec<F_Q6_K>(w, x, xq, y, N, nb, st);
}

hipError_t launch_matvec_q4_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q4_1>(w, xq, nullptr, y, 1, N, nb, st);
}
hipError_t launch_matvec_q5_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q5_0>(w, xq, nullptr, y, 1, N, nb, st);
}
hipError_t launch_matvec_q5_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st) {
    return dispatch_mv<F_Q5_1>(w, xq, nullptr, y, 1, N, nb, st);
}
hipError_t launch_matvec_q4_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st) {
    return dispatch_mv<F_Q4_K>(w, xq, nullptr, y, 1, N, ns, st);
}
hipError_t launch_matvec_q6_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st) {
    return dispatch_mv<F_Q6_K>(w, xq, nullptr, y, 1, N, ns, st);
}

}  // namespace qmm
