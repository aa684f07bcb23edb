// Products of a few tokens (M <= small_tokens(format)) on the decode kernel: TT tokens
// per grid row, each wave's weight slice streamed once per TT tokens (kernel:
// matvec_kernel.h).
#include "matvec_kernel.h"

namespace qmm {

hipError_t launch_matvec_q4_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q8_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q2_k(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q4_k(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q6_k(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q4_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q5_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q5_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);

// A few tokens at once (the product entry points for small M): the decode
// kernel with TT tokens per grid row and the rows per wave chosen as for
// decode (about 5 KB per wave, at least 2048 waves over the grid's rows of
// tokens where the matrix has the rows: Q4_0 512 x 1024, M = 8, 8 rows per
// wave 12.1 us, 1 row 4.8 us; 2048 x 4096, M = 16, 1 row 7.4 us, 2 rows 7.0
// us), a row of more than 64 units or 5 KB walked in 64-unit segments, so
// that TT activation segments and the slices fit in LDS.
template <int F, bool PAIRED, int TT>
static hipError_t pick_mv_tokens(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    using FB = FmtBytes<F>;
    using UT = Unit<F, PAIRED>;
    constexpr int NW = TT >= 8 ? 8 : 4;   // eight waves share the larger activation copy of 8 tokens
    const int nu = (nb / UT::BPU) * UT::UPB;
    const int64_t gy = (M + TT - 1) / TT;
    const int64_t g = min(5000 / ((int64_t)nb * FB::BB), max((int64_t)1, (int64_t)N * gy / kMinDecodeWaves));
    if (nu > kWave || g < 2) return launch_mv<F, PAIRED, 1, 1, false, NW, TT>(w, xq, nullptr, y, M, N, nb, st);
    if (g >= 8) return launch_mv<F, PAIRED, 8, 1, false, NW, TT>(w, xq, nullptr, y, M, N, nb, st);
    if (g >= 4) return launch_mv<F, PAIRED, 4, 1, false, NW, TT>(w, xq, nullptr, y, M, N, nb, st);
    return launch_mv<F, PAIRED, 2, 1, false, NW, TT>(w, xq, nullptr, y, M, N, nb, st);
}

template <int F, bool PAIRED>
static hipError_t mv_tokens(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    if (M <= 2) return pick_mv_tokens<F, PAIRED, 2>(w, xq, y, M, N, nb, st);
    if (M <= 4) return pick_mv_tokens<F, PAIRED, 4>(w, xq, y, M, N, nb, st);
    return pick_mv_tokens<F, PAIRED, 8>(w, xq, y, M, N, nb, st);
}

// Products of 2 .. small_tokens(format) tokens for any weight format.
template <int F>
static hipError_t matvec_tokens(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    if constexpr (!kIsK<F>) {
        if (nb % 2 == 0) return mv_tokens<F, true>(w, xq, y, M, N, nb, st);
    }
    return mv_tokens<F, false>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matvec_tokens(int fmt, const void *w, const void *xq, float *y, int M, int N, int nb,
                                hipStream_t st) {
    if (M < 1 || M > small_tokens(fmt)) return hipErrorInvalidValue;
    if (M == 1) {   // one token: the decode launch itself
        switch (fmt) {
            case F_Q4_0: return launch_matvec_q4_0(w, xq, y, N, nb, st);
            case F_Q8_0: return launch_matvec_q8_0(w, xq, y, N, nb, st);
            case F_Q4_1: return launch_matvec_q4_1(w, xq, y, N, nb, st);
            case F_Q5_0: return launch_matvec_q5_0(w, xq, y, N, nb, st);
            case F_Q5_1: return launch_matvec_q5_1(w, xq, y, N, nb, st);
            case F_Q2_K: return launch_matvec_q2_k(w, xq, y, N, nb, st);
            case F_Q4_K: return launch_matvec_q4_k(w, xq, y, N, nb, st);
            case F_Q6_K: return launch_matvec_q6_k(w, xq, y, N, nb, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (fmt) {
        case F_Q4_0: return matvec_tokens<F_Q4_0>(w, xq, y, M, N, nb, st);
        case F_Q8_0: return matvec_tokens<F_Q8_0>(w, xq, y, M, N, nb, st);
        case F_Q4_1: return matvec_tokens<F_Q4_1>(w, xq, y, M, N, nb, st);
        case F_Q5_0: return matvec_tokens<F_Q5_0>(w, xq, y, M, N, nb, st);
        case F_Q5_1: return matvec_tokens<F_Q5_1>(w, xq, y, M, N, nb, st);
        case F_Q2_K: return matvec_tokens<F_Q2_K>(w, xq, y, M, N, nb, st);
        case F_Q4_K: return matvec_tokens<F_Q4_K>(w, xq, y, M, N, nb, st);
        case F_Q6_K: return matvec_tokens<F_Q6_K>(w, xq, y, M, N, nb, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
