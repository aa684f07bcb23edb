// Embedding rows: out[t][:] = the decoded row ids[t] of a quantized table
// (minfer "The embedding matmul": not a product, a lookup that walks the
// token's row block by block and dequantizes it; one row getter for every
// backend keeps the embeddings byte-for-byte identical).
//
// Bit-exactness: each decoded value is a binary16 scale times a small integer
// (exact in f32: at most 11 + 13 significant bits), or for the formats with
// mins or offsets the difference or sum of two such exact values, rounded once (the library is
// built without contraction, so no fused multiply-add changes that rounding).
// The result is the exactly decoded value rounded to f32, as the oracle's.
#include "qmm_device.h"

namespace qmm {

__device__ __forceinline__ float rd_f16(const uint8_t *p) {
    return f16_bits_to_f32((uint32_t)p[0] | ((uint32_t)p[1] << 8));
}

// Values i0 .. i0+3 (i0 % 4 == 0) of a row in format F.
template <int F>
__device__ __forceinline__ void decode4(const uint8_t *row, int64_t i0, float (&v)[4]) {
    if constexpr (F == F_Q4_0 || F == F_Q8_0) {
        constexpr int BB = (F == F_Q4_0) ? kQ40Bytes : kQ80Bytes;
        const uint8_t *blk = row + (i0 >> 5) * BB;
        const int j = (int)(i0 & 31);
        const float d = rd_f16(blk);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = j + k;
            int c;
            if constexpr (F == F_Q4_0) {
                const int byte = blk[2 + (e & 15)];               // low nibble: element e, high: e + 16
                c = (e < 16 ? (byte & 15) : (byte >> 4)) - 8;
            } else {
                c = (int8_t)blk[2 + e];
            }
            v[k] = d * (float)c;
        }
    } else if constexpr (F == F_Q4_1 || F == F_Q5_0 || F == F_Q5_1) {
        // d*q + m (_1) or d*(q - 16) (Q5_0); qs byte j = value j | value j+16 << 4,
        // bit j of the little-endian qh = value j's fifth bit
        constexpr int BB = F == F_Q4_1 ? kQ41Bytes : (F == F_Q5_0 ? kQ50Bytes : kQ51Bytes);
        constexpr int QS = F == F_Q4_1 ? 4 : (F == F_Q5_0 ? 6 : 8);
        constexpr int QH = F == F_Q5_0 ? 2 : 4;
        const uint8_t *blk = row + (i0 >> 5) * BB;
        const int j = (int)(i0 & 31);
        const float d = rd_f16(blk);
        uint32_t qh = 0;
        if constexpr (F != F_Q4_1)
            qh = (uint32_t)blk[QH] | ((uint32_t)blk[QH + 1] << 8) | ((uint32_t)blk[QH + 2] << 16) |
                 ((uint32_t)blk[QH + 3] << 24);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = j + k;
            const int byte = blk[QS + (e & 15)];
            const int q = (e < 16 ? (byte & 15) : (byte >> 4)) | (int)(((qh >> e) & 1u) << 4);
            if constexpr (F == F_Q5_0)
                v[k] = d * (float)(q - 16);
            else
                v[k] = d * (float)q + rd_f16(blk + 2);
        }
    } else if constexpr (F == F_Q2_K) {
        const uint8_t *blk = row + (i0 >> 8) * kQ2KBytes;
        const float d = rd_f16(blk + 80), dmin = rd_f16(blk + 82);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = (int)(i0 & 255) + k, h = i >> 7, s = (i & 127) >> 5, l = i & 31;
            const int q = (blk[16 + 32 * h + l] >> (2 * s)) & 3;
            const int sm = blk[i >> 4];
            v[k] = d * (float)((sm & 15) * q) - dmin * (float)(sm >> 4);
        }
    } else if constexpr (F == F_Q4_K) {
        const uint8_t *blk = row + (i0 >> 8) * kQ4KBytes;
        const float d = rd_f16(blk), dmin = rd_f16(blk + 2);
        const int i = (int)(i0 & 255), s = i >> 5;                 // the four values share sub-block s
        const uint8_t *b = blk + 4;
        int sc, m;
        if (s < 4) {
            sc = b[s] & 63;
            m = b[s + 4] & 63;
        } else {
            sc = (b[s + 4] & 15) | ((b[s - 4] >> 6) << 4);
            m = (b[s + 4] >> 4) | ((b[s] >> 6) << 4);
        }
        const int jc = i >> 6, hi = (i >> 5) & 1, l = i & 31;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int byte = blk[16 + 32 * jc + l + k];
            const int q = hi ? (byte >> 4) : (byte & 15);
            v[k] = d * (float)(sc * q) - dmin * (float)m;
        }
    } else {
        const uint8_t *blk = row + (i0 >> 8) * kQ6KBytes;
        const float d = rd_f16(blk + 208);
        const int i = (int)(i0 & 255), h = i >> 7, kk = (i & 127) >> 5, l = i & 31;
        const int sc = (int8_t)blk[192 + (i >> 4)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int lb = blk[64 * h + l + k + 32 * (kk & 1)];
            const int lo = (kk < 2) ? (lb & 15) : (lb >> 4);
            const int q = lo | (((blk[128 + 32 * h + l + k] >> (2 * kk)) & 3) << 4);
            v[k] = d * (float)(sc * (q - 32));
        }
    }
}

// Thread g of the launch writes values 4(g % (K/4)) .. +3 of output row
// g / (K/4).  An id outside [0, N) gives a row of quiet NaNs.
template <int F>
__global__ __launch_bounds__(256) void k_get_rows(const uint8_t *__restrict__ w, const int32_t *__restrict__ ids,
                                                  float4 *__restrict__ out, int64_t total, int64_t k4, int64_t N,
                                                  int64_t row_bytes) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= total) return;
    const int64_t t = g / k4, i0 = 4 * (g - t * k4);
    const int64_t id = ids[t];
    float v[4];
    if (id < 0 || id >= N) {
        const float nan = __builtin_bit_cast(float, 0x7fc00000u);
        v[0] = v[1] = v[2] = v[3] = nan;
    } else {
        decode4<F>(w + id * row_bytes, i0, v);
    }
    out[g] = make_float4(v[0], v[1], v[2], v[3]);
}

template <int F>
static hipError_t launch_rows(const void *w, const int32_t *ids, float *out, int64_t n, int64_t N, int64_t K,
                              int64_t row_bytes, hipStream_t st) {
    int64_t k4 = K / 4, total = n * k4;
    const int64_t grid = (total + 255) / 256;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    float4 *op = reinterpret_cast<float4 *>(out);
    void *args[] = {(void *)&wp, (void *)&ids, (void *)&op, (void *)&total, (void *)&k4, (void *)&N,
                    (void *)&row_bytes};
    return hipLaunchKernel((const void *)k_get_rows<F>, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_get_rows(int fmt, const void *w, const int32_t *ids, float *out, int64_t n, int64_t N, int64_t K,
                           int64_t row_bytes, hipStream_t st) {
    switch (fmt) {
        case F_Q4_0: return launch_rows<F_Q4_0>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q8_0: return launch_rows<F_Q8_0>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q2_K: return launch_rows<F_Q2_K>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q4_K: return launch_rows<F_Q4_K>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q6_K: return launch_rows<F_Q6_K>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q4_1: return launch_rows<F_Q4_1>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q5_0: return launch_rows<F_Q5_0>(w, ids, out, n, N, K, row_bytes, st);
        case F_Q5_1: return launch_rows<F_Q5_1>(w, ids, out, n, N, K, row_bytes, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qmm
