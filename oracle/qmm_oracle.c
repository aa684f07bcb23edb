/*
 * qmm oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar C implementation of the block-quantized weight x
 * Q8_0 / Q8_K activation product.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no source,
 * header, table or helper with the HIP library; the two meet only at the
 * byte layouts the pages define.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (SSE arithmetic, so every
 * float operation below is one correctly rounded IEEE binary32 operation).
 *
 * Sources (page titles; each function names the part it follows):
 *   [minfer]  "10 . CPU matmul: quantized weights x Q8_0 activations"
 *   [ggml]    "ggml Q4_0 vec_dot Walkthrough"
 *   [krafla]  "Architecture" (krafla)
 *   [kvad]    "kvad -- the same ideas, at scale"
 *
 * Readings taken where the pages are silent, garbled or disagree are listed
 * in the repository design notes; the ones that shape arithmetic here are
 * repeated at the function that applies them.
 *
 * Parity status: every exported function is pinned by a CPU test (values the
 * pages print, closed forms, invariants, a library routine or brute force).
 * The Q2_K, Q4_K, Q6_K, Q4_1, Q5_0 and Q5_1 weight quantizers follow rules of
 * our own (the pages give their formats, not a quantizer); each rule as
 * stated at its function is pinned by hand-computed blocks (every
 * intermediate worked out by hand, ties, clamp edges, f16-rounded scales)
 * that altered copies of these functions fail.  "Parity unpinned" remains
 * only where the pages give no bits at all: the packing of Q4_K's eight
 * 6-bit scales and mins into 12 bytes, the whole Q6_K block layout, and the
 * Q4_1 / Q5_0 / Q5_1 field and bit order (the pages give the block sizes,
 * Q4_K's field order and its two-term dot, and the d*q + m form; the reading
 * is GGUF's layout, pinned only by round trips and by brute force against
 * the decoded values, which checks the dot, not the layout).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32       /* values per Q4_0 / Q8_0 block                  */
#define QKK 256     /* values per Q2_K / Q8_K super-block            */
#define Q4_0_BYTES 18
#define Q8_0_BYTES 34
#define Q2_K_BYTES 84
#define Q8_K_BYTES 292
#define Q4_1_BYTES 20
#define Q5_0_BYTES 22
#define Q5_1_BYTES 24
#define Q4_K_BYTES 144
#define Q6_K_BYTES 210

/* ------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32                                          */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16 -> binary32, exact for every finite half, inf and NaN. */
float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    if (e == 0) {
        /* zero or subnormal: m * 2^-24, exact in binary32 */
        float v = (float)m * 0x1p-24f;
        return sign ? -v : v;
    }
    if (e == 31) return bits_f32(sign | 0x7f800000u | (m << 13));
    return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

/* binary32 -> binary16, round to nearest, ties to even, with subnormals.
 * The scales are stored as f16 of an f32 value ([minfer] quantize_avx2:
 * "f16(d)"); IEEE's default rounding is the reading. Values at or above
 * 65520 in magnitude become infinity (outside the contract of the method). */
uint16_t orc_f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    x &= 0x7fffffffu;
    if (x >= 0x7f800000u) return sign | (x > 0x7f800000u ? 0x7e00u : 0x7c00u);
    if (x >= 0x477ff000u) return sign | 0x7c00u;          /* >= 65520 */
    if (x < 0x33000000u) return sign;                      /* < 2^-25  */
    uint32_t e = x >> 23;
    uint32_t mant = (x & 0x7fffffu) | 0x800000u;
    uint32_t r, rem, half;
    if (e >= 113u) {                                       /* normal half */
        r = ((e - 112u) << 10) | ((mant >> 13) & 0x3ffu);
        rem = mant & 0x1fffu;
        half = 0x1000u;
    } else {                                               /* subnormal half */
        uint32_t sh = 126u - e;                            /* 14 .. 24 */
        r = mant >> sh;
        rem = mant & ((1u << sh) - 1u);
        half = 1u << (sh - 1u);
    }
    if (rem > half || (rem == half && (r & 1u))) r += 1u;  /* may carry into exponent */
    return sign | (uint16_t)r;
}

static float rd_f16(const uint8_t *p) { return orc_f16_to_f32((uint16_t)(p[0] | (p[1] << 8))); }
static void wr_f16(uint8_t *p, float v) { uint16_t h = orc_f32_to_f16(v); p[0] = (uint8_t)h; p[1] = (uint8_t)(h >> 8); }
static float rd_f32(const uint8_t *p) { float v; memcpy(&v, p, 4); return v; }

/* Round to nearest integer, ties to even, computed without relying on the
 * floating-point environment: for |v| < 2^23 the value floor(v) is exact and
 * v - floor(v) is exact, so the comparison with 0.5 is exact. */
static float rne(float v) {
    if (!(fabsf(v) < 8388608.0f)) return v;               /* already integral */
    float fl = floorf(v);
    float frac = v - fl;
    if (frac > 0.5f) return fl + 1.0f;
    if (frac < 0.5f) return fl;
    return (fmodf(fl, 2.0f) == 0.0f) ? fl : fl + 1.0f;     /* tie: to even */
}

/* ------------------------------------------------------------------ */
/* Activation quantizers                                               */
/* ------------------------------------------------------------------ */

/* Q8_0, per 32 values ([minfer] "The activation quantizers", the
 * quantize_avx2 listing; [ggml] section 1.1; [krafla] "Numerics": the rule
 * is written as exact float32 operations):
 *   amax = max |x_j|;  d = amax / 127 (f32), stored as f16;
 *   id = amax != 0 ? 127 / amax : 0;   q_j = round-to-nearest-even(x_j * id).
 * Block: f16 d (little-endian) at byte 0, int8 q[32] at bytes 2..33.
 * Reading: the inverse scale is 127/amax (the only form printed as code);
 * ties go to even (_MM_ROUND_NEAREST); no clamp (|q| <= 127 always holds). */
void orc_quantize_q8_0(const float *x, uint8_t *out, int64_t M, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + m * K + b * QK;
            uint8_t *ob = out + (m * nb + b) * Q8_0_BYTES;
            float amax = 0.0f;
            for (int j = 0; j < QK; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
            wr_f16(ob, d);
            for (int j = 0; j < QK; ++j) {
                float v = xb[j] * id;
                ob[2 + j] = (uint8_t)(int8_t)(int)rne(v);
            }
        }
    }
}

/* Q8_K, per 256 values ([minfer] quantize_row_q8_k_buf_neon listing and the
 * three details after it): amax; d = amax / 127; q_i = saturate[-128,127]
 * (round(x_i * id)); bsums[g] = sum of the 16 saturated codes of group g.
 * Reading: d is stored as f32 (the ggml-style "f32 d" struct the same page
 * mentions), layout d @0, int8 q[256] @4, int16 bsums[16] @260 = 292 bytes. */
void orc_quantize_q8_k(const float *x, uint8_t *out, int64_t M, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t s = 0; s < ns; ++s) {
            const float *xb = x + m * K + s * QKK;
            uint8_t *ob = out + (m * ns + s) * Q8_K_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < QKK; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
            memcpy(ob, &d, 4);
            int8_t q[QKK];
            for (int i = 0; i < QKK; ++i) {
                float r = rne(xb[i] * id);
                if (r > 127.0f) r = 127.0f;
                if (r < -128.0f) r = -128.0f;
                q[i] = (int8_t)(int)r;
                ob[4 + i] = (uint8_t)q[i];
            }
            for (int g = 0; g < 16; ++g) {
                int sum = 0;
                for (int i = 0; i < 16; ++i) sum += q[16 * g + i];
                int16_t s16 = (int16_t)sum;
                memcpy(ob + 260 + 2 * g, &s16, 2);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Weight quantizers (test-data generation)                            */
/* ------------------------------------------------------------------ */

/* Q4_0, per 32 weights ([ggml] section 1.1, quantize_row_q4_0_ref prose;
 * [kvad] "The scale that wasted a code"): take the value of largest
 * magnitude with its sign (first index on ties), d = max / -8, so that value
 * lands on code 0; code_j = clamp(round(x_j / d) + 8, 0, 15); f16 d stored.
 * Packing ([ggml] section 2 probe, [minfer] scalar kernel): byte j of qs
 * holds element j in its low nibble and element j+16 in its high nibble.
 * Readings: the division uses the f32 d; round is to nearest, ties to even;
 * an all-zero block gets d = 0 and every code 8. */
void orc_quantize_q4_0_w(const float *w, uint8_t *out, int64_t N, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = w + n * K + b * QK;
            uint8_t *ob = out + (n * nb + b) * Q4_0_BYTES;
            float amax = 0.0f, mx = 0.0f;
            for (int j = 0; j < QK; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax) { amax = a; mx = xb[j]; }
            }
            float d = (amax != 0.0f) ? mx / -8.0f : 0.0f;   /* +0 for a zero block */
            wr_f16(ob, d);
            int code[QK];
            for (int j = 0; j < QK; ++j) {
                int c = 8;
                if (d != 0.0f) c = (int)rne(xb[j] / d) + 8;
                if (c < 0) c = 0;
                if (c > 15) c = 15;
                code[j] = c;
            }
            for (int j = 0; j < 16; ++j) ob[2 + j] = (uint8_t)(code[j] | (code[j + 16] << 4));
        }
    }
}

/* Q2_K, per 256 weights in 16 groups of 16 (format: [ggml] section 1.2:
 * scales[16] (low nibble sc, high nibble m), qs[64], f16 d, f16 dmin; a
 * weight decodes as d*sc*q - dmin*m).  The pages give no quantizer; this is
 * the simplest rule that fills the format:
 *   per group: lo = min(0, min x), hi = max x, s = (hi - lo) / 3, mn = -lo;
 *   d = max_g s / 15, dmin = max_g mn / 15 (stored f16);
 *   sc = clamp(round(s / f16(d)), 0, 15), m = clamp(round(mn / f16(dmin)), 0, 15);
 *   q = clamp(round((x + f16(dmin) * m) / (f16(d) * sc)), 0, 3), 0 if the divisor is 0.
 * Bit order of qs (not on the pages; the reading shared by both sides):
 * byte 32h + l holds, at bit shift 2s, the code of weight 128h + 32s + l. */
void orc_quantize_q2_k_w(const float *w, uint8_t *out, int64_t N, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < ns; ++sb) {
            const float *xb = w + n * K + sb * QKK;
            uint8_t *ob = out + (n * ns + sb) * Q2_K_BYTES;
            float s[16], mn[16];
            float smax = 0.0f, mnmax = 0.0f;
            for (int g = 0; g < 16; ++g) {
                float lo = 0.0f, hi = xb[16 * g];
                for (int i = 0; i < 16; ++i) {
                    float v = xb[16 * g + i];
                    if (v < lo) lo = v;
                    if (v > hi) hi = v;
                }
                s[g] = (hi - lo) / 3.0f;
                mn[g] = -lo;
                if (s[g] > smax) smax = s[g];
                if (mn[g] > mnmax) mnmax = mn[g];
            }
            float d = smax / 15.0f, dmin = mnmax / 15.0f;
            wr_f16(ob + 80, d);
            wr_f16(ob + 82, dmin);
            float dh = rd_f16(ob + 80), dminh = rd_f16(ob + 82);
            int sc[16], mm[16];
            for (int g = 0; g < 16; ++g) {
                int a = 0, c = 0;
                if (dh != 0.0f) a = (int)rne(s[g] / dh);
                if (dminh != 0.0f) c = (int)rne(mn[g] / dminh);
                sc[g] = a < 0 ? 0 : (a > 15 ? 15 : a);
                mm[g] = c < 0 ? 0 : (c > 15 ? 15 : c);
                ob[g] = (uint8_t)(sc[g] | (mm[g] << 4));
            }
            uint8_t q[QKK];
            for (int i = 0; i < QKK; ++i) {
                int g = i / 16;
                float off = dminh * (float)mm[g];
                float div = dh * (float)sc[g];
                int c = 0;
                if (div != 0.0f) c = (int)rne((xb[i] + off) / div);
                q[i] = (uint8_t)(c < 0 ? 0 : (c > 3 ? 3 : c));
            }
            memset(ob + 16, 0, 64);
            for (int i = 0; i < QKK; ++i) {
                int h = i / 128, sft = (i % 128) / 32, l = i % 32;
                ob[16 + 32 * h + l] |= (uint8_t)(q[i] << (2 * sft));
            }
        }
    }
}

/* The 32-value formats with an offset or a fifth bit ([ggml] section 1.1:
 * the _1 formats add a per-block offset, value = d * q + m; [minfer]: Q5_0 and
 * Q5_1 add a high-bit plane, 22- and 24-byte blocks).  Field order and bit
 * order are not on the pages; the reading is GGUF's:
 *   Q4_1 (20 B): f16 d @0, f16 m @2, qs[16] @4            value = d * q + m,        q in [0, 15]
 *   Q5_0 (22 B): f16 d @0, qh[4] @2, qs[16] @6            value = d * (q - 16),     q in [0, 31]
 *   Q5_1 (24 B): f16 d @0, f16 m @2, qh[4] @4, qs[16] @8  value = d * q + m,        q in [0, 31]
 * qs byte j holds value j's low four bits (low nibble) and value j+16's (high
 * nibble), as in Q4_0; bit j of the little-endian 32-bit qh is value j's
 * fifth bit. */
static int q41_code(const uint8_t *blk, int j) {
    uint8_t b = blk[4 + (j & 15)];
    return j < 16 ? (b & 15) : (b >> 4);
}
static int q5_code(const uint8_t *qh4, const uint8_t *qs, int j) {
    uint32_t qh = (uint32_t)qh4[0] | ((uint32_t)qh4[1] << 8) | ((uint32_t)qh4[2] << 16) | ((uint32_t)qh4[3] << 24);
    uint8_t b = qs[j & 15];
    int lo = j < 16 ? (b & 15) : (b >> 4);
    return lo | (int)(((qh >> j) & 1u) << 4);
}

/* Value j of a block of format fmt (4 = Q4_1, 5 = Q5_0, 6 = Q5_1), exact in double. */
static double val32(int fmt, const uint8_t *blk, int j) {
    double d = rd_f16(blk);
    if (fmt == 5) return d * (double)(q5_code(blk + 2, blk + 6, j) - 16);
    double m = rd_f16(blk + 2);
    if (fmt == 4) return d * (double)q41_code(blk, j) + m;
    return d * (double)q5_code(blk + 4, blk + 8, j) + m;
}

/* Weight quantizers for the three (test data; the pages give no rule):
 *   Q4_1 / Q5_1: lo = min x, hi = max x over the block (a zero of either sign
 *     taken as +0); d = (hi - lo) / L
 *     (L = 15 or 31), m = lo (both stored f16); q = clamp(round((x - m) / d),
 *     0, L) with the stored d and m, 0 if d is 0.
 *   Q5_0: Q4_0's rule with 32 levels: the value of largest magnitude (first
 *     on ties) lands on code 0, d = max / -16; q = clamp(round(x / d) + 16, 0,
 *     31), 16 if d is 0. */
static void quant_block32(int fmt, const float *xb, uint8_t *ob) {
    int code[QK];
    if (fmt == 5) {
        float amax = 0.0f, mx = 0.0f;
        for (int j = 0; j < QK; ++j) {
            float a = fabsf(xb[j]);
            if (a > amax) { amax = a; mx = xb[j]; }
        }
        float d = (amax != 0.0f) ? mx / -16.0f : 0.0f;
        wr_f16(ob, d);
        for (int j = 0; j < QK; ++j) {
            int c = 16;
            if (d != 0.0f) c = (int)rne(xb[j] / d) + 16;
            code[j] = c < 0 ? 0 : (c > 31 ? 31 : c);
        }
    } else {
        int L = (fmt == 4) ? 15 : 31;
        float lo = xb[0], hi = xb[0];
        for (int j = 1; j < QK; ++j) {
            if (xb[j] < lo) lo = xb[j];
            if (xb[j] > hi) hi = xb[j];
        }
        lo += 0.0f;                      /* a zero of either sign counts as +0 */
        hi += 0.0f;
        wr_f16(ob, (hi - lo) / (float)L);
        wr_f16(ob + 2, lo);
        float dh = rd_f16(ob), mh = rd_f16(ob + 2);
        for (int j = 0; j < QK; ++j) {
            int c = 0;
            if (dh != 0.0f) c = (int)rne((xb[j] - mh) / dh);
            code[j] = c < 0 ? 0 : (c > L ? L : c);
        }
    }
    uint8_t *qs = ob + (fmt == 4 ? 4 : (fmt == 5 ? 6 : 8));
    for (int j = 0; j < 16; ++j) qs[j] = (uint8_t)((code[j] & 15) | ((code[j + 16] & 15) << 4));
    if (fmt != 4) {
        uint32_t qh = 0;
        for (int j = 0; j < QK; ++j) qh |= (uint32_t)((code[j] >> 4) & 1) << j;
        uint8_t *q4 = ob + (fmt == 5 ? 2 : 4);
        for (int k = 0; k < 4; ++k) q4[k] = (uint8_t)(qh >> (8 * k));
    }
}

static int bytes32(int fmt) { return fmt == 4 ? Q4_1_BYTES : (fmt == 5 ? Q5_0_BYTES : Q5_1_BYTES); }

static void quantize32_w(int fmt, const float *w, uint8_t *out, int64_t N, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) quant_block32(fmt, w + n * K + b * QK, out + (n * nb + b) * bytes32(fmt));
}
void orc_quantize_q4_1_w(const float *w, uint8_t *out, int64_t N, int64_t K) { quantize32_w(4, w, out, N, K); }
void orc_quantize_q5_0_w(const float *w, uint8_t *out, int64_t N, int64_t K) { quantize32_w(5, w, out, N, K); }
void orc_quantize_q5_1_w(const float *w, uint8_t *out, int64_t N, int64_t K) { quantize32_w(6, w, out, N, K); }

static void dequantize32(int fmt, const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            for (int j = 0; j < QK; ++j)
                out[r * K + b * QK + j] = val32(fmt, blk + (r * nb + b) * bytes32(fmt), j);
}
void orc_dequantize_q4_1(const uint8_t *b, double *o, int64_t rows, int64_t K) { dequantize32(4, b, o, rows, K); }
void orc_dequantize_q5_0(const uint8_t *b, double *o, int64_t rows, int64_t K) { dequantize32(5, b, o, rows, K); }
void orc_dequantize_q5_1(const uint8_t *b, double *o, int64_t rows, int64_t K) { dequantize32(6, b, o, rows, K); }

/* Q4_K layout ([minfer] block.rs sizes: 144 bytes; the K-quant dot kernel
 * walked in "The payoff": f16 d @0, f16 dmin @2, 12 bytes of scales @4, 128
 * bytes of nibbles @16; 32-byte chunk j holds values 64j + l in its low
 * nibbles and 64j + 32 + l in its high nibbles, l < 32; sub-block s of 32
 * values uses scales[s] and mins[s]).  The packing of the eight 6-bit scales
 * and eight 6-bit mins into the 12 bytes is not on the pages; the reading is
 * GGUF's: for s < 4, scale = b[s] & 63 and min = b[s+4] & 63; for s >= 4,
 * scale = (b[s+4] & 15) | (b[s-4] >> 6) << 4 and min = (b[s+4] >> 4) |
 * (b[s] >> 6) << 4. */
static void q4k_scale_min(const uint8_t *b, int s, int *sc, int *m) {
    if (s < 4) {
        *sc = b[s] & 63;
        *m = b[s + 4] & 63;
    } else {
        *sc = (b[s + 4] & 15) | ((b[s - 4] >> 6) << 4);
        *m = (b[s + 4] >> 4) | ((b[s] >> 6) << 4);
    }
}

static void q4k_pack_scale_min(uint8_t *b, const int *sc, const int *m) {
    for (int s = 0; s < 4; ++s) {
        b[s] = (uint8_t)((sc[s] & 63) | ((sc[s + 4] >> 4) << 6));
        b[s + 4] = (uint8_t)((m[s] & 63) | ((m[s + 4] >> 4) << 6));
        b[s + 8] = (uint8_t)((sc[s + 4] & 15) | ((m[s + 4] & 15) << 4));
    }
}

/* The 4-bit code of value i of a Q4_K block (the chunk order above). */
static int q4k_code(const uint8_t *blk, int i) {
    int j = i / 64, hi = (i % 64) / 32, l = i % 32;
    uint8_t byte = blk[16 + 32 * j + l];
    return hi ? byte >> 4 : byte & 15;
}

/* Q4_K weights, per 256 in 8 sub-blocks of 32 (format above; a weight
 * decodes as d * sc_s * q - dmin * m_s, [minfer] "The payoff": value =
 * q * d_s - min_s).  The pages give no quantizer; the rule here, like Q2_K's:
 *   per sub-block: lo = min(0, min x), hi = max x, s = (hi - lo) / 15, mn = -lo;
 *   d = max s / 63, dmin = max mn / 63 (stored f16);
 *   sc = clamp(round(s / f16(d)), 0, 63), m = clamp(round(mn / f16(dmin)), 0, 63);
 *   q = clamp(round((x + f16(dmin) * m) / (f16(d) * sc)), 0, 15), 0 if the divisor is 0. */
void orc_quantize_q4_k_w(const float *w, uint8_t *out, int64_t N, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < ns; ++sb) {
            const float *xb = w + n * K + sb * QKK;
            uint8_t *ob = out + (n * ns + sb) * Q4_K_BYTES;
            float sv[8], mn[8], smax = 0.0f, mnmax = 0.0f;
            for (int t = 0; t < 8; ++t) {
                float lo = 0.0f, hi = xb[32 * t];
                for (int i = 0; i < 32; ++i) {
                    float v = xb[32 * t + i];
                    if (v < lo) lo = v;
                    if (v > hi) hi = v;
                }
                sv[t] = (hi - lo) / 15.0f;
                mn[t] = -lo;
                if (sv[t] > smax) smax = sv[t];
                if (mn[t] > mnmax) mnmax = mn[t];
            }
            wr_f16(ob, smax / 63.0f);
            wr_f16(ob + 2, mnmax / 63.0f);
            float dh = rd_f16(ob), dminh = rd_f16(ob + 2);
            int sc[8], mm[8];
            for (int t = 0; t < 8; ++t) {
                int a = 0, c = 0;
                if (dh != 0.0f) a = (int)rne(sv[t] / dh);
                if (dminh != 0.0f) c = (int)rne(mn[t] / dminh);
                sc[t] = a < 0 ? 0 : (a > 63 ? 63 : a);
                mm[t] = c < 0 ? 0 : (c > 63 ? 63 : c);
            }
            q4k_pack_scale_min(ob + 4, sc, mm);
            memset(ob + 16, 0, 128);
            for (int i = 0; i < QKK; ++i) {
                int t = i / 32;
                float off = dminh * (float)mm[t];
                float div = dh * (float)sc[t];
                int c = 0;
                if (div != 0.0f) c = (int)rne((xb[i] + off) / div);
                c = c < 0 ? 0 : (c > 15 ? 15 : c);
                int j = i / 64, hi = (i % 64) / 32, l = i % 32;
                ob[16 + 32 * j + l] |= (uint8_t)(hi ? c << 4 : c);
            }
        }
    }
}

/* Q6_K layout ([minfer] block.rs sizes: 210 bytes; the rest is not on the
 * pages, the reading is GGUF's): low 4 bits ql[128] @0, high 2 bits qh[64]
 * @128, int8 scales[16] @192, f16 d @208.  Value i (h = i / 128, r = i % 128,
 * k = r / 32, l = r % 32): low bits from ql[64h + l + 32 (k & 1)] (low nibble
 * for k < 2, high nibble for k >= 2), high bits (qh[32h + l] >> 2k) & 3;
 * q = low | high << 4 in [0, 63]; group g = i / 16; value = d * sc_g * (q - 32). */
static int q6k_code(const uint8_t *blk, int i) {
    int h = i / 128, r = i % 128, k = r / 32, l = r % 32;
    uint8_t lb = blk[64 * h + l + 32 * (k & 1)];
    int lo = (k < 2) ? (lb & 15) : (lb >> 4);
    int hi = (blk[128 + 32 * h + l] >> (2 * k)) & 3;
    return lo | (hi << 4);
}

/* Q6_K weights, per 256 in 16 groups of 16.  The pages give no quantizer; the
 * rule here follows Q4_0's signed maximum (kvad "The scale that wasted a
 * code"): per group the value of largest magnitude mx (first on ties) lands
 * on code 0, s = mx / -32; d = max |s| / 127 (stored f16); sc = clamp(round(
 * s / f16(d)), -128, 127); q = clamp(round(x / (f16(d) * sc)) + 32, 0, 63),
 * 32 if the divisor is 0. */
void orc_quantize_q6_k_w(const float *w, uint8_t *out, int64_t N, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < ns; ++sb) {
            const float *xb = w + n * K + sb * QKK;
            uint8_t *ob = out + (n * ns + sb) * Q6_K_BYTES;
            float sv[16], smax = 0.0f;
            for (int g = 0; g < 16; ++g) {
                float amax = 0.0f, mx = 0.0f;
                for (int i = 0; i < 16; ++i) {
                    float a = fabsf(xb[16 * g + i]);
                    if (a > amax) { amax = a; mx = xb[16 * g + i]; }
                }
                sv[g] = mx / -32.0f;
                if (fabsf(sv[g]) > smax) smax = fabsf(sv[g]);
            }
            wr_f16(ob + 208, smax / 127.0f);
            float dh = rd_f16(ob + 208);
            int sc[16];
            for (int g = 0; g < 16; ++g) {
                int a = 0;
                if (dh != 0.0f) a = (int)rne(sv[g] / dh);
                sc[g] = a < -128 ? -128 : (a > 127 ? 127 : a);
                ob[192 + g] = (uint8_t)(int8_t)sc[g];
            }
            memset(ob, 0, 192);
            for (int i = 0; i < QKK; ++i) {
                float div = dh * (float)sc[i / 16];
                int c = 32;
                if (div != 0.0f) c = (int)rne(xb[i] / div) + 32;
                c = c < 0 ? 0 : (c > 63 ? 63 : c);
                int h = i / 128, r = i % 128, k = r / 32, l = r % 32;
                ob[64 * h + l + 32 * (k & 1)] |= (uint8_t)((k < 2) ? (c & 15) : ((c & 15) << 4));
                ob[128 + 32 * h + l] |= (uint8_t)((c >> 4) << (2 * k));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Decoders (each value exact in double)                               */
/* ------------------------------------------------------------------ */

/* Q8_0 value = d * q ([ggml] section 1.1). */
void orc_dequantize_q8_0(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *p = blk + (r * nb + b) * Q8_0_BYTES;
            double d = rd_f16(p);
            for (int j = 0; j < QK; ++j) out[r * K + b * QK + j] = d * (double)(int8_t)p[2 + j];
        }
}

/* Q4_0 value = d * (nibble - 8); low nibble of byte j is element j, high
 * nibble is element j+16 ([minfer] scalar kernel and its worked byte 0x21;
 * [ggml] section 2). */
void orc_dequantize_q4_0(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *p = blk + (r * nb + b) * Q4_0_BYTES;
            double d = rd_f16(p);
            for (int j = 0; j < 16; ++j) {
                out[r * K + b * QK + j] = d * (double)((p[2 + j] & 0x0f) - 8);
                out[r * K + b * QK + j + 16] = d * (double)((p[2 + j] >> 4) - 8);
            }
        }
}

/* Q2_K value = d * sc_g * q - dmin * m_g, g = i / 16 ([ggml] section 1.2). */
void orc_dequantize_q2_k(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t sb = 0; sb < ns; ++sb) {
            const uint8_t *p = blk + (r * ns + sb) * Q2_K_BYTES;
            double d = rd_f16(p + 80), dmin = rd_f16(p + 82);
            for (int i = 0; i < QKK; ++i) {
                int g = i / 16, h = i / 128, sft = (i % 128) / 32, l = i % 32;
                int q = (p[16 + 32 * h + l] >> (2 * sft)) & 3;
                int sc = p[g] & 0x0f, m = p[g] >> 4;
                out[r * K + sb * QKK + i] = d * sc * q - dmin * m;
            }
        }
}

/* Q4_K value = d * sc_s * q - dmin * m_s, s = i / 32 (layout above). */
void orc_dequantize_q4_k(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t sb = 0; sb < ns; ++sb) {
            const uint8_t *p = blk + (r * ns + sb) * Q4_K_BYTES;
            double d = rd_f16(p), dmin = rd_f16(p + 2);
            for (int i = 0; i < QKK; ++i) {
                int sc, m;
                q4k_scale_min(p + 4, i / 32, &sc, &m);
                out[r * K + sb * QKK + i] = d * sc * q4k_code(p, i) - dmin * m;
            }
        }
}

/* Q6_K value = d * sc_g * (q - 32), g = i / 16 (layout above), formed as the
 * binary16 scale times the integer sc_g * (q - 32) (reading: the pages' row
 * getter decodes every format as "scale x integer"; with a negative sc_g this
 * fixes the sign of a decoded zero to that of d). */
void orc_dequantize_q6_k(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t sb = 0; sb < ns; ++sb) {
            const uint8_t *p = blk + (r * ns + sb) * Q6_K_BYTES;
            double d = rd_f16(p + 208);
            for (int i = 0; i < QKK; ++i)
                out[r * K + sb * QKK + i] = d * (double)((int8_t)p[192 + i / 16] * (q6k_code(p, i) - 32));
        }
}

/* Q8_K value = d * q with f32 d. */
void orc_dequantize_q8_k(const uint8_t *blk, double *out, int64_t rows, int64_t K) {
    int64_t ns = K / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t sb = 0; sb < ns; ++sb) {
            const uint8_t *p = blk + (r * ns + sb) * Q8_K_BYTES;
            double d = rd_f32(p);
            for (int i = 0; i < QKK; ++i) out[r * K + sb * QKK + i] = d * (double)(int8_t)p[4 + i];
        }
}

/* ------------------------------------------------------------------ */
/* Block dot products                                                  */
/* ------------------------------------------------------------------ */

/* One output of a row against one activation row, as the pages define it
 * ([ggml] section 2, right-hand listing; [minfer] scalar kernel; [krafla]
 * "Data flow": the int32 block sum is scaled by d_w * d_x):
 *   y = sum_b d_w[b] * d_x[b] * I_b,   I_b = sum_j w_j * q_j  (exact int32).
 * Terms are formed and summed in double (each term is exact in double);
 * `mag` receives sum_b |d_w d_x| sum_j |w_j q_j|, the magnitude the
 * tolerance is relative to ([krafla] "Numerics": agreement within 1e-5 of the
 * dot product's magnitude). */
static void dot_q4_0_q8_0(const uint8_t *w, const uint8_t *x, int64_t nb, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = w + b * Q4_0_BYTES, *xb = x + b * Q8_0_BYTES;
        int32_t isum = 0, iabs = 0;
        for (int j = 0; j < 16; ++j) {
            int v0 = (wb[2 + j] & 0x0f) - 8, v1 = (wb[2 + j] >> 4) - 8;
            int q0 = (int8_t)xb[2 + j], q1 = (int8_t)xb[2 + j + 16];
            isum += v0 * q0 + v1 * q1;
            iabs += abs(v0 * q0) + abs(v1 * q1);
        }
        double sc = (double)rd_f16(wb) * (double)rd_f16(xb);
        s += sc * (double)isum;
        a += fabs(sc) * (double)iabs;
    }
    *y = s;
    if (mag) *mag = a;
}

/* Q8_0 weights: the same with int8 weight codes ([minfer] Q8_0 kernel). */
static void dot_q8_0_q8_0(const uint8_t *w, const uint8_t *x, int64_t nb, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = w + b * Q8_0_BYTES, *xb = x + b * Q8_0_BYTES;
        int32_t isum = 0, iabs = 0;
        for (int j = 0; j < QK; ++j) {
            int p = (int8_t)wb[2 + j] * (int8_t)xb[2 + j];
            isum += p;
            iabs += abs(p);
        }
        double sc = (double)rd_f16(wb) * (double)rd_f16(xb);
        s += sc * (double)isum;
        a += fabs(sc) * (double)iabs;
    }
    *y = s;
    if (mag) *mag = a;
}

/* Q2_K x Q8_K, per super-block: the two-term form of the K-quant dot
 * ([minfer] "The payoff: a K-quant dot kernel, walked": the min term is a sum
 * over activations only, carried by bsums):
 *   V  = sum_g sc_g * sum_{i in g} q_i * x_i,  Mn = sum_g m_g * bsums_g,
 *   t  = d * d8 * V - dmin * d8 * Mn. */
static void dot_q2_k_q8_k(const uint8_t *w, const uint8_t *x, int64_t ns, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t sb = 0; sb < ns; ++sb) {
        const uint8_t *wb = w + sb * Q2_K_BYTES, *xb = x + sb * Q8_K_BYTES;
        double d = rd_f16(wb + 80), dmin = rd_f16(wb + 82), d8 = rd_f32(xb);
        int64_t V = 0, Mn = 0;
        double aa = 0.0;
        for (int g = 0; g < 16; ++g) {
            int sc = wb[g] & 0x0f, m = wb[g] >> 4;
            int32_t gs = 0;
            for (int t = 0; t < 16; ++t) {
                int i = 16 * g + t, h = i / 128, sft = (i % 128) / 32, l = i % 32;
                int q = (wb[16 + 32 * h + l] >> (2 * sft)) & 3;
                int qx = (int8_t)xb[4 + i];
                gs += q * qx;
                aa += (fabs(d * sc * q) + fabs(dmin * m)) * fabs(d8 * qx);
            }
            int16_t bs;
            memcpy(&bs, xb + 260 + 2 * g, 2);
            V += (int64_t)sc * gs;
            Mn += (int64_t)m * bs;
        }
        s += d * d8 * (double)V - dmin * d8 * (double)Mn;
        a += aa;
    }
    *y = s;
    if (mag) *mag = a;
}

/* Q4_K x Q8_K, per super-block, as [minfer] "The payoff: a K-quant dot
 * kernel, walked" writes it: the min term Mn = sum_s m_s * (bsums[2s] +
 * bsums[2s+1]) (a sub-block of 32 is two bsum groups of 16), the value term
 * V = sum_s sc_s * sum_{i in s} q_i * x_i, then
 *   t = d * d8 * V - dmin * d8 * Mn. */
static void dot_q4_k_q8_k(const uint8_t *w, const uint8_t *x, int64_t ns, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t sb = 0; sb < ns; ++sb) {
        const uint8_t *wb = w + sb * Q4_K_BYTES, *xb = x + sb * Q8_K_BYTES;
        double d = rd_f16(wb), dmin = rd_f16(wb + 2), d8 = rd_f32(xb);
        int64_t V = 0, Mn = 0;
        double aa = 0.0;
        for (int t = 0; t < 8; ++t) {
            int sc, m;
            q4k_scale_min(wb + 4, t, &sc, &m);
            int32_t ts = 0;
            for (int u = 0; u < 32; ++u) {
                int i = 32 * t + u, q = q4k_code(wb, i), qx = (int8_t)xb[4 + i];
                ts += q * qx;
                aa += (fabs(d * sc * q) + fabs(dmin * m)) * fabs(d8 * qx);
            }
            int16_t b0, b1;
            memcpy(&b0, xb + 260 + 2 * (2 * t), 2);
            memcpy(&b1, xb + 260 + 2 * (2 * t + 1), 2);
            V += (int64_t)sc * ts;
            Mn += (int64_t)m * (b0 + b1);
        }
        s += d * d8 * (double)V - dmin * d8 * (double)Mn;
        a += aa;
    }
    *y = s;
    if (mag) *mag = a;
}

/* Q6_K x Q8_K, per super-block: the plain sum of decoded products (the pages
 * give no Q6_K kernel), grouped as the format groups it:
 *   t = d * d8 * sum_g sc_g * sum_{i in g} (q_i - 32) * x_i. */
static void dot_q6_k_q8_k(const uint8_t *w, const uint8_t *x, int64_t ns, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t sb = 0; sb < ns; ++sb) {
        const uint8_t *wb = w + sb * Q6_K_BYTES, *xb = x + sb * Q8_K_BYTES;
        double d = rd_f16(wb + 208), d8 = rd_f32(xb);
        int64_t V = 0;
        double aa = 0.0;
        for (int g = 0; g < 16; ++g) {
            int sc = (int8_t)wb[192 + g];
            int32_t gs = 0;
            for (int u = 0; u < 16; ++u) {
                int i = 16 * g + u, q = q6k_code(wb, i) - 32, qx = (int8_t)xb[4 + i];
                gs += q * qx;
                aa += fabs(d * sc * q) * fabs(d8 * qx);
            }
            V += (int64_t)sc * gs;
        }
        s += d * d8 * (double)V;
        a += aa;
    }
    *y = s;
    if (mag) *mag = a;
}

/* Q4_1 / Q5_0 / Q5_1 weights x Q8_0: the plain sum of decoded products per
 * block, grouped as the format is (scale x integer sum, plus the offset times
 * the activation's code sum for the _1 formats):
 *   t_b = d_w d_x sum_j q'_j x_j + m d_x sum_j x_j,   q' = q (Q5_0: q - 16). */
static void dot_32(int fmt, const uint8_t *w, const uint8_t *x, int64_t nb, double *y, double *mag) {
    double s = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = w + b * bytes32(fmt), *xb = x + b * Q8_0_BYTES;
        double dw = rd_f16(wb), dx = rd_f16(xb), m = (fmt == 5) ? 0.0 : rd_f16(wb + 2);
        int32_t isum = 0, xsum = 0;
        double aa = 0.0;
        for (int j = 0; j < QK; ++j) {
            int qx = (int8_t)xb[2 + j];
            int q = (fmt == 4) ? q41_code(wb, j) : q5_code(wb + (fmt == 5 ? 2 : 4), wb + (fmt == 5 ? 6 : 8), j);
            if (fmt == 5) q -= 16;
            isum += q * qx;
            xsum += qx;
            aa += fabs(val32(fmt, wb, j)) * fabs(dx * qx);
        }
        s += dw * dx * (double)isum + m * dx * (double)xsum;
        a += aa;
    }
    *y = s;
    if (mag) *mag = a;
}

enum { ORC_Q4_0 = 0, ORC_Q8_0 = 1, ORC_Q2_K = 2, ORC_Q4_K = 3, ORC_Q6_K = 4, ORC_Q4_1 = 5, ORC_Q5_0 = 6,
       ORC_Q5_1 = 7 };

static void dot_any(int fmt, const uint8_t *w, const uint8_t *x, int64_t K, double *y, double *mag) {
    if (fmt == ORC_Q4_0) dot_q4_0_q8_0(w, x, K / QK, y, mag);
    else if (fmt == ORC_Q8_0) dot_q8_0_q8_0(w, x, K / QK, y, mag);
    else if (fmt == ORC_Q2_K) dot_q2_k_q8_k(w, x, K / QKK, y, mag);
    else if (fmt == ORC_Q4_K) dot_q4_k_q8_k(w, x, K / QKK, y, mag);
    else if (fmt == ORC_Q6_K) dot_q6_k_q8_k(w, x, K / QKK, y, mag);
    else dot_32(fmt - 1, w, x, K / QK, y, mag);     /* 5, 6, 7 -> the local ids 4, 5, 6 */
}

static int64_t w_row_bytes(int fmt, int64_t K) {
    if (fmt == ORC_Q4_0) return K / QK * Q4_0_BYTES;
    if (fmt == ORC_Q8_0) return K / QK * Q8_0_BYTES;
    if (fmt == ORC_Q2_K) return K / QKK * Q2_K_BYTES;
    if (fmt == ORC_Q4_K) return K / QKK * Q4_K_BYTES;
    if (fmt == ORC_Q6_K) return K / QKK * Q6_K_BYTES;
    return K / QK * bytes32(fmt - 1);
}
static int64_t x_row_bytes(int fmt, int64_t K) {
    if (fmt == ORC_Q2_K || fmt == ORC_Q4_K || fmt == ORC_Q6_K) return K / QKK * Q8_K_BYTES;
    return K / QK * Q8_0_BYTES;
}

/* ------------------------------------------------------------------ */
/* Matrix products                                                     */
/* ------------------------------------------------------------------ */

/* out[t][o] = dot(w row o, x row t): token-major output [M][N], each element
 * written once ([minfer] mm_rows listing and "Pitfalls": the output is
 * [nt][od]).  Work is split by output rows across threads; each element is
 * computed by one thread in one fixed order, so the result does not depend
 * on the thread count ([minfer] "Read the loop order carefully"). */
typedef struct {
    int fmt; const uint8_t *w, *x; float *y; double *y64, *mag;
    int64_t M, N, K, n0, n1;
} orc_job;

static void *orc_rows(void *arg) {
    orc_job *j = (orc_job *)arg;
    int64_t wr = w_row_bytes(j->fmt, j->K), xr = x_row_bytes(j->fmt, j->K);
    for (int64_t o = j->n0; o < j->n1; ++o)
        for (int64_t t = 0; t < j->M; ++t) {
            double v, a;
            dot_any(j->fmt, j->w + o * wr, j->x + t * xr, j->K, &v, &a);
            if (j->y) j->y[t * j->N + o] = (float)v;
            if (j->y64) j->y64[t * j->N + o] = v;
            if (j->mag) j->mag[t * j->N + o] = a;
        }
    return NULL;
}

/* fmt: 0 = Q4_0 weights x Q8_0, 1 = Q8_0 x Q8_0, 2 = Q2_K x Q8_K,
 * 3 = Q4_K x Q8_K, 4 = Q6_K x Q8_K, 5 = Q4_1 x Q8_0, 6 = Q5_0 x Q8_0,
 * 7 = Q5_1 x Q8_0.
 * y (f32), y64 (double) and mag (double) are [M][N]; any may be NULL. */
int orc_matmul(int fmt, const uint8_t *w, const uint8_t *x, float *y, double *y64, double *mag,
               int64_t M, int64_t N, int64_t K, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > N) threads = (int)N;
    orc_job jobs[256];
    pthread_t tid[256];
    for (int i = 0; i < threads; ++i) {
        jobs[i] = (orc_job){fmt, w, x, y, y64, mag, M, N, K, N * i / threads, N * (i + 1) / threads};
    }
    int started = 0;
    for (int i = 1; i < threads; ++i) {
        if (pthread_create(&tid[i], NULL, orc_rows, &jobs[i]) != 0) break;
        started = i;
    }
    orc_rows(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    for (int i = started + 1; i < threads; ++i) orc_rows(&jobs[i]);   /* any thread that failed to start */
    return 0;
}

/* Selected outputs (mi[c], ni[c]) of the same product: for checking a full
 * size GPU result on a sample of its elements. */
int orc_matmul_sampled(int fmt, const uint8_t *w, const uint8_t *x, const int64_t *mi, const int64_t *ni,
                       int64_t count, double *y64, double *mag, int64_t K) {
    int64_t wr = w_row_bytes(fmt, K), xr = x_row_bytes(fmt, K);
    for (int64_t c = 0; c < count; ++c) {
        double v, a;
        dot_any(fmt, w + ni[c] * wr, x + mi[c] * xr, K, &v, &a);
        y64[c] = v;
        if (mag) mag[c] = a;
    }
    return 0;
}

/* Embedding rows ([minfer] "The embedding matmul": for each token id the
 * quantized row of the table is walked block by block and dequantized into
 * the output row; the same row getter serves every backend, so the rows are
 * byte-for-byte identical).  out[t][:] = f32 of the decoded row ids[t] (each
 * value exact in double, rounded once); an id outside [0, N) gives a row of
 * quiet NaNs (reading: the page's code indexes the table directly, an id out
 * of range is outside its contract). */
int orc_get_rows(int fmt, const uint8_t *w, const int32_t *ids, int64_t n, int64_t N, int64_t K, float *out) {
    int64_t rb = w_row_bytes(fmt, K);
    double *row = (double *)malloc(sizeof(double) * (size_t)K);
    if (!row) return -1;
    for (int64_t t = 0; t < n; ++t) {
        int64_t id = ids[t];
        if (id < 0 || id >= N) {
            for (int64_t i = 0; i < K; ++i) out[t * K + i] = bits_f32(0x7fc00000u);
            continue;
        }
        const uint8_t *wr = w + id * rb;
        if (fmt == ORC_Q4_0) orc_dequantize_q4_0(wr, row, 1, K);
        else if (fmt == ORC_Q8_0) orc_dequantize_q8_0(wr, row, 1, K);
        else if (fmt == ORC_Q2_K) orc_dequantize_q2_k(wr, row, 1, K);
        else if (fmt == ORC_Q4_K) orc_dequantize_q4_k(wr, row, 1, K);
        else if (fmt == ORC_Q6_K) orc_dequantize_q6_k(wr, row, 1, K);
        else dequantize32(fmt - 1, wr, row, 1, K);
        for (int64_t i = 0; i < K; ++i) out[t * K + i] = (float)row[i];
    }
    free(row);
    return 0;
}

/* Single block dot, for the pins: returns the exact integer sum of one
 * Q4_0 x Q8_0 (fmt 0) or Q8_0 x Q8_0 (fmt 1) block pair. */
int32_t orc_block_isum(int fmt, const uint8_t *w, const uint8_t *x) {
    int32_t isum = 0;
    for (int j = 0; j < QK; ++j) {
        int wv;
        if (fmt == ORC_Q4_0) wv = (j < 16 ? (w[2 + j] & 0x0f) : (w[2 + j - 16] >> 4)) - 8;
        else wv = (int8_t)w[2 + j];
        isum += wv * (int8_t)x[2 + j];
    }
    return isum;
}

/* Element-wise conversions over arrays (for the exhaustive fp16 pins). */
void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n) {
    for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_f16_to_f32(h[i]);
}
