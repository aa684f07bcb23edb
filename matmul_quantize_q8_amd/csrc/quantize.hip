// Quantizers: f32 rows -> Q8_0 / Q8_K activation blocks, and f32 weight rows
// -> Q4_0 / Q2_K weight blocks.  Each block is independent, so every
// quantizer treats its input as one flat sequence of blocks (row boundaries
// coincide with block boundaries) and maps lanes to blocks.
//
// Bit-exactness: every floating-point step is a single correctly rounded f32
// operation (hipcc's default f32 division is correctly rounded, the library
// is built with -ffp-contract=off so no multiply-add is fused, f32 denormals
// are kept), rounding to integer is v_rndne_f32 (ties to even) and the f16
// store is v_cvt_f16_f32 (nearest even).  Reductions use max/min only, which
// are exact in any order.
#include "qmm_device.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Q8_0 (minfer "The activation quantizers"; ggml section 1.1):
// per 32 values amax, d = amax/127 -> f16, id = amax ? 127/amax : 0,
// q = rne(x * id).  Eight lanes share a block, four values each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q8_0(const float4 *__restrict__ x, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 3;
    const int part = threadIdx.x & 7;
    const bool valid = blk < nblocks;
    float4 v = valid ? x[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    float d;
    const uint32_t packed = q8_0_part(v, d);
    if (valid) store_q8_0_part(out + blk * kQ80Bytes, part, packed, d);
}

// ---------------------------------------------------------------------------
// Q8_K (minfer quantize_row_q8_k_buf): per 256 values amax, f32 d = amax/127,
// q = saturate(rne(x*id)), bsums[g] = sum of the 16 saturated codes of g.
// One wave per block; lane L holds values 4L..4L+3 (group L/4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q8_k(const float4 *__restrict__ x, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;                               // whole wave exits together
    const float4 v = x[blk * 64 + lane];
    int gsum;
    float d;
    const uint32_t packed = q8_k_wave(v, gsum, d);
    store_q8_k_lane(out + blk * kQ8KBytes, lane, packed, gsum, d);   // 292 = 4 * 73: 4-byte aligned
}

// ---------------------------------------------------------------------------
// Q4_0 weights (ggml section 1.1; kvad "The scale that wasted a code"):
// the value of largest magnitude (first index on ties) keeps its sign as
// max; d = max / -8 (0 for an all-zero block); code = clamp(rne(x/d)+8, 0, 15);
// byte j of qs = code_j | code_{j+16} << 4.  Eight lanes per block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q4_0(const float4 *__restrict__ w, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 3;
    const int part = threadIdx.x & 7;
    const bool valid = blk < nblocks;
    const float4 v = valid ? w[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float vv[4] = {v.x, v.y, v.z, v.w};

    // (|value|, index, value) of this lane's four, first index on ties
    float am = fabsf(vv[0]), mx = vv[0];
    int ix = 4 * part;
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const float a = fabsf(vv[k]);
        if (a > am) { am = a; mx = vv[k]; ix = 4 * part + k; }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        const float oam = xor_shfl(am, m);
        const float omx = xor_shfl(mx, m);
        const int oix = xor_shfl(ix, m);
        if (oam > am || (oam == am && oix < ix)) { am = oam; mx = omx; ix = oix; }
    }
    const float d = (am != 0.0f) ? mx / -8.0f : 0.0f;
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int c = 8;
        if (d != 0.0f) c = (int)rintf(vv[k] / d) + 8;
        c = min(max(c, 0), 15);
        codes |= (uint32_t)c << (8 * k);
    }
    // lanes 0..3 hold elements 0..15 (low nibbles), lanes 4..7 elements 16..31
    const uint32_t hi = xor_shfl(codes, 4);
    if (valid && part < 4) {
        const uint32_t bytes = codes | (hi << 4);
        uint8_t *ob = out + blk * kQ40Bytes;
        uint16_t *o16 = reinterpret_cast<uint16_t *>(ob + 2 + 4 * part);
        o16[0] = (uint16_t)(bytes & 0xffffu);
        o16[1] = (uint16_t)(bytes >> 16);
        if (part == 0) *reinterpret_cast<uint16_t *>(ob) = (uint16_t)f32_to_f16_bits(d);
    }
}

// ---------------------------------------------------------------------------
// Q2_K weights.  Format: ggml section 1.2.  The pages give no quantizer; the
// rule (the same in the header's contract) is, per group g of 16:
//   lo = min(0, min x), hi = max x, s = (hi - lo)/3, mn = -lo;
// per block: d = max_g s / 15, dmin = max_g mn / 15 (f16 stored; dh, dminh
// below are the stored values), sc = clamp(rne(s/dh), 0, 15),
// m = clamp(rne(mn/dminh), 0, 15), q = clamp(rne((x + dminh*m)/(dh*sc)), 0, 3).
// qs bit order: byte 32h + l holds, at shift 2s, weight 128h + 32s + l.
// One wave per block; lane L holds weights 4L..4L+3 (group L/4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q2_k(const float4 *__restrict__ w, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const float4 v = w[blk * 64 + lane];
    const float vv[4] = {v.x, v.y, v.z, v.w};

    float lo = fminf(fminf(vv[0], vv[1]), fminf(vv[2], vv[3]));
    float hi = fmaxf(fmaxf(vv[0], vv[1]), fmaxf(vv[2], vv[3]));
    lo = fminf(lo, xor_shfl(lo, 1));
    hi = fmaxf(hi, xor_shfl(hi, 1));
    lo = fminf(lo, xor_shfl(lo, 2));
    hi = fmaxf(hi, xor_shfl(hi, 2));
    lo = fminf(lo, 0.0f);
    const float s = (hi - lo) / 3.0f;
    const float mn = -lo;

    float smax = s, mmax = mn;
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) {
        smax = fmaxf(smax, xor_shfl(smax, m));
        mmax = fmaxf(mmax, xor_shfl(mmax, m));
    }
    smax = (smax > 0.0f) ? smax : 0.0f;        // +0 when no group spans anything
    mmax = (mmax > 0.0f) ? mmax : 0.0f;
    const uint32_t dbits = f32_to_f16_bits(smax / 15.0f);
    const uint32_t dminbits = f32_to_f16_bits(mmax / 15.0f);
    const float dh = f16_bits_to_f32(dbits);
    const float dminh = f16_bits_to_f32(dminbits);

    int sc = 0, mq = 0;
    if (dh != 0.0f) sc = min(max((int)rintf(s / dh), 0), 15);
    if (dminh != 0.0f) mq = min(max((int)rintf(mn / dminh), 0), 15);
    const float off = dminh * (float)mq;
    const float div = dh * (float)sc;
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int c = 0;
        if (div != 0.0f) c = min(max((int)rintf((vv[k] + off) / div), 0), 3);
        codes |= (uint32_t)c << (8 * k);
    }
    // weights 4L..4L+3: h = L/32, s = (L%32)/8, l = 4(L%8)..+3; lanes that
    // share (h, L%8) fill the same qs dword at shifts 0, 2, 4, 6.
    const int sh = (lane >> 3) & 3;
    uint32_t word = codes << (2 * sh);
    word |= xor_shfl(word, 8);
    word |= xor_shfl(word, 16);

    uint8_t *ob = out + blk * kQ2KBytes;                      // 84 = 4 * 21: 4-byte aligned
    if (sh == 0) *reinterpret_cast<uint32_t *>(ob + 16 + 32 * (lane >> 5) + 4 * (lane & 7)) = word;
    if ((lane & 3) == 0) ob[lane >> 2] = (uint8_t)(sc | (mq << 4));
    if (lane == 0) {
        *reinterpret_cast<uint16_t *>(ob + 80) = (uint16_t)dbits;
        *reinterpret_cast<uint16_t *>(ob + 82) = (uint16_t)dminbits;
    }
}

// ---------------------------------------------------------------------------
// Q4_K weights.  Format: 144 bytes, f16 d @0, f16 dmin @2, 12 bytes of 6-bit
// scales and mins @4, 128 bytes of nibbles @16; 32-byte chunk j holds values
// 64j + l (low nibble of byte l) and 64j + 32 + l (high nibble) (minfer "The
// payoff: a K-quant dot kernel, walked"); the 12-byte packing is GGUF's: for
// s < 4, scale = b[s] & 63, min = b[s+4] & 63; for s >= 4, scale =
// (b[s+4] & 15) | (b[s-4] >> 6) << 4, min = (b[s+4] >> 4) | (b[s] >> 6) << 4.
// The pages give no quantizer; the rule (the same as the header's) is, per
// sub-block t of 32: lo = min(0, min x), hi = max x, s = (hi - lo)/15,
// mn = -lo; d = max s / 63, dmin = max mn / 63 (f16; dh, dminh the stored
// values); sc = clamp(rne(s/dh), 0, 63), m = clamp(rne(mn/dminh), 0, 63);
// q = clamp(rne((x + dminh*m)/(dh*sc)), 0, 15).  One wave per block; lane L
// holds values 4L..4L+3 (sub-block L/8).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q4_k(const float4 *__restrict__ w, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const float4 v = w[blk * 64 + lane];
    const float vv[4] = {v.x, v.y, v.z, v.w};

    float lo = fminf(fminf(vv[0], vv[1]), fminf(vv[2], vv[3]));
    float hi = fmaxf(fmaxf(vv[0], vv[1]), fmaxf(vv[2], vv[3]));
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        lo = fminf(lo, xor_shfl(lo, m));
        hi = fmaxf(hi, xor_shfl(hi, m));
    }
    lo = fminf(lo, 0.0f);
    const float s = (hi - lo) / 15.0f;
    const float mn = -lo;
    float smax = s, mmax = mn;
#pragma unroll
    for (int m = 8; m < 64; m <<= 1) {
        smax = fmaxf(smax, xor_shfl(smax, m));
        mmax = fmaxf(mmax, xor_shfl(mmax, m));
    }
    smax = (smax > 0.0f) ? smax : 0.0f;        // +0 when no sub-block spans anything
    mmax = (mmax > 0.0f) ? mmax : 0.0f;
    const uint32_t dbits = f32_to_f16_bits(smax / 63.0f);
    const uint32_t dminbits = f32_to_f16_bits(mmax / 63.0f);
    const float dh = f16_bits_to_f32(dbits);
    const float dminh = f16_bits_to_f32(dminbits);

    int sc = 0, mq = 0;
    if (dh != 0.0f) sc = min(max((int)rintf(s / dh), 0), 63);
    if (dminh != 0.0f) mq = min(max((int)rintf(mn / dminh), 0), 63);
    const float off = dminh * (float)mq;
    const float div = dh * (float)sc;
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int c = 0;
        if (div != 0.0f) c = min(max((int)rintf((vv[k] + off) / div), 0), 15);
        codes |= (uint32_t)c << (8 * k);
    }
    // values 4L..4L+3 are chunk j = L/16, nibble half (L/8)&1, bytes 4(L%8)..+3:
    // lane L (low half) and lane L+8 (high half) fill one qs dword.
    const uint32_t word = codes | (xor_shfl(codes, 8) << 4);
    uint8_t *ob = out + blk * kQ4KBytes;                     // 144 = 16 * 9: 16-byte aligned
    if ((lane & 8) == 0) *reinterpret_cast<uint32_t *>(ob + 16 + 32 * (lane >> 4) + 4 * (lane & 7)) = word;
    // scales: sub-block t = L/8; lanes 8t (t < 4) also hold sub-block t+4's via xor 32
    const int sc4 = xor_shfl(sc, 32), m4 = xor_shfl(mq, 32);
    if (lane < 32 && (lane & 7) == 0) {
        const int t = lane >> 3;
        ob[4 + t] = (uint8_t)((sc & 63) | ((sc4 >> 4) << 6));
        ob[8 + t] = (uint8_t)((mq & 63) | ((m4 >> 4) << 6));
        ob[12 + t] = (uint8_t)((sc4 & 15) | ((m4 & 15) << 4));
    }
    if (lane == 0) {
        *reinterpret_cast<uint16_t *>(ob) = (uint16_t)dbits;
        *reinterpret_cast<uint16_t *>(ob + 2) = (uint16_t)dminbits;
    }
}

// ---------------------------------------------------------------------------
// Q6_K weights.  Format (GGUF's; the pages give only the 210-byte size): low
// 4 bits ql[128] @0, high 2 bits qh[64] @128, int8 scales[16] @192, f16 d
// @208; value i (h = i/128, k = (i%128)/32, l = i%32) has its low bits in
// ql[64h + l + 32(k&1)] (low nibble for k < 2, high for k >= 2) and its high
// bits at bit 2k of qh[32h + l]; value = d * sc_{i/16} * (q - 32).  The pages
// give no quantizer; the rule (the same as the header's) is, per group g of
// 16: mx = the value of largest magnitude (first on ties), s = mx / -32;
// d = max |s| / 127 (f16; dh the stored value); sc = clamp(rne(s/dh), -128,
// 127); q = clamp(rne(x/(dh*sc)) + 32, 0, 63), 32 if the divisor is 0.  One
// wave per block; lane L holds values 4L..4L+3 (group L/4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q6_k(const float4 *__restrict__ w, uint8_t *__restrict__ out,
                                                       int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const float4 v = w[blk * 64 + lane];
    const float vv[4] = {v.x, v.y, v.z, v.w};

    // (|value|, index, value) of the group's largest magnitude, first index on ties
    float am = fabsf(vv[0]), mx = vv[0];
    int ix = 4 * lane;
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const float a = fabsf(vv[k]);
        if (a > am) { am = a; mx = vv[k]; ix = 4 * lane + k; }
    }
#pragma unroll
    for (int m = 1; m < 4; m <<= 1) {
        const float oam = xor_shfl(am, m);
        const float omx = xor_shfl(mx, m);
        const int oix = xor_shfl(ix, m);
        if (oam > am || (oam == am && oix < ix)) { am = oam; mx = omx; ix = oix; }
    }
    const float s = (am != 0.0f) ? mx / -32.0f : 0.0f;
    float smax = fabsf(s);
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) smax = fmaxf(smax, xor_shfl(smax, m));
    const uint32_t dbits = f32_to_f16_bits(smax / 127.0f);
    const float dh = f16_bits_to_f32(dbits);
    int sc = 0;
    if (dh != 0.0f) sc = min(max((int)rintf(s / dh), -128), 127);
    const float div = dh * (float)sc;
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int c = 32;
        if (div != 0.0f) c = min(max((int)rintf(vv[k] / div) + 32, 0), 63);
        codes |= (uint32_t)c << (8 * k);
    }
    // values 4L..4L+3: h = L/32, k = (L%32)/8, l = 4(L%8)..+3.  ql dword at
    // 64h + 32(k&1) + 4(L%8): low nibbles from lane L (k < 2), high nibbles
    // from lane L+16 (k + 2); qh dword at 128 + 32h + 4(L%8) gathers the four k.
    const int kq = (lane >> 3) & 3;
    const uint32_t lo4 = codes & 0x0f0f0f0fu;
    const uint32_t qlw = lo4 | (xor_shfl(lo4, 16) << 4);
    uint32_t qhw = ((codes >> 4) & 0x03030303u) << (2 * kq);
    qhw |= xor_shfl(qhw, 8);
    qhw |= xor_shfl(qhw, 16);
    uint8_t *ob = out + blk * kQ6KBytes;                      // 210: only 2-byte aligned
    const int h = lane >> 5;
    if (kq < 2) {
        uint16_t *o16 = reinterpret_cast<uint16_t *>(ob + 64 * h + 32 * kq + 4 * (lane & 7));
        o16[0] = (uint16_t)(qlw & 0xffffu);
        o16[1] = (uint16_t)(qlw >> 16);
    }
    if (kq == 0) {
        uint16_t *o16 = reinterpret_cast<uint16_t *>(ob + 128 + 32 * h + 4 * (lane & 7));
        o16[0] = (uint16_t)(qhw & 0xffffu);
        o16[1] = (uint16_t)(qhw >> 16);
    }
    if ((lane & 3) == 0) ob[192 + (lane >> 2)] = (uint8_t)(int8_t)sc;
    if (lane == 0) *reinterpret_cast<uint16_t *>(ob + 208) = (uint16_t)dbits;
}

// ---------------------------------------------------------------------------
// Q4_1 / Q5_0 / Q5_1 weights (formats: ggml section 1.1, the _1 formats add a
// per-block offset; minfer, the Q5 formats add a fifth-bit plane; field and
// bit order GGUF's: Q4_1 d m qs, Q5_0 d qh qs, Q5_1 d m qh qs, qs byte j =
// value j | value j+16 << 4, bit j of qh = value j's fifth bit).  The pages
// give no quantizer; the rule (the same as the header's):
//   _1: lo = min x, hi = max x (a zero of either sign as +0); d = (hi - lo)/L
//       (L = 15, 31), m = lo (f16; dh, mh the stored values);
//       q = clamp(rne((x - mh)/dh), 0, L), 0 if dh is 0;
//   Q5_0: the value of largest magnitude (first on ties) gives d = max / -16;
//       q = clamp(rne(x/d) + 16, 0, 31), 16 if d is 0.
// Eight lanes per block, four values each (lane part p: values 4p..4p+3).
// ---------------------------------------------------------------------------
template <int F> struct W32 {
    static constexpr int BYTES = F == F_Q4_1 ? kQ41Bytes : (F == F_Q5_0 ? kQ50Bytes : kQ51Bytes);
    static constexpr int QS = F == F_Q4_1 ? 4 : (F == F_Q5_0 ? 6 : 8);   // qs offset
    static constexpr int QH = F == F_Q5_0 ? 2 : 4;                        // qh offset (Q5 only)
};

template <int F>
__global__ __launch_bounds__(256) void k_quantize_w32(const float4 *__restrict__ w, uint8_t *__restrict__ out,
                                                      int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 3;
    const int part = threadIdx.x & 7;
    const bool valid = blk < nblocks;
    const float4 v = valid ? w[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    int code[4];
    uint32_t dbits, mbits = 0;
    if constexpr (F == F_Q5_0) {
        float am = fabsf(vv[0]), mx = vv[0];
        int ix = 4 * part;
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            const float a = fabsf(vv[k]);
            if (a > am) { am = a; mx = vv[k]; ix = 4 * part + k; }
        }
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
            const float oam = xor_shfl(am, m);
            const float omx = xor_shfl(mx, m);
            const int oix = xor_shfl(ix, m);
            if (oam > am || (oam == am && oix < ix)) { am = oam; mx = omx; ix = oix; }
        }
        const float d = (am != 0.0f) ? mx / -16.0f : 0.0f;
        dbits = f32_to_f16_bits(d);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int c = 16;
            if (d != 0.0f) c = min(max((int)rintf(vv[k] / d) + 16, 0), 31);
            code[k] = c;
        }
    } else {
        constexpr int L = F == F_Q4_1 ? 15 : 31;
        float lo = fminf(fminf(vv[0], vv[1]), fminf(vv[2], vv[3]));
        float hi = fmaxf(fmaxf(vv[0], vv[1]), fmaxf(vv[2], vv[3]));
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
            lo = fminf(lo, xor_shfl(lo, m));
            hi = fmaxf(hi, xor_shfl(hi, m));
        }
        lo += 0.0f;
        hi += 0.0f;
        dbits = f32_to_f16_bits((hi - lo) / (float)L);
        mbits = f32_to_f16_bits(lo);
        const float dh = f16_bits_to_f32(dbits), mh = f16_bits_to_f32(mbits);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int c = 0;
            if (dh != 0.0f) c = min(max((int)rintf((vv[k] - mh) / dh), 0), L);
            code[k] = c;
        }
    }
    uint32_t c4 = 0, qb = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c4 |= (uint32_t)(code[k] & 15) << (8 * k);
        qb |= (uint32_t)((code[k] >> 4) & 1) << (4 * part + k);
    }
    // lanes 0..3 hold values 0..15 (low nibbles), lanes 4..7 values 16..31
    const uint32_t hi4 = xor_shfl(c4, 4);
    qb |= xor_shfl(qb, 1);
    qb |= xor_shfl(qb, 2);
    qb |= xor_shfl(qb, 4);
    if (valid) {
        uint8_t *ob = out + blk * W32<F>::BYTES;                   // 2-byte aligned at least
        if (part < 4) {
            const uint32_t bytes = c4 | (hi4 << 4);
            uint16_t *o16 = reinterpret_cast<uint16_t *>(ob + W32<F>::QS + 4 * part);
            o16[0] = (uint16_t)(bytes & 0xffffu);
            o16[1] = (uint16_t)(bytes >> 16);
        }
        if (part == 0) {
            *reinterpret_cast<uint16_t *>(ob) = (uint16_t)dbits;
            if constexpr (F != F_Q5_0) *reinterpret_cast<uint16_t *>(ob + 2) = (uint16_t)mbits;
            if constexpr (F != F_Q4_1) {
                uint16_t *q16 = reinterpret_cast<uint16_t *>(ob + W32<F>::QH);
                q16[0] = (uint16_t)(qb & 0xffffu);
                q16[1] = (uint16_t)(qb >> 16);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers (called by the C ABI after argument checks).
// ---------------------------------------------------------------------------
hipError_t launch_quantize_q8_0(const float *x, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 31) / 32;
    void *args[] = {(void *)&x, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q8_0, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_quantize_q8_k(const float *x, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 3) / 4;
    void *args[] = {(void *)&x, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q8_k, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_quantize_q4_0(const float *w, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 31) / 32;
    void *args[] = {(void *)&w, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q4_0, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_quantize_q2_k(const float *w, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 3) / 4;
    void *args[] = {(void *)&w, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q2_k, dim3((unsigned)grid), dim3(256), args, 0, st);
}

template <int F>
static hipError_t launch_w32(const float *w, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 31) / 32;
    void *args[] = {(void *)&w, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_w32<F>, dim3((unsigned)grid), dim3(256), args, 0, st);
}
hipError_t launch_quantize_q4_1(const float *w, void *out, int64_t nb, hipStream_t st) {
    return launch_w32<F_Q4_1>(w, out, nb, st);
}
hipError_t launch_quantize_q5_0(const float *w, void *out, int64_t nb, hipStream_t st) {
    return launch_w32<F_Q5_0>(w, out, nb, st);
}
hipError_t launch_quantize_q5_1(const float *w, void *out, int64_t nb, hipStream_t st) {
    return launch_w32<F_Q5_1>(w, out, nb, st);
}

hipError_t launch_quantize_q4_k(const float *w, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 3) / 4;
    void *args[] = {(void *)&w, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q4_k, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_quantize_q6_k(const float *w, void *out, int64_t nblocks, hipStream_t st) {
    const int64_t grid = (nblocks + 3) / 4;
    void *args[] = {(void *)&w, (void *)&out, (void *)&nblocks};
    return hipLaunchKernel((const void *)k_quantize_q6_k, dim3((unsigned)grid), dim3(256), args, 0, st);
}

}  // namespace qmm
