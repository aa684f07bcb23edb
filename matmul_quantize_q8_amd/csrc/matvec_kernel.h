#pragma once
// Decode matvec, one token: y[n] = sum_b d_w[n,b] d_x[b] I_b[n].
//
// Decode is weight streaming: every weight byte is read once per token
// (minfer section 2.1, "the decode physics"), so the kernel is bound by HBM
// and is built to keep the weight stream moving at full rate:
//   * a wave owns G consecutive rows (whole rows: every output is reduced
//     inside one wave, in a fixed order, and written once -- minfer's row
//     ownership, the reason results do not depend on the launch shape);
//   * the rows' bytes form one contiguous span, copied into the wave's own
//     LDS slice by gfx950 LDS-DMA loads (global_load_lds_dwordx4: 16 bytes
//     per lane, coalesced, no registers); Q4_0 / Q8_0 blocks are only 2-byte
//     aligned, so blocks are re-sliced from LDS rather than loaded directly;
//   * the activation row is DMA'd once per workgroup into LDS; each lane then
//     owns fixed "units" of every row (a pair of blocks for Q4_0 / Q8_0 --
//     with an even block count a pair starts 4-byte aligned -- or a quarter
//     of a Q2_K super-block), keeps the matching activation codes in
//     registers and reuses them for all G rows;
//   * integer block sums come from v_dot4_i32_i8; the per-block scale product
//     d_w*d_x of two binary16 values is exact in f32, so each block adds one
//     correctly rounded term;
//   * the G row sums are reduced across the wave by a transposing butterfly
//     (log2(G) exchange steps that halve the live values, then plain steps),
//     all in VALU lane exchanges: gfx950's permlane32/permlane16 swaps for
//     lane bits 5 and 4, DPP for bits 3..0.
// Rows longer than one segment (64*MAXU units) are walked in segments with
// the partial sums kept in registers (only with G = 1).
//
// Fused variant (XF32): the workgroup takes the f32 activation row instead of
// its Q8_0 blocks and quantizes it itself, so a decode step is one launch
// (minfer section 3.3, "Design choices": the quantized row is derived data of
// the product, shared by sibling products; here the quantizer moves into the
// product's launch): each thread loads
// 16-byte pieces of the row before the weight copies are issued, waits for
// those loads alone, quantizes them with the same arithmetic as the Q8_0
// quantizer kernel, and writes the codes to LDS in a lane-friendly layout
// (per unit: the blocks' 32 codes, then their scales as f32).  For the
// K-quant weights the activation is Q8_K: each wave quantizes whole 256-value
// super-blocks (the Q8_K quantizer's arithmetic, lane L holding values
// 4L..4L+3) and writes them to LDS in the row's own 292-byte layout, which
// the K-quant units then read as in the plain kernel.  One workgroup per
// token also stores the quantized row to global memory when asked to.
#include "qmm_device.h"

namespace qmm {

template <int F> struct FmtBytes;
template <> struct FmtBytes<F_Q4_0> { static constexpr int BB = kQ40Bytes, XB = kQ80Bytes; };
template <> struct FmtBytes<F_Q8_0> { static constexpr int BB = kQ80Bytes, XB = kQ80Bytes; };
template <> struct FmtBytes<F_Q2_K> { static constexpr int BB = kQ2KBytes, XB = kQ8KBytes; };
template <> struct FmtBytes<F_Q4_K> { static constexpr int BB = kQ4KBytes, XB = kQ8KBytes; };
template <> struct FmtBytes<F_Q6_K> { static constexpr int BB = kQ6KBytes, XB = kQ8KBytes; };
template <> struct FmtBytes<F_Q4_1> { static constexpr int BB = kQ41Bytes, XB = kQ80Bytes; };
template <> struct FmtBytes<F_Q5_0> { static constexpr int BB = kQ50Bytes, XB = kQ80Bytes; };
template <> struct FmtBytes<F_Q5_1> { static constexpr int BB = kQ51Bytes, XB = kQ80Bytes; };

// A unit is what one lane handles per row: P blocks (P = 2 paired, 1 single)
// of Q4_0 / Q8_0, or a quarter (64 values) of a K-quant super-block.
template <int F, bool PAIRED> struct Unit {
    static constexpr int BPU = kIsK<F> ? 1 : (PAIRED ? 2 : 1);   // blocks per unit
    static constexpr int UPB = kIsK<F> ? 4 : 1;                  // units per block
};

// Activation registers of one unit.
template <int F, bool PAIRED, bool K = kIsK<F>> struct XU {
    int q[8 * Unit<F, PAIRED>::BPU];
    float d[Unit<F, PAIRED>::BPU];
    int sx8[Unit<F, PAIRED>::BPU];                    // 8 * sum of codes (Q4_0 only)
};
template <int F, bool PAIRED> struct XU<F, PAIRED, true> {
    int q[16];                                        // the unit's 64 Q8_K codes
    int bs[4];                                        // the bsums of its four groups of 16
    float d;
};

// --- LDS readers -------------------------------------------------------------
// Q8_0 block (f16 d, 32 codes) at a 2-byte aligned LDS byte offset o.
__device__ __forceinline__ void lds_q8_0_block(const uint8_t *l8, uint32_t o, int *q, float &d) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(l8);
    const uint32_t qd = (o + 2) >> 2, qsh = (o + 2) & 3;
    uint32_t v[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) v[k] = l32[qd + k];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = (int)align_bytes(v[k + 1], v[k], qsh);
    d = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(l8 + o));
}

// The same with the codes' byte offset (o + 2) mod 4 known to the caller.
template <int SH>
__device__ __forceinline__ void lds_q8_0_block_at(const uint8_t *l8, uint32_t o, int *q, float &d) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(l8);
    const uint32_t qd = (o + 2) >> 2;
    if constexpr (SH == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = (int)l32[qd + k];
    } else {
        uint32_t v[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) v[k] = l32[qd + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = (int)align_bytes(v[k + 1], v[k], SH);
    }
    d = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(l8 + o));
}

// A paired unit's activation blocks: rows of an even block count start on
// 4-byte boundaries and xoff keeps that alignment, so block 0's codes sit 2
// bytes past a dword boundary and block 1's on one.
template <int F, bool PAIRED>
__device__ __forceinline__ void load_xu(const uint8_t *xl, uint32_t xoff, int u, XU<F, PAIRED> &x) {
    if constexpr (!kIsK<F>) {
        constexpr int P = Unit<F, PAIRED>::BPU;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const uint32_t o = xoff + (uint32_t)(P * u + j) * kQ80Bytes;
            if constexpr (P == 2) {
                if (j == 0)
                    lds_q8_0_block_at<2>(xl, o, x.q, x.d[0]);
                else
                    lds_q8_0_block_at<0>(xl, o, x.q + 8, x.d[1]);
            } else {
                lds_q8_0_block(xl, o, x.q + 8 * j, x.d[j]);
            }
            int s = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) s = dot4(x.q[8 * j + k], 0x01010101, s);
            x.sx8[j] = 8 * s;        // sum_j (n_j - 8) q_j = sum_j n_j q_j - 8 sum_j q_j
        }
    } else {
        // Q8_K unit u = (super-block c, part p); Q8_K blocks are 4-byte aligned.
        const int c = u >> 2, p = u & 3;
        const uint8_t *b = xl + xoff + (uint32_t)c * kQ8KBytes;
        if constexpr (F == F_Q4_K) {
            // part p = chunk j: values 64j + [0, 64), groups 4j .. 4j+3
            const uint32_t *q32 = reinterpret_cast<const uint32_t *>(b + 4 + 64 * p);
#pragma unroll
            for (int k = 0; k < 16; ++k) x.q[k] = (int)q32[k];
            const uint32_t *bs32 = reinterpret_cast<const uint32_t *>(b + 260 + 8 * p);
#pragma unroll
            for (int k = 0; k < 4; ++k) x.bs[k] = (int)(int16_t)(bs32[k >> 1] >> (16 * (k & 1)));
        } else {
            // Q2_K: part p covers weight qs bytes [16p, 16p+16), i.e. values
            // 128h + 32s + 16(p&1) + [0,16), s < 4, h = p/2 (groups 8h + 2s + (p&1)).
            // Q6_K: part p = (h, g2) covers values 128h + 32k + 16 g2 + [0,16),
            // k < 4 (groups 8h + 2k + g2) -- the same sets of values.
            const int h = p >> 1, odd = p & 1;
            const uint32_t *q32 = reinterpret_cast<const uint32_t *>(b + 4 + 128 * h + 16 * odd);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int k = 0; k < 4; ++k) x.q[4 * s + k] = (int)q32[8 * s + k];
            const uint32_t *bs32 = reinterpret_cast<const uint32_t *>(b + 260 + 16 * h);
#pragma unroll
            for (int s = 0; s < 4; ++s) x.bs[s] = (int)(int16_t)(bs32[s] >> (16 * odd));
        }
        x.d = *reinterpret_cast<const float *>(b);
    }
}

// Fused-variant activation layout in LDS: unit u at (32*P + 16)*u bytes holds
// the P blocks' codes (32 bytes each), then their f16-rounded scales as f32.
template <int P> struct XLayout { static constexpr int US = 32 * P + 16; };

template <int F, bool PAIRED>
__device__ __forceinline__ void load_xu_q(const uint8_t *xl, int u, XU<F, PAIRED> &x) {
    constexpr int P = Unit<F, PAIRED>::BPU;
    const uint8_t *ub = xl + XLayout<P>::US * u;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const uint4 a = reinterpret_cast<const uint4 *>(ub + 32 * j)[0];
        const uint4 b = reinterpret_cast<const uint4 *>(ub + 32 * j)[1];
        int *q = x.q + 8 * j;
        q[0] = (int)a.x; q[1] = (int)a.y; q[2] = (int)a.z; q[3] = (int)a.w;
        q[4] = (int)b.x; q[5] = (int)b.y; q[6] = (int)b.z; q[7] = (int)b.w;
        x.d[j] = reinterpret_cast<const float *>(ub + 32 * P)[j];
        int s = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) s = dot4(q[k], 0x01010101, s);
        x.sx8[j] = 8 * s;
    }
}

// --- one unit of one row ------------------------------------------------------
// Q4_0 block: I = sum_j (nib_j - 8) q_j with low nibbles = elements 0..15 and
// high nibbles = 16..31 (minfer scalar kernel; ggml section 2).
__device__ __forceinline__ int q4_isum(const uint32_t *qs, const int *x, int sx8) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s = dot4((int)(qs[k] & 0x0f0f0f0fu), x[k], s);
        s = dot4((int)((qs[k] >> 4) & 0x0f0f0f0fu), x[k + 4], s);
    }
    return s - sx8;
}

template <int F, bool PAIRED>
__device__ __forceinline__ float unit_dot(const uint8_t *sl, uint32_t bo, int u, const XU<F, PAIRED> &x, float acc);

// Paired Q4_0 at a 4-byte aligned offset: 36 bytes = d0, qs0 (2-byte shifted),
// d1, qs1 (aligned).
template <>
__device__ __forceinline__ float unit_dot<F_Q4_0, true>(const uint8_t *sl, uint32_t bo, int,
                                                        const XU<F_Q4_0, true> &x, float acc) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(sl + bo);
    uint32_t v[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) v[k] = l32[k];
    uint32_t qs0[4], qs1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        qs0[k] = align_bytes(v[k + 1], v[k], 2);
        qs1[k] = v[5 + k];
    }
    const float dw0 = f16_bits_to_f32(v[0]), dw1 = f16_bits_to_f32(v[4] >> 16);
    acc = fmaf(dw0 * x.d[0], (float)q4_isum(qs0, x.q, x.sx8[0]), acc);
    return fmaf(dw1 * x.d[1], (float)q4_isum(qs1, x.q + 8, x.sx8[1]), acc);
}

template <>
__device__ __forceinline__ float unit_dot<F_Q4_0, false>(const uint8_t *sl, uint32_t bo, int,
                                                         const XU<F_Q4_0, false> &x, float acc) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(sl);
    const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
    uint32_t v[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) v[k] = l32[qd + k];
    uint32_t qs[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) qs[k] = align_bytes(v[k + 1], v[k], qsh);
    const float dw = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(sl + bo));
    return fmaf(dw * x.d[0], (float)q4_isum(qs, x.q, x.sx8[0]), acc);
}

// Paired Q8_0 at a 4-byte aligned offset: 68 bytes = d0, codes0 (2-byte
// shifted), d1, codes1 (aligned).
template <>
__device__ __forceinline__ float unit_dot<F_Q8_0, true>(const uint8_t *sl, uint32_t bo, int,
                                                        const XU<F_Q8_0, true> &x, float acc) {
    const uint32_t *l32 = reinterpret_cast<const uint32_t *>(sl + bo);
    uint32_t v[17];
#pragma unroll
    for (int k = 0; k < 17; ++k) v[k] = l32[k];
    int s0 = 0, s1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        s0 = dot4((int)align_bytes(v[k + 1], v[k], 2), x.q[k], s0);
        s1 = dot4((int)v[9 + k], x.q[8 + k], s1);
    }
    const float dw0 = f16_bits_to_f32(v[0]), dw1 = f16_bits_to_f32(v[8] >> 16);
    acc = fmaf(dw0 * x.d[0], (float)s0, acc);
    return fmaf(dw1 * x.d[1], (float)s1, acc);
}

template <>
__device__ __forceinline__ float unit_dot<F_Q8_0, false>(const uint8_t *sl, uint32_t bo, int,
                                                         const XU<F_Q8_0, false> &x, float acc) {
    int q[8];
    float dw;
    lds_q8_0_block(sl, bo, q, dw);
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = dot4(q[k], x.q[k], s);
    return fmaf(dw * x.d[0], (float)s, acc);
}

// Q2_K part p of the super-block at a 4-byte aligned offset:
//   V = sum_s sc_s * sum q x,  Mn = sum_s m_s * bsum_s,
//   t = d d8 V - dmin d8 Mn   (minfer "a K-quant dot kernel, walked").
template <>
__device__ __forceinline__ float unit_dot<F_Q2_K, false>(const uint8_t *sl, uint32_t bo, int u,
                                                         const XU<F_Q2_K, false> &x, float acc) {
    const int p = u & 3, h = p >> 1, odd = p & 1;
    const uint32_t *b32 = reinterpret_cast<const uint32_t *>(sl + bo);
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = b32[4 + 4 * p + k];
    const uint32_t sc01 = b32[2 * h], sc23 = b32[2 * h + 1];
    const uint32_t dd = b32[20];
    // Bit pair s of each byte is used in place: q & (3 << 2s) is 4^s times
    // the code (at most 48, a positive int8, for s < 3); pair 3 is shifted
    // down by two first (16 times the code).  The group dots are then
    // G = (g0, 4 g1, 16 g2, 16 g3) and 16 V = 16 sc0 G0 + 4 sc1 G1 + sc2 G2
    // + sc3 G3 (|16 V| < 2^23, exact in f32).
    int G0 = 0, G1 = 0, G2 = 0, G3 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        G0 = dot4((int)(q[k] & 0x03030303u), x.q[k], G0);
        G1 = dot4((int)(q[k] & 0x0c0c0c0cu), x.q[4 + k], G1);
        G2 = dot4((int)(q[k] & 0x30303030u), x.q[8 + k], G2);
        G3 = dot4((int)((q[k] >> 2) & 0x30303030u), x.q[12 + k], G3);
    }
    // group s's scale byte: byte 2 (s & 1) + odd of sc01 (s < 2) or sc23
    const uint32_t o0 = 8u * (uint32_t)odd, o1 = o0 + 16u;
    const int sc0 = (int)__builtin_amdgcn_ubfe(sc01, o0, 4), m0 = (int)__builtin_amdgcn_ubfe(sc01, o0 + 4u, 4);
    const int sc1 = (int)__builtin_amdgcn_ubfe(sc01, o1, 4), m1 = (int)__builtin_amdgcn_ubfe(sc01, o1 + 4u, 4);
    const int sc2 = (int)__builtin_amdgcn_ubfe(sc23, o0, 4), m2 = (int)__builtin_amdgcn_ubfe(sc23, o0 + 4u, 4);
    const int sc3 = (int)__builtin_amdgcn_ubfe(sc23, o1, 4), m3 = (int)__builtin_amdgcn_ubfe(sc23, o1 + 4u, 4);
    const int V16 = 16 * sc0 * G0 + 4 * sc1 * G1 + sc2 * G2 + sc3 * G3;
    const int Mn = m0 * x.bs[0] + m1 * x.bs[1] + m2 * x.bs[2] + m3 * x.bs[3];
    const float d = f16_bits_to_f32(dd), dmin = f16_bits_to_f32(dd >> 16);
    acc = fmaf(d * x.d * 0.0625f, (float)V16, acc);
    return fmaf(-(dmin * x.d), (float)Mn, acc);
}

// Q4_K chunk j = u & 3 of the super-block at a 16-byte aligned offset (minfer
// "The payoff: a K-quant dot kernel, walked"): low nibbles of the chunk's 32
// bytes are sub-block 2j, high nibbles sub-block 2j+1;
//   V = sc_2j * sum_lo + sc_2j+1 * sum_hi,
//   Mn = m_2j * (bsum_4j + bsum_4j+1) + m_2j+1 * (bsum_4j+2 + bsum_4j+3),
//   t = d d8 V - dmin d8 Mn.
// The 6-bit scales and mins of sub-block s sit in bytes A = s & 3, B = A + 4,
// C = A + 8 of the 12-byte field: s < 4: sc = A & 63, m = B & 63; s >= 4:
// sc = (C & 15) | (A >> 6) << 4, m = (C >> 4) | (B >> 6) << 4.
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int s, int &sc, int &m) {
    const uint32_t sh = 8u * (uint32_t)(s & 3);
    const uint32_t A = (s0 >> sh) & 0xffu, B = (s1 >> sh) & 0xffu, C = (s2 >> sh) & 0xffu;
    if (s < 4) {
        sc = (int)(A & 63u);
        m = (int)(B & 63u);
    } else {
        sc = (int)((C & 15u) | ((A >> 6) << 4));
        m = (int)((C >> 4) | ((B >> 6) << 4));
    }
}

template <>
__device__ __forceinline__ float unit_dot<F_Q4_K, false>(const uint8_t *sl, uint32_t bo, int u,
                                                         const XU<F_Q4_K, false> &x, float acc) {
    const int j = u & 3;
    const uint32_t *b32 = reinterpret_cast<const uint32_t *>(sl + bo);
    const uint32_t dd = b32[0], s0 = b32[1], s1 = b32[2], s2 = b32[3];
    int lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t q = b32[4 + 8 * j + k];
        lo = dot4((int)(q & 0x0f0f0f0fu), x.q[k], lo);
        hi = dot4((int)((q >> 4) & 0x0f0f0f0fu), x.q[8 + k], hi);
    }
    int sc0, m0, sc1, m1;
    q4k_scale_min(s0, s1, s2, 2 * j, sc0, m0);
    q4k_scale_min(s0, s1, s2, 2 * j + 1, sc1, m1);
    const int V = sc0 * lo + sc1 * hi;
    const int Mn = m0 * (x.bs[0] + x.bs[1]) + m1 * (x.bs[2] + x.bs[3]);
    const float d = f16_bits_to_f32(dd), dmin = f16_bits_to_f32(dd >> 16);
    acc = fmaf(d * x.d, (float)V, acc);
    return fmaf(-(dmin * x.d), (float)Mn, acc);
}

// n dwords of LDS starting at a 2-byte aligned byte offset `off`.
template <int NW>
__device__ __forceinline__ void lds_dwords(const uint8_t *sl, uint32_t off, uint32_t (&out)[NW]) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(sl + (off & ~3u));
    const uint32_t sh = off & 3u;
    uint32_t v[NW + 1];
#pragma unroll
    for (int k = 0; k <= NW; ++k) v[k] = p[k];
#pragma unroll
    for (int k = 0; k < NW; ++k) out[k] = align_bytes(v[k + 1], v[k], sh);
}

// Q6_K part p = (h, g2) of the super-block at a 2-byte aligned offset: values
// 128h + 32k + 16 g2 + l (k < 4, l < 16) take their low 4 bits from ql run A =
// ql[64h + 16 g2 ..] (k = 0 low nibble, k = 2 high) or run B = ql[64h + 32 +
// 16 g2 ..] (k = 1 low, k = 3 high), their high 2 bits from qh[32h + 16 g2 ..]
// at bit 2k; group 8h + 2k + g2.  t = d d8 sum_k sc_k (sum q x - 32 bsum_k).
template <>
__device__ __forceinline__ float unit_dot<F_Q6_K, false>(const uint8_t *sl, uint32_t bo, int u,
                                                         const XU<F_Q6_K, false> &x, float acc) {
    const int p = u & 3, h = p >> 1, g2 = p & 1;
    uint32_t ra[4], rb[4], qh[4], sw[2];
    lds_dwords<4>(sl, bo + 64 * h + 16 * g2, ra);
    lds_dwords<4>(sl, bo + 64 * h + 32 + 16 * g2, rb);
    lds_dwords<4>(sl, bo + 128 + 32 * h + 16 * g2, qh);
    lds_dwords<2>(sl, bo + 192 + 8 * h, sw);           // scales 8h .. 8h+7
    const uint32_t dbits = *reinterpret_cast<const uint16_t *>(sl + bo + 208);
    int V = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t src = (k & 1) ? rb[e] : ra[e];
            const uint32_t lo4 = (k < 2) ? (src & 0x0f0f0f0fu) : ((src >> 4) & 0x0f0f0f0fu);
            const uint32_t hi2 = ((qh[e] >> (2 * k)) & 0x03030303u) << 4;
            s = dot4((int)(lo4 | hi2), x.q[4 * k + e], s);
        }
        // scale of group 8h + 2k + g2: byte 2k + g2 of the 8-byte window
        const int sc = __builtin_amdgcn_sbfe((int)sw[k >> 1], 8 * (2 * (k & 1) + g2), 8);
        V += sc * (s - 32 * x.bs[k]);
    }
    return fmaf(f16_bits_to_f32(dbits) * x.d, (float)V, acc);
}

// --- Q4_1 / Q5_0 / Q5_1 (ggml section 1.1: the _1 formats add a per-block
// offset, value = d*q + m; minfer: the Q5 formats add a fifth-bit plane) --------
// One block given as dwords of its fields: the codes of values 4k..4k+3 and
// 16+4k..16+4k+3 come from qs dword k (low / high nibbles) and, for the Q5
// formats, bits 4k.. and 16+4k.. of qh; returns sum_j q_j x_j.
template <bool Q5>
__device__ __forceinline__ int block32_isum(const uint32_t (&qs)[4], uint32_t qh, const int *x) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t lo = qs[k] & 0x0f0f0f0fu, hi = (qs[k] >> 4) & 0x0f0f0f0fu;
        if constexpr (Q5) {
            lo |= bits_to_bytes(__builtin_amdgcn_ubfe(qh, 4 * k, 4)) << 4;
            hi |= bits_to_bytes(__builtin_amdgcn_ubfe(qh, 16 + 4 * k, 4)) << 4;
        }
        s = dot4((int)lo, x[k], s);
        s = dot4((int)hi, x[k + 4], s);
    }
    return s;
}

// t = dw dx I (+ m dx S for the _1 formats); S = sum of the block's
// activation codes = sx8 / 8; Q5_0's codes carry +16: I = sum q x - 16 S.
template <int F>
__device__ __forceinline__ float block32_fold(int I, uint32_t dm, float dx, int sx8, float acc) {
    const float dw = f16_bits_to_f32(dm);
    if constexpr (F == F_Q5_0) {
        I -= 2 * sx8;
        return fmaf(dw * dx, (float)I, acc);
    } else {
        acc = fmaf(dw * dx, (float)I, acc);
        return fmaf(f16_bits_to_f32(dm >> 16) * dx, (float)(sx8 >> 3), acc);
    }
}

template <int F>
__device__ __forceinline__ float block32_term(uint32_t dm, const uint32_t (&qs)[4], uint32_t qh, const int *x,
                                              float dx, int sx8, float acc) {
    constexpr bool Q5 = F != F_Q4_1;
    return block32_fold<F>(block32_isum<Q5>(qs, qh, x), dm, dx, sx8, acc);
}

// Fields of the block at a 2-byte aligned LDS offset o: d (and m) dword, qh, qs.
template <int F>
__device__ __forceinline__ void block32_fields(const uint8_t *sl, uint32_t o, uint32_t &dm, uint32_t &qh,
                                               uint32_t (&qs)[4]) {
    // Q4_1 (20 bytes) and Q5_1 (24 bytes) blocks are 4-byte aligned in a
    // row, and rows land in LDS at their global alignment: direct reads.
    if constexpr (F == F_Q4_1) {          // d m | qs
        const uint32_t *w = reinterpret_cast<const uint32_t *>(sl + o);
        dm = w[0];
        qh = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) qs[k] = w[1 + k];
    } else if constexpr (F == F_Q5_1) {   // d m | qh | qs
        const uint32_t *w = reinterpret_cast<const uint32_t *>(sl + o);
        dm = w[0];
        qh = w[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) qs[k] = w[2 + k];
    } else {                              // 22 bytes: d | qh | qs, fields 2 bytes off the dwords
        uint32_t w[6];
        lds_dwords<6>(sl, o, w);
        dm = w[0] & 0xffffu;
        qh = align_bytes(w[1], w[0], 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) qs[k] = align_bytes(w[2 + k], w[1 + k], 2);
    }
}

template <int F, bool PAIRED>
__device__ __forceinline__ float unit_dot32(const uint8_t *sl, uint32_t bo, const XU<F, PAIRED> &x, float acc) {
    constexpr int P = Unit<F, PAIRED>::BPU;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        uint32_t dm, qh, qs[4];
        block32_fields<F>(sl, bo + (uint32_t)j * FmtBytes<F>::BB, dm, qh, qs);
        acc = block32_term<F>(dm, qs, qh, x.q + 8 * j, x.d[j], x.sx8[j], acc);
    }
    return acc;
}
template <>
__device__ __forceinline__ float unit_dot<F_Q4_1, true>(const uint8_t *sl, uint32_t bo, int,
                                                        const XU<F_Q4_1, true> &x, float acc) {
    return unit_dot32<F_Q4_1, true>(sl, bo, x, acc);
}
template <>
__device__ __forceinline__ float unit_dot<F_Q4_1, false>(const uint8_t *sl, uint32_t bo, int,
                                                         const XU<F_Q4_1, false> &x, float acc) {
    return unit_dot32<F_Q4_1, false>(sl, bo, x, acc);
}
template <>
__device__ __forceinline__ float unit_dot<F_Q5_0, true>(const uint8_t *sl, uint32_t bo, int,
                                                        const XU<F_Q5_0, true> &x, float acc) {
    return unit_dot32<F_Q5_0, true>(sl, bo, x, acc);
}
template <>
__device__ __forceinline__ float unit_dot<F_Q5_0, false>(const uint8_t *sl, uint32_t bo, int,
                                                         const XU<F_Q5_0, false> &x, float acc) {
    return unit_dot32<F_Q5_0, false>(sl, bo, x, acc);
}
template <>
__device__ __forceinline__ float unit_dot<F_Q5_1, true>(const uint8_t *sl, uint32_t bo, int,
                                                        const XU<F_Q5_1, true> &x, float acc) {
    return unit_dot32<F_Q5_1, true>(sl, bo, x, acc);
}
template <>
__device__ __forceinline__ float unit_dot<F_Q5_1, false>(const uint8_t *sl, uint32_t bo, int,
                                                         const XU<F_Q5_1, false> &x, float acc) {
    return unit_dot32<F_Q5_1, false>(sl, bo, x, acc);
}

// Copy bytes [lo, hi) of global memory into LDS at `dst` (16-byte aligned), as
// the 16-byte chunks from lo & ~15 up to the chunk holding byte hi-1; chunk c
// lands at dst + 16 c.  This wave issues the chunk groups (64 chunks, one
// instruction each) k = first, first+step, ...; every lane of an issued
// instruction loads (lanes past the end re-load the last chunk, into slots of
// the group that are never read), so the number of instructions this wave
// issued is exactly the return value.  Global reads never pass the 16-byte
// granule that holds byte hi-1.
template <bool STREAM = false>
__device__ __forceinline__ int dma_span(const uint8_t *src, int64_t lo, int64_t hi, uint4 *dst, int lane,
                                        int first, int step) {
    const int64_t A = lo & ~(int64_t)15;
    const int nch = (int)((((hi + 15) & ~(int64_t)15) - A) >> 4);
    int issued = 0;
    for (int k = first; k * kWave < nch; k += step) {
        const int c = min(k * kWave + lane, nch - 1);
        global_to_lds16<STREAM>(src + A + 16 * (int64_t)c, dst + k * kWave);
        ++issued;
    }
    return issued;
}

// --- a row's weight unit held for several tokens -------------------------------
// The few-token path dots one weight unit with every token.  In general the
// unit is re-read from LDS for each token (unpaired Q4_0 and Q8_0 units);
// the other units keep their codes (expanded to bytes) and scales in
// registers (up to 26 VGPRs), so each further token costs its dot products
// and the folds.
// Same integer sums and the same fmaf order as unit_dot.
template <int F, bool PAIRED> struct UnitW {
    const uint8_t *sl;
    uint32_t bo;
    int u;
    __device__ __forceinline__ void load(const uint8_t *s, uint32_t o, int uu) {
        sl = s;
        bo = o;
        u = uu;
    }
    __device__ __forceinline__ float dot(const XU<F, PAIRED> &x, float acc) const {
        return unit_dot<F, PAIRED>(sl, bo, u, x, acc);
    }
};
// Paired Q4_0: the codes are held as signed bytes 16 (nib - 8) (the nibble in
// the byte's top half, XOR 0x80; krafla "Weight packing"), so a token's dot is
// 16 I with no activation code sum; dw / 16 and 16 I are exact, so each fold
// rounds the same product as unit_dot's.
template <> struct UnitW<F_Q4_0, true> {
    uint32_t c[16];   // block j: low nibbles of qs bytes 4k.. in c[8j + k], high nibbles in c[8j + 4 + k]
    float dw16[2];
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int) {
        const uint32_t *l32 = reinterpret_cast<const uint32_t *>(sl + bo);
        uint32_t v[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) v[k] = l32[k];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q0 = align_bytes(v[k + 1], v[k], 2), q1 = v[5 + k];
            c[k] = ((q0 << 4) & 0xf0f0f0f0u) ^ 0x80808080u;
            c[4 + k] = (q0 & 0xf0f0f0f0u) ^ 0x80808080u;
            c[8 + k] = ((q1 << 4) & 0xf0f0f0f0u) ^ 0x80808080u;
            c[12 + k] = (q1 & 0xf0f0f0f0u) ^ 0x80808080u;
        }
        dw16[0] = f16_bits_to_f32(v[0]) * 0.0625f;
        dw16[1] = f16_bits_to_f32(v[4] >> 16) * 0.0625f;
    }
    __device__ __forceinline__ float dot(const XU<F_Q4_0, true> &x, float acc) const {
        int s0 = 0, s1 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s0 = dot4((int)c[k], x.q[k], s0);
            s0 = dot4((int)c[4 + k], x.q[k + 4], s0);
            s1 = dot4((int)c[8 + k], x.q[8 + k], s1);
            s1 = dot4((int)c[12 + k], x.q[12 + k], s1);
        }
        acc = fmaf(dw16[0] * x.d[0], (float)s0, acc);
        return fmaf(dw16[1] * x.d[1], (float)s1, acc);
    }
};

template <> struct UnitW<F_Q8_0, true> {
    int c[16];        // block j's 32 codes in c[8j .. 8j + 7]
    float dw[2];
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int) {
        const uint32_t *l32 = reinterpret_cast<const uint32_t *>(sl + bo);
        uint32_t v[17];
#pragma unroll
        for (int k = 0; k < 17; ++k) v[k] = l32[k];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            c[k] = (int)align_bytes(v[k + 1], v[k], 2);
            c[8 + k] = (int)v[9 + k];
        }
        dw[0] = f16_bits_to_f32(v[0]);
        dw[1] = f16_bits_to_f32(v[8] >> 16);
    }
    __device__ __forceinline__ float dot(const XU<F_Q8_0, true> &x, float acc) const {
        int s0 = 0, s1 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s0 = dot4(c[k], x.q[k], s0);
            s1 = dot4(c[8 + k], x.q[8 + k], s1);
        }
        acc = fmaf(dw[0] * x.d[0], (float)s0, acc);
        return fmaf(dw[1] * x.d[1], (float)s1, acc);
    }
};

template <> struct UnitW<F_Q4_K, false> {
    int c[16];        // quarter u & 3 of the super-block: low nibbles in c[0..7], high in c[8..15]
    int sc0, m0, sc1, m1;
    float d, dmin;
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int u) {
        const int j = u & 3;
        const uint32_t *b32 = reinterpret_cast<const uint32_t *>(sl + bo);
        const uint32_t dd = b32[0], s0 = b32[1], s1 = b32[2], s2 = b32[3];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t q = b32[4 + 8 * j + k];
            c[k] = (int)(q & 0x0f0f0f0fu);
            c[8 + k] = (int)((q >> 4) & 0x0f0f0f0fu);
        }
        q4k_scale_min(s0, s1, s2, 2 * j, sc0, m0);
        q4k_scale_min(s0, s1, s2, 2 * j + 1, sc1, m1);
        d = f16_bits_to_f32(dd);
        dmin = f16_bits_to_f32(dd >> 16);
    }
    __device__ __forceinline__ float dot(const XU<F_Q4_K, false> &x, float acc) const {
        int lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lo = dot4(c[k], x.q[k], lo);
            hi = dot4(c[8 + k], x.q[8 + k], hi);
        }
        const int V = sc0 * lo + sc1 * hi;
        const int Mn = m0 * (x.bs[0] + x.bs[1]) + m1 * (x.bs[2] + x.bs[3]);
        acc = fmaf(d * x.d, (float)V, acc);
        return fmaf(-(dmin * x.d), (float)Mn, acc);
    }
};

template <> struct UnitW<F_Q6_K, false> {
    int c[16];        // group k's 16 six-bit codes in c[4k .. 4k + 3]
    int sc[4];
    float d;
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int u) {
        const int p = u & 3, h = p >> 1, g2 = p & 1;
        uint32_t ra[4], rb[4], qh[4], sw[2];
        lds_dwords<4>(sl, bo + 64 * h + 16 * g2, ra);
        lds_dwords<4>(sl, bo + 64 * h + 32 + 16 * g2, rb);
        lds_dwords<4>(sl, bo + 128 + 32 * h + 16 * g2, qh);
        lds_dwords<2>(sl, bo + 192 + 8 * h, sw);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t src = (k & 1) ? rb[e] : ra[e];
                const uint32_t lo4 = (k < 2) ? (src & 0x0f0f0f0fu) : ((src >> 4) & 0x0f0f0f0fu);
                const uint32_t hi2 = ((qh[e] >> (2 * k)) & 0x03030303u) << 4;
                c[4 * k + e] = (int)(lo4 | hi2);
            }
            sc[k] = __builtin_amdgcn_sbfe((int)sw[k >> 1], 8 * (2 * (k & 1) + g2), 8);
        }
        d = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(sl + bo + 208));
    }
    __device__ __forceinline__ float dot(const XU<F_Q6_K, false> &x, float acc) const {
        int V = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int s = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) s = dot4(c[4 * k + e], x.q[4 * k + e], s);
            V += sc[k] * (s - 32 * x.bs[k]);
        }
        return fmaf(d * x.d, (float)V, acc);
    }
};

template <> struct UnitW<F_Q2_K, false> {
    int c[16];        // the in-place bit pairs of unit_dot: group s in c[4s .. 4s + 3]
    int sc16[4], m[4];
    float d, dmin;
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int u) {
        const int p = u & 3, h = p >> 1, odd = p & 1;
        const uint32_t *b32 = reinterpret_cast<const uint32_t *>(sl + bo);
        const uint32_t sc01 = b32[2 * h], sc23 = b32[2 * h + 1], dd = b32[20];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q = b32[4 + 4 * p + k];
            c[k] = (int)(q & 0x03030303u);
            c[4 + k] = (int)(q & 0x0c0c0c0cu);
            c[8 + k] = (int)(q & 0x30303030u);
            c[12 + k] = (int)((q >> 2) & 0x30303030u);
        }
        const uint32_t o0 = 8u * (uint32_t)odd, o1 = o0 + 16u;
        // 16 V = 16 sc0 G0 + 4 sc1 G1 + sc2 G2 + sc3 G3 (see unit_dot)
        sc16[0] = 16 * (int)__builtin_amdgcn_ubfe(sc01, o0, 4);
        sc16[1] = 4 * (int)__builtin_amdgcn_ubfe(sc01, o1, 4);
        sc16[2] = (int)__builtin_amdgcn_ubfe(sc23, o0, 4);
        sc16[3] = (int)__builtin_amdgcn_ubfe(sc23, o1, 4);
        m[0] = (int)__builtin_amdgcn_ubfe(sc01, o0 + 4u, 4);
        m[1] = (int)__builtin_amdgcn_ubfe(sc01, o1 + 4u, 4);
        m[2] = (int)__builtin_amdgcn_ubfe(sc23, o0 + 4u, 4);
        m[3] = (int)__builtin_amdgcn_ubfe(sc23, o1 + 4u, 4);
        d = f16_bits_to_f32(dd);
        dmin = f16_bits_to_f32(dd >> 16);
    }
    __device__ __forceinline__ float dot(const XU<F_Q2_K, false> &x, float acc) const {
        int G0 = 0, G1 = 0, G2 = 0, G3 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            G0 = dot4(c[k], x.q[k], G0);
            G1 = dot4(c[4 + k], x.q[4 + k], G1);
            G2 = dot4(c[8 + k], x.q[8 + k], G2);
            G3 = dot4(c[12 + k], x.q[12 + k], G3);
        }
        const int V16 = sc16[0] * G0 + sc16[1] * G1 + sc16[2] * G2 + sc16[3] * G3;
        const int Mn = m[0] * x.bs[0] + m[1] * x.bs[1] + m[2] * x.bs[2] + m[3] * x.bs[3];
        acc = fmaf(d * x.d * 0.0625f, (float)V16, acc);
        return fmaf(-(dmin * x.d), (float)Mn, acc);
    }
};

// The 32-value formats with an offset or a fifth bit: the unit's blocks with
// their codes expanded to bytes (fifth bits included) and the d (m) dword.
template <int F, bool PAIRED> struct UnitW32 {
    static constexpr int P = Unit<F, PAIRED>::BPU;
    uint32_t c[P][8];   // block j: codes of values 4k.. in c[j][k], of 16 + 4k.. in c[j][4 + k]
    uint32_t dm[P];
    __device__ __forceinline__ void load(const uint8_t *sl, uint32_t bo, int) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            uint32_t qh, qs[4];
            block32_fields<F>(sl, bo + (uint32_t)j * FmtBytes<F>::BB, dm[j], qh, qs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t lo = qs[k] & 0x0f0f0f0fu, hi = (qs[k] >> 4) & 0x0f0f0f0fu;
                if constexpr (F != F_Q4_1) {
                    lo |= bits_to_bytes(__builtin_amdgcn_ubfe(qh, 4 * k, 4)) << 4;
                    hi |= bits_to_bytes(__builtin_amdgcn_ubfe(qh, 16 + 4 * k, 4)) << 4;
                }
                c[j][k] = lo;
                c[j][4 + k] = hi;
            }
        }
    }
    __device__ __forceinline__ float dot(const XU<F, PAIRED> &x, float acc) const {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            int I = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                I = dot4((int)c[j][k], x.q[8 * j + k], I);
                I = dot4((int)c[j][4 + k], x.q[8 * j + k + 4], I);
            }
            acc = block32_fold<F>(I, dm[j], x.d[j], x.sx8[j], acc);
        }
        return acc;
    }
};
template <> struct UnitW<F_Q4_1, true> : UnitW32<F_Q4_1, true> {};
template <> struct UnitW<F_Q4_1, false> : UnitW32<F_Q4_1, false> {};
template <> struct UnitW<F_Q5_0, true> : UnitW32<F_Q5_0, true> {};
template <> struct UnitW<F_Q5_0, false> : UnitW32<F_Q5_0, false> {};
template <> struct UnitW<F_Q5_1, true> : UnitW32<F_Q5_1, true> {};
template <> struct UnitW<F_Q5_1, false> : UnitW32<F_Q5_1, false> {};

// --- row-sum reduction across the wave -----------------------------------------
__device__ __forceinline__ uint32_t f_as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u_as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

template <int BIT> struct LaneXchg;       // DPP control pairing lanes across lane bit BIT
template <> struct LaneXchg<8> { static constexpr int CTRL = kDppRowRor8; };        // l ^ 8
template <> struct LaneXchg<4> { static constexpr int CTRL = kDppHalfRowMirror; };  // l ^ 7 within 8
template <> struct LaneXchg<2> { static constexpr int CTRL = kDppQuadXor2; };       // l ^ 2
template <> struct LaneXchg<1> { static constexpr int CTRL = kDppQuadXor1; };       // l ^ 1

// Halving step at lane bit BIT: a lane with the bit clear keeps `lo` plus its
// partner's `lo`, a lane with the bit set keeps `hi` plus its partner's `hi`
// (the partner is a lane with the opposite bit).  For bits 5 and 4 the
// permlane swap of (lo, hi) hands every lane exactly those two values.
template <int BIT>
__device__ __forceinline__ float xsum_half(float lo, float hi, int lane) {
    if constexpr (BIT == 32 || BIT == 16) {
        const auto r = (BIT == 32) ? __builtin_amdgcn_permlane32_swap(f_as_u(lo), f_as_u(hi), false, false)
                                   : __builtin_amdgcn_permlane16_swap(f_as_u(lo), f_as_u(hi), false, false);
        return u_as_f(r[0]) + u_as_f(r[1]);
    } else {
        const bool h = (lane & BIT) != 0;
        const float keep = h ? hi : lo, send = h ? lo : hi;
        return keep + dpp_f32<LaneXchg<BIT>::CTRL>(send);
    }
}

// Plain step at lane bit BIT: the sum of a lane's value and its partner's.
template <int BIT>
__device__ __forceinline__ float xsum(float a) {
    if constexpr (BIT == 32 || BIT == 16) {
        const auto r = (BIT == 32) ? __builtin_amdgcn_permlane32_swap(f_as_u(a), f_as_u(a), false, false)
                                   : __builtin_amdgcn_permlane16_swap(f_as_u(a), f_as_u(a), false, false);
        return u_as_f(r[0]) + u_as_f(r[1]);
    } else {
        return a + dpp_f32<LaneXchg<BIT>::CTRL>(a);
    }
}

// Transposing butterfly over GP row sums (GP a power of two): afterwards lane
// l holds the full sum of row l / (64 / GP).
template <int BIT, int CNT, int GP>
__device__ __forceinline__ void row_butterfly(float (&acc)[GP], int lane) {
    if constexpr (BIT >= 1) {
        if constexpr (CNT > 1) {
#pragma unroll
            for (int j = 0; j < CNT / 2; ++j) acc[j] = xsum_half<BIT>(acc[j], acc[j + CNT / 2], lane);
            row_butterfly<BIT / 2, CNT / 2, GP>(acc, lane);
        } else {
            acc[0] = xsum<BIT>(acc[0]);
            row_butterfly<BIT / 2, 1, GP>(acc, lane);
        }
    }
}

template <int G> struct Pow2Ceil { static constexpr int V = G <= 1 ? 1 : 2 * Pow2Ceil<(G + 1) / 2>::V; };
template <> struct Pow2Ceil<1> { static constexpr int V = 1; };

// --- the kernel ---------------------------------------------------------------
// Dynamic LDS: [TT activation segments of xs bytes][NW wave slices of ss bytes].
// Tokens: grid row j takes tokens TT j .. TT j + TT - 1 (activation rows xrow
// bytes apart; tokens past M re-read the last row and store nothing) and
// writes their output rows.  TT = 1 is the decode step; TT > 1 serves a few
// tokens at once: each wave's weight slice is streamed once and dotted with
// every token's activation (M tokens cost ceil(M / TT) weight passes).
// XF32: `xin` is f32 activations and xq_out (may be null) receives the Q8_0
// rows; otherwise `xin` is Q8_0 / Q8_K activation blocks.
template <int F, bool PAIRED, int G, int MAXU, bool XF32, int NW, int TT>
__global__ __launch_bounds__(64 * NW) void k_matvec(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xin,
                                                float *__restrict__ y, int N, int nb, int64_t xrow, int xs,
                                                int ss, uint8_t *__restrict__ xq_out, int M) {
    using FB = FmtBytes<F>;
    using UT = Unit<F, PAIRED>;
    static_assert(!XF32 || TT == 1, "the fused quantizer serves one token");
    extern __shared__ uint4 lds_dyn[];
    constexpr int SEGU = kWave * MAXU;                 // units per segment
    constexpr int NT = kWave * NW;                     // threads per workgroup
    // 16-byte f32 activation pieces per thread and segment (XF32): Q8_0,
    // 8 per block over the workgroup; Q8_K, one super-block per wave, 4
    // values per lane
    constexpr int XL = !XF32 ? 1
                       : kIsK<F> ? (SEGU / UT::UPB + NW - 1) / NW
                                 : (8 * MAXU * UT::BPU + NW - 1) / NW;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int tok0 = (int)blockIdx.y * TT;
    const int64_t xtok = (int64_t)tok0 * xrow;         // byte offset of the first token's activation row
    y += (int64_t)tok0 * N;
    const int64_t row0 = ((int64_t)blockIdx.x * NW + wave) * G;
    const int nrows = (int)max((int64_t)0, min((int64_t)G, (int64_t)N - row0));
    const int64_t RB = (int64_t)nb * FB::BB;
    const int nu = (nb / UT::BPU) * UT::UPB;           // units per row
    uint4 *xlds = lds_dyn;
    uint4 *slice = lds_dyn + TT * (xs / 16) + wave * (ss / 16);
    const uint8_t *xl8 = reinterpret_cast<const uint8_t *>(xlds);
    const uint8_t *sl8 = reinterpret_cast<const uint8_t *>(slice);

    constexpr int GP = Pow2Ceil<G>::V;                 // row sums, padded to a power of two
    static_assert((TT & (TT - 1)) == 0 && GP * TT <= kWave, "row x token sums: a power of two, at most 64");
    float acc[GP * TT];                                // sum of row r, token t at r TT + t
#pragma unroll
    for (int r = 0; r < GP * TT; ++r) acc[r] = 0.0f;

    for (int u0 = 0; u0 < nu; u0 += SEGU) {
        const int u1 = min(nu, u0 + SEGU);
        const int b0 = u0 / UT::UPB * UT::BPU, b1 = u1 / UT::UPB * UT::BPU;   // blocks of the segment
        // activation of the segment (all waves of the workgroup share it)
        uint32_t xoff = 0, xofft[TT];
        const int nch = 8 * (b1 - b0);                 // its 16-byte f32 pieces (XF32)
        v4f xv[XL];
        if constexpr (XF32 && kIsK<F>) {
            // super-block j of the segment is wave j % NW's, i = j / NW
            const uint8_t *xseg = xin + xtok + (int64_t)b0 * 1024;
#pragma unroll
            for (int i = 0; i < XL; ++i)
                xv[i] = global_load16_async(xseg, 1024u * (uint32_t)min(wave + NW * i, b1 - b0 - 1) + 16u * lane);
        } else if constexpr (XF32) {
            const uint8_t *xseg = xin + xtok + (int64_t)b0 * 128;
#pragma unroll
            for (int i = 0; i < XL; ++i)
                xv[i] = global_load16_async(xseg, 16u * (uint32_t)min((int)threadIdx.x + NT * i, nch - 1));
        } else if constexpr (TT == 1) {
            const int64_t xlo = xtok + (int64_t)b0 * FB::XB, xhi = xtok + (int64_t)b1 * FB::XB;
            xoff = (uint32_t)(xlo & 15);
            dma_span(xin, xlo, xhi, xlds, lane, wave, NW);
        } else {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const int64_t xr = (int64_t)min(tok0 + t, M - 1) * xrow;
                const int64_t xlo = xr + (int64_t)b0 * FB::XB, xhi = xr + (int64_t)b1 * FB::XB;
                xofft[t] = (uint32_t)(xlo & 15);
                dma_span(xin, xlo, xhi, xlds + t * (xs / 16), lane, wave, NW);
            }
        }
        // this wave's weight span
        int wissued = 0;
        int64_t A = 0;
        if (nrows > 0) {
            const int64_t lo = row0 * RB + (int64_t)b0 * FB::BB;
            const int64_t hi = (row0 + nrows - 1) * RB + (int64_t)b1 * FB::BB;
            A = lo & ~(int64_t)15;
            // one token: every weight byte is read once per launch
            wissued = dma_span<TT == 1>(w, lo, hi, slice, lane, 0, 1);
        }
        wait_vmcnt(wissued);                           // this wave's activation loads have landed
        if constexpr (XF32 && kIsK<F>) {
            // the segment's Q8_K super-blocks, laid out in LDS as in the
            // activation row (292 bytes each from offset 0), as the plain
            // kernel's copy lands them
            uint8_t *xw8 = reinterpret_cast<uint8_t *>(xlds);
            uint8_t *xq_row = (xq_out != nullptr && blockIdx.x == 0)
                                  ? xq_out + (int64_t)blockIdx.y * nb * kQ8KBytes + (int64_t)b0 * kQ8KBytes
                                  : nullptr;
#pragma unroll
            for (int i = 0; i < XL; ++i) {
                pin_after_wait(xv[i]);
                const int j = wave + NW * i;
                int gsum;
                float d;
                const uint32_t packed = q8_k_wave(make_float4(xv[i][0], xv[i][1], xv[i][2], xv[i][3]), gsum, d);
                if (j < b1 - b0) {
                    store_q8_k_lane(xw8 + j * kQ8KBytes, lane, packed, gsum, d);
                    if (xq_row != nullptr) store_q8_k_lane(xq_row + (int64_t)j * kQ8KBytes, lane, packed, gsum, d);
                }
            }
            wait_lds_reads();                          // the codes are in LDS
        } else if constexpr (XF32) {
            constexpr int US = XLayout<UT::BPU>::US;
            uint8_t *xw8 = reinterpret_cast<uint8_t *>(xlds);
            uint8_t *xq_row = (xq_out != nullptr && blockIdx.x == 0)
                                  ? xq_out + (int64_t)blockIdx.y * nb * kQ80Bytes + (int64_t)b0 * kQ80Bytes
                                  : nullptr;
#pragma unroll
            for (int i = 0; i < XL; ++i) {
                pin_after_wait(xv[i]);
                const int c = (int)threadIdx.x + NT * i;    // piece c = part c%8 of segment block c/8
                float d;
                const uint32_t packed = q8_0_part(make_float4(xv[i][0], xv[i][1], xv[i][2], xv[i][3]), d);
                if (c < nch) {
                    const int jb = c >> 3, part = c & 7;
                    uint8_t *ub = xw8 + US * (jb / UT::BPU);
                    const int j = jb % UT::BPU;
                    *reinterpret_cast<uint32_t *>(ub + 32 * j + 4 * part) = packed;
                    if (part == 0)
                        reinterpret_cast<float *>(ub + 32 * UT::BPU)[j] = f16_bits_to_f32(f32_to_f16_bits(d));
                    if (xq_row != nullptr) store_q8_0_part(xq_row + (int64_t)jb * kQ80Bytes, part, packed, d);
                }
            }
            wait_lds_reads();                          // the codes are in LDS
        }
        __builtin_amdgcn_s_barrier();                  // ... and every other wave's
        if constexpr (TT > 1) {
            // every token against the whole slice: wait for it, take each
            // row's weight unit once, then one token's activation registers
            // at a time
            static_assert(MAXU == 1, "the few-token path runs one unit per lane and segment");
            wait_vmcnt(0);
            if (nrows > 0) {
                const int ul = lane;                   // unit within the segment
                const bool live = ul < u1 - u0;
                UnitW<F, PAIRED> wu[G];
#pragma unroll
                for (int r = 0; r < G; ++r) {
                    const uint32_t ro = (uint32_t)((min(row0 + r, row0 + nrows - 1)) * RB + (int64_t)b0 * FB::BB - A);
                    wu[r].load(sl8, ro + (uint32_t)(min(ul, u1 - u0 - 1) / UT::UPB * UT::BPU) * FB::BB, u0 + ul);
                }
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    XU<F, PAIRED> xu;
                    load_xu<F, PAIRED>(xl8 + t * xs, xofft[t], min(ul, u1 - u0 - 1), xu);
#pragma unroll
                    for (int r = 0; r < G; ++r)
                        if (r < nrows && live) acc[r * TT + t] = wu[r].dot(xu, acc[r * TT + t]);
                }
            }
            if (u1 < nu) {
                wait_lds_reads();
                __builtin_amdgcn_s_barrier();
            }
            continue;
        }
        XU<F, PAIRED> xu[MAXU];
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            const int ul = min(lane + kWave * i, u1 - u0 - 1);
            if constexpr (XF32 && !kIsK<F>)
                load_xu_q<F, PAIRED>(xl8, ul, xu[i]);
            else
                load_xu<F, PAIRED>(xl8, xoff, ul, xu[i]);
        }
        if (nrows > 0) {
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (r < nrows) {
                    const uint32_t ro = (uint32_t)((row0 + r) * RB + (int64_t)b0 * FB::BB - A);
                    // row r's bytes end in chunk group kr; the groups after it may
                    // still be in flight while this row is computed
                    const int64_t rend = (row0 + r) * RB + (int64_t)b1 * FB::BB;
                    const int kr = (int)((rend - 1 - A) >> 10);
                    wait_vmcnt(wissued - 1 - kr);
#pragma unroll
                    for (int i = 0; i < MAXU; ++i) {
                        const int ul = lane + kWave * i;            // unit within the segment
                        if (ul < u1 - u0) {
                            const uint32_t bo = ro + (uint32_t)(ul / UT::UPB * UT::BPU) * FB::BB;
                            acc[r] = unit_dot<F, PAIRED>(sl8, bo, u0 + ul, xu[i], acc[r]);
                        }
                    }
                }
            }
        }
        wait_vmcnt(0);
        if (u1 < nu) {                                 // the LDS is refilled for the next segment
            wait_lds_reads();
            __builtin_amdgcn_s_barrier();
        }
    }
    if (nrows == 0) return;

    row_butterfly<32, GP * TT, GP * TT>(acc, lane);
    constexpr int LPR = kWave / (GP * TT);             // lanes holding copies of one sum
    const int v = lane / LPR, r = v / TT, t = v % TT;
    if (lane % LPR == 0 && r < nrows && tok0 + t < M) y[(int64_t)t * N + row0 + r] = acc[0];
}

// --- launch configuration -----------------------------------------------------
// The launchers choose the rows per wave so that a launch keeps at least this
// many waves (8 per CU of MI355X) where the matrix has the rows.
constexpr int64_t kMinDecodeWaves = 2048;

template <int F, bool PAIRED, int G, int MAXU, bool XF32, int NW = 4, int TT = 1>
static hipError_t launch_mv(const void *w, const void *xin, uint8_t *xq_out, float *y, int M, int N, int nb,
                            hipStream_t st) {
    using FB = FmtBytes<F>;
    using UT = Unit<F, PAIRED>;
    const int nu = (nb / UT::BPU) * UT::UPB;
    const int segu = min(nu, kWave * MAXU);
    const int segb = (segu + UT::UPB - 1) / UT::UPB * UT::BPU;
    const int64_t span = (G == 1) ? (int64_t)segb * FB::BB : (int64_t)G * nb * FB::BB;
    // whole 1 KB chunk groups (dma_span may fill a full last group) after up to
    // 15 bytes of misalignment at each end
    const int ss = (int)(((span + 32 + 1023) / 1024) * 1024);
    const int xs = (XF32 && !kIsK<F>) ? (XLayout<UT::BPU>::US * segu + 15) / 16 * 16
                                      : (int)((((int64_t)segb * FB::XB + 32 + 1023) / 1024) * 1024);
    const int64_t waves = ((int64_t)N + G - 1) / G;
    const int64_t grid = (waves + NW - 1) / NW;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xin);
    int64_t xrow = XF32 ? (int64_t)nb * (kIsK<F> ? 1024 : 128) : (int64_t)nb * FB::XB;   // f32: 4 bytes a value
    const auto kern = k_matvec<F, PAIRED, G, MAXU, XF32, NW, TT>;
    const size_t lds = (size_t)TT * xs + (size_t)NW * ss;
    static int lds_ok[kLdsDevices] = {};
    const hipError_t e = allow_dynamic_lds((const void *)kern, lds, lds_ok);
    if (e != hipSuccess) return e;
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&N, (void *)&nb,
                    (void *)&xrow, (void *)&xs, (void *)&ss, (void *)&xq_out, (void *)&M};
    const unsigned gy = (unsigned)((M + TT - 1) / TT);
    return hipLaunchKernel((const void *)kern, dim3((unsigned)grid, gy), dim3(kWave * NW), args, lds, st);
}

}  // namespace qmm
