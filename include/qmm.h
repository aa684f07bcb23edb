/*
 * qmm -- block-quantized weight x Q8_0 / Q8_K activation products on MI355X
 * (gfx950).  C ABI of libqmm.so.
 *
 * The method (pages: "10 . CPU matmul: quantized weights x Q8_0 activations"
 * (minfer), "ggml Q4_0 vec_dot Walkthrough", krafla "Architecture", "kvad --
 * the same ideas, at scale"): weights stay in their GGUF block layouts;
 * activations are quantized on the fly to Q8_0 (per 32 values) or Q8_K (per
 * 256); each output is a sum over blocks of an exact int32 block dot product
 * scaled by the two block scales, accumulated in f32.
 *
 * Byte layouts (little-endian; "f16" is IEEE binary16):
 *   Q8_0  34 B / 32 values : f16 d @0, int8 q[32] @2.          value = d*q
 *   Q4_0  18 B / 32 values : f16 d @0, uint8 qs[16] @2; byte j holds element
 *                            j in its low nibble and j+16 in its high nibble.
 *                                                               value = d*(nib-8)
 *   Q2_K  84 B / 256 values: uint8 scales[16] @0 (low nibble sc, high nibble
 *                            m, one byte per group of 16), uint8 qs[64] @16,
 *                            f16 d @80, f16 dmin @82.   value = d*sc*q - dmin*m
 *                            qs byte 32h+l holds, at bit shift 2s, the 2-bit
 *                            code of value 128h+32s+l (h<2, s<4, l<32).
 *   Q8_K 292 B / 256 values: f32 d @0, int8 q[256] @4, int16 bsums[16] @260
 *                            (bsums[g] = sum of codes 16g..16g+15).
 *   Q4_K 144 B / 256 values: f16 d @0, f16 dmin @2, 12 B of 6-bit scales and
 *                            mins @4, uint8 qs[128] @16; byte l of 32-byte
 *                            chunk j holds value 64j+l (low nibble) and
 *                            64j+32+l (high nibble); sub-block s = i/32 has
 *                            scale sc_s and min m_s: for s < 4 sc = b[s] & 63,
 *                            m = b[s+4] & 63; for s >= 4 sc = (b[s+4] & 15) |
 *                            (b[s-4] >> 6) << 4, m = (b[s+4] >> 4) |
 *                            (b[s] >> 6) << 4 (b = the 12 bytes).
 *                                                  value = d*sc_s*q - dmin*m_s
 *   Q6_K 210 B / 256 values: ql[128] @0 (low 4 bits), qh[64] @128 (high 2
 *                            bits), int8 scales[16] @192, f16 d @208; value
 *                            i (h = i/128, k = (i%128)/32, l = i%32): low bits
 *                            in ql[64h + l + 32(k&1)] (low nibble for k < 2,
 *                            high for k >= 2), high bits at bit 2k of
 *                            qh[32h + l].        value = d*scales[i/16]*(q-32)
 *   Q4_1  20 B / 32 values : f16 d @0, f16 m @2, uint8 qs[16] @4   value = d*q + m
 *   Q5_0  22 B / 32 values : f16 d @0, uint32 qh @2, uint8 qs[16] @6
 *                                                          value = d*(q-16)
 *   Q5_1  24 B / 32 values : f16 d @0, f16 m @2, uint32 qh @4, uint8 qs[16] @8
 *                                                          value = d*q + m
 *                            (qs as Q4_0; bit j of qh is value j's fifth bit)
 *   (The Q4_K scale packing, the Q6_K layout and the Q4_1 / Q5 field and bit
 *   order are GGUF's; the pages give the block sizes, Q4_K's field and chunk
 *   order and its two-term dot, and the d*q + m form of the _1 formats.)
 * A matrix of R rows and K columns in format F is R*K/blk(F) blocks, row-major
 * (row r starts at byte r*(K/blk)*bytes(F)), with no padding.
 *
 * Conventions for every entry point below:
 *   - All data pointers are DEVICE pointers on the current HIP device and must
 *     be 16-byte aligned (QMM_E_ALIGN otherwise).  The caller owns every
 *     buffer; the library never allocates, frees, synchronizes or keeps state
 *     between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; the return value reports argument and launch
 *     errors only.
 *   - Outputs must not alias inputs.  Outputs are overwritten, never
 *     accumulated into.
 *   - Kernels may read up to 15 bytes past the end of an input buffer (never
 *     past the end of the 16-byte-aligned granule that holds its last byte, so
 *     never into another page); those bytes do not affect any result.
 *   - Calls are thread-safe.  No entry point aborts the process.
 *   - Sizes: M, N >= 1, K >= one block, K a multiple of the block length of
 *     the format (32, or 256 for Q8_K and the K-quants), every dimension < 2^31 and every
 *     buffer < 2^40 bytes; QMM_E_SHAPE otherwise.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMM_OK = 0,
    QMM_E_SHAPE = 1,  /* bad M, N or K, or a byte size that overflows   */
    QMM_E_NULL = 2,   /* a required pointer is NULL                      */
    QMM_E_ALIGN = 3,  /* a pointer is not 16-byte aligned                */
    QMM_E_DEVICE = 4, /* no current device, or it is not gfx950          */
    QMM_E_LAUNCH = 5  /* the HIP runtime refused a kernel launch         */
} qmm_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *qmm_status_string(qmm_status s);

/* Version of this ABI (incremented on any incompatible change). */
int qmm_abi_version(void);

/* ---- activation quantizers ------------------------------------------------ */

/* Q8_0 quantization of M rows of K f32 values (minfer "The activation
 * quantizers", quantize_avx2; ggml section 1.1; krafla "Numerics").  For each
 * block of 32: amax = max|x|, d = amax/127 (f32, stored as f16 rounded to
 * nearest even), id = amax ? 127/amax : 0, q = round-half-even(x*id).
 * Bit-exact: every step is one correctly rounded f32 operation.
 *   x  : f32 [M][K], read only.
 *   xq : Q8_0 [M][K/32] blocks, M*K/32*34 bytes, written.
 * Also the quantizer of Q8_0 weight matrices (same rule, rows = N). */
qmm_status qmm_quantize_q8_0(const float *x, void *xq, int64_t M, int64_t K, void *stream);

/* Q8_K quantization (minfer quantize_row_q8_k_buf and its three details):
 * per 256 values amax, d = amax/127 stored as f32, q = saturate[-128,127]
 * (round-half-even(x*id)), bsums from the saturated codes.
 *   x  : f32 [M][K], K % 256 == 0.   xq : Q8_K [M][K/256] blocks (292 B). */
qmm_status qmm_quantize_q8_k(const float *x, void *xq, int64_t M, int64_t K, void *stream);

/* ---- weight quantizers (prepare weight matrices; not on the product path) -- */

/* Q4_0 quantization of N rows of K f32 weights (ggml section 1.1 prose;
 * kvad "The scale that wasted a code"): per 32, the value of largest
 * magnitude (first on ties) keeps its sign as max, d = max/-8 (d = 0 for an
 * all-zero block), code = clamp(round-half-even(x/d)+8, 0, 15), f16 d.
 *   w : f32 [N][K].   wq : Q4_0 [N][K/32] blocks (18 B). */
qmm_status qmm_quantize_q4_0(const float *w, void *wq, int64_t N, int64_t K, void *stream);

/* Q2_K quantization of N rows of K f32 weights, K % 256 == 0.  The pages
 * define the format (ggml section 1.2) but no quantizer; the rule is: per
 * group of 16, lo = min(0, min x), hi = max x, s = (hi-lo)/3, mn = -lo;
 * d = max s / 15, dmin = max mn / 15 (f16); sc = clamp(rne(s/d),0,15),
 * m = clamp(rne(mn/dmin),0,15); q = clamp(rne((x + dmin*m)/(d*sc)),0,3),
 * with 0 for a zero divisor (d and dmin here are the stored f16 values).
 *   w : f32 [N][K].   wq : Q2_K [N][K/256] blocks (84 B). */
qmm_status qmm_quantize_q2_k(const float *w, void *wq, int64_t N, int64_t K, void *stream);

/* Q4_K and Q6_K quantization of N rows of K f32 weights, K % 256 == 0 (test
 * and benchmark data; the pages give no quantizer).  Q4_K: Q2_K's rule with
 * 15 levels, s = (hi-lo)/15, and 6-bit sc, m: d = max s / 63, dmin = max mn /
 * 63, sc = clamp(rne(s/d), 0, 63), m = clamp(rne(mn/dmin), 0, 63),
 * q = clamp(rne((x + dmin*m)/(d*sc)), 0, 15), per sub-block of 32.  Q6_K, per
 * group of 16: the value of largest magnitude (first on ties) mx gives
 * s = mx / -32; d = max |s| / 127; sc = clamp(rne(s/d), -128, 127);
 * q = clamp(rne(x/(d*sc)) + 32, 0, 63), 32 for a zero divisor.  d, dmin are
 * the stored f16 values in every step after they are stored.
 *   w : f32 [N][K].   wq : Q4_K (144 B) / Q6_K (210 B) blocks, N*K/256 of them. */
qmm_status qmm_quantize_q4_k(const float *w, void *wq, int64_t N, int64_t K, void *stream);

/* Q4_1 / Q5_0 / Q5_1 quantization of N rows of K f32 weights (test and
 * benchmark data; the pages give no quantizer).  Q4_1 / Q5_1, per block of 32:
 * lo = min x, hi = max x (a zero of either sign as +0), d = (hi - lo)/L with
 * L = 15 / 31, m = lo, q = clamp(rne((x - m)/d), 0, L) (0 for d = 0); Q5_0:
 * Q4_0's rule with 32 levels, d = max/-16, q = clamp(rne(x/d) + 16, 0, 31)
 * (16 for d = 0); d and m are the stored f16 values after they are stored. */
qmm_status qmm_quantize_q4_1(const float *w, void *wq, int64_t N, int64_t K, void *stream);
qmm_status qmm_quantize_q5_0(const float *w, void *wq, int64_t N, int64_t K, void *stream);
qmm_status qmm_quantize_q5_1(const float *w, void *wq, int64_t N, int64_t K, void *stream);
qmm_status qmm_quantize_q6_k(const float *w, void *wq, int64_t N, int64_t K, void *stream);

/* ---- products ----------------------------------------------------------------
 * y[t][n] = sum over blocks b of d_w[n,b] * d_x[t,b] * I_b[t,n], where I_b is
 * the exact int32 dot product of the block's codes (minfer mm_rows and the
 * scalar kernel; ggml section 2; krafla "Data flow for one token").  Integer
 * block sums are exact; only the f32 accumulation order is free, so results
 * agree with an exact evaluation within 1e-5 of sum |d_w d_x w_j q_j| per
 * output (krafla "Numerics").  Output is token-major [M][N] f32 (minfer
 * "Pitfalls": out[t*od + o]).
 * Pairing (minfer "Two activation formats, one pairing rule"): the 32-value
 * formats (Q4_0, Q8_0, Q4_1, Q5_0, Q5_1) take Q8_0 activations; the K-quants
 * (Q2_K, Q4_K, Q6_K) take Q8_K activations.  The _1 formats add the offset
 * term m*dx*sum q per block.  K-quant dots (minfer "The payoff: a K-quant dot kernel,
 * walked"): per super-block d*d8*sum_s sc_s*sum q x, minus dmin*d8*sum_s m_s *
 * (the bsums of s) for the formats with mins; Q6_K: d*d8*sum_g sc_g *
 * sum (q-32) x. */

/* Decode matvec, one token (M = 1).
 *   w  : N rows of K/32 weight blocks.   xq : one row of Q8_0 (or Q8_K) blocks.
 *   y  : f32 [N], written. */
qmm_status qmm_matvec_q8_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q4_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q4_1(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q5_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q5_1(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q2_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q4_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream);
qmm_status qmm_matvec_q6_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream);

/* Decode matvec with the activation quantization fused into the same launch
 * (minfer section 3.3, "Design choices", on sibling products sharing one
 * quantized row; krafla "Data flow for one token"): every workgroup quantizes
 * the row it needs into LDS, so a decode step is one launch.  The result is the same as qmm_quantize_q8_0
 * of x followed by qmm_matvec_q4_0 / qmm_matvec_q8_0 on its output, bit for
 * bit.  For long rows (more than 4096 values, or more than 2048 with an odd
 * block count) and a non-NULL xq, the library runs exactly those two launches
 * instead, because re-quantizing a long row in every workgroup costs more
 * than the second launch; with xq NULL it always runs the single launch.
 *   w  : N rows of K/32 Q4_0 (or Q8_0) weight blocks.
 *   x  : f32 [K], read only.
 *   xq : NULL, or a Q8_0 row of K/32 blocks (K/32*34 bytes, 16-byte aligned)
 *        that receives the quantized activation, bit-identical to
 *        qmm_quantize_q8_0 -- for a caller that applies several weight
 *        matrices to the same activation (QKV, gate and up) and runs the
 *        others with qmm_matvec_* on it.
 *   y  : f32 [N], written. */
qmm_status qmm_quantize_matvec_q4_0(const void *w, const float *x, void *xq, float *y, int64_t N, int64_t K,
                                    void *stream);
qmm_status qmm_quantize_matvec_q8_0(const void *w, const float *x, void *xq, float *y, int64_t N, int64_t K,
                                    void *stream);
/* The same fused decode step for the K-quant weights (minfer "The payoff: a
 * K-quant dot kernel, walked": they pair with Q8_K activations): every
 * workgroup quantizes the row to Q8_K super-blocks in LDS with the arithmetic
 * of qmm_quantize_q8_k, so the result equals qmm_quantize_q8_k followed by
 * qmm_matvec_q2_k / _q4_k / _q6_k bit for bit; rows of more than 4096 values
 * with a non-NULL xq8k run those two launches.
 *   w    : N rows of K/256 Q2_K, Q4_K or Q6_K super-blocks (K % 256 == 0).
 *   x    : f32 [K], read only.
 *   xq8k : NULL, or a Q8_K row of K/256 blocks (K/256*292 bytes, 16-byte
 *          aligned) that receives the quantized activation.
 *   y    : f32 [N], written. */
qmm_status qmm_quantize_matvec_q2_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream);
qmm_status qmm_quantize_matvec_q4_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream);
qmm_status qmm_quantize_matvec_q6_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream);

/* Matmul, M tokens (prefill, or a few tokens at once).
 *   w  : N rows of weight blocks.   xq : M rows of Q8_0 (Q8_K) blocks.
 *   y  : f32 [M][N], written.
 * Up to 8 tokens (Q4_0; 2 for Q2_K, 4 for the other formats) run on the
 * decode matvec kernel, which streams each weight slice once per group of
 * 2, 4 or 8 tokens (one token: the decode launch itself); more tokens run
 * on the MFMA kernels below (32-token tiles up to 128 tokens for Q2_K and
 * Q4_K and up to 64 for the other formats, 128-token tiles beyond).  Results
 * agree within the same tolerance either way (they are not bitwise
 * identical: the two paths sum the blocks in different orders).
 * An MFMA launch of at most 256 output tiles (32 or 128 tokens x 128 or 256
 * weight rows) splits K in two: y is first zeroed on the stream, then the two
 * halves of each output are added into it with f32 atomic adds (device
 * memory from hipMalloc; two addends give the same bits in either order, so
 * repeated calls are bitwise reproducible; a launch of fewer than 128
 * tiles first sums each half from two quarters, in a fixed order).  The
 * 32-token launches of fewer than 128 such tiles (every format but Q6_K)
 * instead sum all of K inside each workgroup (four quarters, in a fixed
 * order) and write y with plain stores.
 * The 32-value formats (Q4_0, Q8_0, Q4_1, Q5_0, Q5_1) run on int8 MFMA (4-bit
 * codes enter as 16 * (q - 8), 5-bit codes as 8 * (q - 16); the offset term
 * of Q4_1 / Q5_1, m * dx * sum x per block, runs on an f32 MFMA) and also
 * return QMM_E_SHAPE when 128 rows of Q8_0 activations (128 * K/32 * 34
 * bytes) exceed 2^31 - 1 bytes, i.e. K > 15,790,304.  qmm_matmul_q2_k runs on int8 MFMA
 * (the group scales folded into the codes, one scale fold per 256 values)
 * plus an f16 MFMA for the min term; qmm_matmul_q4_k runs one int8 MFMA tile
 * per 32-value sub-block on the 4-bit codes, applies the 6-bit sub-block
 * scales in int32 and takes the min term from the same f16 MFMA over the
 * activation's block sums; qmm_matmul_q6_k runs one int8 MFMA tile per
 * 16-value group on the unsigned 6-bit codes, applies the signed group scales
 * in int32 and takes the offset of 32 from an f16 MFMA over the block sums.
 * All three return QMM_E_SHAPE when 128 rows of Q8_K activations
 * (128 * K/256 * 292 bytes) exceed 2^31 - 1 bytes. */
qmm_status qmm_matmul_q4_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q8_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q4_1(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q5_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q5_1(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q2_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q4_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);
qmm_status qmm_matmul_q6_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream);

/* ---- embedding rows ---------------------------------------------------------
 * out[t][:] = the decoded row ids[t] of the quantized table w (N rows of K
 * values), as f32: minfer "The embedding matmul" (a lookup, not a product: the
 * token's row is dequantized block by block; one row getter for every backend
 * keeps the embeddings byte-for-byte identical).  Every value is the exactly
 * decoded one rounded once to f32 (Q4_0, Q8_0, Q6_K values are exact in f32;
 * Q2_K and Q4_K subtract two exact products).
 *   w   : N rows of blocks in the entry point's format.
 *   ids : int32 [n_ids], device memory; an id outside [0, N) yields a row of
 *         quiet NaNs (no read outside the table).
 *   out : f32 [n_ids][K], written. */
qmm_status qmm_get_rows_q4_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q8_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q2_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q4_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q6_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q4_1(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q5_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);
qmm_status qmm_get_rows_q5_1(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
