// Prefill matmul, Q2_K weights x Q8_K activations, on MFMA.
//
// Per super-block s of 256 values (minfer "The payoff: a K-quant dot kernel,
// walked": a value term and a min term):
//   Y[m][n] += d8[m,s] * ( d[n,s] * V[m,n,s]  -  dmin[n,s] * Mn[m,n,s] )
//   V  = sum_i (sc_g(i) q_i) x_i       (g = i/16: the group scale folded into the code)
//   Mn = sum_g m_g bsum_g
// sc_g q_i <= 15 * 3 = 45 is an exact int8, so V is a 256-deep int8 contraction:
// eight v_mfma_i32_32x32x32_i8 accumulating in int32, and the f32 scale fold
// happens once per 256 values, not once per 32 as for Q4_0.  Mn is a 16-deep
// contraction of bsums (|b| <= 2048, exact in f16) with mins (<= 15): one
// v_mfma_f32_32x32x16_f16, exact (|Mn| < 2^24).
//
// Workgroup tile 128 tokens x 128 weight rows, 4 waves of 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32), one workgroup per CU (two stage buffers of 52 KB).
// Staging: a stage is one super-block.  Each activation row's 292 bytes
// arrive as 19 chunks of 16 bytes (LDS row: codes 0..255 at 0, bsums at 256,
// the chunk holding d8 at 288; 304-byte stride, so the 32 rows of a 16-byte
// read fall in distinct banks) and each weight row's 84 bytes as 7 chunks
// (scales at 0, qs at 16, the chunk holding d and dmin at 80, one spare;
// 112-byte stride).  Consecutive lanes take consecutive chunks of a row, so
// every load is coalesced; each lane's global offsets are fixed for the
// whole K loop and the stage position rides in the scalar offset.  The DMA of
// stage s+1 runs while stage s is computed.
//
// Operands.  K-step t of a super-block covers values 32t .. 32t+31, which are
// the 2-bit fields at shift 2(t%4) of qs bytes 32(t/4) .. +31 (the qs bit
// order of Q2_K), groups 2t and 2t+1.  Lane half h feeds values 32t + 16h ..
// +15 of both operands (the same values, so the pairing agrees): the A
// operand is 16 activation codes read straight from LDS; the B operand takes
// the 16 qs bytes once per four K-steps and turns each dword into sc*q bytes
// with a shift, a mask and a v_perm from the table [0, sc, 2sc, 3sc].
//
// Fold (exact-integer bias as in the Q4_0 kernel): the int32 accumulator
// starts at 0x4B400000, so the result read as f32 is F = 1.5*2^23 + V
// (|V| <= 256*45*128 < 2^22); u = fma(F, d, -1.5*2^23*d) = V*d (one rounding),
// t = fma(-dmin, Mn, u), acc = fma(t, d8, acc).
// Output lane layout of a 32x32 MFMA tile: lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4 and column l%32.
#include "qmm_device.h"

#include <type_traits>

namespace qmm {

namespace mk {
constexpr int BM = 128;                        // tokens per workgroup tile
constexpr int BN = 128;                        // weight rows per workgroup tile
constexpr int NT = 256;                        // 4 waves, 2 x 2 of 64 x 64
constexpr int XC = 19;                         // 16-byte chunks per activation row per stage
constexpr int WC = 7;                          // per weight row
constexpr int XQ = BM * XC / kWave;            // 38 wave loads of activation chunks
constexpr int WQ = BN * WC / kWave;            // 14 of weight chunks
constexpr int PER_WAVE = (XQ + WQ) / 4;        // 13 DMA loads per wave per stage
constexpr int XROW = 16 * XC;                  // 304-byte LDS activation row
constexpr int WROW = 16 * WC;                  // 112-byte LDS weight row
constexpr int WOFF = BM * XROW;                // weight rows start (bytes into a stage buffer)
constexpr int STAGE = (BM * XC + BN * WC) * 16;   // 53,248 bytes
constexpr int NBUF = 2;
constexpr int D8 = NBUF * STAGE;               // per-wave f32 d8 of its 64 rows
constexpr int LDS_BYTES = D8 + 4 * 64 * 4;     // 107,520
constexpr float kBias = 12582912.0f;           // 1.5 * 2^23, bit pattern 0x4B400000
// global offsets (within a super-block) of the chunks of a row
constexpr int xchunk(int c) { return c < 16 ? 4 + 16 * c : (c == 16 ? 260 : (c == 17 ? 276 : 0)); }
constexpr int wchunk(int c) { return c < 5 ? 16 * c : 68; }
static_assert(XQ * kWave == BM * XC && WQ * kWave == BN * WC && (XQ + WQ) % 4 == 0,
              "a stage splits into whole wave loads, evenly over the waves");
}  // namespace mk

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// BYTES per lane from a buffer into LDS at m0base + OFF + 16 * lane (see the
// Q4_0 prefill kernel: inline assembly so that the compiler neither waits for
// these loads before LDS reads nor keeps one LDS address per load alive).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF>
__device__ __forceinline__ void buffer16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t m0base, uint32_t voff, int soff) {
    asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0base), "v"(voff), "s"(r), "s"(soff), "i"(OFF) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

__global__ __launch_bounds__(mk::NT, 1) void k_matmul_q2_k(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int ns, int tiles_m) {
    using namespace mk;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = uniform(t >> 6);
    const int mt = blockIdx.x % tiles_m, nt = blockIdx.x / tiles_m;
    const int m0 = mt * BM, n0 = nt * BN;
    const uint32_t xrow = (uint32_t)ns * kQ8KBytes, wrow = (uint32_t)ns * kQ2KBytes;

    // DMA: wave load q = wave + 4k (k < 13) of a stage is chunk load q of the
    // stage image (activation chunks for q < 38, weight chunks after) and
    // lands at byte 1024 q of the stage buffer.  Rows past the matrix re-read
    // its last row (their results are not stored).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + (int64_t)m0 * xrow), 0, (int)((uint32_t)min(M - m0, BM) * xrow), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + (int64_t)n0 * wrow), 0, (int)((uint32_t)min(N - n0, BN) * wrow), 0x00020000);
    uint32_t voff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int q = wave + 4 * k;
        if (q < XQ) {
            const int f = kWave * q + lane, row = f / XC, c = f - XC * row;
            voff[k] = (uint32_t)(min(m0 + row, M - 1) - m0) * xrow + (uint32_t)xchunk(c);
        } else {
            const int f = kWave * (q - XQ) + lane, row = f / WC, c = f - WC * row;
            voff[k] = (uint32_t)(min(n0 + row, N - 1) - n0) * wrow + (uint32_t)wchunk(c);
        }
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
    const uint32_t m0w = (uint32_t)uniform((int)(lds0 + 1024u * wave));
    static_assert(XQ == 38 && PER_WAVE == 13, "the load roles below are written for this split");
    auto dma = [&](int s, int b) __attribute__((always_inline)) {
        const int sx = s * kQ8KBytes, sw = s * kQ2KBytes;
        const uint32_t base = m0w + (uint32_t)(b * STAGE);
        // loads 0..8 are activation chunks for every wave; load 9 for waves 0
        // and 1 (q = 36, 37), weight chunks for waves 2 and 3; loads 10..12 weights
        auto one = [&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const bool isw = k == 9 ? wave >= 2 : k >= 10;
            buffer16_to_lds<4096 * k>(isw ? wr : xr, base, voff[k], isw ? sw : sx);
        };
        one(std::integral_constant<int, 0>());
        one(std::integral_constant<int, 1>());
        one(std::integral_constant<int, 2>());
        one(std::integral_constant<int, 3>());
        one(std::integral_constant<int, 4>());
        one(std::integral_constant<int, 5>());
        one(std::integral_constant<int, 6>());
        one(std::integral_constant<int, 7>());
        one(std::integral_constant<int, 8>());
        one(std::integral_constant<int, 9>());
        one(std::integral_constant<int, 10>());
        one(std::integral_constant<int, 11>());
        one(std::integral_constant<int, 12>());
    };

    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 31, lh = lane >> 5;
    const int xa = XROW * (64 * wm + lr);                // A row 64wm+lr (tile i: +32 rows)
    const int wb = WOFF + WROW * (64 * wn + lr);         // B row 64wn+lr (tile j: +32 rows)
    const int xd = XROW * (64 * wm + lane) + 288;        // the d8 chunk of the row this lane converts
    float *d8w = reinterpret_cast<float *>(lds + D8 + 256 * wave);

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0x4B400000;
    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto rd16 = [](const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); };
    auto rd4 = [](const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); };
    auto as_v4i = [](const uint4 &u) { return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}; };
    // 8 int16 (one uint4) -> 8 f16, exact for |x| <= 2048
    auto i16x8_to_h = [](const uint4 &u) {
        v8h r;
        const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[2 * e] = (_Float16)(int)(int16_t)(a[e] & 0xffffu);
            r[2 * e + 1] = (_Float16)(int)(int16_t)(a[e] >> 16);
        }
        return r;
    };
    // the high nibbles (mins) of 8 scale bytes (two dwords) -> 8 f16
    auto mins_to_h = [](uint32_t lo, uint32_t hi) {
        v8h r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = (_Float16)(int)((lo >> (8 * e + 4)) & 15u);
            r[4 + e] = (_Float16)(int)((hi >> (8 * e + 4)) & 15u);
        }
        return r;
    };
    auto half_lo = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); };
    auto half_hi = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); };

    auto compute = [&](const uint8_t *sb) __attribute__((always_inline)) {
        // d8 of the wave's 64 activation rows into its private array
        d8w[lane] = *reinterpret_cast<const float *>(sb + xd);
        // per B tile: the 16 scale bytes and d, dmin
        uint4 scl[2];
        float dw[2], nbw[2], ndm[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            scl[j] = rd16(sb + wb + WROW * 32 * j);
            const uint32_t dd = rd4(sb + wb + WROW * 32 * j + 92);
            dw[j] = half_lo(dd);
            asm volatile("" : "+v"(dw[j]));          // keep the f32 value (see the Q4_0 kernel)
            nbw[j] = dw[j] * -kBias;                 // exact: 11 + 2 significant bits
            ndm[j] = -half_hi(dd);
        }
        // min term: one f16 MFMA per tile
        v16f mn[2][2];
        {
            v8h am[2], bm[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) am[i] = i16x8_to_h(rd16(sb + xa + XROW * 32 * i + 256 + 16 * lh));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t lo = lh ? scl[j].z : scl[j].x, hi = lh ? scl[j].w : scl[j].y;   // groups 8h .. 8h+7
                bm[j] = mins_to_h(lo, hi);
            }
            const v16f z = {};
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mn[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[i], bm[j], z, 0, 0, 0);
        }
        // value term: eight K-steps of int8 MFMA, int32 accumulation from the bias
        v16i v[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) v[i][j] = bias;
        uint4 qs[2];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const int h = kt >> 2, sft = 2 * (kt & 3);
            if ((kt & 3) == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) qs[j] = rd16(sb + wb + WROW * 32 * j + 16 + 32 * h + 16 * lh);
            }
            v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = as_v4i(rd16(sb + xa + XROW * 32 * i + 32 * kt + 16 * lh));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // group 2kt + lh: scale byte, table [0, sc, 2sc, 3sc]
                const int g = 2 * kt + lh;
                const uint32_t sw = (g < 4) ? scl[j].x : (g < 8) ? scl[j].y : (g < 12) ? scl[j].z : scl[j].w;
                const uint32_t sc = (sw >> (8 * (g & 3))) & 15u;
                const uint32_t tab = sc * 0x03020100u;
                const uint32_t d4[4] = {qs[j].x, qs[j].y, qs[j].z, qs[j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t qb = (d4[e] >> sft) & 0x03030303u;
                    b[j][e] = (int)__builtin_amdgcn_perm(0u, tab, qb);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) v[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], v[i][j], 0, 0, 0);
        }
        // fold: acc += d8 * (d * V - dmin * Mn)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float d8[16];
            const float4 *p = reinterpret_cast<const float4 *>(d8w + 32 * i + 4 * lh);
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const float4 qd = p[2 * a4];
                d8[4 * a4] = qd.x;
                d8[4 * a4 + 1] = qd.y;
                d8[4 * a4 + 2] = qd.z;
                d8[4 * a4 + 3] = qd.w;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int e = v[i][j][r];
                    const float u = fmaf(__int_as_float(e), dw[j], nbw[j]);
                    const float tt = fmaf(ndm[j], mn[i][j][r], u);
                    acc[i][j][r] = fmaf(tt, d8[r], acc[i][j][r]);
                }
        }
    };

    // Stage s lives in buffer s % 2.  At step s: wait for this wave's loads of
    // stage s, the barrier publishes every wave's (and tells that stage s-1's
    // buffer is free), the DMA of stage s+1 goes into it, then stage s is
    // computed.
    dma(0, 0);
    for (int s = 0; s < ns; ++s) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (s + 1 < ns) dma(s + 1, (s + 1) & 1);
        compute(lds + (s & 1) * STAGE);
    }
    // no LDS-DMA write may still be in flight when the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + lr;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m < M) y[(int64_t)m * N + n] = acc[i][j][r];
            }
        }
}

// Largest super-block count whose tile offsets fit the 32-bit buffer offsets
// (128 activation rows of ns * 292 bytes).
constexpr int64_t kMatmulKMaxBlocks = (((int64_t)1 << 31) - 1) / (mk::BM * kQ8KBytes);

int64_t matmul_q2_k_max_blocks() { return kMatmulKMaxBlocks; }

hipError_t launch_matmul_q2_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    if (ns > kMatmulKMaxBlocks) return hipErrorInvalidValue;
    static int lds_ok = 0;
    const hipError_t e = allow_dynamic_lds((const void *)k_matmul_q2_k, (size_t)mk::LDS_BYTES, lds_ok);
    if (e != hipSuccess) return e;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    int tiles_m = (M + mk::BM - 1) / mk::BM;
    const int64_t tiles = (int64_t)tiles_m * ((N + mk::BN - 1) / mk::BN);
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&ns, (void *)&tiles_m};
    return hipLaunchKernel((const void *)k_matmul_q2_k, dim3((unsigned)tiles), dim3(mk::NT), args,
                           (size_t)mk::LDS_BYTES, st);
}

}  // namespace qmm
