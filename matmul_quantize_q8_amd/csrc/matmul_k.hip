// Prefill matmul, Q2_K, Q4_K or Q6_K weights x Q8_K activations, on MFMA.
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
// Workgroup tile 128 tokens x 256 weight rows, 8 waves of all 128 tokens x
// 32 weight rows (four MFMA tiles of 32 x 32 sharing one B operand, so each
// B operand is built once per workgroup), one workgroup per CU: two waves per
// SIMD, so that one issues while the other waits, and two stage buffers of
// 66 KB (the DMA of stage s+1 runs while stage s is computed).
// Staging: a stage is one super-block.  Each activation row's 292 bytes
// arrive as 19 chunks of 16 bytes (LDS row: codes 0..255 at 0, bsums at 256,
// the chunk holding d8 at 288; 304-byte stride, so the 32 rows of a 16-byte
// read fall in distinct banks) and each weight row's 84 bytes as 7 chunks
// (scales at 0, qs at 16, the chunk holding d and dmin at 80, one spare;
// 112-byte stride).  Consecutive lanes take consecutive chunks of a row, so
// every load is coalesced; each lane's global offsets are fixed for the
// whole K loop and the stage position rides in the scalar offset.
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
//
// Q4_K weights (the same staging, weight rows of 144 bytes in nine chunks):
// sub-block j of 32 values has a 6-bit scale sc_j and min m_j (minfer "The
// payoff: a K-quant dot kernel, walked"), and sc_j q <= 63 * 15 is no int8;
// but sc_j = 8 sh_j + sl_j with sh_j, sl_j <= 7, and sh_j q, sl_j q <= 105
// are, so two 256-deep int8 contractions A1 = sum sh q x and A2 = sum sl q x
// (eight v_mfma_i32_32x32x32_i8 each, int32, |A| < 2^22) give
// V = sum_j sc_j sum q x = 8 A1 + A2 exactly (|V| < 2^25); the min term is
// the same f16 MFMA over the block sums (m <= 63, |Mn| < 2^22, exact), and
// the fold is acc += d8 * ((float)V * d - dmin * Mn).
// Output lane layout of a 32x32 MFMA tile: lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4 and column l%32.
#include "qmm_device.h"

#include <type_traits>

namespace qmm {

namespace mk {
constexpr int BM = 128;                        // tokens per workgroup tile
constexpr int NW = 8;                          // waves per workgroup
constexpr int NT = NW * kWave;
constexpr int XC = 19;                         // 16-byte chunks per activation row per stage
constexpr int XQ = BM * XC / kWave;            // 38 wave loads of activation chunks
constexpr int XROW = 16 * XC;                  // 304-byte LDS activation row
constexpr int WOFF = BM * XROW;                // weight rows start (bytes into a stage buffer)
constexpr int NBUF = 2;
constexpr float kBias = 12582912.0f;           // 1.5 * 2^23, bit pattern 0x4B400000
// global offsets (within a super-block) of the chunks of an activation row
constexpr int xchunk(int c) { return c < 16 ? 4 + 16 * c : (c == 16 ? 260 : (c == 17 ? 276 : 0)); }

// Per weight format: Q2_K rows of 84 bytes in 7 chunks (scales at 0, qs at
// 16, the chunk holding d and dmin at 80, one spare), Q4_K rows of 144 bytes
// in 9 chunks (d, dmin, scales, qs: the super-block as it is), Q6_K rows of
// 210 bytes in 14 (ql at 0, qh at 128, scales at 192, the chunk holding d at
// 208).  Q2_K and Q4_K: 256 weight rows per workgroup, each wave all 128
// tokens (four A tiles) x 32 rows; Q6_K, whose rows do not leave room for
// 256 in two stage buffers: 128 weight rows, each wave 64 tokens (two A
// tiles) x 32 rows.
template <int F> struct KW {
    static constexpr int WB = F == F_Q2_K ? kQ2KBytes : F == F_Q4_K ? kQ4KBytes : kQ6KBytes;
    static constexpr int WC = F == F_Q2_K ? 7 : F == F_Q4_K ? 9 : 14;   // 16-byte chunks per weight row
    static constexpr int BN = F == F_Q6_K ? 128 : 256;          // weight rows per workgroup tile
    static constexpr int TI = F == F_Q6_K ? 2 : 4;              // A tiles (of 32 tokens) per wave
    static constexpr int WROW = 16 * WC;                        // LDS weight row
    static constexpr int WQ = BN * WC / kWave;                  // wave loads of weight chunks
    static constexpr int NQ = XQ + WQ;                          // 66, 74 or 66 wave loads per stage
    static constexpr int PER_WAVE = (NQ + NW - 1) / NW;         // 9, 10 or 9
    static constexpr int STAGE = (BM * XC + BN * WC) * 16;      // 67,584, 75,776 or 67,584 bytes
    static constexpr int D8 = NBUF * STAGE;                     // per-wave f32 d8 of its 32 TI rows
    static constexpr int LDS_BYTES = D8 + NW * 32 * TI * 4;
    static constexpr int wchunk(int c) {
        return F == F_Q2_K ? (c < 5 ? 16 * c : 68) : F == F_Q4_K ? 16 * c : (c < 13 ? 16 * c : 194);
    }
    static_assert(XQ * kWave == BM * XC && WQ * kWave == BN * WC && NQ > NW * (PER_WAVE - 1),
                  "a stage splits into whole wave loads; only the last round of loads has gaps");
    static_assert(NW * 32 * TI == BM * BN / 32, "the waves cover the workgroup tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

// Narrow tile for launches of a few tokens: 32 tokens x 128 weight rows
// per group of four waves, wave w alone on weight rows 32w .. 32w+31 (one A
// tile), so that a few tokens do not pay for the 96 rows of a 128-token tile
// past M.  A stage image is the 32 activation rows (608 chunks in ten wave
// loads; lanes past the last chunk re-load it into padding), then the 128
// weight rows.  A launch of fewer workgroups than CUs runs K groups per
// workgroup, each with its own stage buffers on its share of the
// super-blocks, stepping through the same barriers; groups 1.. hand their
// sums to group 0 through LDS at the end (the same order on every call).
// Q2_K and Q4_K run four groups of two waves on 64 weight rows with K whole
// and plain stores (no fill kernel, no atomic adds: Q4_K M = 32, N = 12288,
// K = 4096: 13.5 us with two groups on a split launch, 11.3 with four), and
// up to two workgroups per CU two groups of two waves (M = 64: 25.6 us with
// one group on a split launch, 23.9 with two); Q6_K, whose four groups of
// stage buffers do not fit LDS, two groups of four on each half of a split
// launch.
constexpr int NBM = 32;                        // tokens per narrow tile
// Token counts up to which the narrow tile runs: up to 128 for Q2_K and
// Q4_K, whose full tiles of 256 weight rows leave most CUs idle below 129
// tokens (96 workgroups at N = 12288), 64 for Q6_K (12288 x 4096, us, full
// / narrow: Q2_K M = 65 32.1 / 24.0, M = 128 37.1 / 25.7; Q4_K 46.2 / 35.9,
// 52.7 / 37.3; Q6_K 44.3 / 62.3, 49.8 / 63.7).
constexpr int narrow_tokens(int f) { return f == F_Q6_K ? 2 * NBM : 4 * NBM; }
constexpr int NXQ = 10;                        // wave loads of activation chunks
template <int F, int G, int WPG = 4> struct KN {   // G groups of WPG waves (32 weight rows each)
    using W = KW<F>;
    static constexpr int NW = WPG * G;                       // waves per workgroup
    static constexpr int BN = 32 * WPG;                      // weight rows per workgroup tile
    static constexpr int WQ = BN * W::WC / kWave;            // 14, 18 or 28 wave loads of weight chunks (WPG = 4)
    static constexpr int NQ = NXQ + WQ;                      // 24, 28 or 38
    static constexpr int PER_WAVE = (NQ + WPG - 1) / WPG;    // 6, 7 or 10
    static constexpr int WOFF = NXQ * 1024;
    static constexpr int STAGE = NQ * 1024;                  // 24,576, 28,672 or 38,912 bytes
    static constexpr int D8 = G * NBUF * STAGE;              // per-wave f32 d8 of its 32 rows
    static constexpr int LDS_BYTES = D8 + NW * 32 * 4;
    static_assert(NBM * XC <= NXQ * kWave && WQ * kWave == BN * W::WC && NQ > WPG * (PER_WAVE - 1),
                  "a stage splits into whole wave loads; only the last round of loads has gaps");
};
}  // namespace mk

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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

// f(integral_constant<int, K>) for K = 0 .. N-1, in order.
template <class Fn, int... K>
__device__ __forceinline__ void for_each_index(Fn &&f, std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>()), ...);
}

// Q4_K's packed 6-bit scales: scale and min of sub-block s from the three
// scale dwords (bytes 4..15 of the super-block).
__device__ __forceinline__ void q4k_sc_m(uint32_t s0, uint32_t s1, uint32_t s2, int s, int &sc, int &m) {
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

template <int F, bool SPLIT, bool NARROW = false, int G = 1, int WPG = 4>
__device__ __forceinline__ void matmul_k_body(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                              float *__restrict__ y, int M, int N, int ns, int tiles_m) {
    using namespace mk;
    using W = KW<F>;
    using KT = KN<F, G, WPG>;
    static_assert(G == 1 || (G == 2 && NARROW && SPLIT && WPG == 4) || ((G == 2 || G == 4) && NARROW && !SPLIT && WPG == 2),
                  "two K groups on split narrow launches, groups of two waves on unsplit ones");
    constexpr int WC = W::WC, WROW = W::WROW;
    constexpr int NWG = NARROW ? WPG : NW;               // waves per K group
    constexpr int XQN = NARROW ? NXQ : XQ;               // wave loads of activation chunks
    constexpr int NQ = NARROW ? KT::NQ : W::NQ, PER_WAVE = NARROW ? KT::PER_WAVE : W::PER_WAVE;
    constexpr int STAGE = NARROW ? KT::STAGE : W::STAGE, D8 = NARROW ? KT::D8 : W::D8;
    constexpr int BN = NARROW ? KT::BN : W::BN, TI = NARROW ? 1 : W::TI, TBM = NARROW ? NBM : BM;
    constexpr int WO = NARROW ? KT::WOFF : WOFF;         // weight rows start (bytes into a stage buffer)
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = uniform(NARROW ? (t >> 6) % WPG : t >> 6);
    const int grp = G == 1 ? 0 : uniform((t >> 6) / WPG);   // K group: its own stage buffers and super-blocks
    // SPLIT: the grid holds every tile twice, one per part of K, and both
    // parts add into the zeroed output.  Part p of P = ksplit * G (grid part
    // and K group) takes super-blocks [ceil(p ns / P), ceil((p + 1) ns / P))
    // (the caller keeps ns >= P).
    constexpr int ksplit = SPLIT ? 2 : 1;
    constexpr int P = ksplit * G;
    const int tiles = (int)gridDim.x / ksplit;
    const int tile = (int)blockIdx.x % tiles, gpart = (int)blockIdx.x / tiles;
    const int mt = tile % tiles_m, nt = tile / tiles_m;
    const int m0 = mt * TBM, n0 = nt * BN;
    auto first_sb = [&](int p) { return (p * ns + P - 1) / P; };
    const int sh = (ns + 1) / 2;
    const int s0 = G == 1 ? (gpart ? sh : 0) : first_sb(G * gpart + grp);       // this part's [s0, s1)
    const int s1 = G == 1 ? (SPLIT && !gpart ? sh : ns) : first_sb(G * gpart + grp + 1);
    // every wave of the workgroup passes the same barriers: the K groups
    // step together for the larger of their super-block counts
    int nsteps = s1 - s0;
#pragma unroll
    for (int g = 0; g < G; ++g)
        if (G > 1) nsteps = max(nsteps, first_sb(G * gpart + g + 1) - first_sb(G * gpart + g));
    const uint32_t xrow = (uint32_t)ns * kQ8KBytes, wrow = (uint32_t)ns * W::WB;

    // DMA: wave load q = wave + 8k (k < PER_WAVE; narrow: 4k) of a stage is
    // chunk load q of the stage image (activation chunks for q < 38, or 10,
    // weight chunks after) and lands at byte 1024 q of the stage buffer; a
    // wave whose last q is past NQ repeats its previous load instead (same
    // bytes to the same place), so that every wave issues the same count.
    // Rows past the matrix re-read its last row (their results are not
    // stored).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + (int64_t)m0 * xrow), 0, (int)((uint32_t)min(M - m0, TBM) * xrow), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + (int64_t)n0 * wrow), 0, (int)((uint32_t)min(N - n0, BN) * wrow), 0x00020000);
    uint32_t voff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int q = wave + NWG * k;
        if (q >= NQ) {
            voff[k] = voff[k - 1];
        } else if (q < XQN) {
            const int f0 = kWave * q + lane, f = NARROW ? min(f0, NBM * XC - 1) : f0;
            const int row = f / XC, c = f - XC * row;
            voff[k] = (uint32_t)(min(m0 + row, M - 1) - m0) * xrow + (uint32_t)xchunk(c);
        } else {
            const int f = kWave * (q - XQN) + lane, row = f / WC, c = f - WC * row;
            voff[k] = (uint32_t)(min(n0 + row, N - 1) - n0) * wrow + (uint32_t)W::wchunk(c);
        }
    }
    uint8_t *const ldsg = lds + grp * (NBUF * STAGE);   // this K group's stage buffers
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(ldsg);
    const uint32_t m0w = (uint32_t)uniform((int)(lds0 + 1024u * wave));
    constexpr int KL = PER_WAVE - 1;
    // LDS offset of the last load of a stage (or of the load it repeats)
    const uint32_t last_off = (uint32_t)uniform(1024 * NWG * (wave + NWG * KL >= NQ ? KL - 1 : KL));
    auto dma = [&](int s, int b) __attribute__((always_inline)) {
        const int sx = s * kQ8KBytes, sw = s * W::WB;
        const uint32_t base = m0w + (uint32_t)(b * STAGE);
        auto one = [&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const bool isw = wave + NWG * k >= XQN;   // a repeated load is a weight load
            const int soff = uniform(isw ? sw : sx);
            if constexpr (k == KL)
                buffer16_to_lds<0>(isw ? wr : xr, base + last_off, voff[k], soff);
            else
                buffer16_to_lds<1024 * NWG * k>(isw ? wr : xr, base, voff[k], soff);
        };
        for_each_index(one, std::make_integer_sequence<int, PER_WAVE>());
    };

    const int lr = lane & 31, lh = lane >> 5;
    // the wave's tokens 32 TI wm .. and weight rows 32 wn ..
    const int wm = (NARROW || TI == 4) ? 0 : wave & 1, wn = (NARROW || TI == 4) ? wave : wave >> 1;
    const int xa = XROW * (32 * TI * wm + lr);           // A row lr of the wave (tile i: +32i rows)
    const int wb = WO + WROW * (32 * wn + lr);           // B row 32 wn + lr
    float *d8w = reinterpret_cast<float *>(lds + D8 + 4 * 32 * TI * (NWG * grp + wave));
    // d8 of the wave's activation rows into its private array (narrow: 32
    // rows, lanes 32..63 writing the same values as 0..31)
    auto store_d8 = [&](const uint8_t *sb) __attribute__((always_inline)) {
        if constexpr (NARROW) {
            d8w[lr] = *reinterpret_cast<const float *>(sb + XROW * lr + 288);
        } else if constexpr (TI == 4) {
            d8w[lane] = *reinterpret_cast<const float *>(sb + XROW * lane + 288);
            d8w[64 + lane] = *reinterpret_cast<const float *>(sb + XROW * (64 + lane) + 288);
        } else {
            d8w[lane] = *reinterpret_cast<const float *>(sb + XROW * (64 * wm + lane) + 288);
        }
    };

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0x4B400000;
    float acc[TI][16];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

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

    // One stage: the wave's B tile (32 weight rows) against all four A tiles
    // (128 tokens), so that each B operand is built once per workgroup.
    auto compute = [&](const uint8_t *sb) __attribute__((always_inline)) {
        if constexpr (F == F_Q2_K) {
            store_d8(sb);
            // the B tile's 16 scale bytes and d, dmin
            const uint4 scl = rd16(sb + wb);
            const uint32_t dd = rd4(sb + wb + 92);
            uint4 qs = rd16(sb + wb + 16 + 16 * lh);
            // B operand of K-step kt: group 2kt + lh, table [0, sc, 2sc, 3sc]
            auto build_b = [&](int kt, const uint4 &q) __attribute__((always_inline)) {
                const int g = 2 * kt + lh, sft = 2 * (kt & 3);
                const uint32_t sw = (g < 4) ? scl.x : (g < 8) ? scl.y : (g < 12) ? scl.z : scl.w;
                const uint32_t sc = (sw >> (8 * (g & 3))) & 15u;
                const uint32_t tab = __umul24(sc << 8, 0x030201u);   // sc * 0x03020100
                const uint32_t d4[4] = {q.x, q.y, q.z, q.w};
                v4i b;
    #pragma unroll
                for (int e = 0; e < 4; ++e) b[e] = (int)__builtin_amdgcn_perm(0u, tab, (d4[e] >> sft) & 0x03030303u);
                return b;
            };
            // value term: eight K-steps of int8 MFMA, int32 accumulation from the bias
            v16i v[TI];
    #pragma unroll
            for (int i = 0; i < TI; ++i) v[i] = bias;
    #pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                if (kt == 4) qs = rd16(sb + wb + 16 + 32 + 16 * lh);
                const v4i b = build_b(kt, qs);
    #pragma unroll
                for (int i = 0; i < TI; ++i) {
                    const v4i a = as_v4i(rd16(sb + xa + XROW * 32 * i + 32 * kt + 16 * lh));
                    v[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, v[i], 0, 0, 0);
                }
            }
            float dw = half_lo(dd), ndm = -half_hi(dd);
            // keep the f32 values (an f16 operand would make each fold FMA a
            // half-rate v_fma_mix)
            asm volatile("" : "+v"(dw), "+v"(ndm));
            const float nbw = dw * -kBias;   // exact: 11 + 2 significant bits
            // min term, one f16 MFMA per A tile, and the fold:
            // acc += d8 * (d * V - dmin * Mn)
            const uint32_t mlo = lh ? scl.z : scl.x, mhi = lh ? scl.w : scl.y;   // groups 8h .. 8h+7
            const v8h bm = mins_to_h(mlo, mhi);
            const v16f z = {};
    #pragma unroll
            for (int i = 0; i < TI; ++i) {
                const v8h am = i16x8_to_h(rd16(sb + xa + XROW * 32 * i + 256 + 16 * lh));
                const v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(am, bm, z, 0, 0, 0);
                // d8 of output rows 8a4 + 4lh + c, four at a time
                const float4 *p = reinterpret_cast<const float4 *>(d8w + 32 * i + 4 * lh);
    #pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const float4 qd = p[2 * a4];
                    const float d8[4] = {qd.x, qd.y, qd.z, qd.w};
    #pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * a4 + c;
                        const int e = v[i][r];
                        const float u = fmaf(__int_as_float(e), dw, nbw);
                        const float tt = fmaf(ndm, mn[r], u);
                        acc[i][r] = fmaf(tt, d8[c], acc[i][r]);
                    }
                }
            }
        } else if constexpr (F == F_Q4_K) {
            store_d8(sb);
            // the B tile row's d, dmin and packed scales
            const uint32_t dd = rd4(sb + wb), s0 = rd4(sb + wb + 4), s1 = rd4(sb + wb + 8), s2 = rd4(sb + wb + 12);
            int sc[8], mm[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q4k_sc_m(s0, s1, s2, j, sc[j], mm[j]);
            // value term: sub-block kt is K-step kt, on the 4-bit codes of qs
            // chunk kt/2 (low nibbles for even kt, high for odd).  The scale
            // splits as sc = 8 sh + sl (sh, sl <= 7), so sh q and sl q (<= 105)
            // are exact int8 operands: two 256-deep int32 contractions
            // A1 = sum sh q x and A2 = sum sl q x on MFMA give
            // V = sum sc I = 8 A1 + A2 (|A1|, |A2| <= 256*105*128 < 2^22),
            // with no vector work per sub-block and output (one v_mad_i32_i24
            // per sub-block and output before: four VALU cycles each, twice
            // the MFMA time)
            v16i A1[TI], A2[TI];
            const v16i zero = {};
#pragma unroll
            for (int i = 0; i < TI; ++i) A1[i] = A2[i] = zero;
            uint4 qs = rd16(sb + wb + 16 + 16 * lh);   // chunk 0 (K-steps 0, 1)
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                if (kt >= 2 && (kt & 1) == 0) qs = rd16(sb + wb + 16 + 32 * (kt >> 1) + 16 * lh);
                const uint32_t sft = 4u * (uint32_t)(kt & 1);
                // byte-wise products by a multiply of the two 16-bit halves
                // (v_pk_mul_lo_u16): each half holds two codes b0 + 256 b1,
                // and b0 s <= 105, 256 b1 s < 2^16, so no carry crosses a byte
                const unsigned short sh = (unsigned short)(sc[kt] >> 3), sl = (unsigned short)(sc[kt] & 7);
                const u16x2 sh2 = {sh, sh}, sl2 = {sl, sl};
                const uint32_t q4[4] = {qs.x, qs.y, qs.z, qs.w};
                v4i b1, b2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u16x2 nib = __builtin_bit_cast(u16x2, (q4[e] >> sft) & 0x0f0f0f0fu);   // four codes
                    b1[e] = __builtin_bit_cast(int, nib * sh2);
                    b2[e] = __builtin_bit_cast(int, nib * sl2);
                }
#pragma unroll
                for (int i = 0; i < TI; ++i) {
                    const v4i a = as_v4i(rd16(sb + xa + XROW * 32 * i + 32 * kt + 16 * lh));
                    A1[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, A1[i], 0, 0, 0);
                    A2[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b2, A2[i], 0, 0, 0);
                }
            }
            float dw = half_lo(dd), ndm = -half_hi(dd);
            // keep the f32 values (an f16 operand would make each fold FMA a
            // half-rate v_fma_mix)
            asm volatile("" : "+v"(dw), "+v"(ndm));
            // min term, one f16 MFMA per A tile: groups 8h .. 8h+7 are
            // sub-blocks 4h .. 4h+3, two groups each
            v8h bm;
#pragma unroll
            for (int e = 0; e < 8; ++e) bm[e] = (_Float16)(lh ? mm[4 + (e >> 1)] : mm[e >> 1]);
            const v16f z = {};
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const v8h am = i16x8_to_h(rd16(sb + xa + XROW * 32 * i + 256 + 16 * lh));
                const v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(am, bm, z, 0, 0, 0);
                // d8 of output rows 8a4 + 4lh + c, four at a time
                const float4 *p = reinterpret_cast<const float4 *>(d8w + 32 * i + 4 * lh);
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const float4 qd = p[2 * a4];
                    const float d8[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * a4 + c;
                        const int V = A1[i][r] * 8 + A2[i][r];   // |V| < 2^25
                        const float tt = fmaf(ndm, mn[r], (float)V * dw);
                        acc[i][r] = fmaf(tt, d8[c], acc[i][r]);
                    }
                }
            }
        } else {
            // Q6_K: value 128hh + 32k + l of a super-block takes its low 4 bits
            // from ql[64hh + 32(k&1) + l] (low nibble for k < 2, high for
            // k >= 2) and its high 2 bits from qh[32hh + l] >> 2k, and group
            // g = 8hh + 2k + l/16 of 16 values has the signed scale sc[g].
            // A K=16 MFMA per group on the unsigned codes q (0..63) gives
            // I_g = sum q x; V = sum_g sc_g I_g in int32 (v_mad_i32_i24), and
            // the offset of 32 is sum_g 32 sc_g bsum_g, one f16 MFMA over the
            // block sums: the product is d8 d (V - Mn).
            store_d8(sb);
            const uint4 scl = rd16(sb + wb + 192);
            auto scale = [&](int g) __attribute__((always_inline)) {
                const uint32_t sw = g < 4 ? scl.x : g < 8 ? scl.y : g < 12 ? scl.z : scl.w;
                return (int)(int8_t)(sw >> (8 * (g & 3)));
            };
            auto rd8 = [](const uint8_t *p) { return *reinterpret_cast<const uint2 *>(p); };
            int V[TI][16];
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) V[i][r] = 0;
            // Steps t = TI (4 (2 hh + gg) + k) + i, software-pipelined as for
            // Q4_K: the MFMA of step t+1 goes out before the mads of step t,
            // A operands are read one step ahead, and the code bytes of the
            // next (hh, gg) pair (this lane's 8 values of its groups 8hh + 2k
            // + gg: l = 16gg + 8lh ..) one pair ahead.
            struct Codes {
                uint2 qa, qb, qh;
            };
            auto read_codes = [&](int p) __attribute__((always_inline)) {
                const int hh = p >> 1, gg = p & 1;
                return Codes{rd8(sb + wb + 64 * hh + 16 * gg + 8 * lh), rd8(sb + wb + 64 * hh + 32 + 16 * gg + 8 * lh),
                             rd8(sb + wb + 128 + 32 * hh + 16 * gg + 8 * lh)};
            };
            // group of step t: index gi = t / TI = 4 (2 hh + gg) + k
            auto group = [](int t) {
                const int gi = t / TI;
                return 8 * (gi >> 3) + 2 * (gi & 3) + ((gi >> 2) & 1);
            };
            auto build_b = [](const Codes &q, int k) __attribute__((always_inline)) {
                const uint2 ql = (k & 1) ? q.qb : q.qa;
                const uint32_t nsh = 4u * (uint32_t)(k >> 1), hsh = 2u * (uint32_t)k;
                const uint32_t b0 = ((ql.x >> nsh) & 0x0f0f0f0fu) | (((q.qh.x >> hsh) & 0x03030303u) << 4);
                const uint32_t b1 = ((ql.y >> nsh) & 0x0f0f0f0fu) | (((q.qh.y >> hsh) & 0x03030303u) << 4);
                return (long)(((uint64_t)b1 << 32) | b0);
            };
            auto read_a = [&](int t) __attribute__((always_inline)) {
                const uint2 av = rd8(sb + xa + XROW * 32 * (t % TI) + 16 * group(t) + 8 * lh);
                return (long)(((uint64_t)av.y << 32) | av.x);
            };
            constexpr int T = 16 * TI;
            const v16i zero = {};
            Codes qc = read_codes(0), qn = read_codes(1);
            long b = build_b(qc, 0);
            long an = read_a(1);
            v16i I = __builtin_amdgcn_mfma_i32_32x32x16_i8(read_a(0), b, zero, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int i = t % TI;
                v16i In = zero;
                if (t + 1 < T) {
                    const int t1 = t + 1, g1 = t1 / TI;
                    if (t1 % TI == 0) {                        // a new group: new B operand
                        if ((g1 & 3) == 0) {                   // and a new (hh, gg) pair
                            qc = qn;
                            if ((g1 >> 2) + 1 < 4) qn = read_codes((g1 >> 2) + 1);
                        }
                        b = build_b(qc, g1 & 3);
                    }
                    In = __builtin_amdgcn_mfma_i32_32x32x16_i8(an, b, zero, 0, 0, 0);
                    if (t + 2 < T) an = read_a(t + 2);
                }
                const int sc = scale(group(t));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int e = I[r];
                    V[i][r] = __mul24(sc, e) + V[i][r];   // v_mad_i32_i24
                    asm volatile("" : "+v"(V[i][r]));    // keep the running sum (see Q4_K)
                }
                __builtin_amdgcn_sched_barrier(0);
                I = In;
            }
            float dw = half_hi(rd4(sb + wb + 220));   // d: bytes 208..209 of the super-block
            asm volatile("" : "+v"(dw));
            const float ndw = -dw;
            // offset term: groups 8h .. 8h+7, 32 sc_g exact in f16
            v8h bm;
#pragma unroll
            for (int e = 0; e < 8; ++e) bm[e] = (_Float16)(32 * (lh ? scale(8 + e) : scale(e)));
            const v16f z = {};
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const v8h am = i16x8_to_h(rd16(sb + xa + XROW * 32 * i + 256 + 16 * lh));
                const v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(am, bm, z, 0, 0, 0);
                const float4 *p = reinterpret_cast<const float4 *>(d8w + 32 * i + 4 * lh);
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const float4 qd = p[2 * a4];
                    const float d8[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * a4 + c;
                        const float tt = fmaf(ndw, mn[r], (float)V[i][r] * dw);
                        acc[i][r] = fmaf(tt, d8[c], acc[i][r]);
                    }
                }
            }
        }
    };

    // Super-block s0 + j lives in buffer j % 2.  At step j: wait for this
    // wave's loads of it, the barrier publishes every wave's (and tells that
    // the previous one's buffer is free), the DMA of the next goes into it,
    // then it is computed.  A K group with fewer super-blocks than the other
    // passes its extra step's barrier without work or loads.
    dma(s0, 0);
    if constexpr (G == 1) {
        for (int s = s0; s < s1; ++s) {
            asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (s + 1 < s1) dma(s + 1, (s + 1 - s0) & 1);
            compute(lds + ((s - s0) & 1) * STAGE);
        }
    } else {
        for (int j = 0; j < nsteps; ++j) {
            asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (s0 + j + 1 < s1) dma(s0 + j + 1, (j + 1) & 1);
            if (s0 + j < s1) compute(ldsg + (j & 1) * STAGE);
        }
    }
    // no LDS-DMA write may still be in flight when the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (G > 1) {
        // groups 1 .. G-1 hand their sums to group 0 through LDS ([group -
        // 1][wave][r][lane], over the stage buffers), which adds them to its
        // own in group order
        float *red = reinterpret_cast<float *>(lds) + 1024 * wave + lane;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (grp > 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) red[1024 * NWG * (grp - 1) + 64 * r] = acc[0][r];
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[0][r] += red[1024 * NWG * (g - 1) + 64 * r];
    }

    const int n = n0 + 32 * wn + lr;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * TI * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m >= M) continue;
                // two addends on a zeroed output: the same sum in either order
                if constexpr (SPLIT)
                    atomicAdd(y + (int64_t)m * N + n, acc[i][r]);
                else
                    y[(int64_t)m * N + n] = acc[i][r];
            }
    }
}

template <int F>
__global__ __launch_bounds__(mk::NT) void k_matmul_k(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                                     float *__restrict__ y, int M, int N, int ns, int tiles_m) {
    matmul_k_body<F, false>(w, xq, y, M, N, ns, tiles_m);
}

template <int F>
__global__ __launch_bounds__(mk::NT) void k_matmul_k_split(const uint8_t *__restrict__ w,
                                                           const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                           int M, int N, int ns, int tiles_m) {
    matmul_k_body<F, true>(w, xq, y, M, N, ns, tiles_m);
}

// The narrow tile (32 tokens x 128 weight rows) for launches of up to
// narrow_tokens tokens: one group of four waves, K whole or split in two,
// or (G = 2) two groups on the halves of each split part.
template <int F, bool SPLIT, int G, int WPG = 4>
__global__ __launch_bounds__(64 * WPG * G) void k_matmul_k_narrow(const uint8_t *__restrict__ w,
                                                                  const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                  int M, int N, int ns, int tiles_m) {
    static_assert(mk::KN<F, G, WPG>::LDS_BYTES <= 160 * 1024, "LDS of one CU");
    matmul_k_body<F, SPLIT, true, G, WPG>(w, xq, y, M, N, ns, tiles_m);
}

// Largest super-block count whose tile offsets fit the 32-bit buffer offsets
// (128 activation rows of ns * 292 bytes; 256 weight rows take fewer).
constexpr int64_t kMatmulKMaxBlocks = (((int64_t)1 << 31) - 1) / (mk::BM * kQ8KBytes);

int64_t matmul_k_max_blocks() { return kMatmulKMaxBlocks; }

template <int F>
static hipError_t launch_k(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    if (ns > kMatmulKMaxBlocks) return hipErrorInvalidValue;
    if (M <= small_tokens(F)) return launch_matvec_tokens(F, w, xq, y, M, N, ns, st);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    // up to narrow_tokens: the 32-token tile (a 128-token tile would compute
    // and drop the rows past M)
    const bool narrow = M <= mk::narrow_tokens(F);
    const int bm = narrow ? mk::NBM : mk::BM, bn = narrow ? mk::KN<F, 1>::BN : mk::KW<F>::BN;
    int tiles_m = (M + bm - 1) / bm;
    const int64_t tiles = (int64_t)tiles_m * ((N + bn - 1) / bn);
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&ns, (void *)&tiles_m};
    // Fewer narrow workgroups than CUs (Q2_K, Q4_K): four groups of two
    // waves on 64 weight rows per workgroup, each on a quarter of K (at
    // least two super-blocks each), written with plain stores.  Four groups
    // of Q6_K stage buffers do not fit one CU's LDS.
    if constexpr (F != F_Q6_K) {
        if (narrow && tiles * 2 < kCUs && ns >= 8) {
            using K4 = mk::KN<F, 4, 2>;
            static int lds_ok4[kLdsDevices] = {};
            const void *k4 = (const void *)k_matmul_k_narrow<F, false, 4, 2>;
            const hipError_t e4 = allow_dynamic_lds(k4, (size_t)K4::LDS_BYTES, lds_ok4);
            if (e4 != hipSuccess) return e4;
            const int64_t tiles4 = (int64_t)tiles_m * ((N + K4::BN - 1) / K4::BN);
            return hipLaunchKernel(k4, dim3((unsigned)tiles4), dim3(64 * K4::NW), args, (size_t)K4::LDS_BYTES, st);
        }
        // up to two such workgroups per CU: two groups of two waves, each on
        // half of K (at least two super-blocks each)
        if (narrow && tiles <= kCUs && ns >= 4) {
            using K2 = mk::KN<F, 2, 2>;
            static_assert(2 * K2::LDS_BYTES <= 160 * 1024, "two workgroups per CU");
            static int lds_ok2[kLdsDevices] = {};
            const void *k2 = (const void *)k_matmul_k_narrow<F, false, 2, 2>;
            const hipError_t e2 = allow_dynamic_lds(k2, (size_t)K2::LDS_BYTES, lds_ok2);
            if (e2 != hipSuccess) return e2;
            const int64_t tiles2 = (int64_t)tiles_m * ((N + K2::BN - 1) / K2::BN);
            return hipLaunchKernel(k2, dim3((unsigned)tiles2), dim3(64 * K2::NW), args, (size_t)K2::LDS_BYTES, st);
        }
    }
    const bool split = tiles <= kSplitTiles && ns >= 2;
    // fewer narrow workgroups than CUs otherwise: two K groups per
    // workgroup, each on half of its part of K (at least one super-block
    // each)
    const bool groups = narrow && split && tiles * 2 < kCUs && ns >= 4;
    static int lds_ok[5][kLdsDevices] = {};
    const int v = groups ? 4 : narrow ? (split ? 3 : 2) : (split ? 1 : 0);
    const void *kern = v == 4   ? (const void *)k_matmul_k_narrow<F, true, 2>
                       : v == 3 ? (const void *)k_matmul_k_narrow<F, true, 1>
                       : v == 2 ? (const void *)k_matmul_k_narrow<F, false, 1>
                       : v == 1 ? (const void *)k_matmul_k_split<F>
                                : (const void *)k_matmul_k<F>;
    const int lds_bytes = groups ? mk::KN<F, 2>::LDS_BYTES : narrow ? mk::KN<F, 1>::LDS_BYTES : mk::KW<F>::LDS_BYTES;
    const int threads = groups ? 512 : narrow ? 256 : mk::NT;
    const hipError_t e = allow_dynamic_lds(kern, (size_t)lds_bytes, lds_ok[v]);
    if (e != hipSuccess) return e;
    if (split) {
        const hipError_t ez = launch_zero_f32(y, (int64_t)M * N, st);
        if (ez != hipSuccess) return ez;
    }
    const int ksplit = split ? 2 : 1;
    return hipLaunchKernel(kern, dim3((unsigned)(tiles * ksplit)), dim3(threads), args, (size_t)lds_bytes, st);
}

hipError_t launch_matmul_q2_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    return launch_k<F_Q2_K>(w, xq, y, M, N, ns, st);
}

hipError_t launch_matmul_q4_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    return launch_k<F_Q4_K>(w, xq, y, M, N, ns, st);
}

hipError_t launch_matmul_q6_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st) {
    return launch_k<F_Q6_K>(w, xq, y, M, N, ns, st);
}

}  // namespace qmm
