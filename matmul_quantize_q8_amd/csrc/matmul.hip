// Prefill matmul, Q4_0 or Q8_0 weights x Q8_0 activations, on int8 MFMA.
//
//   Y[m][n] = sum_b dx[m,b] dw[n,b] I_b[m,n],   I_b = sum_{k<32} q[m,32b+k] w'[n,32b+k]
//   (w' = nibble - 8 for Q4_0, the int8 code for Q8_0)
//
// Once a weight tile is reused across many tokens the product is a dense
// contraction (kvad "Batched prefill, and i8mm"; krafla "Batched prompt
// prefill"), and one 32-value block is exactly the K of
// v_mfma_i32_32x32x32_i8, so every block gets its own exact int32 tile.
//
// Workgroup tile: 128 tokens x 128 weight rows, 4 waves of 64 x 64 (2 x 2
// MFMA tiles of 32 x 32); two workgroups share a CU, so the two waves on a
// SIMD belong to different workgroups and do not meet at the same barriers.
// The K loop moves two blocks per stage.  Launches of up to 64 tokens run a
// narrow tile of 32 tokens, and launches of fewer workgroups than CUs two K
// groups per workgroup (both below).
//
// Staging.  A stage is copied into LDS by buffer LDS-DMA loads of 16 bytes
// per lane (these loads accept the 2-byte aligned addresses of the blocks).
// Each row's 68 activation bytes of the stage (two 34-byte blocks) arrive as
// five 16-byte chunks at segment offsets 0, 16, 32, 48 and 52 (the last one
// overlaps the fourth, so nothing past the segment is read), and each row's
// 36 weight bytes as three chunks at 0, 16 and 20.  Consecutive lanes take
// consecutive chunks of a row, so a load is coalesced; chunks land in LDS in
// the same order, 80 and 48 bytes per row.  Each lane's global offset is
// fixed for the whole K loop and the stage position rides in the scalar
// offset: four loads per wave per stage and no address arithmetic.
// Stages rotate through three buffers: the DMA runs two stages ahead, spread
// over the folds of the current stage, and a stage costs one barrier.
//
// Operands.  Lane half h of an MFMA lane feeds 16 of the 32 codes of its row,
// the same 16 for both operands; which 16, and in what order, only has to
// agree between the two, so it follows the chunks:
//   block 0: half 0 = codes 14..29 (chunk 1); half 1 = codes 30, 31, 0..13
//            (chunk 0 with its first two bytes, the scale, replaced by the
//            first two of chunk 2: one v_perm)
//   block 1: half 0 = codes 12..27 (chunk 3); half 1 = codes 28..31 (last
//            dword of chunk 4), 0..11 (last three dwords of chunk 2)
// Every read is 16 bytes; at an 80- or 48-byte row stride the 32 rows of a
// read fall in distinct banks.  Weight nibbles become signed bytes
// 16*(nib-8) with one shift and one bitop3 per dword (XOR 0x88 on the
// nibbles, krafla "Weight packing"), taken from the bytes that hold the
// weights matching each code position: for block 0 the 16 nibble bytes
// rotated by two (bytes 14, 15, 0..13), low or high nibble per byte as the
// code index is below or above 16; for block 1 bytes 12..15, 0..11.
//
// Scale fold.  The MFMA's C input is the constant 0x4B400000, so the int32
// result read as f32 is exactly F = 1.5*2^23 + 16 I (|16 I| < 2^22); then
//   u = fma(F, dw, -1.5*2^23*dw) = 16 I dw   (one rounding)
//   acc = fma(u, dx, acc)                    (one rounding)
// and the store multiplies by 1/16 (exact).  Both are plain f32 FMAs: on
// gfx950 v_fma_f32 issues at twice the rate of v_fma_mix_f32 and
// v_cvt_f32_f16, so the f16 scales are converted once per stage, not in the
// fold.  Each wave converts the dx of its 64 activation rows into a private
// f32 array in LDS, where four consecutive rows are one 16-byte read.
// Output lane layout of a 32x32 MFMA tile: lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4 and column l%32.
//
// Q8_0 weights (minfer Q8_0 kernel: both operands are 34-byte blocks): the
// weight rows are staged exactly like the activation rows (five chunks, 80
// bytes per row, so a stage is 20 KB and every wave issues five loads), the
// B operand is built like the A operand (the same code order per lane half,
// so the pairing agrees), with no nibble transform; each lane reads its
// weight rows' two scales from chunk 0 and chunk 2.  |I| <= 32*127*127 <
// 2^22, so the bias trick holds with F = 1.5*2^23 + I and the store does not
// rescale.
#include "qmm_device.h"

#include <type_traits>
#include <utility>

namespace qmm {

namespace mm {
constexpr int BM = 128;                   // tokens per workgroup tile
constexpr int BN = 128;                   // weight rows per workgroup tile
constexpr int NT = 256;                   // 4 waves, 2 x 2 of 64 x 64
constexpr int XC = 5;                     // 16-byte chunks per activation row per stage
constexpr int XQ = BM * XC / kWave;       // 10 wave loads of activation chunks
constexpr int WOFF = BM * XC * 16;        // weight chunks start (bytes into a stage buffer)
constexpr int NBUF = 3;                   // stage buffers: DMA runs two stages ahead
constexpr float kBias = 12582912.0f;      // 1.5 * 2^23, bit pattern 0x4B400000
// segment offsets of the activation chunks (and of Q8_0 weight chunks)
constexpr int xchunk(int c) { return c < 4 ? 16 * c : 52; }

// Per weight format (Q4_0, Q8_0, Q5_0, Q4_1 or Q5_1).
template <int WFMT> struct WF {
    static constexpr bool Q8W = WFMT == F_Q8_0, Q41 = WFMT == F_Q4_1, Q51 = WFMT == F_Q5_1;
    static constexpr bool Q5 = WFMT == F_Q5_0 || Q51;          // five-bit codes, high bits in qh
    static constexpr bool MIN = Q41 || Q51;                    // value d q + m: an offset term per block
    static constexpr int WB = Q8W ? kQ80Bytes : WFMT == F_Q5_0 ? kQ50Bytes : Q41 ? kQ41Bytes : Q51 ? kQ51Bytes
                                                                                          : kQ40Bytes;
    static constexpr int WC = Q8W ? 5 : 3;                    // 16-byte chunks per weight row per stage
    static constexpr int WQ = BN * WC / kWave;                // 10 or 6 wave loads of weight chunks
    static constexpr int STAGE = (BM * XC + BN * WC) * 16;    // 20,480 or 16,384 bytes
    static constexpr int PER_WAVE = (XQ + WQ) / 4;            // 5 or 4 DMA loads per wave per stage
    // per-wave f32 dx (and dx * code sum with an offset term): [wave][kind][block][64 rows]
    static constexpr int DXF = NBUF * STAGE;
    static constexpr int DXW = (MIN ? 4 : 2) * 64 * 4;        // bytes per wave
    static constexpr int LDS_BYTES = DXF + 4 * DXW;
    // two K groups of four waves, each with its own stage buffers
    static constexpr int DXF2 = 2 * NBUF * STAGE;
    static constexpr int LDS_BYTES2 = DXF2 + 8 * DXW;
    // 4-bit codes enter as 16*(q-8), 5-bit codes as 8*(q-16)
    static constexpr float OUT_SCALE = Q8W ? 1.0f : Q5 ? 0.125f : 0.0625f;
    // segment offsets of the weight chunks (segment = two blocks): Q4_0 36
    // bytes in chunks at 0, 16, 20; Q5_0 44 at 0, 16, 28; Q4_1 40 at 0, 16,
    // 24; Q5_1 48 at 0, 16, 32
    static constexpr int wchunk(int c) { return Q8W ? xchunk(c) : c < 2 ? 16 * c : 2 * WB - 16; }
    static_assert(XQ * kWave == BM * XC && WQ * kWave == BN * WC && (XQ + WQ) % 4 == 0,
                  "stage splits into whole wave loads, evenly over the waves");
};

// Narrow tile for launches of a few tokens: 32 tokens x 128 weight rows,
// wave w alone on weight rows 32w .. 32w+31 (one 32 x 32 MFMA tile per
// block).  A stage image is the tile's 32 activation rows (160 chunks, three
// wave loads; lanes past the last chunk re-load it into padding slots), then
// per wave its own 32 weight rows (2 or 3 wave loads).  Every wave issues one
// activation load (wave 3 repeats wave 2's: the same bytes to the same
// place) and its weight loads, so all waves wait for the same count.
// A launch of fewer workgroups than CUs runs eight waves per workgroup
// instead, in K groups, each with its own stage buffers on its share of the
// stages, stepping through the same barriers; at the end groups 1.. pass
// their sums to group 0 through LDS, which adds them to its own before the
// store (the same order on every call).  With one workgroup of four waves
// per CU or fewer, the stage chain of a lone wave per SIMD sets the time;
// two waves per SIMD halve it.  The narrow tile runs four groups of two
// waves on 64 weight rows and K whole (no fill kernel, no atomic adds:
// Q4_0 M = 32, N = 12288, K = 4096: 19.9 us with one group and K split in
// two, 17.2 with two groups of four, 14.8 with four of two); the full tile
// runs two groups of four on each half of a split launch (Q5_1 M = 65 48.4
// -> 39.8 us, Q8_0 37.9 -> 33.9 us).
constexpr int NBM = 32;                    // tokens per narrow tile
// Token counts up to which the narrow tile runs.  Past 64 tokens it would
// run three or four token tiles per weight tile, and the full tile with two
// K groups per workgroup is faster for every format (12288 x 4096, us,
// narrow / full with two K groups: Q4_0 M = 65 36.1 / 32.2, M = 128 39.8 /
// 37.2; Q5_0 39.5 / 34.7, 44.1 / 39.8).
constexpr int narrow_tokens(int) { return 2 * NBM; }
constexpr int NXL = 3;                     // wave loads of activation chunks
template <int WFMT, int WPG = 4> struct WN {   // WPG waves per K group (32 weight rows each)
    using F = WF<WFMT>;
    static constexpr int WL = (32 * F::WC + kWave - 1) / kWave;   // 2, or 3 for Q8_0 weights
    static constexpr int NA = (NXL + WPG - 1) / WPG;              // activation loads per wave
    static constexpr int PER_WAVE = NA + WL;
    static constexpr int AREA = NXL * 1024;                        // activation chunks of a stage
    static constexpr int STAGE = AREA + WPG * WL * 1024;           // 11,264 or 15,360 bytes (WPG = 4)
    static constexpr int NBUF = 3;                                 // stage buffers per K group
    // G groups of WPG waves, each on its own part of K
    template <int G> static constexpr int DXF = G * NBUF * STAGE;
    template <int G> static constexpr int LDS_BYTES = DXF<G> + WPG * G * F::DXW;
    static_assert(NBM * XC <= NXL * kWave && 32 * F::WC <= WL * kWave, "chunks fit the wave loads");
};
}  // namespace mm

// BYTES (4 or 16) per lane from a buffer into LDS: lane i's bytes land at LDS
// byte m0base + OFF + BYTES*i (m0base wave-uniform); the write completes with
// the vector-memory counter.  Issued as inline assembly so that the compiler
// does not see an LDS store: for the intrinsic it conservatively waits for
// every outstanding LDS-DMA load before each later LDS read and before every
// barrier, which would serialise the copy of stage s+2 with the work on stage
// s.  The waits are explicit instead (vmcnt before the barrier that publishes
// a stage).  M0 is formed inside the statement so that the compiler does not
// keep one LDS address per load and stage alive in scalar registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES, int OFF>
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t m0base, uint32_t voff, int soff) {
    static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4");
    if constexpr (BYTES == 16)
        asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(m0base), "v"(voff), "s"(r), "s"(soff), "i"(OFF) : "memory", "m0", "scc");
    else
        asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :: "s"(m0base), "v"(voff), "s"(r), "s"(soff), "i"(OFF) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// fn(integral_constant<I>) for each I of the sequence, in order
template <int... I, class Fn>
__device__ __forceinline__ void each_index(std::integer_sequence<int, I...>, Fn &&fn) {
    (fn(std::integral_constant<int, I>()), ...);
}

// Workgroup barrier that orders LDS accesses but does not wait for
// outstanding vector-memory loads (the LDS-DMA copies in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int WFMT, bool SPLIT, bool NARROW = false, int G = 1, int WPG = 4>
__device__ __forceinline__ void matmul_body(uint8_t *lds, const uint8_t *__restrict__ w,
                                            const uint8_t *__restrict__ xq, float *__restrict__ y, int M, int N,
                                            int nb, int tiles_m) {
    using namespace mm;
    using F = WF<WFMT>;
    constexpr bool Q8W = F::Q8W, Q5 = F::Q5, MIN = F::MIN;
    constexpr int WC = F::WC, WQ = F::WQ;
    using NW_ = WN<WFMT, WPG>;
    constexpr int STAGE = NARROW ? NW_::STAGE : F::STAGE;
    constexpr int PER_WAVE = NARROW ? NW_::PER_WAVE : F::PER_WAVE;
    constexpr int DXF = NARROW ? NW_::template DXF<G> : G == 2 ? F::DXF2 : F::DXF;
    constexpr int NB = NARROW ? NW_::NBUF : NBUF;        // stage buffers; the DMA runs NB - 1 stages ahead
    static_assert(G == 1 || (G == 2 && SPLIT && !NARROW) || (G == 4 && NARROW && WPG == 2 && !SPLIT),
                  "two K groups on split full-tile launches; four groups of two waves on unsplit narrow launches");
    static_assert(NARROW || WPG == 4, "the full tile has four waves per K group");
    constexpr int TBM = NARROW ? NBM : BM;           // tokens per tile
    constexpr int TI = NARROW ? 1 : 2, TJ = NARROW ? 1 : 2;   // A and B tiles per wave
    const int t = threadIdx.x, lane = t & 63;
    const int wave = uniform(G == 1 ? t >> 6 : (t >> 6) % WPG);
    const int grp = G == 1 ? 0 : uniform((t >> 6) / WPG);   // K group: its own stage buffers and blocks
    // SPLIT: the grid holds every tile twice, one per part of K, and both
    // parts add into the zeroed output.  With one K group part 0 takes the
    // first kb1 blocks of each row (whole stages) and part 1 the rest; with
    // G groups part p of P = ksplit * G (grid part and K group) takes stages
    // [p S / P, (p + 1) S / P) of the S = ceil(nb / 2) two-block stages of a
    // row (the caller keeps S >= P).
    constexpr int ksplit = SPLIT ? 2 : 1;
    constexpr int P = ksplit * G;
    const int tiles = (int)gridDim.x / ksplit;
    const int tile = (int)blockIdx.x % tiles, gpart = (int)blockIdx.x / tiles;
    const int mt = tile % tiles_m, nt = tile / tiles_m;
    constexpr int TBN = NARROW ? 32 * WPG : BN;          // weight rows per tile
    const int m0 = mt * TBM, n0 = nt * TBN;
    const uint32_t xrow = (uint32_t)nb * kQ80Bytes, wrow = (uint32_t)nb * F::WB;
    const int S_all = (nb + 1) >> 1;
    auto first_stage = [&](int p) { return p * S_all / P; };
    const int part = G * gpart + grp;
    const int kb1 = 2 * ((nb + 2) / 4);   // G = 1: part 0's blocks (whole stages)
    const int kb0 = G == 1 ? (part ? kb1 : 0) : 2 * first_stage(part);                     // this part's first block
    const int nbp = G == 1 ? (SPLIT ? (part ? nb - kb1 : kb1) : nb) : min(2 * first_stage(part + 1), nb) - kb0;   // its count
    const int nst = (nbp + 1) >> 1;   // an odd block count leaves a last stage of one block
    // every wave of the workgroup passes the same barriers: the K groups
    // step together for the larger of their stage counts
    int nst_wg = nst;
#pragma unroll
    for (int g = 0; g < G; ++g)
        if (G > 1) nst_wg = max(nst_wg, first_stage(G * gpart + g + 1) - first_stage(G * gpart + g));

    // DMA: wave load q = w + 4k (k < 4) of a stage is chunk load q of the
    // stage image (activation chunks for q < 10, weight chunks after) and
    // lands at byte 1024 q of the stage buffer.  Rows past the matrix re-read
    // its last row (their results are not stored).  In the last stage of an
    // odd block count the segments start one block earlier, so that the
    // copy stays inside the row: block 1 of that stage holds the real block
    // and block 0 a copy of the block before it, whose weight scales are
    // taken as 0 (it adds nothing).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + (int64_t)m0 * xrow), 0, (int)((uint32_t)min(M - m0, TBM) * xrow), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + (int64_t)n0 * wrow), 0, (int)((uint32_t)min(N - n0, TBN) * wrow), 0x00020000);
    uint32_t voff[PER_WAVE];
    uint32_t m0k[PER_WAVE];   // narrow: the LDS base of each of this wave's loads
    if constexpr (!NARROW) {
#pragma unroll
        for (int k = 0; k < PER_WAVE; ++k) {
            const int q = wave + 4 * k;
            if (q < XQ) {
                const int f = kWave * q + lane, row = f / XC, c = f - XC * row;
                voff[k] = (uint32_t)(min(m0 + row, M - 1) - m0) * xrow + (uint32_t)xchunk(c);
            } else {
                const int f = kWave * (q - XQ) + lane, row = f / WC, c = f - WC * row;
                voff[k] = (uint32_t)(min(n0 + row, N - 1) - n0) * wrow + (uint32_t)F::wchunk(c);
            }
        }
    }
    // the low half of a generic LDS address is the LDS offset
    uint8_t *const ldsg = lds + grp * (NB * STAGE);   // this K group's stage buffers
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(ldsg);
    const uint32_t m0w = (uint32_t)uniform((int)(lds0 + 1024u * wave));
    if constexpr (NARROW) {
        constexpr int NA = NW_::NA;
#pragma unroll
        for (int k = 0; k < PER_WAVE; ++k) {
            if (k < NA) {
                // activation load min(wave + WPG k, NXL - 1): the last one may
                // repeat another wave's (the same bytes to the same place)
                const int a = min(wave + WPG * k, NXL - 1);
                const int f = min(kWave * a + lane, NBM * XC - 1), row = f / XC, c = f - XC * row;
                voff[k] = (uint32_t)(min(m0 + row, M - 1) - m0) * xrow + (uint32_t)xchunk(c);
                m0k[k] = (uint32_t)uniform((int)(lds0 + 1024u * a));
            } else {
                const int f = min(kWave * (k - NA) + lane, 32 * WC - 1), row = f / WC, c = f - WC * row;
                voff[k] = (uint32_t)(min(n0 + 32 * wave + row, N - 1) - n0) * wrow + (uint32_t)F::wchunk(c);
                m0k[k] = (uint32_t)uniform((int)(lds0 + NW_::AREA + 1024u * (NW_::WL * wave + k - NA)));
            }
        }
    }
    // stage s starts at block kb0 + 2s, or one block earlier for the last
    // stage of an odd count (kb0 >= 2 whenever part 1 has an odd count)
    auto seg = [&](int s) { return kb0 + 2 * s - (2 * s + 1 == nbp ? 1 : 0); };
    auto dma_load = [&](auto kc, int s, int b) {
        constexpr int k = decltype(kc)::value;
        const int sx = seg(s) * kQ80Bytes, sw = seg(s) * F::WB;
        if constexpr (NARROW) {
            constexpr bool isw = k >= NW_::NA;
            buffer_to_lds<16, 0>(isw ? wr : xr, m0k[k] + (uint32_t)(b * STAGE), voff[k], isw ? sw : sx);
        } else {
            const uint32_t base = m0w + (uint32_t)(b * STAGE);
            // load 2: activation chunks for waves 0 and 1, weight chunks for 2 and 3
            const bool isw = k == 2 ? wave >= 2 : k >= 3;
            buffer_to_lds<16, 4096 * k>(isw ? wr : xr, base, voff[k], isw ? sw : sx);
        }
    };
    static_assert(NARROW || (XQ == 10 && (WQ == 6 || WQ == 10) && PER_WAVE == (XQ + WQ) / 4),
                  "the load roles above are written for these splits");
    auto dma = [&](int s, int b) {
        dma_load(std::integral_constant<int, 0>(), s, b);
        dma_load(std::integral_constant<int, 1>(), s, b);
        dma_load(std::integral_constant<int, 2>(), s, b);
        if constexpr (PER_WAVE >= 4) dma_load(std::integral_constant<int, 3>(), s, b);
        if constexpr (PER_WAVE == 5) dma_load(std::integral_constant<int, 4>(), s, b);
    };

    const int wm = NARROW ? 0 : wave & 1, wn = NARROW ? wave : wave >> 1;
    const int lr = lane & 31, lh = lane >> 5;
    // A row 64wm+lr (tile i: +32 rows); narrow: row lr of the tile's 32
    const int xa = NARROW ? 16 * XC * lr : 16 * XC * (64 * wm + lr);
    const int xa_main = xa + (lh ? 0 : 16);              // block 0: chunk 1 (half 0) or 0 (half 1); block 1: +32
    // B row 64wn+lr (tile j: +32 rows); narrow: row lr of this wave's 32
    const int wb = NARROW ? NW_::AREA + 1024 * NW_::WL * wave + 16 * WC * lr
                          : WOFF + 16 * WC * (64 * wn + lr);
    const int wb_main = wb + (lh ? 0 : 16);              // Q8_0 weights: as xa_main
    // the row whose dx this lane converts (narrow: lanes 32..63 repeat 0..31)
    const int xd = NARROW ? 16 * XC * lr : 16 * XC * (64 * wm + lane);
    const int dxw = DXF + F::DXW * (WPG * grp + wave);   // this wave's f32 dx: [block][64 rows 64wm..]
    const uint32_t selA = lh ? 0x03020504u : 0x03020100u;   // half 1: codes 30, 31 into bytes 0, 1
    const uint32_t selB = lh ? 0x07060100u : 0x03020504u;   // block 0, first dword: which bytes take low nibbles
    const uint32_t shHi = lh ? 4u : 0u;                  // shift for a dword that half 0 takes high nibbles of
    const uint32_t shLo = lh ? 0u : 4u;                  // shift for a dword that half 0 takes low nibbles of

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0x4B400000;
    // kept in vector registers for the whole loop; left to itself the
    // allocator rebuilds it from scalar registers in every unrolled stage
    // (8 v_mov_b64 reading the scalar bus, which do not issue in pairs)
    asm volatile("" : "+v"(bias));
    float acc[TI][TJ][16];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // 16*(nib-8) as int8 from a nibble in the high half of each byte
    // The two masks live in vector registers: with either in a scalar
    // register the v_bitop3 this becomes reads the scalar bus and no longer
    // issues in pairs with the other wave's VALU work (measured at two waves
    // per SIMD: 2.7 against 4.8 clocks per instruction).
    uint32_t kHiNib = 0xF0F0F0F0u, kSign = 0x80808080u;
    asm volatile("" : "+v"(kHiNib), "+v"(kSign));
    auto nib = [&](uint32_t v) { return (v & kHiNib) ^ kSign; };
    // Q5_0: 8*(q-16) as int8, q = nibble + 16 * fifth bit, from the nibbles in
    // the high half of each byte of v and the inverted fifth bits nq of the
    // lane's 16 codes (dword k: bits 4k..4k+3): 8*nib in bits 3..6, bit 7 set
    // when the fifth bit is clear (8*nib - 128 as a byte).  The multiply by
    // 0x204081 spreads four bits to the low bit of four bytes (the shifted
    // copies never overlap); the shift by 7 moves them to bit 7.
    auto q5code = [](uint32_t v, uint32_t nq, int k) {
        const uint32_t b = (nq >> (4 * k)) & 15u;
        return ((v >> 1) & 0x78787878u) | (((b * 0x00204081u) << 7) & 0x80808080u);
    };
    auto half_lo = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); };
    auto half_hi = [](uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); };
    auto rd16 = [](const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); };
    auto rd4 = [](const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); };
    auto mfma = [&](const v4i &a, const v4i &b) { return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, bias, 0, 0, 0); };
    // The wave's dx for one stage as f32: lane l converts row 64wm+l's scale
    // of each block (bytes 0..1 of chunk 0 and 2..3 of chunk 2).  Only this
    // wave reads them back, and a wave's LDS accesses complete in order.
    // With an offset term it also stores dx * sx (sx = the block's code sum,
    // exact in f32: 11 + 12 significant bits) at [2 + block][64 rows]: the
    // row's segment bytes 0..63 sit at row offsets 0..63 and bytes 64..67 at
    // 76..79 (chunk 4); block 0's codes are bytes 2..33, block 1's 36..67.
    auto convert_dx = [&](const uint8_t *sb) {
        float *d = reinterpret_cast<float *>(lds + dxw);
        if constexpr (MIN) {
            const uint4 q0 = rd16(sb + xd), q1 = rd16(sb + xd + 16), q2 = rd16(sb + xd + 32),
                        q3 = rd16(sb + xd + 48);
            const uint32_t q19 = rd4(sb + xd + 76);
            constexpr int ones = 0x01010101;
            int s0 = dot4((int)q0.x, 0x01010000, 0);
            s0 = dot4((int)q0.y, ones, dot4((int)q0.z, ones, dot4((int)q0.w, ones, s0)));
            s0 = dot4((int)q1.x, ones, dot4((int)q1.y, ones, dot4((int)q1.z, ones, dot4((int)q1.w, ones, s0))));
            s0 = dot4((int)q2.x, 0x00000101, s0);
            int s1 = dot4((int)q2.y, ones, dot4((int)q2.z, ones, dot4((int)q2.w, ones, 0)));
            s1 = dot4((int)q3.x, ones, dot4((int)q3.y, ones, dot4((int)q3.z, ones, dot4((int)q3.w, ones, s1))));
            s1 = dot4((int)q19, ones, s1);
            const float dx0 = half_lo(q0.x), dx1 = half_hi(q2.x);
            d[lane] = dx0;
            d[64 + lane] = dx1;
            d[128 + lane] = dx0 * (float)s0;
            d[192 + lane] = dx1 * (float)s1;
        } else {
            d[lane] = half_lo(rd4(sb + xd));
            d[64 + lane] = half_hi(rd4(sb + xd + 32));
        }
    };
    // dx of the lane's 16 output rows of A tile i, block kb: rows 8a + 4lh + c
    // of the tile, four 16-byte reads
    auto load_dx = [&](int kb, int i, float (&d)[16]) {
        const float4 *p = reinterpret_cast<const float4 *>(lds + dxw + 4 * (64 * kb + 32 * i + 4 * lh));
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float4 q = p[2 * a];
            d[4 * a] = q.x;
            d[4 * a + 1] = q.y;
            d[4 * a + 2] = q.z;
            d[4 * a + 3] = q.w;
        }
    };
    // The 16 u values first, then the 16 accumulator updates, with a fence
    // between: left to itself the scheduler pairs each u with its update
    // through one temporary, and every pair then waits out the FMA latency.
    auto fold = [&](const v16i &d, int i, int j, const float (&dx)[16], float dw, float nbias) {
        float u[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // element first, then reinterpret: __builtin_bit_cast applied
            // directly to a vector element reads element 0 with this
            // toolchain (hipcc 7.2), so it must not be used here
            const int e = d[r];
            u[r] = fmaf(__int_as_float(e), dw, nbias);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(u[r], dx[r], acc[i][j][r]);
    };

    // Chunks of one stage for this lane: per A tile the block-0 and block-1
    // main chunks and chunk 4; per B tile the three Q4_0 weight chunks, or for
    // Q8_0 weights the same three chunks as for A plus the two scale dwords.
    struct RawQ4 {
        uint4 a0[2], a1[2], a4[2], w0[2], w1[2], w2[2];
    };
    struct RawQ8 {
        uint4 a0[2], a1[2], a4[2], b0[2], b1[2], b4[2];
        uint32_t s0[2], s2[2];
    };
    using Raw = std::conditional_t<Q8W, RawQ8, RawQ4>;
    struct Ops {
        v4i a[2], b[2];
        float dw[2], nb[2];
    };
    auto load_raw = [&](const uint8_t *sb, Raw &r) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            r.a0[i] = rd16(sb + xa_main + 16 * XC * 32 * i);
            r.a1[i] = rd16(sb + xa_main + 32 + 16 * XC * 32 * i);
            r.a4[i] = rd16(sb + xa + 64 + 16 * XC * 32 * i);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if constexpr (Q8W) {
                r.b0[j] = rd16(sb + wb_main + 16 * WC * 32 * j);
                r.b1[j] = rd16(sb + wb_main + 32 + 16 * WC * 32 * j);
                r.b4[j] = rd16(sb + wb + 64 + 16 * WC * 32 * j);
                r.s0[j] = rd4(sb + wb + 16 * WC * 32 * j);
                r.s2[j] = rd4(sb + wb + 32 + 16 * WC * 32 * j);
            } else {
                r.w0[j] = rd16(sb + wb + 16 * WC * 32 * j);
                r.w1[j] = rd16(sb + wb + 16 + 16 * WC * 32 * j);
                r.w2[j] = rd16(sb + wb + 32 + 16 * WC * 32 * j);
            }
        }
    };
    auto set_scale = [&](Ops &o, int j, float dw) {
        o.dw[j] = dw;
        // keep dw an f32 register: folded back into the fold, the f16
        // conversion would turn each v_fma_f32 into a half-rate v_fma_mix
        asm volatile("" : "+v"(o.dw[j]));
        o.nb[j] = o.dw[j] * -kBias;   // exact: 11 + 2 significant bits
    };
    auto build0 = [&](const Raw &r, bool absent, Ops &o) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const uint4 c = r.a0[i];   // chunk 1 (half 0) or chunk 0 (half 1)
            o.a[i] = v4i{(int)__builtin_amdgcn_perm(r.a1[i].x, c.x, selA), (int)c.y, (int)c.z, (int)c.w};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if constexpr (Q8W) {
                const uint4 c = r.b0[j];
                o.b[j] = v4i{(int)__builtin_amdgcn_perm(r.b1[j].x, c.x, selA), (int)c.y, (int)c.z, (int)c.w};
                set_scale(o, j, absent ? 0.0f : half_lo(r.s0[j]));
            } else if constexpr (F::Q41 || F::Q51) {
                // block 0: d, m at 0, 2, then (Q5_1) qh at 4..7, and qs at 4
                // (Q4_1) or 8 (Q5_1); the rotated nibble bytes 14, 15, 0..13
                // are two bytes off the dword grid
                const uint4 c0 = r.w0[j], c1 = r.w1[j];
                const uint32_t a = F::Q41 ? c0.y : c0.z, b = F::Q41 ? c0.z : c0.w, c = F::Q41 ? c0.w : c1.x,
                               e = F::Q41 ? c1.x : c1.y;   // nibble bytes 0..3, 4..7, 8..11, 12..15
                const uint32_t P = __builtin_amdgcn_perm(e, a, 0x01000706u);   // bytes 14, 15, 0, 1
                const uint32_t Pm = __builtin_amdgcn_perm(P << 4, P, selB);
                const uint32_t D1 = __builtin_amdgcn_alignbyte(b, a, 2), D2 = __builtin_amdgcn_alignbyte(c, b, 2),
                               D3 = __builtin_amdgcn_alignbyte(e, c, 2);
                if constexpr (F::Q51) {
                    const uint32_t nq = ~__builtin_amdgcn_alignbit(c0.y, c0.y, lh ? 30u : 14u);
                    o.b[j] = v4i{(int)q5code(Pm, nq, 0), (int)q5code(D1 << shHi, nq, 1),
                                 (int)q5code(D2 << shHi, nq, 2), (int)q5code(D3 << shHi, nq, 3)};
                } else {
                    o.b[j] = v4i{(int)nib(Pm), (int)nib(D1 << shHi), (int)nib(D2 << shHi), (int)nib(D3 << shHi)};
                }
                set_scale(o, j, absent ? 0.0f : half_lo(c0.x));
            } else if constexpr (Q5) {
                // block 0 of the 44-byte segment: d at 0, qh at 2..5, qs at
                // 6..21; its nibble bytes 14, 15, 0..13 are segment bytes
                // 20, 21, 6..19
                const uint4 c0 = r.w0[j], c1 = r.w1[j];
                const uint32_t P = __builtin_amdgcn_perm(c1.y, c0.y, 0x03020504u);
                const uint32_t Pm = __builtin_amdgcn_perm(P << 4, P, selB);
                const uint32_t qh = __builtin_amdgcn_alignbyte(c0.y, c0.x, 2);
                const uint32_t nq = ~__builtin_amdgcn_alignbit(qh, qh, lh ? 30u : 14u);   // codes 14.. or 30, 31, 0..
                o.b[j] = v4i{(int)q5code(Pm, nq, 0), (int)q5code(c0.z << shHi, nq, 1),
                             (int)q5code(c0.w << shHi, nq, 2), (int)q5code(c1.x << shHi, nq, 3)};
                set_scale(o, j, absent ? 0.0f : half_lo(c0.x));
            } else {
                const uint4 c0 = r.w0[j];
                const uint32_t P = __builtin_amdgcn_perm(r.w1[j].x, c0.x, 0x03020504u);   // nibble bytes 14, 15, 0, 1
                const uint32_t Pm = __builtin_amdgcn_perm(P << 4, P, selB);
                o.b[j] = v4i{(int)nib(Pm), (int)nib(c0.y << shHi), (int)nib(c0.z << shHi), (int)nib(c0.w << shHi)};
                set_scale(o, j, absent ? 0.0f : half_lo(c0.x));
            }
        }
    };
    auto build1 = [&](const Raw &r, Ops &o) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const uint4 c = r.a1[i];   // chunk 3 (half 0) or chunk 2 (half 1)
            const uint32_t d0 = lh ? r.a4[i].w : c.x;
            o.a[i] = v4i{(int)d0, (int)c.y, (int)c.z, (int)c.w};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if constexpr (Q8W) {
                const uint4 c = r.b1[j];
                const uint32_t d0 = lh ? r.b4[j].w : c.x;
                o.b[j] = v4i{(int)d0, (int)c.y, (int)c.z, (int)c.w};
                set_scale(o, j, half_hi(r.s2[j]));
            } else if constexpr (F::Q41 || F::Q51) {
                // block 1: d, m at segment 20 (Q4_1) or 24 (Q5_1), Q5_1's qh
                // at 28..31, the nibble bytes in chunk 2
                const uint4 c1 = r.w1[j], c2 = r.w2[j];
                if constexpr (F::Q51) {
                    const uint32_t nq = ~__builtin_amdgcn_alignbit(c1.w, c1.w, lh ? 28u : 12u);
                    o.b[j] = v4i{(int)q5code(c2.w << shLo, nq, 0), (int)q5code(c2.x << shHi, nq, 1),
                                 (int)q5code(c2.y << shHi, nq, 2), (int)q5code(c2.z << shHi, nq, 3)};
                } else {
                    o.b[j] = v4i{(int)nib(c2.w << shLo), (int)nib(c2.x << shHi), (int)nib(c2.y << shHi),
                                 (int)nib(c2.z << shHi)};
                }
                set_scale(o, j, half_lo(F::Q41 ? c1.y : c1.z));
            } else if constexpr (Q5) {
                // block 1: d at segment 22, qh at 24..27, qs at 28..43 (chunk 2)
                const uint4 c1 = r.w1[j], c2 = r.w2[j];
                const uint32_t nq = ~__builtin_amdgcn_alignbit(c1.z, c1.z, lh ? 28u : 12u);   // codes 12.. or 28..31, 0..
                o.b[j] = v4i{(int)q5code(c2.w << shLo, nq, 0), (int)q5code(c2.x << shHi, nq, 1),
                             (int)q5code(c2.y << shHi, nq, 2), (int)q5code(c2.z << shHi, nq, 3)};
                set_scale(o, j, half_hi(c1.y));
            } else {
                const uint4 c2 = r.w2[j];   // nibble bytes 0..15 of block 1
                o.b[j] = v4i{(int)nib(c2.w << shLo), (int)nib(c2.x << shHi), (int)nib(c2.y << shHi),
                             (int)nib(c2.z << shHi)};
                set_scale(o, j, half_hi(r.w1[j].x));
            }
        }
    };

    // Offset term of the formats whose value is d q + m (Q4_1, Q5_1).  With
    // the codes entering as 16 (q - 8) (Q4_1) or 8 (q - 16) (Q5_1) the MFMA
    // gives I' = sum q' x, and the block adds (to the accumulator, which the
    // store scales by S = OUT_SCALE)
    //   dx d I' + (dx sx) (128 d + m / S),   sx = the activation's code sum.
    // The second part is an outer product summed over the stage's two blocks:
    // one v_mfma_f32_32x32x2_f32 per tile and stage, straight into the f32
    // accumulator, K = block.  Lane half h supplies block h: A = dx sx of row
    // lr of the tile (from convert_dx), B = 128 d + m/S of column lr (one
    // rounding; 0 for the duplicated block 0 of an odd last stage).
    auto offset_operands = [&](const Raw &r, bool absent0, float (&ao)[2], float (&bo)[2]) {
        const float *d = reinterpret_cast<const float *>(lds + dxw);
#pragma unroll
        for (int i = 0; i < TI; ++i) ao[i] = d[128 + 64 * lh + 32 * i + lr];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if constexpr (MIN) {
                const uint32_t sc = lh ? (F::Q41 ? r.w1[j].y : r.w1[j].z) : r.w0[j].x;
                const float c = fmaf(half_lo(sc), 128.0f, half_hi(sc) * (1.0f / F::OUT_SCALE));
                bo[j] = (absent0 && !lh) ? 0.0f : c;
            }
        }
    };
    auto offset_mfma = [&](int i, int j, float a, float b) {
        v16f c;
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = acc[i][j][r];
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = c[r];
    };

    // One stage: 2 blocks x 4 tiles in an explicit order, fenced against the
    // scheduler.  The MFMA of tile t+1 is issued before the fold of tile t
    // (a fold never waits for its MFMA and two MFMAs never queue back to
    // back), dx reads go out one fold ahead, and the DMA of stage sd into
    // buffer bd is spread over the first four folds so that a workgroup's
    // loads do not queue up at the texture unit at once.
    auto compute = [&](const uint8_t *sb, bool absent0, int sd, int bd) __attribute__((always_inline)) {
        Raw r;
        Ops o0, o1;
        float dxa[16], dxb[16];
        if constexpr (NARROW) {
            // one tile: the MFMA of block 1 is issued before the fold of block 0
            float ao[2], bo[2];
            convert_dx(sb);
            load_raw(sb, r);
            if constexpr (MIN) offset_operands(r, absent0, ao, bo);
            load_dx(0, 0, dxa);
            load_dx(1, 0, dxb);
            build0(r, absent0, o0);
            v16i d0 = mfma(o0.a[0], o0.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            dma(sd, bd);
            __builtin_amdgcn_sched_barrier(0);
            build1(r, o1);
            v16i d1 = mfma(o1.a[0], o1.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d0, 0, 0, dxa, o0.dw[0], o0.nb[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d1, 0, 0, dxb, o1.dw[0], o1.nb[0]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MIN) {
                offset_mfma(0, 0, ao[0], bo[0]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            auto dma_after = [&](auto kc) {
                dma_load(kc, sd, bd);
                __builtin_amdgcn_sched_barrier(0);
            };
            float ao[2], bo[2];
            convert_dx(sb);
            load_raw(sb, r);
            if constexpr (MIN) offset_operands(r, absent0, ao, bo);
            load_dx(0, 0, dxa);
            build0(r, absent0, o0);
            v16i d0 = mfma(o0.a[0], o0.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            load_dx(0, 1, dxb);
            v16i d1 = mfma(o0.a[0], o0.b[1]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d0, 0, 0, dxa, o0.dw[0], o0.nb[0]);
            dma_after(std::integral_constant<int, 0>());
            d0 = mfma(o0.a[1], o0.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d1, 0, 1, dxa, o0.dw[1], o0.nb[1]);
            dma_after(std::integral_constant<int, 1>());
            d1 = mfma(o0.a[1], o0.b[1]);
            load_dx(1, 0, dxa);
            __builtin_amdgcn_sched_barrier(0);
            fold(d0, 1, 0, dxb, o0.dw[0], o0.nb[0]);
            dma_after(std::integral_constant<int, 2>());
            build1(r, o1);
            d0 = mfma(o1.a[0], o1.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d1, 1, 1, dxb, o0.dw[1], o0.nb[1]);
            dma_after(std::integral_constant<int, 3>());
            d1 = mfma(o1.a[0], o1.b[1]);
            load_dx(1, 1, dxb);
            __builtin_amdgcn_sched_barrier(0);
            fold(d0, 0, 0, dxa, o1.dw[0], o1.nb[0]);
            if constexpr (PER_WAVE == 5) dma_load(std::integral_constant<int, 4>(), sd, bd);
            __builtin_amdgcn_sched_barrier(0);
            d0 = mfma(o1.a[1], o1.b[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d1, 0, 1, dxa, o1.dw[1], o1.nb[1]);
            __builtin_amdgcn_sched_barrier(0);
            d1 = mfma(o1.a[1], o1.b[1]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d0, 1, 0, dxb, o1.dw[0], o1.nb[0]);
            __builtin_amdgcn_sched_barrier(0);
            fold(d1, 1, 1, dxb, o1.dw[1], o1.nb[1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MIN) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) offset_mfma(i, j, ao[i], bo[j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Stage s lives in buffer s % NB.  At step s this wave's loads of stage
    // s have landed once at most the PER_WAVE loads of each later stage in
    // flight are outstanding; the barrier publishes every wave's and frees
    // buffer (s-1) % NB, which the DMA of stage s+NB-1 then fills.  The last
    // steps have no such stage and copy the last stage again into that idle
    // buffer instead, so that every step issues the same loads and waits for
    // the same count.  A K group with fewer stages than the other passes its
    // extra step's barrier without work or loads.
    auto step = [&](int s, auto bc) {
        constexpr int b = decltype(bc)::value;
        asm volatile("s_waitcnt vmcnt(%0)" :: "i"((NB - 2) * PER_WAVE) : "memory");
        lds_barrier();
        if (G == 1 || s < nst) compute(ldsg + b * STAGE, 2 * s + 1 == nbp, min(s + NB - 1, nst - 1), (b + NB - 1) % NB);
    };
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k) dma(min(k, nst - 1), k);
    for (int s = 0; s < nst_wg; s += NB) {
        each_index(std::make_integer_sequence<int, NB>(), [&](auto bc) {
            if (decltype(bc)::value == 0 || s + decltype(bc)::value < nst_wg) step(s + decltype(bc)::value, bc);
        });
    }
    // no LDS-DMA write may still be in flight when the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (G > 1) {
        // groups 1 .. G-1 hand their sums to group 0 through LDS
        // ([group - 1][tile][wave][r][lane], over the stage buffers), which
        // adds them to its own in group order: the same order on every call
        constexpr int TS = 1024 * WPG;                   // floats per tile and group
        float *red = reinterpret_cast<float *>(lds) + 1024 * wave + lane;
        lds_barrier();
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[TS * (TI * TJ * (grp - 1) + TJ * i + j) + 64 * r] = acc[i][j][r];
        }
        lds_barrier();
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < G; ++g)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += red[TS * (TI * TJ * (g - 1) + TJ * i + j) + 64 * r];
    }

    // store: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int n = n0 + (NARROW ? 32 * wave : 64 * wn + 32 * j) + lr;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + (NARROW ? 0 : 64 * wm + 32 * i) + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m >= M) continue;
                // two addends on a zeroed output: the same sum in either order
                if constexpr (SPLIT)
                    atomicAdd(y + (int64_t)m * N + n, acc[i][j][r] * F::OUT_SCALE);
                else
                    y[(int64_t)m * N + n] = acc[i][j][r] * F::OUT_SCALE;
            }
        }
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_0(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q4_0>::LDS_BYTES];
    matmul_body<F_Q4_0, false>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_0_split(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q4_0>::LDS_BYTES];
    matmul_body<F_Q4_0, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q8_0(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q8_0>::LDS_BYTES];
    matmul_body<F_Q8_0, false>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q8_0_split(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q8_0>::LDS_BYTES];
    matmul_body<F_Q8_0, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q5_0(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q5_0>::LDS_BYTES];
    matmul_body<F_Q5_0, false>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q5_0_split(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q5_0>::LDS_BYTES];
    matmul_body<F_Q5_0, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_1(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q4_1>::LDS_BYTES];
    matmul_body<F_Q4_1, false>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_1_split(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q4_1>::LDS_BYTES];
    matmul_body<F_Q4_1, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q5_1(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                          int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q5_1>::LDS_BYTES];
    matmul_body<F_Q5_1, false>(lds, w, xq, y, M, N, nb, tiles_m);
}

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q5_1_split(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                int M, int N, int nb, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<F_Q5_1>::LDS_BYTES];
    matmul_body<F_Q5_1, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

// The 128-token tile with two groups of four waves, each on half of the
// workgroup's part of K, for split launches of fewer workgroups than CUs.
template <int WFMT>
__global__ __launch_bounds__(2 * mm::NT, 1) void k_matmul_wide2(const uint8_t *__restrict__ w,
                                                               const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                               int M, int N, int nb, int tiles_m) {
    static_assert(mm::WF<WFMT>::LDS_BYTES2 <= 160 * 1024, "LDS of one CU");
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WF<WFMT>::LDS_BYTES2];
    matmul_body<WFMT, true, false, 2>(lds, w, xq, y, M, N, nb, tiles_m);
}

// The narrow tile of 32 tokens x 64 weight rows with four groups of two
// waves, each on a quarter of K, for launches of fewer narrow workgroups
// than CUs: the K parallelism of a split launch with two groups, without
// the fill kernel and the atomic adds.
template <int WFMT>
__global__ __launch_bounds__(2 * mm::NT, 1) void k_matmul_narrow4(const uint8_t *__restrict__ w,
                                                                 const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                                 int M, int N, int nb, int tiles_m) {
    static_assert(mm::WN<WFMT, 2>::template LDS_BYTES<4> <= 160 * 1024, "LDS of one CU");
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WN<WFMT, 2>::template LDS_BYTES<4>];
    matmul_body<WFMT, false, true, 4, 2>(lds, w, xq, y, M, N, nb, tiles_m);
}

// The narrow tile (32 tokens x 128 weight rows) for launches of up to
// narrow_tokens tokens, every 32-value format, K in one part or split in two.
template <int WFMT, bool SPLIT>
__global__ __launch_bounds__(mm::NT, 2) void k_matmul_narrow(const uint8_t *__restrict__ w,
                                                            const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                            int M, int N, int nb, int tiles_m) {
    static_assert(2 * mm::WN<WFMT>::template LDS_BYTES<1> <= 160 * 1024, "two workgroups per CU");
    __shared__ __attribute__((aligned(16))) uint8_t lds[mm::WN<WFMT>::template LDS_BYTES<1>];
    matmul_body<WFMT, SPLIT, true>(lds, w, xq, y, M, N, nb, tiles_m);
}

// K = 32: one block per row, too short for the two-block stages above (the
// window of an odd last stage would start before the row).  One thread per
// output: Y[m][n] = dx dw I with I the exact int32 block dot.
__global__ __launch_bounds__(256) void k_matmul_q4_0_one_block(const uint8_t *__restrict__ w,
                                                               const uint8_t *__restrict__ xq,
                                                               float *__restrict__ y, int M, int N) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= (int64_t)M * N) return;
    const int m = (int)(o / N), n = (int)(o - (int64_t)m * N);
    const uint8_t *xb = xq + (int64_t)m * kQ80Bytes;
    const uint8_t *wb = w + (int64_t)n * kQ40Bytes;
    int isum = 0;
    for (int j = 0; j < 16; ++j) {
        const int b = wb[2 + j];
        isum += (int)(int8_t)xb[2 + j] * ((b & 15) - 8) + (int)(int8_t)xb[18 + j] * ((b >> 4) - 8);
    }
    const float dx = f16_bits_to_f32((uint32_t)xb[0] | (uint32_t)xb[1] << 8);
    const float dw = f16_bits_to_f32((uint32_t)wb[0] | (uint32_t)wb[1] << 8);
    y[o] = (float)isum * dw * dx;
}

__global__ __launch_bounds__(256) void k_matmul_q8_0_one_block(const uint8_t *__restrict__ w,
                                                               const uint8_t *__restrict__ xq,
                                                               float *__restrict__ y, int M, int N) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= (int64_t)M * N) return;
    const int m = (int)(o / N), n = (int)(o - (int64_t)m * N);
    const uint8_t *xb = xq + (int64_t)m * kQ80Bytes;
    const uint8_t *wb = w + (int64_t)n * kQ80Bytes;
    int isum = 0;
    for (int j = 0; j < 32; ++j) isum += (int)(int8_t)xb[2 + j] * (int)(int8_t)wb[2 + j];
    const float dx = f16_bits_to_f32((uint32_t)xb[0] | (uint32_t)xb[1] << 8);
    const float dw = f16_bits_to_f32((uint32_t)wb[0] | (uint32_t)wb[1] << 8);
    y[o] = (float)isum * dw * dx;
}

// The same for the 32-value formats with a fifth bit or an offset (Q4_1,
// Q5_0, Q5_1): Y[m][n] = dx (dw sum q' x + m sum x), q' = q (Q5_0: q - 16),
// both integer sums exact.
template <int WFMT>
__global__ __launch_bounds__(256) void k_matmul_32_one_block(const uint8_t *__restrict__ w,
                                                             const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                             int M, int N) {
    constexpr int WB = WFMT == F_Q4_1 ? kQ41Bytes : WFMT == F_Q5_0 ? kQ50Bytes : kQ51Bytes;
    constexpr int QH = WFMT == F_Q5_0 ? 2 : 4;                               // qh offset (Q5_0, Q5_1)
    constexpr int QS = WFMT == F_Q4_1 ? 4 : WFMT == F_Q5_0 ? 6 : 8;          // qs offset
    constexpr int OFF = WFMT == F_Q5_0 ? 16 : 0;
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= (int64_t)M * N) return;
    const int m = (int)(o / N), n = (int)(o - (int64_t)m * N);
    const uint8_t *xb = xq + (int64_t)m * kQ80Bytes;
    const uint8_t *wb = w + (int64_t)n * WB;
    const uint32_t qh = WFMT == F_Q4_1 ? 0u
                                        : (uint32_t)wb[QH] | (uint32_t)wb[QH + 1] << 8 |
                                              (uint32_t)wb[QH + 2] << 16 | (uint32_t)wb[QH + 3] << 24;
    int isum = 0, xsum = 0;
    for (int j = 0; j < 16; ++j) {
        const int b = wb[QS + j];
        const int lo = (b & 15) | (int)((qh >> j) & 1u) << 4, hi = (b >> 4) | (int)((qh >> (j + 16)) & 1u) << 4;
        const int x0 = (int8_t)xb[2 + j], x1 = (int8_t)xb[18 + j];
        isum += x0 * (lo - OFF) + x1 * (hi - OFF);
        xsum += x0 + x1;
    }
    const float dx = f16_bits_to_f32((uint32_t)xb[0] | (uint32_t)xb[1] << 8);
    const float dw = f16_bits_to_f32((uint32_t)wb[0] | (uint32_t)wb[1] << 8);
    const float mw = WFMT == F_Q5_0 ? 0.0f : f16_bits_to_f32((uint32_t)wb[2] | (uint32_t)wb[3] << 8);
    y[o] = fmaf(dw, (float)isum, mw * (float)xsum) * dx;
}

// Largest block count whose tile offsets fit the 32-bit buffer offsets
// (128 activation or Q8_0 weight rows of nb * 34 bytes).
constexpr int64_t kMatmulMaxBlocks = (((int64_t)1 << 31) - 1) / (mm::BM * kQ80Bytes);

int64_t matmul_q4_0_max_blocks() { return kMatmulMaxBlocks; }

__global__ __launch_bounds__(256) void k_zero_f32(float *__restrict__ y, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        *reinterpret_cast<float4 *>(y + i) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
        for (int64_t k = i; k < n; ++k) y[k] = 0.0f;
    }
}

hipError_t launch_zero_f32(float *y, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t grid = (n + 1023) / 1024;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)grid), dim3(256), 0, st, y, n);
    return hipGetLastError();
}

template <int WFMT>
static hipError_t launch_mm(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    if (nb > kMatmulMaxBlocks) return hipErrorInvalidValue;
    if (M <= small_tokens(WFMT)) return launch_matvec_tokens(WFMT, w, xq, y, M, N, nb, st);
    if (nb == 1) {
        const int64_t outs = (int64_t)M * N;
        const int64_t grid = (outs + 255) / 256;
        if (grid > 0x7fffffff) return hipErrorInvalidValue;
        const auto one = WFMT == F_Q8_0 ? k_matmul_q8_0_one_block
                         : WFMT == F_Q4_0 ? k_matmul_q4_0_one_block
                                          : k_matmul_32_one_block<WFMT>;
        hipLaunchKernelGGL(one, dim3((unsigned)grid), dim3(256), 0, st, wp, xp, y, M, N);
        return hipGetLastError();
    }
    // up to narrow_tokens: the 32-token tile (a 128-token tile would compute
    // and drop the rows past M)
    const bool narrow = M <= mm::narrow_tokens(WFMT);
    int tiles_m = narrow ? (M + mm::NBM - 1) / mm::NBM : (M + mm::BM - 1) / mm::BM;
    const int64_t tiles = (int64_t)tiles_m * ((N + mm::BN - 1) / mm::BN);
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&nb, (void *)&tiles_m};
    // Fewer narrow workgroups than CUs: four groups of two waves on 64
    // weight rows per workgroup, each on a quarter of K (at least two stages
    // each), written with plain stores.
    if (narrow && tiles * 2 < kCUs && nb >= 16) {
        const int64_t tiles64 = (int64_t)tiles_m * ((N + 63) / 64);
        return hipLaunchKernel((const void *)k_matmul_narrow4<WFMT>, dim3((unsigned)tiles64), dim3(2 * mm::NT), args,
                               0, st);
    }
    // A launch of at most one workgroup per CU leaves the CUs half idle and
    // each workgroup alone on its CU: split K in two, the parts adding into
    // an output zeroed first.
    const bool split = tiles <= kSplitTiles && nb >= 4;
    if (split) {
        const hipError_t e = launch_zero_f32(y, (int64_t)M * N, st);
        if (e != hipSuccess) return e;
    }
    const int ksplit = split ? 2 : 1;
    // Fewer full-tile workgroups than CUs: two groups of four waves per
    // workgroup, each on half of its part of K (at least four stages each).
    const bool groups = !narrow && split && tiles * 2 < kCUs && nb >= 16;
    const void *kern = groups           ? (const void *)k_matmul_wide2<WFMT>
                       : narrow         ? (split ? (const void *)k_matmul_narrow<WFMT, true>
                                                 : (const void *)k_matmul_narrow<WFMT, false>)
                       : WFMT == F_Q8_0 ? (split ? (const void *)k_matmul_q8_0_split : (const void *)k_matmul_q8_0)
                       : WFMT == F_Q5_0 ? (split ? (const void *)k_matmul_q5_0_split : (const void *)k_matmul_q5_0)
                       : WFMT == F_Q4_1 ? (split ? (const void *)k_matmul_q4_1_split : (const void *)k_matmul_q4_1)
                       : WFMT == F_Q5_1 ? (split ? (const void *)k_matmul_q5_1_split : (const void *)k_matmul_q5_1)
                       : split          ? (const void *)k_matmul_q4_0_split
                                        : (const void *)k_matmul_q4_0;
    return hipLaunchKernel(kern, dim3((unsigned)(tiles * ksplit)), dim3(groups ? 2 * mm::NT : mm::NT), args, 0, st);
}

hipError_t launch_matmul_q4_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    return launch_mm<F_Q4_0>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matmul_q8_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    return launch_mm<F_Q8_0>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matmul_q5_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    return launch_mm<F_Q5_0>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matmul_q4_1(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    return launch_mm<F_Q4_1>(w, xq, y, M, N, nb, st);
}

hipError_t launch_matmul_q5_1(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    return launch_mm<F_Q5_1>(w, xq, y, M, N, nb, st);
}

}  // namespace qmm
