// Prefill matmul, Q4_0 weights x Q8_0 activations, on int8 MFMA.
//
//   Y[m][n] = sum_b dx[m,b] dw[n,b] I_b[m,n],   I_b = sum_{k<32} q[m,32b+k] (w[n,32b+k]-8)
//
// Once a weight tile is reused across many tokens the product is a dense
// contraction (kvad "Batched prefill, and i8mm"; krafla "Batched prompt
// prefill"), and one 32-value block is exactly the K of
// v_mfma_i32_32x32x32_i8, so every block gets its own exact int32 tile.
//
// Workgroup tile: 128 tokens x 128 weight rows, 4 waves of 64x64 (2x2 MFMA
// tiles of 32x32); two workgroups share a CU (80 KB of LDS each), so the two
// waves on a SIMD belong to different workgroups and do not meet at the same
// barriers.  The K loop moves KB = 2 blocks per stage through LDS:
//   1. the tile's row segments are copied raw into LDS by gfx950 LDS-DMA
//      loads (16 bytes per lane, coalesced, no registers), one stage ahead;
//   2. a re-layout pass slices the 2-byte-aligned blocks out of the raw rows:
//      activation codes go to [kb][m][32] int8 and their f16 scales to
//      [kb][m]; weight nibbles are unpacked once per workgroup into signed
//      bytes 16*(nib-8) (XOR 0x88 then shift/mask, krafla "Weight packing")
//      and their scales to [kb][n] as f32 dw/16 (exact: a power of two);
//   3. each wave reads its MFMA operands with one ds_read_b128 per 32x32 tile
//      (lane = row, lane half = which 16 of the 32 codes; A and B use the same
//      split, so the k order inside the instruction does not matter).
// Raw and re-laid-out buffers are both double-buffered, so a stage costs one
// barrier: DMA for stage s+2, re-layout of stage s+1 and the MFMA work of
// stage s all run between two barriers.
// Scale fold: the MFMA's C input is the constant 0x4B400000, so the int32
// result read as f32 is exactly 1.5*2^23 + 16 I (|16 I| < 2^22); then
//   u = fma(F, dw/16, -1.5*2^23*dw/16) = I*dw   (one rounding)
//   acc = fma(u, dx, acc)                       (one rounding; dx read as f16)
// Output lane layout of a 32x32 MFMA tile: lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4 and column l%32.
#include "qmm_device.h"

namespace qmm {

namespace mm {
constexpr int BM = 128;                 // tokens per workgroup tile
constexpr int BN = 128;                 // weight rows per workgroup tile
constexpr int KB = 2;                   // blocks (of 32) per stage
constexpr int NT = 256;                 // threads (4 waves: 2 along tokens x 2 along weight rows)
// 16-byte chunks per raw row segment: 2 blocks plus up to 14 bytes of
// misalignment need at most 6 (activations, 68 B) and 4 (weights, 36 B); the
// weight rows get one more slot to spread consecutive rows over the LDS banks
constexpr int XCH = 6;
constexpr int WCH = 5;
constexpr int RAWX = BM * XCH;          // chunks of raw activation rows per stage (768)
constexpr int RAW = RAWX + BN * WCH;    // chunks per stage (1408)
constexpr int DMA_GROUPS = (RAW + kWave - 1) / kWave;   // 64-chunk DMA instructions per stage (22)
constexpr float kBias = 12582912.0f;    // 1.5 * 2^23, bit pattern 0x4B400000
}  // namespace mm

// 80,896 bytes: two workgroups fit in the 160 KB of LDS of a CU
struct MmShared {
    uint4 raw[2][mm::DMA_GROUPS * kWave];  // 2 x 22 KB (DMA groups are whole)
    uint4 a[2][mm::KB][mm::BM][2];         // activation codes, 2 x 8 KB
    uint4 b[2][mm::KB][mm::BN][2];         // weight codes * 16, 2 x 8 KB
    _Float16 dx[2][mm::KB][mm::BM];        // 2 x 512 B
    float dw[2][mm::KB][mm::BN];           // dw / 16, 2 x 1 KB
};
static_assert(sizeof(MmShared) <= 81920, "two workgroups per CU");

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_0_any(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                                        float *__restrict__ y, int M, int N, int nb, int tiles_m) {
    using namespace mm;
    extern __shared__ uint4 lds_dyn[];
    MmShared &sh = *reinterpret_cast<MmShared *>(lds_dyn);
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int mt = blockIdx.x % tiles_m, nt = blockIdx.x / tiles_m;
    const int m0 = mt * BM, n0 = nt * BN;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t xrow = (int64_t)nb * kQ80Bytes, wrow = (int64_t)nb * kQ40Bytes;
    const int nst = (nb + KB - 1) / KB;

    // Raw stage image: chunk q < RAWX is chunk q % XCH of activation row q / XCH,
    // chunk q >= RAWX chunk (q-RAWX) % WCH of weight row (q-RAWX) / WCH; DMA group
    // g (chunks 64g..64g+63) is all-activation for g < 12 and all-weight after.
    // A row segment starts at its 16-byte granule; slots past the segment's
    // last chunk re-read that chunk (the same address as a neighbouring lane,
    // so the load is merged), and rows past the matrix re-read its last row,
    // so every load stays inside the buffer.
    static_assert(RAWX % kWave == 0, "activation and weight chunks must not share a DMA group");
    constexpr int MAXG = (DMA_GROUPS + NT / kWave - 1) / (NT / kWave);   // groups per wave (6)
    const int ndma = (DMA_GROUPS - wave + NT / kWave - 1) / (NT / kWave); // groups this wave issues
    int64_t gbase[MAXG];          // byte offset of this lane's row start
    int gc[MAXG];                 // chunk index within the row segment
#pragma unroll
    for (int j = 0; j < MAXG; ++j) {
        const int g = wave + j * (NT / kWave);
        const int q = min(g * kWave + lane, RAW - 1);
        if (q < RAWX) {
            const int r = q / XCH;
            gbase[j] = (int64_t)min(m0 + r, M - 1) * xrow;
            gc[j] = q - r * XCH;
        } else {
            const int r = (q - RAWX) / WCH;
            gbase[j] = (int64_t)min(n0 + r, N - 1) * wrow;
            gc[j] = q - RAWX - r * WCH;
        }
    }
    auto dma_stage = [&](int s) {
        const int b0 = s * KB, bl = min(KB, nb - b0);
        uint4 *dst = sh.raw[s & 1];
#pragma unroll
        for (int j = 0; j < MAXG; ++j) {
            const int g = wave + j * (NT / kWave);
            if (g < DMA_GROUPS) {
                const bool isx = g * kWave < RAWX;
                const int bb = isx ? kQ80Bytes : kQ40Bytes;
                const int64_t lo = gbase[j] + (int64_t)b0 * bb;
                const int last = ((int)(lo & 15) + bl * bb - 1) >> 4;
                const int64_t a = (lo & ~(int64_t)15) + 16 * min(gc[j], last);
                global_to_lds16((isx ? xq : w) + a, dst + g * kWave);
            }
        }
    };

    const uint32_t xrbase = (uint32_t)((int64_t)min(m0 + (t >> 1), M - 1) * xrow);   // low bits suffice:
    const uint32_t wrbase = (uint32_t)((int64_t)min(n0 + (t >> 1), N - 1) * wrow);   // only & 15 is used
    auto relayout = [&](int s) {
        const int b0 = s * KB, bl = min(KB, nb - b0), buf = s & 1;
        const uint8_t *rb = reinterpret_cast<const uint8_t *>(sh.raw[s & 1]);
        const uint32_t *r32 = reinterpret_cast<const uint32_t *>(rb);
        {
            const int r = t >> 1, kb = t & 1;
            uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0;
            _Float16 d = (_Float16)0.0f;
            if (kb < bl) {
                const uint32_t lo = xrbase + (uint32_t)b0 * kQ80Bytes;
                const uint32_t bo = (uint32_t)r * (XCH * 16) + (lo & 15) + 34u * kb;
                const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
                uint32_t v[9];
#pragma unroll
                for (int i = 0; i < 9; ++i) v[i] = r32[qd + i];
                c0 = make_uint4(align_bytes(v[1], v[0], qsh), align_bytes(v[2], v[1], qsh),
                                align_bytes(v[3], v[2], qsh), align_bytes(v[4], v[3], qsh));
                c1 = make_uint4(align_bytes(v[5], v[4], qsh), align_bytes(v[6], v[5], qsh),
                                align_bytes(v[7], v[6], qsh), align_bytes(v[8], v[7], qsh));
                d = __builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(rb + bo));
            }
            sh.a[buf][kb][r][0] = c0;
            sh.a[buf][kb][r][1] = c1;
            sh.dx[buf][kb][r] = d;
        }
        {
            const int r = t >> 1, kb = t & 1;
            uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0;
            float d16 = 0.0f;
            if (kb < bl) {
                const uint32_t lo = wrbase + (uint32_t)b0 * kQ40Bytes;
                const uint32_t bo = (uint32_t)(RAWX * 16) + (uint32_t)r * (WCH * 16) + (lo & 15) + 18u * kb;
                const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
                uint32_t v[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) v[i] = r32[qd + i];
                uint32_t q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = align_bytes(v[i + 1], v[i], qsh) ^ 0x88888888u;
                // byte = 16*(nib-8) as int8: low nibbles are elements 0..15, high 16..31
                c0 = make_uint4((q[0] << 4) & 0xf0f0f0f0u, (q[1] << 4) & 0xf0f0f0f0u, (q[2] << 4) & 0xf0f0f0f0u,
                                (q[3] << 4) & 0xf0f0f0f0u);
                c1 = make_uint4(q[0] & 0xf0f0f0f0u, q[1] & 0xf0f0f0f0u, q[2] & 0xf0f0f0f0u, q[3] & 0xf0f0f0f0u);
                d16 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(rb + bo)) * 0.0625f;
            }
            sh.b[buf][kb][r][0] = c0;
            sh.b[buf][kb][r][1] = c1;
            sh.dw[buf][kb][r] = d16;
        }
    };

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

    const int lr = lane & 31, lh = lane >> 5;
    // Operands of one block for this wave: two 32-token A tiles, two 32-row B
    // tiles, the weight scales of the lane's columns and the token scales of
    // the lane's 16 rows in each A tile.
    struct Ops {
        v4i a[2], b[2];
        float dw[2], nb[2];
        _Float16 dx[2][16];
    };
    auto load_ops = [&](int buf, int kb, Ops &o) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 a4 = sh.a[buf][kb][64 * wm + 32 * i + lr][lh];
            o.a[i] = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 b4 = sh.b[buf][kb][64 * wn + 32 * j + lr][lh];
            o.b[j] = v4i{(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
            o.dw[j] = sh.dw[buf][kb][64 * wn + 32 * j + lr];
            o.nb[j] = -kBias * o.dw[j];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) o.dx[i][4 * a + b] = sh.dx[buf][kb][64 * wm + 32 * i + 8 * a + 4 * lh + b];
    };
    auto mfma = [&](const Ops &o, int i, int j) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[i], o.b[j], bias, 0, 0, 0);
    };
    auto fold = [&](const v16i &d, const Ops &o, int i, int j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // element first, then reinterpret: __builtin_bit_cast applied
            // directly to a vector element reads element 0 with this
            // toolchain (hipcc 7.2), so it must not be used here
            const int e = d[r];
            const float u = fmaf(__int_as_float(e), o.dw[j], o.nb[j]);
            acc[i][j][r] = fmaf(u, (float)o.dx[i][r], acc[i][j][r]);
        }
    };
    // One stage = 2 blocks x 4 tiles, written as a software pipeline: the MFMA
    // of tile t+1 is issued before tile t is folded, so the matrix unit and the
    // VALU can overlap inside the wave.  Blocks
    // past the end of K (a partial last stage) were re-laid out as zero codes
    // with dw = 0, so they add exactly 0: u = fma(1.5*2^23, 0, -0) = 0.
    auto compute = [&](int s) {
        const int buf = s & 1;
        Ops o0, o1;
        load_ops(buf, 0, o0);
        v16i d0 = mfma(o0, 0, 0);
        load_ops(buf, 1, o1);
        v16i d1 = mfma(o0, 0, 1);
        fold(d0, o0, 0, 0);
        d0 = mfma(o0, 1, 0);
        fold(d1, o0, 0, 1);
        d1 = mfma(o0, 1, 1);
        fold(d0, o0, 1, 0);
        d0 = mfma(o1, 0, 0);
        fold(d1, o0, 1, 1);
        d1 = mfma(o1, 0, 1);
        fold(d0, o1, 0, 0);
        d0 = mfma(o1, 1, 0);
        fold(d1, o1, 0, 1);
        d1 = mfma(o1, 1, 1);
        fold(d0, o1, 1, 0);
        fold(d1, o1, 1, 1);
    };
    static_assert(KB == 2, "the pipelined stage is written for two blocks");

    // Stage s is DMA'd (into raw[s&1]) one iteration before it is re-laid out
    // (into a/b[s&1]) and two before its MFMA work.
    dma_stage(0);
    if (nst > 1) dma_stage(1);
    wait_vmcnt(nst > 1 ? ndma : 0);          // stage 0 has landed (loads complete in order)
    __syncthreads();
    relayout(0);
    for (int s = 0; s < nst; ++s) {
        wait_global_loads();                 // this wave's DMA of stage s+1 has landed
        __syncthreads();                     // every wave's; re-layout(s) done; compute(s-1) done
        if (s + 2 < nst) dma_stage(s + 2);   // into raw[s&1], consumed by re-layout(s)
        if (s + 1 < nst) relayout(s + 1);    // into a/b[(s+1)&1], last read by compute(s-1)
        compute(s);
    }

    // store: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
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

static hipError_t launch_matmul_q4_0_any(const uint8_t *wp, const uint8_t *xp, float *y, int M, int N, int nb,
                                         hipStream_t st) {
    int tiles_m = (M + mm::BM - 1) / mm::BM;
    const int64_t tiles = (int64_t)tiles_m * ((N + mm::BN - 1) / mm::BN);
    static int lds_ok = 0;
    const hipError_t e = allow_dynamic_lds((const void *)k_matmul_q4_0_any, sizeof(MmShared), lds_ok);
    if (e != hipSuccess) return e;
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&nb, (void *)&tiles_m};
    return hipLaunchKernel((const void *)k_matmul_q4_0_any, dim3((unsigned)tiles), dim3(mm::NT), args,
                           sizeof(MmShared), st);
}

// ---------------------------------------------------------------------------
// Even block count, so every row starts on a 4-byte boundary.  The K loop
// moves two blocks per stage: 68 bytes (17 dwords) of each activation row and
// 36 bytes (9 dwords) of each weight row.  A stage is copied into LDS by
// buffer LDS-DMA loads of one dword per lane, 64 consecutive dwords per
// instruction: the activation rows row-major at a 17-dword stride, the weight
// rows at a 9-dword stride (odd strides, so a wave reading one dword of 32
// different rows touches 32 different banks).  Each lane's global offset for
// each of its 13 loads is fixed for the whole K loop; the stage position
// rides in the scalar offset.
//
// Nothing is re-laid out: each wave reads its MFMA operands from those rows.
// The stage's second block is 4-byte aligned (codes in dwords 9..16); the
// first is not (its codes start 2 bytes into dword 0), so for it the
// contraction order inside the block is rotated by two: lane half 0 takes
// codes 2..17 (dwords 1..4) and half 1 takes codes 18..31, 0, 1 (dwords 5..7
// and one v_perm of dwords 8 and 0).  The weight codes are unpacked in the
// same order; the MFMA sums over the 32 byte positions, so any order that
// both operands share gives the same I_b.
// Weight nibbles are unpacked per wave as in the kernel above (16*(nib-8)).
// The fold is the same two FMAs, in plain f32: on gfx950 v_fma_f32 issues at
// twice the rate of v_fma_mix_f32 and v_cvt_f32_f16, so each scale is
// converted once per stage instead of inside the fold.  Each wave converts
// the dx of its 64 activation rows into a private f32 array in LDS (four
// consecutive rows are then one 16-byte read); dw enters without the 1/16,
// so every accumulator is 16x too large and the store scales it back (a
// power of two, exact).
namespace mmr {
constexpr int BM = 128;                  // tokens per workgroup tile
constexpr int BN = 128;                  // weight rows per workgroup tile
constexpr int NT = 256;                  // 4 waves, 2 x 2 of 64 x 64
constexpr int XD = 17;                   // activation dwords per row per stage
constexpr int WD = 9;                    // weight dwords per row per stage
constexpr int WOFF = BM * XD;            // weight rows start (dwords into a stage buffer)
constexpr int STAGE = WOFF + BN * WD;    // 3328 dwords = 13,312 bytes
constexpr int XQ = BM * XD / kWave;      // 34 wave loads of activation rows
constexpr int WQ = BN * WD / kWave;      // 18 of weight rows
constexpr int NQ = STAGE / kWave;        // 52 in all
constexpr int PER_WAVE = NQ / 4;         // 13
constexpr int NBUF = 3;                  // stage buffers: DMA runs two stages ahead
constexpr int DXF = NBUF * STAGE;        // per-wave f32 dx arrays: [wave][block][64 rows]
constexpr float kBias = 12582912.0f;     // 1.5 * 2^23, bit pattern 0x4B400000
}  // namespace mmr
static_assert(mmr::BM * mmr::XD % kWave == 0 && mmr::BN * mmr::WD % kWave == 0 && mmr::NQ % 4 == 0,
              "stage image splits into whole wave loads, evenly over the waves");

// 4 bytes per lane from a buffer into LDS: lane i's dword lands at LDS byte
// m0base + OFF + 4i (m0base wave-uniform); the write completes with the
// vector-memory counter.  Issued as inline assembly so that the compiler does
// not see an LDS store: for the intrinsic it conservatively waits for every
// outstanding LDS-DMA load before each later LDS read and before every
// barrier, which would serialise the copy of stage s+2 with the work on stage
// s.  The waits are explicit instead (vmcnt before the barrier that publishes
// a stage).  M0 is formed inside the statement so that the compiler does not
// keep one LDS address per load and stage alive in scalar registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF>
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t r, uint32_t m0base, uint32_t voff, int soff) {
    asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m0base), "v"(voff), "s"(r), "s"(soff), "i"(OFF) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// Workgroup barrier that orders LDS accesses but does not wait for
// outstanding vector-memory loads (the LDS-DMA copies in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(mmr::NT, 2) void k_matmul_q4_0(const uint8_t *__restrict__ w,
                                                            const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                            int M, int N, int nb, int tiles_m) {
    using namespace mmr;
    __shared__ __attribute__((aligned(16))) uint32_t lds[NBUF * STAGE + 4 * 2 * 64];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = uniform(t >> 6);
    const int mt = blockIdx.x % tiles_m, nt = blockIdx.x / tiles_m;
    const int m0 = mt * BM, n0 = nt * BN;
    const uint32_t xrow = (uint32_t)nb * kQ80Bytes, wrow = (uint32_t)nb * kQ40Bytes;
    const int nst = nb >> 1;

    // DMA: wave w issues wave loads q = w, w+4, ..., w+48 of each stage.  Rows
    // past the matrix re-read its last row; their results are not stored.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + (int64_t)m0 * xrow), 0, (int)((uint32_t)min(M - m0, BM) * xrow), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + (int64_t)n0 * wrow), 0, (int)((uint32_t)min(N - n0, BN) * wrow), 0x00020000);
    uint32_t voff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int q = wave + 4 * k;
        if (q < XQ) {
            const int f = kWave * q + lane, row = f / XD;
            voff[k] = (uint32_t)(min(m0 + row, M - 1) - m0) * xrow + 4u * (uint32_t)(f - XD * row);
        } else {
            const int f = kWave * (q - XQ) + lane, row = f / WD;
            voff[k] = (uint32_t)(min(n0 + row, N - 1) - n0) * wrow + 4u * (uint32_t)(f - WD * row);
        }
    }
    // Wave load q = w + 4k lands at dwords 64q.. of the stage buffer: loads
    // k = 0..7 are activation rows, k = 8 too for waves 0 and 1 (weight rows
    // for waves 2 and 3), k = 9..12 weight rows.
    // the low half of a generic LDS address is the LDS offset
    const uint32_t lds_w = (uint32_t)uniform((int)((uint32_t)reinterpret_cast<uintptr_t>(lds) + 256u * wave));
    auto dma_load = [&](auto kc, uint32_t base, int sx, int sw) {
        constexpr int k = decltype(kc)::value;
        const bool isw = k == 8 ? wave >= 2 : (k >= 9 && k <= 12);
        buffer_to_lds4<k * 1024>(isw ? wr : xr, base, voff[k], isw ? sw : sx);
    };
    // loads 2p and 2p+1 (p < 6), or load 12 (p = 6), of stage s into buffer b
    auto dma_pair = [&](auto pc, int s, int b) {
        constexpr int p = decltype(pc)::value;
        const uint32_t base = lds_w + (uint32_t)(b * STAGE * 4);
        const int sx = s * (2 * kQ80Bytes), sw = s * (2 * kQ40Bytes);
        dma_load(std::integral_constant<int, 2 * p>(), base, sx, sw);
        if constexpr (2 * p + 1 < PER_WAVE) dma_load(std::integral_constant<int, 2 * p + 1>(), base, sx, sw);
    };
    auto dma = [&](int s, int b) {
        dma_pair(std::integral_constant<int, 0>(), s, b);
        dma_pair(std::integral_constant<int, 1>(), s, b);
        dma_pair(std::integral_constant<int, 2>(), s, b);
        dma_pair(std::integral_constant<int, 3>(), s, b);
        dma_pair(std::integral_constant<int, 4>(), s, b);
        dma_pair(std::integral_constant<int, 5>(), s, b);
        dma_pair(std::integral_constant<int, 6>(), s, b);
    };
    static_assert(XQ == 34 && WQ == 18 && PER_WAVE == 13, "the load list above is written for this split");

    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 31, lh = lane >> 5;
    const int xz = (64 * wm + lr) * XD;          // dword 0 of A row 64wm+lr (tile i: +32 rows)
    const int xa = xz + 4 * lh;                  // the lane half's first code dword, less one
    const int wb = WOFF + (64 * wn + lr) * WD;   // B row 64wn+lr (tile j: +32 rows)
    const int dxw = DXF + 128 * wave;            // this wave's f32 dx: [block][64 rows 64wm..]
    const int xd = (64 * wm + lane) * XD;        // dword 0 of the row whose dx this lane converts
    // byte selectors (v_perm: 0-3 pick the second source, 4-7 the first)
    const uint32_t selA = lh ? 0x03020504u : 0x07060504u;   // half 1: codes 30, 31 then 0, 1
    const uint32_t selB = lh ? 0x07060100u : 0x03020504u;   // which bytes take the low nibble
    const uint32_t shB = lh ? 0u : 4u;                       // half 0: low nibbles, half 1: high

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

    // 16*(nib-8) as int8 from a nibble in the high half of each byte
    auto nib = [](uint32_t v) { return (v & 0xF0F0F0F0u) ^ 0x80808080u; };
    auto half_lo = [](uint32_t v) { return __builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); };
    auto half_hi = [](uint32_t v) { return __builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); };
    auto mfma = [&](const v4i &a, const v4i &b) { return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, bias, 0, 0, 0); };
    // The wave's dx for one stage as f32: lane l converts row 64wm+l's scales
    // (block 0: low half of dword 0, block 1: high half of dword 8).  Only this
    // wave reads them back, and a wave's LDS accesses complete in order.
    auto convert_dx = [&](const uint32_t *sb) {
        float *d = reinterpret_cast<float *>(lds + dxw);
        d[lane] = (float)half_lo(sb[xd]);
        d[64 + lane] = (float)half_hi(sb[xd + 8]);
    };
    // dx of the lane's 16 output rows of A tile i, block kb: rows 8a + 4lh + c
    // of the tile, four 16-byte reads
    auto load_dx = [&](int kb, int i, float (&d)[16]) {
        const float4 *p = reinterpret_cast<const float4 *>(lds + dxw + 64 * kb + 32 * i + 4 * lh);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float4 q = p[2 * a];
            d[4 * a] = q.x;
            d[4 * a + 1] = q.y;
            d[4 * a + 2] = q.z;
            d[4 * a + 3] = q.w;
        }
    };
    auto fold = [&](const v16i &d, int i, int j, const float (&dx)[16], float dw, float nbias) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = d[r];   // element first: see the bit_cast note above
            const float u = fmaf(__int_as_float(e), dw, nbias);
            acc[i][j][r] = fmaf(u, dx[r], acc[i][j][r]);
        }
    };

    // Operands of one block: two A tiles, two B tiles, the B rows' scales.
    struct Ops {
        v4i a[2], b[2];
        float dw[2], nb[2];
    };
    // raw dwords of one block for this lane: A row dwords 1..4 or 5..8 and
    // dword 0 (block 0) or 9..12 or 13..16 (block 1); B row dwords 0..4
    // (block 0) or 4..8 (block 1)
    struct Raw {
        uint32_t a[2][5], w[2][5];
    };
    auto load_raw = [&](const uint32_t *sb, int kb, Raw &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t *pa = sb + xa + 32 * XD * i + (kb ? 8 : 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) r.a[i][k] = pa[1 + k];
            r.a[i][4] = kb ? 0u : sb[xz + 32 * XD * i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t *pw = sb + wb + 32 * WD * j + (kb ? 4 : 0);
#pragma unroll
            for (int e = 0; e < 5; ++e) r.w[j][e] = pw[e];
        }
    };
    auto build = [&](const Raw &r, int kb, Ops &o) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t q3 = kb ? r.a[i][3] : __builtin_amdgcn_perm(r.a[i][3], r.a[i][4], selA);
            o.a[i] = v4i{(int)r.a[i][0], (int)r.a[i][1], (int)r.a[i][2], (int)q3};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t *E = r.w[j];
            if (kb == 0) {
                // nibble bytes 2..15 are dwords 1..3 and the first half of
                // dword 4; bytes 0, 1 are the second half of dword 0
                const uint32_t P = __builtin_amdgcn_perm(E[4], E[0], 0x03020504u);   // bytes 14, 15, 0, 1
                const uint32_t Pm = __builtin_amdgcn_perm(P << 4, P, selB);
                o.b[j] = v4i{(int)nib(E[1] << shB), (int)nib(E[2] << shB), (int)nib(E[3] << shB), (int)nib(Pm)};
                o.dw[j] = (float)half_lo(E[0]);
            } else {
                o.b[j] = v4i{(int)nib(E[1] << shB), (int)nib(E[2] << shB), (int)nib(E[3] << shB),
                             (int)nib(E[4] << shB)};
                o.dw[j] = (float)half_hi(E[0]);
            }
            // keep dw an f32 register: folded back into the fold, the f16
            // conversion would turn each v_fma_f32 into a half-rate v_fma_mix
            asm volatile("" : "+v"(o.dw[j]));
            o.nb[j] = o.dw[j] * -kBias;   // exact: 11 + 2 significant bits
        }
    };
    // Explicit order, fenced against the scheduler: the MFMA of tile t+1 is
    // issued before the fold of tile t (so a fold never waits for its MFMA
    // and two MFMAs never queue back to back), and the dx reads of the next
    // A tile go out one fold ahead.
    // The DMA of stage sd into buffer bd is spread over the step, two loads
    // after each of the first seven folds (one after the seventh), so that
    // the 52 loads of a workgroup do not queue up at the texture unit at once.
    auto compute = [&](const uint32_t *sb, int sd, int bd) __attribute__((always_inline)) {
        Raw r0, r1;
        Ops o0, o1;
        float dxa[16], dxb[16];
        auto dma_after = [&](auto pc) {
            dma_pair(pc, sd, bd);
            __builtin_amdgcn_sched_barrier(0);
        };
        convert_dx(sb);
        load_raw(sb, 0, r0);
        load_dx(0, 0, dxa);
        build(r0, 0, o0);
        v16i d0 = mfma(o0.a[0], o0.b[0]);
        __builtin_amdgcn_sched_barrier(0);
        load_raw(sb, 1, r1);
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
        build(r1, 1, o1);
        d0 = mfma(o1.a[0], o1.b[0]);
        __builtin_amdgcn_sched_barrier(0);
        fold(d1, 1, 1, dxb, o0.dw[1], o0.nb[1]);
        dma_after(std::integral_constant<int, 3>());
        d1 = mfma(o1.a[0], o1.b[1]);
        load_dx(1, 1, dxb);
        __builtin_amdgcn_sched_barrier(0);
        fold(d0, 0, 0, dxa, o1.dw[0], o1.nb[0]);
        dma_after(std::integral_constant<int, 4>());
        d0 = mfma(o1.a[1], o1.b[0]);
        __builtin_amdgcn_sched_barrier(0);
        fold(d1, 0, 1, dxa, o1.dw[1], o1.nb[1]);
        dma_after(std::integral_constant<int, 5>());
        d1 = mfma(o1.a[1], o1.b[1]);
        __builtin_amdgcn_sched_barrier(0);
        fold(d0, 1, 0, dxb, o1.dw[0], o1.nb[0]);
        dma_after(std::integral_constant<int, 6>());
        fold(d1, 1, 1, dxb, o1.dw[1], o1.nb[1]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Stage s lives in buffer s % 3.  At step s this wave's loads of stage s
    // have landed once at most the 13 of stage s+1 are outstanding; the
    // barrier publishes every wave's and frees buffer (s-1) % 3, which the
    // DMA of stage s+2 then fills.  The last two steps have no stage s+2 and
    // copy the last stage again into that idle buffer instead, so that every
    // step issues the same 13 loads and waits for the same count.
    static_assert(PER_WAVE == 13, "the wait below counts 13 loads per stage");
    auto step = [&](int s, auto bc) {
        constexpr int b = decltype(bc)::value;
        asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
        lds_barrier();
        compute(lds + b * STAGE, min(s + 2, nst - 1), (b + 2) % NBUF);
    };
    dma(0, 0);
    dma(min(1, nst - 1), 1);
    for (int s = 0; s < nst; s += NBUF) {
        step(s, std::integral_constant<int, 0>());
        if (s + 1 < nst) step(s + 1, std::integral_constant<int, 1>());
        if (s + 2 < nst) step(s + 2, std::integral_constant<int, 2>());
    }
    // no LDS-DMA write may still be in flight when the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // store: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + lr;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m < M) y[(int64_t)m * N + n] = acc[i][j][r] * 0.0625f;
            }
        }
}

hipError_t launch_matmul_q4_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    // the plane kernel needs 4-byte aligned rows and 32-bit tile offsets
    if ((nb & 1) || (int64_t)mmr::BM * nb * kQ80Bytes >= (int64_t(1) << 31))
        return launch_matmul_q4_0_any(wp, xp, y, M, N, nb, st);
    int tiles_m = (M + mmr::BM - 1) / mmr::BM;
    const int64_t tiles = (int64_t)tiles_m * ((N + mmr::BN - 1) / mmr::BN);
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&nb, (void *)&tiles_m};
    return hipLaunchKernel((const void *)k_matmul_q4_0, dim3((unsigned)tiles), dim3(mmr::NT), args, 0, st);
}

}  // namespace qmm
