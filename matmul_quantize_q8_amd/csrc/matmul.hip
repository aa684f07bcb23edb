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

__global__ __launch_bounds__(mm::NT, 2) void k_matmul_q4_0(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
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

hipError_t launch_matmul_q4_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st) {
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *xp = static_cast<const uint8_t *>(xq);
    int tiles_m = (M + mm::BM - 1) / mm::BM;
    const int64_t tiles = (int64_t)tiles_m * ((N + mm::BN - 1) / mm::BN);
    static int lds_ok = 0;
    const hipError_t e = allow_dynamic_lds((const void *)k_matmul_q4_0, sizeof(MmShared), lds_ok);
    if (e != hipSuccess) return e;
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&nb, (void *)&tiles_m};
    return hipLaunchKernel((const void *)k_matmul_q4_0, dim3((unsigned)tiles), dim3(mm::NT), args,
                           sizeof(MmShared), st);
}

}  // namespace qmm
