// Prefill matmul, Q4_0 weights x Q8_0 activations, on int8 MFMA.
//
//   Y[m][n] = sum_b dx[m,b] dw[n,b] I_b[m,n],   I_b = sum_{k<32} q[m,32b+k] (w[n,32b+k]-8)
//
// Once a weight tile is reused across many tokens the product is a dense
// contraction (kvad "Batched prefill, and i8mm"; krafla "Batched prompt
// prefill"), and one 32-value block is exactly the K of
// v_mfma_i32_32x32x32_i8, so every block gets its own exact int32 tile.
//
// Workgroup tile 128 tokens x 128 weight rows, 4 waves of 64x64 (2x2 MFMA
// tiles of 32x32).  The K loop moves KB blocks per stage:
//   1. coalesced 16-byte loads of the tile's row segments (prefetched into
//      registers one stage ahead) are written raw into LDS;
//   2. a re-layout pass slices the 2-byte-aligned blocks out of the raw rows:
//      activation codes go to [kb][m][32] int8, their f16 scales to [kb][m];
//      weight nibbles are unpacked once per workgroup into signed bytes
//      16*(nib-8) (XOR 0x88 then shift/mask, krafla "Weight packing"), and
//      their scales to [kb][n] as f32 dw/16 (the 16 is a power of two, so the
//      rescale is exact);
//   3. each wave reads its MFMA operands with one ds_read_b128 per 32x32 tile
//      (lane = row, lane half = which 16 of the 32 codes; A and B use the same
//      split, so the k order inside the instruction does not matter).
// Scale fold: the MFMA's C input is the constant 0x4B400000, so the int32
// result read as f32 is exactly 1.5*2^23 + 16 I (|16 I| < 2^22); then
//   u = fma(F, dw/16, -1.5*2^23*dw/16) = I*dw   (one rounding)
//   acc = fma(u, dx, acc)                       (one rounding)
// Output lane layout of a 32x32 MFMA tile: lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4 and column l%32.
#include "qmm_device.h"

namespace qmm {

namespace mm {
constexpr int BM = 128;                 // tokens per workgroup tile
constexpr int BN = 128;                 // weight rows per workgroup tile
constexpr int KB = 4;                   // blocks (of 32) per stage
constexpr int XCH = 10;                 // 16-B chunks per raw activation row segment (136 B + misalignment)
constexpr int WCH = 6;                  // 16-B chunks per raw weight row segment (72 B + misalignment)
constexpr int XLOADS = BM * XCH / 256;  // chunk loads per thread per stage (5)
constexpr int WLOADS = BN * WCH / 256;  // (3)
static_assert(BM * XCH % 256 == 0 && BN * WCH % 256 == 0, "loads must split evenly");
constexpr float kBias = 12582912.0f;    // 1.5 * 2^23, bit pattern 0x4B400000
}  // namespace mm

struct MmShared {
    uint4 rawx[mm::BM * mm::XCH];         // 20480 B
    uint4 raww[mm::BN * mm::WCH];         // 12288 B
    uint4 a[mm::KB][mm::BM][2];           // activation codes, 16384 B
    uint4 b[mm::KB][mm::BN][2];           // weight codes * 16, 16384 B
    _Float16 dx[mm::KB][mm::BM];          // 1024 B
    float dw[mm::KB][mm::BN];             // dw / 16, 2048 B
};

__global__ __launch_bounds__(256, 2) void k_matmul_q4_0(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                                        float *__restrict__ y, int M, int N, int nb) {
    using namespace mm;
    __shared__ MmShared sh;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t xrow = (int64_t)nb * kQ80Bytes, wrow = (int64_t)nb * kQ40Bytes;

    // ---- stage loader: row segments of blocks [b0, b0+KB) ------------------
    uint4 xr[XLOADS], wr[WLOADS];
    auto load_stage = [&](int b0) {
        const int bl = min(KB, nb - b0);
#pragma unroll
        for (int k = 0; k < XLOADS; ++k) {
            const int idx = t + 256 * k, r = idx / XCH, c = idx % XCH;
            const int m = m0 + r;
            xr[k] = make_uint4(0, 0, 0, 0);
            if (m < M) {
                const int64_t lo = m * xrow + (int64_t)b0 * kQ80Bytes;
                const int64_t hi = lo + (int64_t)bl * kQ80Bytes;
                const int64_t A = lo & ~(int64_t)15;
                if (A + 16 * c < hi) xr[k] = *reinterpret_cast<const uint4 *>(xq + A + 16 * c);
            }
        }
#pragma unroll
        for (int k = 0; k < WLOADS; ++k) {
            const int idx = t + 256 * k, r = idx / WCH, c = idx % WCH;
            const int n = n0 + r;
            wr[k] = make_uint4(0, 0, 0, 0);
            if (n < N) {
                const int64_t lo = n * wrow + (int64_t)b0 * kQ40Bytes;
                const int64_t hi = lo + (int64_t)bl * kQ40Bytes;
                const int64_t A = lo & ~(int64_t)15;
                if (A + 16 * c < hi) wr[k] = *reinterpret_cast<const uint4 *>(w + A + 16 * c);
            }
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

    const int nstages = (nb + KB - 1) / KB;
    load_stage(0);
    for (int s = 0; s < nstages; ++s) {
        const int b0 = s * KB;
        const int bl = min(KB, nb - b0);
#pragma unroll
        for (int k = 0; k < XLOADS; ++k) sh.rawx[t + 256 * k] = xr[k];
#pragma unroll
        for (int k = 0; k < WLOADS; ++k) sh.raww[t + 256 * k] = wr[k];
        __syncthreads();

        // ---- re-layout: 512 activation blocks and 512 weight blocks --------
        const uint8_t *rx = reinterpret_cast<const uint8_t *>(sh.rawx);
        const uint8_t *rw = reinterpret_cast<const uint8_t *>(sh.raww);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int p = t + 256 * k, r = p & (BM - 1), kb = p >> 7;
            uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0;
            _Float16 d = (_Float16)0.0f;
            if (kb < bl) {
                const int64_t lo = (int64_t)(m0 + r) * xrow + (int64_t)b0 * kQ80Bytes;
                const uint32_t bo = (uint32_t)r * (XCH * 16) + (uint32_t)(lo & 15) + 34u * kb;
                const uint32_t *l32 = reinterpret_cast<const uint32_t *>(rx);
                const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
                uint32_t v[9];
#pragma unroll
                for (int i = 0; i < 9; ++i) v[i] = l32[qd + i];
                c0 = make_uint4(align_bytes(v[1], v[0], qsh), align_bytes(v[2], v[1], qsh),
                                align_bytes(v[3], v[2], qsh), align_bytes(v[4], v[3], qsh));
                c1 = make_uint4(align_bytes(v[5], v[4], qsh), align_bytes(v[6], v[5], qsh),
                                align_bytes(v[7], v[6], qsh), align_bytes(v[8], v[7], qsh));
                d = __builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(rx + bo));
            }
            sh.a[kb][r][0] = c0;
            sh.a[kb][r][1] = c1;
            sh.dx[kb][r] = d;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int p = t + 256 * k, r = p & (BN - 1), kb = p >> 7;
            uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0;
            float d16 = 0.0f;
            if (kb < bl) {
                const int64_t lo = (int64_t)(n0 + r) * wrow + (int64_t)b0 * kQ40Bytes;
                const uint32_t bo = (uint32_t)r * (WCH * 16) + (uint32_t)(lo & 15) + 18u * kb;
                const uint32_t *l32 = reinterpret_cast<const uint32_t *>(rw);
                const uint32_t qd = (bo + 2) >> 2, qsh = (bo + 2) & 3;
                uint32_t v[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) v[i] = l32[qd + i];
                uint32_t q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = align_bytes(v[i + 1], v[i], qsh) ^ 0x88888888u;
                // byte = 16*(nib-8) as int8: low nibbles are elements 0..15, high 16..31
                c0 = make_uint4((q[0] << 4) & 0xf0f0f0f0u, (q[1] << 4) & 0xf0f0f0f0u, (q[2] << 4) & 0xf0f0f0f0u,
                                (q[3] << 4) & 0xf0f0f0f0u);
                c1 = make_uint4(q[0] & 0xf0f0f0f0u, q[1] & 0xf0f0f0f0u, q[2] & 0xf0f0f0f0u, q[3] & 0xf0f0f0f0u);
                d16 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(rw + bo)) * 0.0625f;
            }
            sh.b[kb][r][0] = c0;
            sh.b[kb][r][1] = c1;
            sh.dw[kb][r] = d16;
        }
        __syncthreads();

        if (s + 1 < nstages) load_stage(b0 + KB);     // in flight during the MFMA work

        // ---- MFMA + scale fold --------------------------------------------
        const int lr = lane & 31, lh = lane >> 5;
        for (int kb = 0; kb < bl; ++kb) {
            v4i av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 a4 = sh.a[kb][64 * wm + 32 * i + lr][lh];
                av[i] = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 b4 = sh.b[kb][64 * wn + 32 * j + lr][lh];
                bv[j] = v4i{(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
            }
            float dwj[2], nbj[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dwj[j] = sh.dw[kb][64 * wn + 32 * j + lr];
                nbj[j] = -kBias * dwj[j];
            }
            _Float16 dxi[2][16];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) dxi[i][4 * a + b] = sh.dx[kb][64 * wm + 32 * i + 8 * a + 4 * lh + b];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const v16i dmf = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[i], bv[j], bias, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // element first, then reinterpret: __builtin_bit_cast applied
                        // directly to a vector element reads element 0 with this
                        // toolchain (hipcc 7.2), so it must not be used here
                        const int e = dmf[r];
                        const float F = __int_as_float(e);
                        const float u = fmaf(F, dwj[j], nbj[j]);
                        acc[i][j][r] = fmaf(u, (float)dxi[i][r], acc[i][j][r]);
                    }
                }
        }
        __syncthreads();
    }

    // ---- store: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
    const int lr = lane & 31, lh = lane >> 5;
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
    dim3 grid((unsigned)((N + mm::BN - 1) / mm::BN), (unsigned)((M + mm::BM - 1) / mm::BM));
    void *args[] = {(void *)&wp, (void *)&xp, (void *)&y, (void *)&M, (void *)&N, (void *)&nb};
    return hipLaunchKernel((const void *)k_matmul_q4_0, grid, dim3(256), args, 0, st);
}

}  // namespace qmm
