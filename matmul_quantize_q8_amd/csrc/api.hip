// C ABI of libqmm: argument checks, device check, launch.  Declarations and
// the contract of every entry point are in include/qmm.h.
#include <atomic>
#include <cstring>

#include "qmm.h"
#include "qmm_device.h"

namespace qmm {
hipError_t launch_quantize_q8_0(const float *x, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q8_k(const float *x, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q4_0(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q2_k(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q4_k(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q4_1(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q5_0(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_quantize_q5_1(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_matvec_q4_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q5_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q5_1(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matmul_q4_1(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st);
hipError_t launch_matmul_q5_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st);
hipError_t launch_matmul_q5_1(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st);
hipError_t launch_quantize_q6_k(const float *w, void *out, int64_t nblocks, hipStream_t st);
hipError_t launch_matvec_q4_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q8_0(const void *w, const void *xq, float *y, int N, int nb, hipStream_t st);
hipError_t launch_matvec_q2_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st);
hipError_t launch_matvec_q4_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st);
hipError_t launch_matvec_q6_k(const void *w, const void *xq, float *y, int N, int ns, hipStream_t st);
hipError_t launch_quantize_matvec_q4_0(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st);
hipError_t launch_quantize_matvec_q2_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st);
hipError_t launch_quantize_matvec_q4_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st);
hipError_t launch_quantize_matvec_q6_k(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st);
hipError_t launch_quantize_matvec_q8_0(const void *w, const float *x, void *xq, float *y, int N, int nb,
                                       hipStream_t st);
hipError_t launch_matmul_q4_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st);
hipError_t launch_matmul_q8_0(const void *w, const void *xq, float *y, int M, int N, int nb, hipStream_t st);
int64_t matmul_q4_0_max_blocks();
hipError_t launch_get_rows(int fmt, const void *w, const int32_t *ids, float *out, int64_t n, int64_t N, int64_t K,
                           int64_t row_bytes, hipStream_t st);
hipError_t launch_matmul_q2_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st);
hipError_t launch_matmul_q4_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st);
hipError_t launch_matmul_q6_k_mfma(const void *w, const void *xq, float *y, int M, int N, int ns, hipStream_t st);
int64_t matmul_k_max_blocks();

}  // namespace qmm

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxBytes = int64_t(1) << 40;
constexpr int kMaxDevices = 64;

std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

qmm_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMM_E_DEVICE;
    int s = g_device_state[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return QMM_E_DEVICE;
        s = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_state[dev].store(s, std::memory_order_release);
    }
    return s == 1 ? QMM_OK : QMM_E_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// rows x (K / blk) blocks of `bytes` each must stay below kMaxBytes.
bool size_ok(int64_t rows, int64_t K, int64_t blk, int64_t bytes) {
    if (rows < 0 || rows > kMaxDim || K > kMaxDim) return false;
    const int64_t nb = K / blk;
    return nb == 0 || rows <= kMaxBytes / (nb * bytes);
}

// Shape checks shared by all entry points: M, N >= 1 and K a positive
// multiple of the block length, every dimension below 2^31 (krafla "Error
// handling": a bad size is a status, never a launch).
qmm_status check_shape(int64_t M, int64_t N, int64_t K, int64_t blk) {
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim) return QMM_E_SHAPE;
    if (K < blk || K > kMaxDim || K % blk != 0) return QMM_E_SHAPE;
    return QMM_OK;
}

qmm_status check_ptrs(std::initializer_list<const void *> ps) {
    for (const void *p : ps)
        if (p == nullptr) return QMM_E_NULL;
    for (const void *p : ps)
        if (!aligned16(p)) return QMM_E_ALIGN;
    return QMM_OK;
}

qmm_status launched(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_E_LAUNCH; }

typedef hipError_t (*quant_launch)(const float *, void *, int64_t, hipStream_t);

qmm_status quantize(quant_launch fn, const float *x, void *out, int64_t rows, int64_t K, int64_t blk,
                    int64_t in_bytes, int64_t out_bytes, void *stream) {
    qmm_status s = check_shape(rows, 1, K, blk);
    if (s != QMM_OK) return s;
    if (!size_ok(rows, K, blk, in_bytes) || !size_ok(rows, K, blk, out_bytes)) return QMM_E_SHAPE;
    if ((s = check_ptrs({x, out})) != QMM_OK) return s;
    if ((s = check_device()) != QMM_OK) return s;
    return launched(fn(x, out, rows * (K / blk), static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char *qmm_status_string(qmm_status s) {
    switch (s) {
        case QMM_OK: return "QMM_OK";
        case QMM_E_SHAPE: return "QMM_E_SHAPE: bad M, N or K, or a byte size that overflows";
        case QMM_E_NULL: return "QMM_E_NULL: a required pointer is NULL";
        case QMM_E_ALIGN: return "QMM_E_ALIGN: a pointer is not 16-byte aligned";
        case QMM_E_DEVICE: return "QMM_E_DEVICE: no current device, or it is not gfx950";
        case QMM_E_LAUNCH: return "QMM_E_LAUNCH: the HIP runtime refused a kernel launch";
    }
    return "QMM: unknown status";
}

int qmm_abi_version(void) { return 1; }

qmm_status qmm_quantize_q8_0(const float *x, void *xq, int64_t M, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q8_0, x, xq, M, K, 32, 128, qmm::kQ80Bytes, stream);
}

qmm_status qmm_quantize_q8_k(const float *x, void *xq, int64_t M, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q8_k, x, xq, M, K, 256, 1024, qmm::kQ8KBytes, stream);
}

qmm_status qmm_quantize_q4_0(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q4_0, w, wq, N, K, 32, 128, qmm::kQ40Bytes, stream);
}

qmm_status qmm_quantize_q2_k(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q2_k, w, wq, N, K, 256, 1024, qmm::kQ2KBytes, stream);
}

qmm_status qmm_quantize_q4_1(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q4_1, w, wq, N, K, 32, 128, qmm::kQ41Bytes, stream);
}

qmm_status qmm_quantize_q5_0(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q5_0, w, wq, N, K, 32, 128, qmm::kQ50Bytes, stream);
}

qmm_status qmm_quantize_q5_1(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q5_1, w, wq, N, K, 32, 128, qmm::kQ51Bytes, stream);
}

qmm_status qmm_quantize_q4_k(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q4_k, w, wq, N, K, 256, 1024, qmm::kQ4KBytes, stream);
}

qmm_status qmm_quantize_q6_k(const float *w, void *wq, int64_t N, int64_t K, void *stream) {
    return quantize(qmm::launch_quantize_q6_k, w, wq, N, K, 256, 1024, qmm::kQ6KBytes, stream);
}

typedef hipError_t (*mv_launch)(const void *, const void *, float *, int, int, hipStream_t);

static qmm_status matvec(mv_launch fn, const void *w, const void *xq, float *y, int64_t N, int64_t K, int64_t blk,
                         int64_t wbytes, int64_t xbytes, void *stream) {
    qmm_status s = check_shape(1, N, K, blk);
    if (s != QMM_OK) return s;
    if (!size_ok(N, K, blk, wbytes) || !size_ok(1, K, blk, xbytes)) return QMM_E_SHAPE;
    if ((s = check_ptrs({w, xq, y})) != QMM_OK) return s;
    if ((s = check_device()) != QMM_OK) return s;
    return launched(fn(w, xq, y, (int)N, (int)(K / blk), static_cast<hipStream_t>(stream)));
}

qmm_status qmm_matvec_q8_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q8_0, w, xq, y, N, K, 32, qmm::kQ80Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matvec_q4_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q4_0, w, xq, y, N, K, 32, qmm::kQ40Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matvec_q2_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q2_k, w, xq8k, y, N, K, 256, qmm::kQ2KBytes, qmm::kQ8KBytes, stream);
}

qmm_status qmm_matvec_q4_1(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q4_1, w, xq, y, N, K, 32, qmm::kQ41Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matvec_q5_0(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q5_0, w, xq, y, N, K, 32, qmm::kQ50Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matvec_q5_1(const void *w, const void *xq, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q5_1, w, xq, y, N, K, 32, qmm::kQ51Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matvec_q4_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q4_k, w, xq8k, y, N, K, 256, qmm::kQ4KBytes, qmm::kQ8KBytes, stream);
}

qmm_status qmm_matvec_q6_k(const void *w, const void *xq8k, float *y, int64_t N, int64_t K, void *stream) {
    return matvec(qmm::launch_matvec_q6_k, w, xq8k, y, N, K, 256, qmm::kQ6KBytes, qmm::kQ8KBytes, stream);
}

typedef hipError_t (*qmv_launch)(const void *, const float *, void *, float *, int, int, hipStream_t);

static qmm_status quantize_matvec(qmv_launch fn, const void *w, const float *x, void *xq, float *y, int64_t N,
                                  int64_t K, int64_t blk, int64_t wbytes, void *stream) {
    qmm_status s = check_shape(1, N, K, blk);
    if (s != QMM_OK) return s;
    if (!size_ok(N, K, blk, wbytes) || !size_ok(1, K, blk, 4 * blk)) return QMM_E_SHAPE;
    if ((s = check_ptrs({w, x, y})) != QMM_OK) return s;
    if (xq != nullptr && !aligned16(xq)) return QMM_E_ALIGN;
    if ((s = check_device()) != QMM_OK) return s;
    return launched(fn(w, x, xq, y, (int)N, (int)(K / blk), static_cast<hipStream_t>(stream)));
}

qmm_status qmm_quantize_matvec_q4_0(const void *w, const float *x, void *xq, float *y, int64_t N, int64_t K,
                                    void *stream) {
    return quantize_matvec(qmm::launch_quantize_matvec_q4_0, w, x, xq, y, N, K, 32, qmm::kQ40Bytes, stream);
}

qmm_status qmm_quantize_matvec_q8_0(const void *w, const float *x, void *xq, float *y, int64_t N, int64_t K,
                                    void *stream) {
    return quantize_matvec(qmm::launch_quantize_matvec_q8_0, w, x, xq, y, N, K, 32, qmm::kQ80Bytes, stream);
}

qmm_status qmm_quantize_matvec_q2_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream) {
    return quantize_matvec(qmm::launch_quantize_matvec_q2_k, w, x, xq8k, y, N, K, 256, qmm::kQ2KBytes, stream);
}

qmm_status qmm_quantize_matvec_q4_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream) {
    return quantize_matvec(qmm::launch_quantize_matvec_q4_k, w, x, xq8k, y, N, K, 256, qmm::kQ4KBytes, stream);
}

qmm_status qmm_quantize_matvec_q6_k(const void *w, const float *x, void *xq8k, float *y, int64_t N, int64_t K,
                                    void *stream) {
    return quantize_matvec(qmm::launch_quantize_matvec_q6_k, w, x, xq8k, y, N, K, 256, qmm::kQ6KBytes, stream);
}

typedef hipError_t (*mm_launch)(const void *, const void *, float *, int, int, int, hipStream_t);

static qmm_status matmul(mm_launch fn, const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K,
                         int64_t blk, int64_t wbytes, int64_t xbytes, void *stream) {
    qmm_status s = check_shape(M, N, K, blk);
    if (s != QMM_OK) return s;
    if (!size_ok(N, K, blk, wbytes) || !size_ok(M, K, blk, xbytes)) return QMM_E_SHAPE;
    if (N > 0 && M > kMaxBytes / 4 / N) return QMM_E_SHAPE;
    if ((s = check_ptrs({w, xq, y})) != QMM_OK) return s;
    if ((s = check_device()) != QMM_OK) return s;
    return launched(fn(w, xq, y, (int)M, (int)N, (int)(K / blk), static_cast<hipStream_t>(stream)));
}

qmm_status qmm_matmul_q4_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    if (K / 32 > qmm::matmul_q4_0_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q4_0, w, xq, y, M, N, K, 32, qmm::kQ40Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matmul_q8_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    if (K / 32 > qmm::matmul_q4_0_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q8_0, w, xq, y, M, N, K, 32, qmm::kQ80Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matmul_q4_1(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    if (K / 32 > qmm::matmul_q4_0_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q4_1, w, xq, y, M, N, K, 32, qmm::kQ41Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matmul_q5_0(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    if (K / 32 > qmm::matmul_q4_0_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q5_0, w, xq, y, M, N, K, 32, qmm::kQ50Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matmul_q5_1(const void *w, const void *xq, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    if (K / 32 > qmm::matmul_q4_0_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q5_1, w, xq, y, M, N, K, 32, qmm::kQ51Bytes, qmm::kQ80Bytes, stream);
}

qmm_status qmm_matmul_q2_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream) {
    if (K / 256 > qmm::matmul_k_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q2_k_mfma, w, xq8k, y, M, N, K, 256, qmm::kQ2KBytes, qmm::kQ8KBytes, stream);
}

qmm_status qmm_matmul_q4_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream) {
    if (K / 256 > qmm::matmul_k_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q4_k_mfma, w, xq8k, y, M, N, K, 256, qmm::kQ4KBytes, qmm::kQ8KBytes, stream);
}

qmm_status qmm_matmul_q6_k(const void *w, const void *xq8k, float *y, int64_t M, int64_t N, int64_t K,
                           void *stream) {
    if (K / 256 > qmm::matmul_k_max_blocks()) return QMM_E_SHAPE;
    return matmul(qmm::launch_matmul_q6_k_mfma, w, xq8k, y, M, N, K, 256, qmm::kQ6KBytes, qmm::kQ8KBytes, stream);
}

static qmm_status get_rows(int fmt, const void *w, const int32_t *ids, float *out, int64_t n, int64_t N, int64_t K,
                           int64_t blk, int64_t wbytes, void *stream) {
    qmm_status s = check_shape(n, N, K, blk);
    if (s != QMM_OK) return s;
    if (!size_ok(N, K, blk, wbytes) || !size_ok(n, K, 1, 4)) return QMM_E_SHAPE;
    if ((n * (K / 4) + 255) / 256 > kMaxDim) return QMM_E_SHAPE;
    if ((s = check_ptrs({w, ids, out})) != QMM_OK) return s;
    if ((s = check_device()) != QMM_OK) return s;
    return launched(qmm::launch_get_rows(fmt, w, ids, out, n, N, K, K / blk * wbytes, static_cast<hipStream_t>(stream)));
}

qmm_status qmm_get_rows_q4_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q4_0, w, ids, out, n_ids, N, K, 32, qmm::kQ40Bytes, stream);
}
qmm_status qmm_get_rows_q8_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q8_0, w, ids, out, n_ids, N, K, 32, qmm::kQ80Bytes, stream);
}
qmm_status qmm_get_rows_q2_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q2_K, w, ids, out, n_ids, N, K, 256, qmm::kQ2KBytes, stream);
}
qmm_status qmm_get_rows_q4_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q4_K, w, ids, out, n_ids, N, K, 256, qmm::kQ4KBytes, stream);
}
qmm_status qmm_get_rows_q6_k(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q6_K, w, ids, out, n_ids, N, K, 256, qmm::kQ6KBytes, stream);
}
qmm_status qmm_get_rows_q4_1(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q4_1, w, ids, out, n_ids, N, K, 32, qmm::kQ41Bytes, stream);
}
qmm_status qmm_get_rows_q5_0(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q5_0, w, ids, out, n_ids, N, K, 32, qmm::kQ50Bytes, stream);
}
qmm_status qmm_get_rows_q5_1(const void *w, const int32_t *ids, float *out, int64_t n_ids, int64_t N, int64_t K,
                             void *stream) {
    return get_rows(qmm::F_Q5_1, w, ids, out, n_ids, N, K, 32, qmm::kQ51Bytes, stream);
}

}  // extern "C"
