"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle parses blocks with hand-computed byte offsets and runs its
products on pthreads over a fixed array of jobs; a C driver built together
with it under -fsanitize=address,undefined (and float-cast-overflow, which
the undefined group leaves out) runs every exported function on small and
odd shapes: one-block rows, odd block and super-block counts, a single row,
more threads than rows, the 256-thread cap, zero blocks, ids outside the
table, and every class of float for the f16 conversions.  Every buffer is
allocated at its exact size, so a read or write one byte past any of them is
reported.  Any sanitizer report fails the test (no recovery, exit code 1).
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);
void orc_quantize_q8_0(const float *x, uint8_t *out, int64_t M, int64_t K);
void orc_quantize_q8_k(const float *x, uint8_t *out, int64_t M, int64_t K);
void orc_quantize_q4_0_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q2_k_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q4_k_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q6_k_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q4_1_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q5_0_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_quantize_q5_1_w(const float *w, uint8_t *out, int64_t N, int64_t K);
void orc_dequantize_q8_0(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q4_0(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q2_k(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q4_k(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q6_k(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q8_k(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q4_1(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q5_0(const uint8_t *b, double *o, int64_t rows, int64_t K);
void orc_dequantize_q5_1(const uint8_t *b, double *o, int64_t rows, int64_t K);
int orc_matmul(int fmt, const uint8_t *w, const uint8_t *x, float *y, double *y64, double *mag,
               int64_t M, int64_t N, int64_t K, int threads);
int orc_matmul_sampled(int fmt, const uint8_t *w, const uint8_t *x, const int64_t *mi, const int64_t *ni,
                       int64_t count, double *y64, double *mag, int64_t K);
int orc_get_rows(int fmt, const uint8_t *w, const int32_t *ids, int64_t n, int64_t N, int64_t K, float *out);
int32_t orc_block_isum(int fmt, const uint8_t *w, const uint8_t *x);
void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n);
void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n);

typedef void (*quant_fn)(const float *, uint8_t *, int64_t, int64_t);
typedef void (*deq_fn)(const uint8_t *, double *, int64_t, int64_t);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double unif(void) {            /* splitmix64 -> [0, 1) */
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (double)((z ^ (z >> 31)) >> 11) * 0x1p-53;
}

/* n values: uniform in [-s, s), with the first block of each row zero and
 * one value per row scaled up 20x */
static float *values(int64_t rows, int64_t K, float s) {
    float *v = (float *)malloc(sizeof(float) * (size_t)(rows * K));
    for (int64_t i = 0; i < rows * K; ++i) v[i] = (float)((2.0 * unif() - 1.0) * s);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < 32 && i < K; ++i) v[r * K + i] = 0.0f;
        v[r * K + K - 1] *= 20.0f;
    }
    return v;
}

struct fmt { int id; const char *name; int blk; int wbytes; int xq8k; quant_fn q; deq_fn dq; };

int main(void) {
    const struct fmt F[] = {
        {0, "q4_0", 32, 18, 0, orc_quantize_q4_0_w, orc_dequantize_q4_0},
        {1, "q8_0", 32, 34, 0, orc_quantize_q8_0, orc_dequantize_q8_0},
        {2, "q2_k", 256, 84, 1, orc_quantize_q2_k_w, orc_dequantize_q2_k},
        {3, "q4_k", 256, 144, 1, orc_quantize_q4_k_w, orc_dequantize_q4_k},
        {4, "q6_k", 256, 210, 1, orc_quantize_q6_k_w, orc_dequantize_q6_k},
        {5, "q4_1", 32, 20, 0, orc_quantize_q4_1_w, orc_dequantize_q4_1},
        {6, "q5_0", 32, 22, 0, orc_quantize_q5_0_w, orc_dequantize_q5_0},
        {7, "q5_1", 32, 24, 0, orc_quantize_q5_1_w, orc_dequantize_q5_1},
    };
    const int64_t nblocks[] = {1, 3, 5};
    const int64_t Ms[] = {1, 3};
    const int64_t Ns[] = {1, 7};
    const int threads[] = {1, 3, 300};
    long calls = 0;
    for (size_t f = 0; f < sizeof(F) / sizeof(F[0]); ++f) {
        for (size_t kb = 0; kb < 3; ++kb) {
            const int64_t K = nblocks[kb] * F[f].blk;
            for (size_t mi = 0; mi < 2; ++mi)
                for (size_t ni = 0; ni < 2; ++ni) {
                    const int64_t M = Ms[mi], N = Ns[ni];
                    float *w = values(N, K, 0.05f), *x = values(M, K, 1.0f);
                    const int64_t wb = N * (K / F[f].blk) * F[f].wbytes;
                    const int64_t xb = F[f].xq8k ? M * (K / 256) * 292 : M * (K / 32) * 34;
                    uint8_t *wq = (uint8_t *)malloc((size_t)wb), *xq = (uint8_t *)malloc((size_t)xb);
                    F[f].q(w, wq, N, K);
                    if (F[f].xq8k) orc_quantize_q8_k(x, xq, M, K); else orc_quantize_q8_0(x, xq, M, K);
                    double *dw = (double *)malloc(sizeof(double) * (size_t)(N * K));
                    double *dx = (double *)malloc(sizeof(double) * (size_t)(M * K));
                    F[f].dq(wq, dw, N, K);
                    if (F[f].xq8k) orc_dequantize_q8_k(xq, dx, M, K); else orc_dequantize_q8_0(xq, dx, M, K);
                    float *y = (float *)malloc(sizeof(float) * (size_t)(M * N));
                    double *y64 = (double *)malloc(sizeof(double) * (size_t)(M * N));
                    double *mag = (double *)malloc(sizeof(double) * (size_t)(M * N));
                    for (size_t t = 0; t < 3; ++t) {
                        if (orc_matmul(F[f].id, wq, xq, y, y64, mag, M, N, K, threads[t]) != 0) return 2;
                        if (orc_matmul(F[f].id, wq, xq, y, NULL, NULL, M, N, K, threads[t]) != 0) return 2;
                        calls += 2;
                    }
                    int64_t smi[2] = {0, M - 1}, sni[2] = {N - 1, 0};
                    double sy[2], sm[2];
                    orc_matmul_sampled(F[f].id, wq, xq, smi, sni, 2, sy, sm, K);
                    orc_matmul_sampled(F[f].id, wq, xq, smi, sni, 2, sy, NULL, K);
                    int32_t ids[4] = {0, (int32_t)(N - 1), -1, (int32_t)N};
                    float *rows = (float *)malloc(sizeof(float) * (size_t)(4 * K));
                    if (orc_get_rows(F[f].id, wq, ids, 4, N, K, rows) != 0) return 3;
                    if (!isnan(rows[2 * K]) || !isnan(rows[4 * K - 1])) return 4;
                    if (F[f].id <= 1) (void)orc_block_isum(F[f].id, wq, xq);
                    free(rows); free(y); free(y64); free(mag); free(dw); free(dx);
                    free(wq); free(xq); free(w); free(x);
                    calls += 4;
                }
        }
    }
    /* f16 conversions: every half, and floats of every class */
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    float *hf = (float *)malloc(sizeof(float) * 65536);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    orc_f16_to_f32_array(h, hf, 65536);
    const float special[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 65504.0f, 65520.0f, 1e30f, -1e30f,
                             5.9604645e-8f, 2.9802322e-8f, 1e-40f, -1e-45f, 3.4028235e38f};
    const int ns = (int)(sizeof(special) / sizeof(special[0]));
    float *sf = (float *)malloc(sizeof(float) * (size_t)ns);
    uint16_t *sh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)ns);
    memcpy(sf, special, sizeof(special));
    orc_f32_to_f16_array(sf, sh, ns);
    orc_f32_to_f16_array(hf, h, 65536);
    for (int i = 0; i < ns; ++i) (void)orc_f16_to_f32(orc_f32_to_f16(special[i]));
    free(h); free(hf); free(sf); free(sh);
    printf("ok %ld\n", calls);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_sanitized"
    cc = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all", "-pthread",
          "-o", str(exe), str(drv), os.path.join(ROOT, "oracle", "qmm_oracle.c"), "-lm"]
    out = subprocess.run(cc, capture_output=True, text=True, timeout=300)
    if out.returncode != 0 and "asan" in (out.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not available: " + out.stderr[-300:])
    assert out.returncode == 0, out.stderr
    # the environment is passed on as it is; a library preloaded by the host
    # would come before the sanitizer runtime, which is allowed here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    report = run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert run.stdout.startswith("ok "), (run.stdout, report[-2000:])
