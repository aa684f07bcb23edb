/*
 * qmm probes -- measurement only, NOT part of the product.  C ABI of
 * libqmm_probe.so, a library of its own beside libqmm.so.
 *
 * The product kernels are reported against MI355X's published peaks and,
 * beside them, against ceilings measured on the same part with these
 * probes: a streaming read of device memory (the bound of every decode
 * product, which streams its weights once per token -- minfer section 2.1,
 * "The bandwidth argument"), a loop of back-to-back int8 MFMAs (the bound
 * of the prefill product, a dense contraction once weights are reused across
 * tokens -- kvad "Batched prefill, and i8mm"), and an issue-rate loop of f32
 * FMAs and int8 MFMAs (the prefill's per-block scale fold runs on the vector
 * ALU beside the MFMAs).  Nothing here computes any part of the quantized
 * products.
 *
 * Conventions as in qmm.h: device pointers on the current HIP device, a
 * hipStream_t passed as void* (NULL = the null stream), asynchronous work,
 * status codes returned (never an abort), the library allocates nothing.
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QMM_PROBE_OK = 0,
    QMM_PROBE_E_SHAPE = 1,  /* a size or parameter outside the ranges below      */
    QMM_PROBE_E_NULL = 2,   /* a required pointer is NULL                          */
    QMM_PROBE_E_ALIGN = 3,  /* buf or out not 16-byte aligned, sink not 4-byte     */
    QMM_PROBE_E_DEVICE = 4, /* no current device, or it is not gfx950              */
    QMM_PROBE_E_LAUNCH = 5  /* the HIP runtime refused the launch                  */
};

/* Bytes one workgroup of the read probe covers: loads_per_lane * waves_per_wg
 * * 1024, or 0 when either parameter is not one of the supported values
 * (loads_per_lane 1, 2, 4, 8, 16; waves_per_wg 4, 8, 16). */
int64_t qmm_probe_read_span(int loads_per_lane, int waves_per_wg);

/* Streams `bytes` of device memory once.  Workgroup b (waves_per_wg waves)
 * covers bytes [S b, S b + S), S = qmm_probe_read_span(...); each lane issues
 * loads_per_lane 16-byte loads (64 lanes x 16 B = one 1 KB chunk per load)
 * before using any, and writes nothing but sink[b] = XOR of the span's 32-bit
 * words (words past `bytes` count as 0), for the host to check.
 * nontemporal != 0 gives the loads the non-temporal cache policy.
 *   buf   : device memory, 16-byte aligned, read only.
 *   bytes : > 0, a multiple of 16, at most 2^40 (and ceil(bytes / S) < 2^31).
 *   sink  : uint32 [ceil(bytes / S)], device memory, 4-byte aligned, written. */
int qmm_peak_read(const void *buf, int64_t bytes, uint32_t *sink, int loads_per_lane, int waves_per_wg,
                  int nontemporal, void *stream);

/* Issue-rate loop: 256 workgroups of 4 * waves_per_simd waves (one workgroup
 * per CU, so waves_per_simd waves on every SIMD), each wave `iters`
 * iterations of
 *   mode 0: 128 v_fma_f32 with vector-register operands (16 independent
 *           chains c = c * 0.9999 + 1.0001),
 *   mode 1: 4 v_mfma_i32_32x32x32_i8 (4 independent accumulators),
 *   mode 2: both, 32 of the FMAs after each MFMA,
 *   mode 3: mode 0's FMAs with one operand in a scalar register.
 * Timing the modes gives the cost of an FMA and of an MFMA per SIMD, how
 * much FMA issue time an MFMA takes when both run, and what a scalar operand
 * costs an FMA.
 *   out  : float [256 * 256 * waves_per_simd], device memory, 4-byte aligned,
 *          written with each lane's sum of its chains (finite).
 *   outi : int32 [same count], device memory, 4-byte aligned, written:
 *          2048 * iters in modes 1 and 2, 0 in mode 0.
 *   mode 0..3, waves_per_simd 1 or 2, iters 1 .. 1,000,000. */
int qmm_probe_issue(int mode, int waves_per_simd, int64_t iters, float *out, int32_t *outi, void *stream);

/* `workgroups` workgroups of four waves, each wave four independent chains of
 * `iters` back-to-back v_mfma_i32_32x32x32_i8 on register operands
 * (2 * 32 * 32 * 32 int8 operations each); with every operand byte 1,
 * out[t] = 2048 * iters for every lane t.
 *   out        : int32 [workgroups * 256], device memory, 16-byte aligned, written.
 *   workgroups : 1 .. 2^20.   iters : 1 .. 1,000,000 (out stays below 2^31). */
int qmm_peak_mfma_i8(int32_t *out, int64_t workgroups, int64_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_PROBE_H */
