/* Microbenchmarks of the machine roofs that the attention kernels are measured
 * against: HBM streaming, reads served by the on-package caches, the bf16
 * matrix cores, the fp32 vector FMA rate and the exp2 rate of one GPU.
 *
 * These calls serve measurement only: none of them computes any part of the
 * attention.  The figures they give replace the vendor's peak numbers where a
 * measured ceiling is wanted beside the published one.
 *
 * Conventions: every call launches one kernel on `stream` (a hipStream_t, NULL
 * for the default stream) and returns at once; the caller times it with events
 * on that stream.  Pointers are device pointers owned by the caller.  Return
 * values: RPE_ROOF_OK, RPE_ROOF_E_ARG (a null pointer, a size that is not a
 * positive multiple of 16 bytes, or a non-positive iteration count; nothing is
 * launched) or RPE_ROOF_E_HIP (the launch failed).  The work a call does (bytes
 * moved or operations) is returned through `work` so that the caller needs no
 * knowledge of the grid the library picks.
 */
#ifndef RPE_ROOFS_H
#define RPE_ROOFS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RPE_ROOF_OK = 0, RPE_ROOF_E_ARG = -1, RPE_ROOF_E_HIP = -9 };

/* dst[0, bytes) = src[0, bytes): 16-byte loads and stores, each byte read once
 * and written once.  *work = 2 * bytes (bytes read plus bytes written). */
int32_t rpe_roof_copy(const void* src, void* dst, int64_t bytes, void* stream, double* work);

/* Reads src[0, bytes) `passes` times over (passes >= 1) with 16-byte loads and
 * folds it into one word that is stored to *sink only when it equals a value it
 * never takes in practice (so the reads cannot be dropped).  With a buffer that
 * the caches hold (a few tens of MB, many passes per launch so that the launch
 * itself costs little) this measures cache read bandwidth.
 * *work = passes * bytes. */
int32_t rpe_roof_read(const void* src, int64_t bytes, int32_t passes, uint32_t* sink, void* stream, double* work);

/* v_mfma_f32_32x32x16_bf16 on register operands: every wave of a grid that
 * fills each SIMD twice runs `iters` rounds of four independent accumulation
 * chains.  *work = floating-point operations (2 * 32 * 32 * 16 per product). */
int32_t rpe_roof_mfma_bf16(int32_t iters, float* sink, void* stream, double* work);

/* Scalar fp32 fused multiply-adds (no packed-fp32 forms), eight independent
 * chains per lane, `iters` rounds.  *work = floating-point operations (2 per
 * FMA). */
int32_t rpe_roof_fma_f32(int32_t iters, float* sink, void* stream, double* work);

/* The hardware exp2 (v_exp_f32), eight independent chains per lane, `iters`
 * rounds.  *work = exp2 evaluations. */
int32_t rpe_roof_exp2_f32(int32_t iters, float* sink, void* stream, double* work);

#ifdef __cplusplus
}
#endif

#endif /* RPE_ROOFS_H */
