/*
 * libfkbaseline: the two standard formulations that FlashAssign and the
 * sort-inverse update replace, built on MI355X for contrast measurements.
 * They are not part of the Lloyd path of libfkmeans and share none of its
 * kernels.
 *
 * The two bottlenecks the pages start from ([itinai], the paragraphs on the
 * first and second bottleneck; [iaemfoco], the section on conventional
 * assignment; [paixiang], the update section and its 50 GB/s figure): the
 * standard assign builds the full (B, N, K) distance matrix in HBM and reads
 * it back for the argmin; the standard update adds every point into its
 * cluster's sums with scatter atomics, which contend on popular clusters.
 *
 * Source tags and conventions are those of fkmeans.h: contiguous row-major
 * tensors, caller-owned device memory, asynchronous on `stream`,
 * fk_status_t results.
 */
#ifndef FKMEANS_BASELINES_H
#define FKMEANS_BASELINES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "fkmeans.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Materialised-distance assign:
 *   dist[b,n,k] = -2 x[b,n] . c_lp[b,k]        (one batched library GEMM,
 *                                                rocBLAS, fp32 accumulate)
 *   ids[b,n]    = argmin_k (cnorm[b,k] + dist[b,n,k]), lowest k on ties
 *                                               (a separate kernel that reads
 *                                                the whole matrix back)
 *   x (B,N,d) dt, c_lp (B,K,d) dt, cnorm (B,K) fp32; dist (B,N,K) fp32 is
 *   caller-provided scratch of B*N*K*4 bytes; ids (B,N) int32 out.
 * The library keeps one rocBLAS handle per device, created at the first
 * call. FK_ERR_INVALID: B, N, d or K <= 0 or >= 2^31, a null pointer, or
 * an unknown dt. FK_ERR_HIP: a launch or rocBLAS call failed.
 */
fk_status_t fkb_assign_materialized(const void* x, const void* c_lp, const float* cnorm,
                                    fk_dtype_t dt, int64_t B, int64_t N, int64_t d, int64_t K,
                                    float* dist, int32_t* ids, hipStream_t stream);

/*
 * Scatter-atomic update:
 *   sums[b,k,:] = 0, counts[b,k] = 0; then for every point, one fp32
 *   atomic add per element of x[b,n] into sums[b,ids[b,n],:] and one
 *   integer atomic add into counts[b,ids[b,n]]; then c = sums / counts for
 *   non-empty clusters, empty clusters keep c.
 *   x (B,N,d) dt, ids (B,N) int32 in [0,K); c (B,K,d) fp32 in/out;
 *   counts (B,K) int32 out; sums (B,K,d) fp32 caller-provided scratch.
 * The order of the atomic additions is not fixed, so the sums may differ
 * between runs by fp32 reassociation. FK_ERR_INVALID, FK_ERR_HIP as above.
 */
fk_status_t fkb_update_atomic(const void* x, const int32_t* ids, fk_dtype_t dt, int64_t B,
                              int64_t N, int64_t d, int64_t K, float* c, int32_t* counts,
                              float* sums, hipStream_t stream);


/*
 * MFMA peak probe (a measurement of the chip, not a K-Means step): `blocks`
 * blocks of 256 threads; every wave issues `iters` x 32 back-to-back
 * v_mfma_f32_32x32x16_f16 (the instruction the small-D FlashAssign kernel
 * uses) over 8 independent accumulators, on operands drawn in [-1, 1) from a
 * counter-based hash of `seed` and the thread index. Each MFMA is 32768 flop,
 * so the call performs blocks * 4 * iters * 32 * 32768 flop.
 *   out    (blocks * 256) fp32: per-thread sums of the accumulators;
 *   stamps (blocks * 4) int64: per block, s_memtime at start and end, then
 *          s_memrealtime (constant rate, hipDeviceAttributeWallClockRate kHz)
 *          at start and end; the shader clock follows from their ratio.
 * FK_ERR_INVALID: blocks < 1, iters < 1 or a null pointer.
 */
fk_status_t fkb_mfma_peak(int64_t blocks, int32_t iters, uint32_t seed, float* out,
                          long long* stamps, hipStream_t stream);

/* Rate of the constant-rate counter read by s_memrealtime on the current
 * device, in kHz (hipDeviceAttributeWallClockRate); 0 if it cannot be read. */
int32_t fkb_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* FKMEANS_BASELINES_H */
