/*
 * libfkmeans -- exact batched Lloyd's K-Means on AMD Instinct MI355X (gfx950).
 *
 * One Lloyd iteration over a batch of B independent problems, each with N
 * points in d dimensions and K clusters:
 *   - fk_norms : round the fp32 master centroids to the element type and
 *                compute their squared norms;
 *   - fk_assign: FlashAssign -- fused distance + online argmin that streams
 *                point and centroid tiles through on-chip memory and never
 *                writes the B x N x K distance matrix;
 *   - fk_update: sort-inverse update -- counting sort of the assignment into
 *                per-cluster segments (an inverse permutation of point
 *                indices; the points themselves never move), on-chip segment
 *                reductions, one stored piece per run of 256 sorted positions
 *                for long segments (no scatter atomics), then the new
 *                centroids and the centre shift;
 *   - fk_lloyd : the loop over those steps with the tol test;
 *   - fk_lloyd_host: the same loop for points kept in host memory, streamed
 *                through the device in chunks every iteration.
 *
 * Sources (web pages describing flash-kmeans):
 *   [hysenlabs] "flash-kmeans and the return of exact K-Means on the GPU"
 *   [itinai]    itinai.com summary "Flash-KMeans boosts k-means speed ... exact, fast"
 *   [arxiv]     "Flash-KMeans: Fast and Memory-Efficient Exact K-Means" (mlsanity.com)
 *   [paixiang]  "Flash-KMeans：IO感知的精确K-Means，在GPU上比FAISS快200倍以上"
 *   [iaemfoco]  "Flash-KMeans: Implementação Exata de K-Means Roda 200× Mais
 *               Rápido que FAISS em GPUs"
 *
 * Conventions for every entry point
 *   Layout     : dense row-major. x (B,N,d) and centroid copies (B,K,d) are in
 *                the element type dt; ids (B,N) and counts (B,K) are int32;
 *                master centroids (B,K,d), norms (B,K) and shift (B) are fp32.
 *   Memory     : every pointer except n_iter and fk_lloyd_host's x_host
 *                (host) is device memory owned by the caller. The library allocates no device memory and keeps
 *                no state between calls except the optional timing trace.
 *   Streams    : work is enqueued on `stream` and is asynchronous, except that
 *                fk_lloyd with tol > 0 reads each iteration's shift back
 *                (while the next iteration already runs) and returns once
 *                the stream is idle, and fk_lloyd_host always returns done.
 *   Sizes      : B >= 0, N >= 0, d >= 1, K >= 1, N < 2^31, K < 2^31,
 *                B*N*d, B*K*d < 2^62. B == 0 or N == 0 is a valid empty
 *                problem: nothing is read, outputs are set as documented.
 *   Errors     : arguments are validated before anything is enqueued; a
 *                failing call returns a status and leaves outputs
 *                unspecified. No exception crosses the ABI.
 *   Values     : inputs must be finite; otherwise results are undefined.
 */
#ifndef FKMEANS_H
#define FKMEANS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of points and centroid copies. */
typedef enum { FK_F32 = 0, FK_F16 = 1, FK_BF16 = 2 } fk_dtype_t;

typedef enum {
  FK_OK = 0,
  FK_ERR_INVALID = 1,      /* bad size, null pointer, bad dt, max_iter < 0, tol < 0 or NaN */
  FK_ERR_UNSUPPORTED = 2,  /* a shape no kernel path can run                                */
  FK_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than fk_workspace_size()   */
  FK_ERR_HIP = 4           /* a HIP launch or runtime call failed                           */
} fk_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* fk_status_string(fk_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t fk_version(void);

/*
 * Bytes of device workspace fk_update and fk_lloyd need for this problem
 * (one size serves both; at least 256). Returns 0 for invalid arguments.
 * The workspace must be 256-byte aligned. Pure host call.
 */
size_t fk_workspace_size(fk_dtype_t dt, int64_t B, int64_t N, int64_t d, int64_t K);

/*
 * Centroid precompute (the ||c||^2 term of the expanded distance).
 *   c     (B,K,d) fp32 in : master centroids.
 *   c_lp  (B,K,d) dt  out: c rounded to nearest-even in dt (a copy when dt is fp32).
 *   cnorm (B,K)  fp32 out: sum over j of c_lp^2, accumulated in fp32.
 * Reading of [paixiang] "它攻克的两大瓶颈" and [iaemfoco] "FlashAssign": the
 * fused assignment needs only x.c and ||c||^2 per pair; ||x||^2 is the same
 * for every centroid and is dropped.
 */
fk_status_t fk_norms(const float* c, void* c_lp, float* cnorm, fk_dtype_t dt,
                     int64_t B, int64_t K, int64_t d, hipStream_t stream);

/*
 * FlashAssign: ids[b,n] = argmin_k ( cnorm[b,k] - 2 x[b,n].c_lp[b,k] ),
 * i.e. the nearest centroid to x[b,n] among c_lp[b,:].
 * Every type runs on the matrix cores with fp32 accumulation: fp16/bf16
 * products are exact, fp32 products are rounded to fp32. Ties: centroids
 * whose fp32 scores are equal, or (small-D path, and the LDS-staged
 * split-D kernel: aligned rows of a multiple of 128 units, with K <= 128 or
 * enough points to give every CU a block) agree to within 2^-19 of their size --
 * the rounding of the fp32 sum itself, since those kernels carry each
 * score's row in its 4 low mantissa bits -- may resolve to either one;
 * between 32-row blocks and in the other split-D kernel exact ties go to the
 * lower index. The small-D path covers fp16/bf16 d <= 512 and fp32 d <= 256. The
 * result is the same on every run.
 * [hysenlabs] "The point of the kernel is that the distance matrix never
 * exists": points processed in tiles, centroids streamed in chunks, the
 * partial dot products kept in registers across the d loop; small-D path
 * for rows of at most 1 KB (d <= 512 fp16/bf16, d <= 256 fp32) and split-D
 * path otherwise, chosen automatically.
 * [itinai] second paragraph, [iaemfoco] "FlashAssign", [arxiv] Abstract.
 *   x (B,N,d) dt, c_lp (B,K,d) dt, cnorm (B,K) fp32 in; ids (B,N) int32 out.
 */
fk_status_t fk_assign(const void* x, const void* c_lp, const float* cnorm, fk_dtype_t dt,
                      int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                      hipStream_t stream);

/*
 * Sort-inverse update.
 *   counts[b,k] = #{n : ids[b,n] == k}                                  (exact)
 *   c[b,k]      = mean of x[b,n] over ids[b,n] == k, if counts > 0 (fp32 sums);
 *                 unchanged otherwise (empty cluster keeps its centroid)
 *   shift[b]    = sum_k || c_new[b,k] - c_old[b,k] ||^2                (fp32)
 * The ids are counting-sorted into per-cluster segments through an inverse
 * permutation of point indices (the point matrix is never permuted); each
 * segment is reduced on chip, a segment longer than 256 sorted positions in
 * pieces (one per run of 256 positions it touches, combined in a fixed
 * order), instead of one scatter atomic per point: [itinai] third paragraph, [paixiang]
 * "它攻克的两大瓶颈" and the update-contention panel of "交互式讲解",
 * [iaemfoco] "Sort-Inverse Update", [arxiv] Abstract.
 *   x (B,N,d) dt, ids (B,N) int32 in (each in [0,K));
 *   c (B,K,d) fp32 in/out; counts (B,K) int32 out; shift (B) fp32 out;
 *   ws: device workspace of at least fk_workspace_size(dt,B,N,d,K) bytes.
 * Ids outside [0,K) give undefined results (not checked on the device).
 * Deterministic for K <= 65536: the sort keeps a fixed order of each
 * cluster's points and every fp32 sum is formed in a fixed order, so the
 * same inputs give bit-identical centroids, counts and shift on every run.
 * Above that the sort ranks points with global atomics and centroids may
 * differ in the last bits between runs; counts never do.
 */
fk_status_t fk_update(const void* x, const int32_t* ids, fk_dtype_t dt,
                      int64_t B, int64_t N, int64_t d, int64_t K,
                      float* c, int32_t* counts, float* shift,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fk_update without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results as fk_update, with
 * the workspace taken from a device array that is part of the library
 * (FK_NOALLOC_SCRATCH_BYTES bytes on each GPU that runs it, held until the
 * process ends). The call allocates nothing. Problems whose
 * fk_workspace_size(dt,B,N,d,K) exceeds FK_NOALLOC_SCRATCH_BYTES are
 * rejected with FK_ERR_WORKSPACE. Every call on one GPU uses that GPU's one
 * array: calls that overlap on a GPU (other streams, other threads) race and
 * give undefined results; calls ordered on one stream are safe. The array
 * keeps the last call's contents; nothing in it is assumed zero.
 * Arguments, layouts and the other errors as fk_update.
 */
#define FK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fk_status_t fk_update_noalloc(const void* x, const int32_t* ids, fk_dtype_t dt,
                              int64_t B, int64_t N, int64_t d, int64_t K,
                              float* c, int32_t* counts, float* shift, hipStream_t stream);

/*
 * One shard's part of a data-parallel update: the points of this call are
 * one contiguous block of each problem's rows, and their per-cluster sums
 * and counts are added to sums and counts, undivided; once every shard has
 * added its part (an all-reduce of K*d + K values per problem), dividing
 * gives the centroids. Same sort-inverse path as fk_update (per-cluster
 * segments reduced on chip), with the segment sums added to sums.
 * [hysenlabs] "Multi-GPU scaling without a NCCL dependency" (contiguous
 * blocks of points per GPU, partial sums reduced across GPUs).
 *   x (B,N,d) dt, ids (B,N) int32 in; sums (B,K,d) fp32, counts (B,K) int32
 *   in/out (accumulated; zero them before the first shard).
 *   ws: fk_workspace_size(dt, B, N, d, K) bytes, 256-byte aligned.
 * Sums are fp32 adds in a fixed order per call (deterministic for K <=
 * 65536); adding into non-zero sums rounds once more per call.
 */
fk_status_t fk_update_partial(const void* x, const int32_t* ids, fk_dtype_t dt, int64_t B,
                              int64_t N, int64_t d, int64_t K, float* sums, int32_t* counts,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Lloyd's loop: centers <- init (widened to fp32); then for t < max_iter:
 * fk_norms, fk_assign, fk_update; stop after iteration t when
 * max_b shift[b] < tol (strict, so tol == 0 runs exactly max_iter iterations).
 *   x (B,N,d) dt, init (B,K,d) dt in; ids (B,N) int32 out (from the last
 *   assignment; all 0 when max_iter == 0); centers (B,K,d) fp32 in/out:
 *   after the last update on return; *n_iter (host) = completed iterations.
 *   init == NULL resumes: the loop starts from the fp32 centres `centers`
 *   already holds (an earlier call's result), so T iterations and then
 *   T' more from its centres give bit for bit the results of T + T'
 *   iterations in one call (a fixed iteration count; with tol > 0 the
 *   second call's first shift is taken against those same centres).
 * With tol > 0, iteration t + 1 is enqueued before t's shift has reached the
 * host; when t turns out to be the last, the ids and centres of t (kept in
 * the workspace) replace what t + 1 wrote, so the results are exactly those
 * of stopping after t. Deterministic like fk_update (K <= 65536).
 * Passing an earlier call's centres as init instead, rounded to dt, is an
 * approximate resume: clusters that stay empty keep the rounded centre.
 * The batched API and its tol argument: [hysenlabs] "Exact K-Means, with the
 * assignment step written in Triton"; one step = one assignment plus one
 * centroid update: [paixiang] "什么是 Flash-KMeans".
 */
fk_status_t fk_lloyd(const void* x, fk_dtype_t dt, int64_t B, int64_t N, int64_t d, int64_t K,
                     const void* init, int32_t max_iter, float tol,
                     int32_t* ids, float* centers, int32_t* n_iter,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Host-streamed Lloyd's loop, for points that stay in host memory (more
 * than fits the device, or not worth a resident copy). Every iteration
 * streams x through two device buffers of `chunk` points per problem: the
 * copy of one chunk overlaps the assign and the accumulating update of the
 * previous one, and the next iteration's first chunks overlap the end of
 * the current one. The update adds each chunk's sorted segments into
 * running fp32 sums (atomics) and counts, and divides after the last chunk.
 * [hysenlabs] section on multi-GPU scaling for large N: contiguous blocks of
 * points, a double-buffered host-to-device and compute pipeline, the next
 * iteration's first block prefetched during the reduction (one GPU here).
 *   x_host (B,N,d) dt in host memory; page-locked memory (hipHostMalloc)
 *   lets the copies overlap, pageable memory still works. init, ids,
 *   centers, n_iter, max_iter, tol and the stop rule as fk_lloyd.
 *   chunk >= 1: points per problem per copy (clamped to N).
 *   ws: fk_workspace_size_host(dt, B, chunk, d, K) bytes, 256-byte aligned.
 *   init == NULL resumes from `centers` as in fk_lloyd.
 * The call creates one non-blocking copy stream and four events, and
 * returns after all its work is done (it synchronises `stream`). Centroids
 * may differ from fk_lloyd's in the last bits (summation order).
 */
fk_status_t fk_lloyd_host(const void* x_host, fk_dtype_t dt, int64_t B, int64_t N, int64_t d,
                          int64_t K, const void* init, int32_t max_iter, float tol,
                          int64_t chunk, int32_t* ids, float* centers, int32_t* n_iter,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes fk_lloyd_host needs; 0 for invalid arguments. */
size_t fk_workspace_size_host(fk_dtype_t dt, int64_t B, int64_t chunk, int64_t d, int64_t K);

/*
 * Optional timing trace of fk_lloyd (process-wide, not thread-safe).
 * fk_trace_begin(capacity) turns it on for up to `capacity` iterations in
 * total. Each traced iteration's norms and assign kernels are launched with
 * HIP events that the launches themselves stamp at the kernel's start and end
 * (hipExtLaunchKernel), so the trace puts nothing between kernels; an
 * iteration's update runs from its assign's end to the next iteration's
 * norms start, and the last iteration a call traces ends on one stream
 * marker after its update. fk_trace_end waits for the events, writes the
 * per-phase totals and turns the trace off.
 */
typedef struct {
  int32_t iterations;   /* iterations recorded (with tol > 0, the one
                           run past a stop and undone is included)    */
  double norms_ms;      /* summed GPU time of fk_norms phases        */
  double assign_ms;     /* summed GPU time of the assign kernel      */
  double update_ms;     /* summed GPU time of the update kernels     */
} fk_trace_t;

fk_status_t fk_trace_begin(int32_t capacity);
fk_status_t fk_trace_end(fk_trace_t* out);

#ifdef __cplusplus
}
#endif
#endif /* FKMEANS_H */
