// Sort-inverse centroid update for gfx950.
//
// The assignment vector is counting-sorted by cluster id into contiguous
// segments through an inverse permutation of point indices; the point matrix
// itself never moves. Each segment is then reduced on chip, and a cluster
// whose segment is longer than one run of sorted positions is summed in
// pieces, one per run it touches, instead of one scatter atomic per point
// (itinai.com summary, third paragraph; "Flash-KMeans：IO感知的精确K-Means…",
// section "它攻克的两大瓶颈" and the update-contention panel of "交互式讲解";
// "Flash-KMeans: Implementação Exata…", section "Sort-Inverse Update";
// "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", Abstract).
//
// Terms. Sorted positions of a problem are cut into runs of kSegRun; the
// segment [lo, hi) of cluster k is short when it holds at most kSegRun
// positions, long otherwise.
//
// Every result is independent of how the GPU schedules its work: the sort is
// stable (a cluster's points keep their index order in perm), each segment
// is summed in a fixed order, and long clusters' pieces are combined in an
// order fixed by their positions. Ids, counts and centroids are therefore
// bit-identical from run to run (clusters up to 2^16: larger K takes an
// atomic-cursor scatter).
//
// Steps:
//   sort      counts, offsets (exclusive prefix sum of counts), perm
//             (perm[offsets[id] + rank] = n, rank = order of n among the
//             points of its cluster) and, per run, the cluster that holds
//             its first position.
//             Split sort (K <= 32768): per-chunk LDS histograms into a count
//             matrix, column prefixes and offsets (no global atomics); then
//             either each chunk is sorted stably in LDS and scattered
//             (chunks that fit LDS), or perm comes from LSD radix passes over
//             the whole problem, 8 key bits per pass, each pass a stable
//             counting sort (per-chunk digit counts, their prefixes, a
//             scatter ranked by wave order and lane order).
//             Larger K: per-range LDS histograms with one global atomic per
//             non-empty bin, scan, prep, then the radix passes (K <= 2^16) or
//             an atomic-cursor scatter.
//   segreduce one wave per (run, column slice). A short segment is summed
//             whole by the wave whose run holds its first position (it may
//             read up to kSegRun - 1 positions past its run) and its mean
//             (sum / count) is written straight into c, the squared move into
//             the wave's shift partial. A long segment is summed piecewise,
//             one piece per run it touches, each piece stored to its run's
//             slot (see LongPieces).
//   q1/q2     sums of the head pieces of every full block of 32 runs (Q1),
//             and of 32 Q1 rows (Q2), in order; only for problems of more
//             than kPieceDirectRuns runs (below that a long sum adds its
//             pieces one by one).
//   finalize  elementwise over (cluster, column) of long clusters:
//             c = (sum of its pieces in fixed order) / count, squared moves
//             into the block's partial; with a shift buffer, shift_reduce
//             sums a problem's partials (its segreduce waves', then its
//             finalize blocks') in a fixed order into shift[b].
// Empty clusters are never touched, so they keep their centroid. Ids outside
// [0, K) are skipped: they count nowhere and add to no cluster.
#include <limits.h>
#include <stdlib.h>

#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsBins = 32768;            // 128 KB of LDS bins per block
constexpr int kSortThreads = 1024;
constexpr int kSortUnroll = 16;               // ids in flight per thread in the sort kernels
constexpr int64_t kFusedOffsetsMax = 1 << 16; // G*K up to this: one offsets block per problem
constexpr int kRadixDigits = 256;             // values of one radix pass's key byte
constexpr int kRadixGroup = 64;               // radix chunks per group of column sums
constexpr size_t kStableLdsMax = 144 * 1024;  // dynamic LDS of one stable-scatter block, at most

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }


// Runs whose first position lies in [lo, hi) start inside cluster k.
__device__ __forceinline__ void mark_runs(int32_t* rf, int k, int lo, int hi) {
  for (int64_t r = (lo + (int64_t)kSegRun - 1) / kSegRun; r * kSegRun < hi; ++r) rf[r] = k;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

__global__ __launch_bounds__(kThreads) void fill_f32_kernel(float* __restrict__ p, float v,
                                                            int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Inclusive prefix sum / maximum over the 64 lanes of a wave by DPP: within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 lanes (lanes with no source
// take 0, or keep their value for the maximum), then across rows by the
// broadcast of lane 15 into rows 1 and 3 and of lane 31 into rows 2 and 3.
// Six VALU steps, where a shuffle per step would be an LDS permute each.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_inclusive_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x143, 0xc, 0xf, false));
  return v;
}

// Exclusive prefix sum over the kSortThreads threads of a block; `total`
// receives the block sum. wtot: kSortThreads / 64 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int32_t* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_inclusive_sum(v);
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSortThreads / 64; ++i) {
    const int t = wtot[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// Exclusive prefix maximum over the kSortThreads threads of a block (-1 for
// thread 0). wtot: kSortThreads / 64 ints of LDS.
__device__ __forceinline__ int block_exclusive_max(int v, int32_t* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_inclusive_max(v);
  const int excl_in_wave = __shfl_up(incl, 1, 64);
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = -1;
#pragma unroll
  for (int i = 0; i < kSortThreads / 64; ++i) before = i < w ? max(before, wtot[i]) : before;
  __syncthreads();
  return lane > 0 ? max(before, excl_in_wave) : before;
}

constexpr int kWavesSort = kSortThreads / 64;   // 16 waves per sort block

// Elements a wave walks in a stable pass over n elements: consecutive ranges
// of whole 64-element steps, wave 0 first.
__device__ __forceinline__ int wave_span(int n) {
  return (n + kSortThreads - 1) / kSortThreads * 64;
}

// One counting-sort pass over the n words of src (LDS) into dst (LDS), by
// the digit (word >> shift) & (2^nbits - 1). Wave w walks its own
// consecutive range of elements 64 at a time and counts into its own
// counters (hist: 16 x 2^nbits ints, wave-major), so no two waves share a
// counter; a word's new position is the number of words with a smaller
// digit, plus those with the same digit in earlier waves, plus what its
// wave's counter returns (earlier steps of the walk, and within a step the
// order in which the LDS unit serves the lanes of one instruction). Nothing
// depends on how the waves are scheduled. The starts come from one exclusive
// scan over (digit, wave) in digit-major order.
__device__ void lds_stable_pass(const uint32_t* src, uint32_t* dst, int n, int shift, int nbits,
                                int32_t* hist, int32_t* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int R = 1 << nbits;
  const int per = wave_span(n);
  const int s0 = min(w * per, n), s1 = min(s0 + per, n);
  for (int r = lane; r < R; r += 64) hist[w * R + r] = 0;
  for (int i = s0 + lane; i < s1; i += 64)
    atomicAdd(&hist[w * R + ((src[i] >> shift) & (uint32_t)(R - 1))], 1);
  __syncthreads();
  const int M = R * kWavesSort;
  const int E = (M + kSortThreads - 1) / kSortThreads;
  const int e0 = min((int)threadIdx.x * E, M), e1 = min(e0 + E, M);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += hist[(e % kWavesSort) * R + e / kWavesSort];
  int total;
  int run = block_exclusive_scan(sum, wtot, total);
  for (int e = e0; e < e1; ++e) {
    int* h = &hist[(e % kWavesSort) * R + e / kWavesSort];
    const int c = *h;
    *h = run;
    run += c;
  }
  __syncthreads();
  for (int i = s0 + lane; i < s1; i += 64) {
    const uint32_t word = src[i];
    dst[atomicAdd(&hist[w * R + ((word >> shift) & (uint32_t)(R - 1))], 1)] = word;
  }
  __syncthreads();
}

// Bits needed for the values 0 .. K (K itself marks an id outside [0, K)).
__host__ __device__ __forceinline__ int key_bits(int64_t K) {
  int b = 1;
  while (((int64_t)1 << b) <= K) ++b;
  return b;
}

// ---------------------------------------------------------------------------
// Split sort (K <= kMaxLdsBins): each problem's ids are cut into G chunks, one
// block each.
//   hist2    block (b, g): LDS histogram of its chunk, stored as row g of the
//            problem's (G, K) count matrix H (no global atomics);
//   offsets  per problem: H's columns become exclusive prefix sums over g,
//            their totals are the counts, whose exclusive prefix sum gives
//            the segment offsets; also the run starts and the long-cluster
//            flag (one block per problem when G*K is small; colscan +
//            offsets_runs on a grid otherwise);
//   perm     chunks that fit LDS: scatter_stable_kernel; otherwise the radix
//            passes.
// When radix passes follow (large G*K, chunks of at most one step below or a
// whole number of steps), hist2 also gives the first pass what its histogram
// kernel would: each step of kSortThreads * kSortUnroll ids is one radix chunk
// whose counts per low key byte (ids outside [0, K) taken as K) go to rdig row
// (b, g * steps + step), and the blocks clear `zero` (the later passes' group
// sums) for their atomics.
__global__ __launch_bounds__(kSortThreads) void hist2_kernel(const int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ H, int N, int K,
                                                             int G, int chunk,
                                                             int32_t* __restrict__ rdig,
                                                             int32_t* __restrict__ zero,
                                                             int64_t nzero) {
  extern __shared__ int32_t bins[];
  __shared__ int32_t dig[kRadixDigits];          // the current step's digit counts (rdig only)
  constexpr int STEP = kSortThreads * kSortUnroll;
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int steps = (chunk + STEP - 1) / STEP;   // rdig rows per chunk
  for (int i = t; i < K; i += kSortThreads) bins[i] = 0;
  if (zero)
    for (int64_t i = (int64_t)blockIdx.x * kSortThreads + t; i < nzero;
         i += (int64_t)gridDim.x * kSortThreads)
      zero[i] = 0;
  const int32_t* ib = ids + (int64_t)b * N;
  const int n0 = g * chunk, n1 = min(n0 + chunk, N);
  for (int j = 0; j < steps; ++j) {
    const int m = n0 + j * STEP;
    if (rdig && t < kRadixDigits) dig[t] = 0;
    __syncthreads();
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int n = m + q * kSortThreads + t;
      kk[q] = ib[min(n, n1 - 1)];                // unconditional: loads in flight together
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      if (m + q * kSortThreads + t >= n1) continue;
      const bool in = (unsigned)kk[q] < (unsigned)K;
      if (in) atomicAdd(&bins[kk[q]], 1);
      if (rdig) atomicAdd(&dig[(in ? kk[q] : K) & (kRadixDigits - 1)], 1);
    }
    __syncthreads();
    if (rdig && t < kRadixDigits)
      rdig[(((int64_t)b * G + g) * steps + j) * kRadixDigits + t] = dig[t];
  }
  __syncthreads();
  int32_t* hr = H + ((int64_t)b * G + g) * K;
  for (int i = t; i < K; i += kSortThreads) hr[i] = bins[i];
}

// Column k of a problem's H: exclusive prefix over g in place; returns the total.
__device__ __forceinline__ int column_prefix(int32_t* hb, int64_t K, int G, int k) {
  int run = 0;
  int g = 0;
  for (; g + 8 <= G; g += 8) {
    int v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = hb[(g + q) * K + k];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      hb[(g + q) * K + k] = run;
      run += v[q];
    }
  }
  for (; g < G; ++g) {
    const int v = hb[g * K + k];
    hb[g * K + k] = run;
    run += v;
  }
  return run;
}

// Column k of a problem's H: its total only (H left as it is).
__device__ __forceinline__ int column_total(const int32_t* hb, int64_t K, int G, int k) {
  int run = 0;
  int g = 0;
  for (; g + 8 <= G; g += 8) {
    int v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = hb[(g + q) * K + k];
#pragma unroll
    for (int q = 0; q < 8; ++q) run += v[q];
  }
  for (; g < G; ++g) run += hb[g * K + k];
  return run;
}

// offsets (one block per problem, G*K small): column prefixes of H and the
// counts first, then offsets, run starts and the long-cluster flag.
__global__ __launch_bounds__(kSortThreads) void offsets_kernel(
    int32_t* __restrict__ H, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ run_first, int32_t* __restrict__ has_long, int K, int G, int runs) {
  extern __shared__ int32_t cnt[];              // K + 1
  __shared__ int32_t wtot[kSortThreads / 64];
  __shared__ int32_t nlong;
  const int b = blockIdx.x, t = threadIdx.x;
  if (t == 0) nlong = 0;
  int32_t* hb = H + (int64_t)b * G * K;
  int32_t* cb = counts + (int64_t)b * K;
  for (int k = t; k < K; k += kSortThreads) cnt[k] = column_prefix(hb, K, G, k);
  __syncthreads();
  const int per = (K + kSortThreads - 1) / kSortThreads;
  const int lo = min(t * per, K), hi = min(lo + per, K);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += cnt[i];
  int total;
  int run = block_exclusive_scan(s, wtot, total);
  int32_t* ob = offsets + (int64_t)b * (K + 1);
  int32_t* rf = run_first + (int64_t)b * runs;
  int mylong = 0;
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cb[i] = c;
    cnt[i] = run;
    if (c > 0) mark_runs(rf, i, run, run + c);
    mylong += is_long(run, run + c) ? 1 : 0;
    run += c;
  }
  if (mylong) atomicAdd(&nlong, mylong);
  if (t == 0) cnt[K] = total;
  __syncthreads();
  for (int k = t; k <= K; k += kSortThreads) ob[k] = cnt[k];   // coalesced
  if (t == 0) has_long[b] = nlong;
  for (int64_t r = (total + (int64_t)kSegRun - 1) / kSegRun + t; r < runs; r += kSortThreads)
    rf[r] = K;                                   // runs past the last valid position
}

// Sum over the kThreads threads of a block (every thread gets it). wsum:
// kThreads / 64 ints of LDS.
__device__ __forceinline__ int block_sum256(int v, int32_t* wsum) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) all += wsum[i];
  __syncthreads();
  return all;
}

// First output position of each radix digit in each group of chunks of one
// problem, from the groups' digit counts cs (RG x kRadixDigits): the keys
// with a smaller digit plus the keys with this digit in earlier groups. A
// block of kRadixDigits threads, thread r for digit r. wsum: 4 ints of LDS.
__device__ void radix_group_starts(const int32_t* __restrict__ cs, int32_t* __restrict__ out,
                                   int RG, int32_t* wsum) {
  static_assert(kThreads == kRadixDigits, "one thread per digit");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int tot = 0;
  for (int rg = 0; rg < RG; ++rg) tot += cs[(int64_t)rg * kRadixDigits + t];
  const int incl = wave_inclusive_sum(tot);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kRadixDigits / 64; ++i) before += i < w ? wsum[i] : 0;
  int run = before + incl - tot;
  for (int rg = 0; rg < RG; ++rg) {
    const int c = cs[(int64_t)rg * kRadixDigits + t];
    out[(int64_t)rg * kRadixDigits + t] = run;
    run += c;
  }
}

// Large G*K: column prefixes on a grid, one thread per (problem, cluster);
// block j of a problem also stores the total count of its kThreads clusters
// in ktot[b * kblocks + j]. Without prefix (radix passes build perm, so no
// scatter reads the per-chunk starts) only the column totals are taken.
// With rdig (radix passes follow): B * RG more blocks, block (b, rg) summing
// the first pass's digit counts of radix chunks [rg * kRadixGroup, ...) (GR
// per problem) into csum0 (no atomics).
__global__ __launch_bounds__(kThreads) void colscan_kernel(int32_t* __restrict__ H,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ ktot, int K,
                                                           int G, int kblocks, int B,
                                                           const int32_t* __restrict__ rdig,
                                                           int32_t* __restrict__ csum0, int GR,
                                                           int RG, bool prefix) {
  __shared__ int32_t wsum[kThreads / 64];
  if ((int64_t)blockIdx.x >= (int64_t)B * kblocks) {
    const int i = (int)(blockIdx.x - B * kblocks);
    const int b = i / RG, rg = i % RG, t = threadIdx.x;
    const int g0 = rg * kRadixGroup, g1 = min(g0 + kRadixGroup, GR);
    const int32_t* rd = rdig + (int64_t)b * GR * kRadixDigits;
    int c = 0;
#pragma unroll 8
    for (int gg = g0; gg < g1; ++gg) c += rd[(int64_t)gg * kRadixDigits + t];
    csum0[((int64_t)b * RG + rg) * kRadixDigits + t] = c;
    return;
  }
  const int b = blockIdx.x / kblocks, j = blockIdx.x % kblocks;
  const int k = j * kThreads + threadIdx.x;
  int c = 0;
  if (k < K) {
    c = prefix ? column_prefix(H + (int64_t)b * G * K, K, G, k)
               : column_total(H + (int64_t)b * G * K, K, G, k);
    counts[(int64_t)b * K + k] = c;
  }
  const int tot = block_sum256(c, wsum);
  if (threadIdx.x == 0) ktot[blockIdx.x] = tot;
}

// Large G*K, after colscan: block j of problem b owns clusters
// [j * kThreads, (j + 1) * kThreads). Their first sorted positions are the
// sum of the totals of the blocks before (ktot) plus an exclusive scan of
// their counts. A run whose first position lies in one of these clusters
// gets it: the last cluster of the block that starts at or before that
// position (an empty cluster starts where the next one does). The last block
// writes the total and gives the runs past it K. The long-cluster flag is set
// (finalize checks every cluster).
// With csum0 (radix passes follow): B more blocks, block b turning problem
// b's first-pass group digit counts into the group starts rgbase.
__global__ __launch_bounds__(kThreads) void offsets_runs_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ ktot,
    int32_t* __restrict__ offsets, int32_t* __restrict__ run_first,
    int32_t* __restrict__ has_long, int K, int runs, int kblocks, int B,
    const int32_t* __restrict__ csum0, int32_t* __restrict__ rgbase, int RG) {
  __shared__ int32_t wsum[kThreads / 64];
  __shared__ int32_t start[kThreads + 1];
  if ((int64_t)blockIdx.x >= (int64_t)B * kblocks) {
    const int bb = (int)(blockIdx.x - B * kblocks);
    radix_group_starts(csum0 + (int64_t)bb * RG * kRadixDigits,
                       rgbase + (int64_t)bb * RG * kRadixDigits, RG, wsum);
    return;
  }
  const int b = blockIdx.x / kblocks, j = blockIdx.x % kblocks, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  int before = 0;
  for (int i = t; i < j; i += kThreads) before += ktot[(int64_t)b * kblocks + i];
  const int base = block_sum256(before, wsum);
  const int k = j * kThreads + t;
  const int c = k < K ? counts[(int64_t)b * K + k] : 0;
  const int incl = wave_inclusive_sum(c);        // inclusive scan within the wave
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int wbefore = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const int v = wsum[i];
    wbefore += i < w ? v : 0;
    all += v;
  }
  const int lo = base + wbefore + incl - c;
  int32_t* ob = offsets + (int64_t)b * (K + 1);
  if (k < K) ob[k] = lo;
  start[t] = lo;
  if (t == 0) start[kThreads] = base + all;
  const bool last = j == kblocks - 1;
  if (last && t == 0) ob[K] = base + all;
  if (j == 0 && t == 0) has_long[b] = 1;
  __syncthreads();
  int32_t* rf = run_first + (int64_t)b * runs;
  const int64_t pa = start[0], pe = start[kThreads];
  for (int64_t r = (pa + kSegRun - 1) / kSegRun + t; r * kSegRun < pe; r += kThreads) {
    const int pos = (int)(r * kSegRun);
    int a = 0, z = kThreads - 1;                 // start[a] <= pos throughout
    while (a < z) {
      const int m = (a + z + 1) >> 1;
      if (start[m] <= pos) a = m;
      else z = m - 1;
    }
    rf[r] = j * kThreads + a;
  }
  if (last)
    for (int64_t r = (pe + kSegRun - 1) / kSegRun + t; r < runs; r += kThreads)
      rf[r] = K;                                 // runs past the last valid position
}

// Direct scatter (ids in at most kDirectKeyBits bits, chunks of at most
// kStableChunk ids): wave w loads its own consecutive range of the chunk
// into registers and walks it once in steps of 64, counting into its own
// counters; each atomic returns the point's rank among the wave's earlier
// points of its id. Prefixes over the waves (per id) and over the ids then
// give each (id, wave) its first rank among the chunk's points of that id,
// and where the id's points start in the chunk's id order. With r = the
// wave's first rank plus the point's rank in the wave, point n goes to
//   perm[offsets[id] + H[g][id] + r]
// The ranks follow the walk (earlier waves, earlier steps, and within a step
// the order in which the LDS unit serves one instruction's lanes), never the
// scheduling of the waves. The stores are staged in LDS in id order first,
// so they go out as runs of consecutive addresses. The counters are 16-bit
// halves of 32-bit words (waves 2j and 2j+1 share a word; a chunk holds at
// most 2^14 ids, so a half never carries into the other).
constexpr int kDirectKeyBits = 11;
constexpr int kLocalBits = 14;                 // point index within a chunk
constexpr int kStableChunk = 1 << kLocalBits;  // ids per chunk of an LDS sort, at most

size_t direct_lds_bytes(int64_t chunk, int64_t K) {
  return (size_t)chunk * 8 + (size_t)(K + 1) * 8 + (size_t)(K + 1) * (kSortThreads / 128) * 4;
}

__global__ __launch_bounds__(kSortThreads) void scatter_direct_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ H,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int N, int K, int G,
    int chunk) {
  extern __shared__ int32_t sdir[];
  __shared__ int32_t wtot[kWavesSort];
  constexpr int SMAX = kStableChunk / kSortThreads;   // steps of 64 per wave, at most
  constexpr int WP = kWavesSort / 2;                   // counter words per id
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int n0 = g * chunk;
  const int n = min(chunk, N - n0);
  if (n <= 0) return;                            // whole block: no barrier follows
  const int K1 = K + 1;
  int32_t* spos = sdir;                          // chunk: global positions in id order
  int32_t* sval = sdir + chunk;                  // chunk: point indices in id order
  int32_t* gstart = sval + chunk;                // K + 1
  int32_t* lstart = gstart + K1;                 // K + 1
  uint32_t* cnt = reinterpret_cast<uint32_t*>(lstart + K1);   // WP x (K + 1)
  uint32_t* mycnt = cnt + (w >> 1) * K1;
  const uint32_t inc = 1u << (16 * (w & 1));
  const int sh = 16 * (w & 1);
  // the wave's consecutive range of the chunk; its ids stay in registers
  const int per = wave_span(n);
  const int s0 = min(w * per, n), s1 = min(s0 + per, n);
  const int32_t* ib = ids + (int64_t)b * N + n0;
  int kk[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    const int i = s0 + j * 64 + lane;
    if (j * 64 < per) {                          // wave-uniform
      const int k = ib[min(i, n - 1)];
      kk[j] = (unsigned)k < (unsigned)K ? k : K;
    }
  }
  const int32_t* hr = H + ((int64_t)b * G + g) * K;
  const int32_t* ob = offsets + (int64_t)b * K1;
  for (int k = t; k < K; k += kSortThreads) gstart[k] = ob[k] + hr[k];
  for (int e = t; e < WP * K1; e += kSortThreads) cnt[e] = 0;
  __syncthreads();
  // one walk: each point's rank among the wave's earlier points of its id
  int rk[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    rk[j] = -1;
    if (j * 64 < per && s0 + j * 64 + lane < s1)
      rk[j] = (int)((atomicAdd(&mycnt[kk[j]], inc) >> sh) & 0xFFFFu);
  }
  __syncthreads();
  // per id: prefix over the waves and the id's total; ids are spread over
  // the threads in consecutive groups so one scan gives their local starts
  const int KPT = (K1 + kSortThreads - 1) / kSortThreads;
  const int k0 = min(t * KPT, K1), k1 = min(k0 + KPT, K1);
  int tsum = 0;
  for (int k = k0; k < k1; ++k) {
    uint32_t cw[WP];
#pragma unroll
    for (int j = 0; j < WP; ++j) cw[j] = cnt[j * K1 + k];
    int run = 0;
#pragma unroll
    for (int j = 0; j < WP; ++j) {
      const int ce = (int)(cw[j] & 0xFFFFu), co = (int)(cw[j] >> 16);
      cnt[j * K1 + k] = (uint32_t)run | ((uint32_t)(run + ce) << 16);
      run += ce + co;
    }
    lstart[k] = run;                             // the id's total, for now
    tsum += run;
  }
  int all;
  int run = block_exclusive_scan(tsum, wtot, all);
  for (int k = k0; k < k1; ++k) {
    const int c = lstart[k];
    lstart[k] = run;
    run += c;
  }
  __syncthreads();
  // each point's place in the chunk's id order and its global position
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    if (rk[j] >= 0) {
      const int key = kk[j];
      const int r = (int)((mycnt[key] >> sh) & 0xFFFFu) + rk[j];
      const int lp = lstart[key] + r;
      spos[lp] = key < K ? gstart[key] + r : -1;
      sval[lp] = n0 + s0 + j * 64 + lane;
    }
  }
  __syncthreads();
  int32_t* pb = perm + (int64_t)b * N;
  for (int l = t; l < n; l += kSortThreads) {
    const int pos = spos[l];
    if (pos >= 0) pb[pos] = sval[l];
  }
}

// scatter2, stable form (chunks of at most kStableChunk ids): the chunk's
// words (id << kLocalBits | local index; ids outside [0, K) become K) are
// sorted in LDS by stable passes of at most 8 id bits, which orders them by
// (id, index). Position p of the sorted chunk belongs to the segment that
// starts at the last p0 <= p with a new id, and goes to
//   perm[offsets[id] + H[g][id] + (p - p0)]
// (H holds the column prefixes: where the chunk's piece of each cluster
// starts). The start of each p is found with a block-wide prefix maximum, the
// segment's base read from global memory once per segment.

__global__ __launch_bounds__(kSortThreads) void scatter_stable_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ H,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int N, int K, int G,
    int chunk, int kbits) {
  extern __shared__ uint32_t swords[];
  __shared__ int32_t wtot[kWavesSort];
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int n0 = g * chunk;
  const int n = min(chunk, N - n0);
  if (n <= 0) return;                            // whole block: no barrier follows
  uint32_t* src = swords;
  uint32_t* dst = swords + chunk;
  int32_t* hist = reinterpret_cast<int32_t*>(swords + 2 * chunk);
  const int32_t* ib = ids + (int64_t)b * N + n0;
  for (int m = 0; m < n; m += kSortThreads * kSortUnroll) {
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int i = m + q * kSortThreads + t;
      kk[q] = ib[min(i, n - 1)];                 // unconditional: loads in flight together
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int i = m + q * kSortThreads + t;
      const uint32_t key = (unsigned)kk[q] < (unsigned)K ? (uint32_t)kk[q] : (uint32_t)K;
      if (i < n) src[i] = key << kLocalBits | (uint32_t)i;
    }
  }
  __syncthreads();
  const int passes = (kbits + 7) / 8;
  const int db = (kbits + passes - 1) / passes;
  for (int q = 0; q < passes; ++q) {
    lds_stable_pass(src, dst, n, kLocalBits + q * db, min(db, kbits - q * db), hist, wtot);
    uint32_t* tmp = src;
    src = dst;
    dst = tmp;
  }
  // src: sorted words; dst: free. Segment starts write their base minus their
  // position into dst; then every position takes the base of its segment.
  const int32_t* hr = H + ((int64_t)b * G + g) * K;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  constexpr int EMAX = kStableChunk / kSortThreads;
  const int E = (n + kSortThreads - 1) / kSortThreads;
  const int q0 = min(t * E, n), q1 = min(q0 + E, n);
  int last = -1;
  uint32_t sk[EMAX];
  int sb[EMAX];
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {               // segment starts of my range
    const int p = q0 + j;
    const uint32_t key = p < q1 ? src[p] >> kLocalBits : (uint32_t)K;
    const bool st = p < q1 && (p == 0 || key != (src[p - 1] >> kLocalBits));
    sk[j] = st && key < (uint32_t)K ? key : (uint32_t)K;
    last = st ? p : last;
  }
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {               // their bases, every load in flight
    const uint32_t kc = min(sk[j], (uint32_t)(K - 1));
    sb[j] = ob[kc] + hr[kc];
  }
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const int p = q0 + j;
    const bool st = p < q1 && (p == 0 || (src[p] >> kLocalBits) != (src[p - 1] >> kLocalBits));
    if (st) dst[p] = (uint32_t)(sb[j] - p);
  }
  const int carry = block_exclusive_max(last, wtot);   // barrier inside: dst complete
  int cur = (q0 < q1 && carry >= 0) ? (int)dst[carry] : 0;
  __syncthreads();                               // every carried base read before overwrites
  for (int p = q0; p < q1; ++p) {
    const uint32_t key = src[p] >> kLocalBits;
    if (p == 0 || key != (src[p - 1] >> kLocalBits)) cur = (int)dst[p];
    dst[p] = (uint32_t)(cur + p);
  }
  __syncthreads();
  int32_t* pb = perm + (int64_t)b * N;
  for (int p = t; p < n; p += kSortThreads) {
    const uint32_t w = src[p];
    if ((w >> kLocalBits) < (uint32_t)K) pb[dst[p]] = n0 + (int)(w & (kStableChunk - 1));
  }
}

// ---------------------------------------------------------------------------
// LSD radix passes over a whole problem (chunks too large for LDS, or large
// K): pass q sorts stably by bits [8q, 8q + 8) of the key, so after the last
// pass the order is by key and, within a key, by point index. Each pass is a
// counting sort over chunks of positions (kRadixChunk, or the split sort's
// chunks when it ran first with a large count matrix):
//   radix_hist     block (b, g): counts of each digit in chunk g -> rhist row
//                  g, also added (integer atomics) to its group of
//                  kRadixRows chunks' column sums
//   radix_scan     per problem: digit starts (exclusive prefix of the digit
//                  totals) plus the column sums of earlier chunk groups ->
//                  each group's first output position per digit
//   radix_scatter  block (b, g): its chunk's start per digit (its group's
//                  start plus the earlier chunks of the group), then
//                  sub-chunks of kRadixSub keys staged in LDS; wave w walks
//                  its own consecutive range in steps of 64, and a key's
//                  position is its digit's running start plus the same-digit
//                  keys of earlier waves, earlier steps and lower lanes.
//                  Writes the key and the point index, or after the last pass
//                  only the point index, into perm.
// Keys outside [0, K) are taken as K: they sort after every real key.
// Two passes over at most 2^24 points keep one 32-bit word per point between
// them: the first pass writes (key >> 8) << 24 | point index (the low digit
// is no longer needed), the second sorts by its top byte; both run
// radix_scatter_packed, which holds one word per key in LDS as well.
constexpr int kRadix = kRadixDigits;
constexpr int kRadixChunk = 16384;             // chunk length without a split sort before
constexpr int kRadixSub = 4096;
constexpr int kRadixRows = kRadixGroup;

__device__ __forceinline__ uint32_t radix_key(int32_t k, int K) {
  return (unsigned)k < (unsigned)K ? (uint32_t)k : (uint32_t)K;
}

// raw: the keys are packed words of the first pass, taken as they are.
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(
    const int32_t* __restrict__ keys, int32_t* __restrict__ rhist, int32_t* __restrict__ colsum,
    int N, int K, int G, int RG, int shift, bool raw, int rc) {
  __shared__ int32_t h[kWavesSort][kRadix];       // one histogram per wave
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int w = t >> 6;
  for (int r = t; r < kWavesSort * kRadix; r += kSortThreads) (&h[0][0])[r] = 0;
  __syncthreads();
  const int n0 = g * rc, n1 = min(n0 + rc, N);
  const int32_t* kb = keys + (int64_t)b * N;
  for (int m = n0; m < n1; m += kSortThreads * kSortUnroll) {
    uint32_t dg[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int i = m + q * kSortThreads + t;
      const int32_t kr = kb[min(i, n1 - 1)];     // unconditional: loads in flight together
      const uint32_t kv = raw ? (uint32_t)kr : radix_key(kr, K);
      dg[q] = i < n1 ? (kv >> shift) & (kRadix - 1) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q)
      if (dg[q] != 0xFFFFFFFFu) atomicAdd(&h[w][dg[q]], 1);
  }
  __syncthreads();
  int32_t* row = rhist + ((int64_t)b * G + g) * kRadix;
  int32_t* cs = colsum + ((int64_t)b * RG + g / kRadixRows) * kRadix;
  for (int r = t; r < kRadix; r += kSortThreads) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < kWavesSort; ++ww) c += h[ww][r];
    row[r] = c;
    if (c) atomicAdd(&cs[r], c);
  }
}

// One block per problem: rgbase[b][rg][r] = (keys with a smaller digit) +
// (keys with digit r in chunk groups before rg).
__global__ __launch_bounds__(kThreads) void radix_scan_kernel(const int32_t* __restrict__ colsum,
                                                              int32_t* __restrict__ rgbase,
                                                              int RG) {
  __shared__ int32_t wsum[kThreads / 64];
  const int b = blockIdx.x;
  radix_group_starts(colsum + (int64_t)b * RG * kRadix, rgbase + (int64_t)b * RG * kRadix, RG,
                     wsum);
}

// keys_in null: the keys are the ids themselves and the point index is the
// position (first pass). keys_out null: last pass, only the index goes out.
// (Sorts of two passes over at most 2^24 points take the packed kernel
// below.) Each sub-chunk is reordered by digit in LDS first (the second walk keeps
// its keys in registers, then stores them at their local sorted places), so
// the global stores go out as runs of consecutive addresses, one run per
// digit.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ keys_in,
    const int32_t* __restrict__ idx_in, const int32_t* __restrict__ rhist,
    const int32_t* __restrict__ rgbase, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ idx_out, int N, int K, int G, int RG, int shift, int rc) {
  __shared__ int32_t skey[kRadixSub];
  __shared__ int32_t sidx[kRadixSub];
  __shared__ int32_t hist[kRadix * kWavesSort];
  __shared__ int32_t carry[kRadix];              // next global position of each digit
  __shared__ int32_t gbase[kRadix];              // global position minus local position
  __shared__ int32_t wtot[kWavesSort];
  constexpr int QS = kSortThreads / kRadix;      // row quarters for the chunk start
  constexpr int SPW = kRadixSub / kSortThreads;  // steps of 64 per wave per sub-chunk
  static_assert(kRadixRows % QS == 0, "rows per quarter");
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int32_t* kb = (keys_in ? keys_in : ids) + (int64_t)b * N;
  const int32_t* xb = idx_in ? idx_in + (int64_t)b * N : nullptr;
  // chunk start per digit: its group's start plus the group's earlier chunks
  {
    const int r = t % kRadix, q = t / kRadix;
    const int gs = g / kRadixRows * kRadixRows;
    const int a0 = gs + q * (kRadixRows / QS), a1 = min(a0 + kRadixRows / QS, g);
    const int32_t* hr = rhist + (int64_t)b * G * kRadix;
    int v[kRadixRows / QS];
#pragma unroll
    for (int j = 0; j < kRadixRows / QS; ++j)   // unconditional: loads in flight together
      v[j] = hr[(int64_t)min(a0 + j, G - 1) * kRadix + r];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kRadixRows / QS; ++j) sum += a0 + j < a1 ? v[j] : 0;
    hist[q * kRadix + r] = sum;
  }
  __syncthreads();
  if (t < kRadix) {
    int c = rgbase[((int64_t)b * RG + g / kRadixRows) * kRadix + t];
#pragma unroll
    for (int q = 0; q < QS; ++q) c += hist[q * kRadix + t];
    carry[t] = c;
  }
  __syncthreads();
  int32_t* ko = keys_out ? keys_out + (int64_t)b * N : nullptr;
  int32_t* xo = idx_out ? idx_out + (int64_t)b * N : nullptr;
  const int n0 = g * rc, n1 = min(n0 + rc, N);
  // a sub-chunk's keys (and indices) are loaded while the one before is
  // being sorted (clamped, unconditional loads: all in flight together)
  int kk[SPW], xx[SPW];
  auto load_sub = [&](int m0, int (&kv)[SPW], int (&xv)[SPW]) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int i = min(m0 + j * kSortThreads + t, n1 - 1);
      kv[j] = kb[i];
      xv[j] = xb ? xb[i] : i;
    }
  };
  if (n0 < n1) load_sub(n0, kk, xx);
  for (int m0 = n0; m0 < n1; m0 += kRadixSub) {
    const int m = min(kRadixSub, n1 - m0);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int l = j * kSortThreads + t;
      skey[l] = (int32_t)radix_key(kk[j], K);
      sidx[l] = xx[j];
    }
    if (m0 + kRadixSub < n1) load_sub(m0 + kRadixSub, kk, xx);
    for (int r = lane; r < kRadix; r += 64) hist[w * kRadix + r] = 0;
    __syncthreads();
    const int per = wave_span(m);
    const int s0 = min(w * per, m), s1 = min(s0 + per, m);
    for (int i = s0 + lane; i < s1; i += 64)
      atomicAdd(&hist[w * kRadix + (((uint32_t)skey[i] >> shift) & (kRadix - 1))], 1);
    __syncthreads();
    // local start of each (digit, wave): digits in order, waves in order
    int hv[kWavesSort];
    int tot = 0;
    if (t < kRadix) {
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) hv[ww] = hist[ww * kRadix + t];
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) tot += hv[ww];
    }
    int all;
    const int lstart = block_exclusive_scan(t < kRadix ? tot : 0, wtot, all);
    if (t < kRadix) {
      int run = lstart;
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) {
        hist[ww * kRadix + t] = run;
        run += hv[ww];
      }
      gbase[t] = carry[t] - lstart;
      carry[t] += tot;
    }
    __syncthreads();
    // local sorted place of each key, kept in registers until every wave has
    // read its keys
    int lp[SPW], lk[SPW], lx[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int i = s0 + j * 64 + lane;
      lp[j] = -1;
      lk[j] = lx[j] = 0;
      if (i < s1) {
        const uint32_t key = (uint32_t)skey[i];
        lp[j] = atomicAdd(&hist[w * kRadix + ((key >> shift) & (kRadix - 1))], 1);
        lk[j] = (int)key;
        lx[j] = sidx[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      if (lp[j] >= 0) {
        skey[lp[j]] = lk[j];
        sidx[lp[j]] = lx[j];
      }
    }
    __syncthreads();
    for (int l = t; l < m; l += kSortThreads) {
      const int key = skey[l];
      const int pos = gbase[((uint32_t)key >> shift) & (kRadix - 1)] + l;
      if (ko) ko[pos] = key;
      xo[pos] = sidx[l];
    }
    __syncthreads();
  }
}

// The two passes of a packed sort (keys below 2^16, at most 2^24 points):
// one 32-bit word per key, both in registers and in LDS.
//   FIRST: keys are the ids and the point index is the position; the word
//          is key << 12 | the key's index within its sub-chunk, and the
//          pass writes the packed word (key >> 8) << 24 | point index;
//   else:  keys are those packed words, sorted by their top byte, and the
//          pass writes the point index (the low 24 bits) into perm.
// Wave w loads its own consecutive range of a sub-chunk (64 keys per step),
// so the keys stay in registers: one LDS atomic per key on the wave's digit
// counts gives its rank among the same-digit keys before it in the wave
// (in the walk's order: earlier steps, and within a step the order in which
// the LDS unit serves one instruction's lanes), the counts become starts by a
// scan over (digit, wave), and each word goes to start + rank in LDS. The
// global stores then go out in local sorted order: runs of consecutive
// addresses, one per digit. The next sub-chunk's keys load during the
// current one.
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_packed_kernel(
    const int32_t* __restrict__ keys, const int32_t* __restrict__ rhist,
    const int32_t* __restrict__ rgbase, int32_t* __restrict__ out, int N, int K, int G, int RG,
    int rc) {
  __shared__ uint32_t sw[kRadixSub];               // words in local sorted order
  __shared__ int32_t hist[kWavesSort * kRadix];    // per-wave digit counts, then starts
  __shared__ int32_t carry[kRadix];                // next global position of each digit
  __shared__ int32_t gbase[kRadix];                // global position minus local position
  __shared__ int32_t wtot[kWavesSort];
  constexpr int QS = kSortThreads / kRadix;        // row quarters for the chunk start
  constexpr int SPW = kRadixSub / kSortThreads;    // keys per lane per sub-chunk
  constexpr int SHIFT = FIRST ? 12 : 24;           // digit position in a word
  static_assert(kRadixSub <= 4096, "local index in 12 bits");
  static_assert(kRadixRows % QS == 0, "rows per quarter");
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int32_t* kb = keys + (int64_t)b * N;
  // chunk start per digit: its group's start plus the group's earlier chunks
  {
    const int r = t % kRadix, q = t / kRadix;
    const int gs = g / kRadixRows * kRadixRows;
    const int a0 = gs + q * (kRadixRows / QS), a1 = min(a0 + kRadixRows / QS, g);
    const int32_t* hr = rhist + (int64_t)b * G * kRadix;
    int v[kRadixRows / QS];
#pragma unroll
    for (int j = 0; j < kRadixRows / QS; ++j)   // unconditional: loads in flight together
      v[j] = hr[(int64_t)min(a0 + j, G - 1) * kRadix + r];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kRadixRows / QS; ++j) sum += a0 + j < a1 ? v[j] : 0;
    hist[q * kRadix + r] = sum;
  }
  __syncthreads();
  if (t < kRadix) {
    int c = rgbase[((int64_t)b * RG + g / kRadixRows) * kRadix + t];
#pragma unroll
    for (int q = 0; q < QS; ++q) c += hist[q * kRadix + t];
    carry[t] = c;
  }
  __syncthreads();
  for (int r = lane; r < kRadix; r += 64) hist[w * kRadix + r] = 0;
  int32_t* ob = out + (int64_t)b * N;
  const int n0 = g * rc, n1 = min(n0 + rc, N);
  // the wave's range of sub-chunk m0 and the lane's keys in it (clamped,
  // unconditional loads: all in flight together)
  auto span = [&](int m0, int& s0, int& s1) {
    const int m = min(kRadixSub, n1 - m0), per = wave_span(m);
    s0 = min(w * per, m);
    s1 = min(s0 + per, m);
  };
  int kk[SPW];
  auto load_sub = [&](int m0, int (&kv)[SPW]) {
    int s0, s1;
    span(m0, s0, s1);
#pragma unroll
    for (int j = 0; j < SPW; ++j) kv[j] = kb[min(m0 + s0 + j * 64 + lane, n1 - 1)];
  };
  if (n0 < n1) load_sub(n0, kk);
  __syncthreads();
  for (int m0 = n0; m0 < n1; m0 += kRadixSub) {
    const int m = min(kRadixSub, n1 - m0);
    int s0, s1;
    span(m0, s0, s1);
    uint32_t wd[SPW];
    int rk[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int i = s0 + j * 64 + lane;
      wd[j] = FIRST ? radix_key(kk[j], K) << 12 | (uint32_t)i : (uint32_t)kk[j];
    }
    if (m0 + kRadixSub < n1) load_sub(m0 + kRadixSub, kk);
    // rank within the wave
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      rk[j] = 0;
      if (s0 + j * 64 + lane < s1)
        rk[j] = atomicAdd(&hist[w * kRadix + ((wd[j] >> SHIFT) & (kRadix - 1))], 1);
    }
    __syncthreads();
    // local start of each (digit, wave): digits in order, waves in order
    int hv[kWavesSort];
    int tot = 0;
    if (t < kRadix) {
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) hv[ww] = hist[ww * kRadix + t];
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) tot += hv[ww];
    }
    int all;
    const int lstart = block_exclusive_scan(t < kRadix ? tot : 0, wtot, all);
    if (t < kRadix) {
      int run = lstart;
#pragma unroll
      for (int ww = 0; ww < kWavesSort; ++ww) {
        hist[ww * kRadix + t] = run;
        run += hv[ww];
      }
      gbase[t] = carry[t] - lstart;
      carry[t] += tot;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      if (s0 + j * 64 + lane < s1)
        sw[hist[w * kRadix + ((wd[j] >> SHIFT) & (kRadix - 1))] + rk[j]] = wd[j];
    __syncthreads();
    for (int r = lane; r < kRadix; r += 64) hist[w * kRadix + r] = 0;
    for (int l = t; l < m; l += kSortThreads) {
      const uint32_t x = sw[l];
      const int pos = gbase[(x >> SHIFT) & (kRadix - 1)] + l;
      ob[pos] = FIRST ? (int32_t)((x >> 20) << 24 | (uint32_t)(m0 + (int)(x & 4095)))
                      : (int32_t)(x & 0xFFFFFF);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sort for K > kMaxLdsBins (bins in several LDS ranges).
// hist: block (chunk, bin range, b). Bins of this range live in dynamic LDS.
template <int IPT>
__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ ids,
                                                        int32_t* __restrict__ counts, int N,
                                                        int K, int nchunks, int nranges) {
  extern __shared__ int32_t bins[];
  constexpr int CH = kThreads * IPT;
  const int chunk = blockIdx.x % nchunks;
  const int range = (blockIdx.x / nchunks) % nranges;
  const int b = blockIdx.x / (nchunks * nranges);
  const int k0 = range * kMaxLdsBins;
  const int nb = (K - k0) < kMaxLdsBins ? (K - k0) : kMaxLdsBins;
  for (int i = threadIdx.x; i < nb; i += kThreads) bins[i] = 0;
  __syncthreads();
  const int32_t* ib = ids + (int64_t)b * N;
  const int n0 = chunk * CH;
#pragma unroll 4
  for (int q = 0; q < IPT; ++q) {
    const int n = n0 + q * kThreads + threadIdx.x;
    if (n < N) {
      const int k = ib[n] - k0;
      if ((unsigned)k < (unsigned)nb && k0 + k < K) atomicAdd(&bins[k], 1);
    }
  }
  __syncthreads();
  int32_t* cb = counts + (int64_t)b * K + k0;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const int v = bins[i];
    if (v) atomicAdd(&cb[i], v);
  }
}

// scan: one block per problem; offsets = exclusive prefix sum of counts,
// cursor = offsets (cursor null: not needed).
__global__ __launch_bounds__(kSortThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ cursor, int K) {
  __shared__ int32_t wtot[kSortThreads / 64];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t per = ((int64_t)K + kSortThreads - 1) / kSortThreads;
  const int64_t lo = t * per < K ? t * per : K;
  const int64_t hi = lo + per < K ? lo + per : K;
  const int32_t* cb = counts + (int64_t)b * K;
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += cb[i];
  int total;
  int run = block_exclusive_scan(s, wtot, total);
  int32_t* ob = offsets + (int64_t)b * (K + 1);
  int32_t* kb = cursor ? cursor + (int64_t)b * K : nullptr;
  for (int64_t i = lo; i < hi; ++i) {
    ob[i] = run;
    if (kb) kb[i] = run;
    run += cb[i];
  }
  if (t == 0) ob[K] = total;
}

// prep: one wave per cluster marks the runs that start inside it; runs past
// the last position get K; the long-cluster flag is set (finalize checks
// every cluster).
__global__ __launch_bounds__(kThreads) void prep_kernel(const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ run_first,
                                                        int32_t* __restrict__ has_long,
                                                        int K, int runs,
                                                        int blocks_per_batch) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.x / blocks_per_batch;
  const int j = blockIdx.x % blocks_per_batch;
  if (j == 0 && threadIdx.x == 0) has_long[b] = 1;   // not counted here: finalize checks all
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  int32_t* rf = run_first + (int64_t)b * runs;
  const int total = ob[K];
  for (int k = j * (kThreads / 64) + wv; k < K; k += blocks_per_batch * (kThreads / 64)) {
    const int lo = ob[k], hi = ob[k + 1];
    if (hi <= lo) continue;
    for (int64_t r = (lo + (int64_t)kSegRun - 1) / kSegRun + lane; r * kSegRun < hi; r += 64)
      rf[r] = k;
  }
  const int64_t r0 = (total + (int64_t)kSegRun - 1) / kSegRun;
  for (int64_t r = r0 + (int64_t)j * kThreads + threadIdx.x; r < runs;
       r += (int64_t)blocks_per_batch * kThreads)
    rf[r] = K;
}

// scatter: perm[offset of cluster + rank] = n.
template <int IPT>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ ids,
                                                           int32_t* __restrict__ cursor,
                                                           int32_t* __restrict__ perm, int N,
                                                           int K, int nchunks, int nranges) {
  extern __shared__ int32_t bins[];
  constexpr int CH = kThreads * IPT;
  const int chunk = blockIdx.x % nchunks;
  const int range = (blockIdx.x / nchunks) % nranges;
  const int b = blockIdx.x / (nchunks * nranges);
  const int k0 = range * kMaxLdsBins;
  const int nb = (K - k0) < kMaxLdsBins ? (K - k0) : kMaxLdsBins;
  for (int i = threadIdx.x; i < nb; i += kThreads) bins[i] = 0;
  __syncthreads();
  const int32_t* ib = ids + (int64_t)b * N;
  const int n0 = chunk * CH;
  int key[IPT], rank[IPT];
#pragma unroll
  for (int q = 0; q < IPT; ++q) {
    const int n = n0 + q * kThreads + threadIdx.x;
    key[q] = -1;
    rank[q] = 0;
    if (n < N) {
      const int k = ib[n] - k0;
      if ((unsigned)k < (unsigned)nb && k0 + k < K) {
        key[q] = k;
        rank[q] = atomicAdd(&bins[k], 1);
      }
    }
  }
  __syncthreads();
  int32_t* cb = cursor + (int64_t)b * K + k0;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const int v = bins[i];
    if (v) bins[i] = atomicAdd(&cb[i], v);
  }
  __syncthreads();
  int32_t* pb = perm + (int64_t)b * N;
#pragma unroll
  for (int q = 0; q < IPT; ++q) {
    if (key[q] >= 0) pb[bins[key[q]] + rank[q]] = n0 + q * kThreads + threadIdx.x;
  }
}

// ---------------------------------------------------------------------------
// segreduce: one wave per (run, column slice).
//
// The positions a wave owns form one contiguous range [s, E): the piece of a
// long segment that covers the run's first position (if any), then every
// segment that starts inside the run, the last of them possibly ending in the
// next run (short) or cut at the run's end (long). The wave stages perm for
// its run and the next one in LDS and lists its segments (cluster, end of its
// rows, count) in three VGPRs, one segment per lane, 64 at a time. It then
// streams [s, E) in batches of BR rows regardless of segment boundaries, with
// the next batch's loads issued before the current batch is summed. Rows are
// read as 16-byte vectors: LPR lanes cover the slice's SPAN columns of a row,
// so one wave instruction reads R = 64/LPR rows. Inside a batch each
// segment's rows are added under a 0/1 position weight; when a segment ends,
// the R row groups are summed across lanes and the sum goes out: divided by
// the count into the cluster's row of c for a short segment (the finished
// mean), stored to the run's slot for a piece of a long one (see
// LongPieces), or, when accumulating over chunks of points, added with
// atomics to its sums row.
template <int DT>
__device__ __forceinline__ void widen16(const uint4 v, float* out) {
  if constexpr (DT == FK_F32) {
    out[0] = __builtin_bit_cast(float, v.x);
    out[1] = __builtin_bit_cast(float, v.y);
    out[2] = __builtin_bit_cast(float, v.z);
    out[3] = __builtin_bit_cast(float, v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = Elem<DT>::widen((uint16_t)(w[i] & 0xFFFFu));
      out[2 * i + 1] = Elem<DT>::widen((uint16_t)(w[i] >> 16));
    }
  }
}

// Lane swaps of gfx950 (VALU, no LDS): v_permlane16_swap exchanges the odd
// 16-lane rows of a with the even rows of b; v_permlane32_swap exchanges the
// upper half of a with the lower half of b. Written as instructions with two
// in-out operands (the compiler's own lowering of these swaps here reads the
// first result twice); the s_nop gives the wait states a VALU write needs
// before a permlane reads the register.
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Sum of v over the lanes that share lane % LPR (LPR = 4, 8 or 16), left in
// every lane: rotations by 8 and 4 inside each 16-lane row (DPP), then the
// row pairs and the two halves added through the lane swaps above.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
  if constexpr (LPR <= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128,
                                                            0xF, 0xF, false));   // row_ror:8
  if constexpr (LPR <= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124,
                                                            0xF, 0xF, false));   // row_ror:4
  float a = v, b = v;
  permlane16_swap(a, b);                         // a: rows 0,0,2,2   b: rows 1,1,3,3
  a += b;
  b = a;
  permlane32_swap(a, b);                         // a: lower half twice, b: upper half twice
  return a + b;
}

template <int DT, int LPR, bool VEC>
__global__ __launch_bounds__(kThreads) void segreduce_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ run_first,
    float* __restrict__ sums, float* __restrict__ c, float* __restrict__ part, int part_stride,
    float* __restrict__ pieces, int N, int d, int K, int runs, int slices, int64_t total_waves,
    bool acc_all) {
  constexpr int R = 64 / LPR;                    // rows per wave instruction
  constexpr int EB = DT == FK_F32 ? 4 : 2;
  constexpr int EV = 16 / EB;                    // elements per 16-byte vector
  constexpr int SPAN = LPR * EV;                 // columns per slice
  constexpr int U = 4;                           // row-iterations per batch
  constexpr int BR = U * R;                      // rows per batch
  constexpr int STAGE = 2 * kSegRun;
  __shared__ int32_t lperm[kThreads / 64][STAGE];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int g = lane / LPR, li = lane % LPR;
  const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + wv;
  if (wid >= total_waves) return;                // whole wave; no block barrier follows
  const int per_batch = runs * slices;
  // Problems in the order that finds the most of x still in the memory-side
  // cache (MALL): the assign walks each XCD's contiguous eighth of the
  // (problem, point block) range in order, so the last problem of every
  // eighth was read last; take those first, then the ones before them. The
  // next assign then starts on the problems read last here.
  int b = (int)(wid / per_batch);
  const int64_t nb = total_waves / per_batch;
  if (nb % 8 == 0) {
    const int b8 = (int)(nb / 8);
    b = (b % 8) * b8 + (b8 - 1 - b / 8);
  }
  const int rem = (int)(wid % per_batch);
  const int run = rem / slices, slice = rem % slices;
  const int p0 = run * kSegRun;
  const int p1 = min(p0 + kSegRun, N);
  const int col = slice * SPAN + li * EV;        // my first column
  const bool colok = col < d;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  const char* xb = reinterpret_cast<const char*>(x) + (int64_t)b * N * d * EB;
  float* sb = acc_all ? sums + (int64_t)b * K * d : nullptr;
  float* cb = acc_all ? nullptr : c + (int64_t)b * K * d;
  float* pr = acc_all ? nullptr : pieces + ((int64_t)b * runs + run) * 2 * d;   // this run's slots
  float moved = 0.f;                             // squared moves of this wave's short clusters
  [&]() {

  // the run's staged positions are loaded together with its first cluster
  // (clamped loads, all in flight at once), then stored to LDS once known
  // to be needed
  const int pend = min(p0 + STAGE, N);
  const int32_t* pp = perm + (int64_t)b * N + p0;
  int pv[STAGE / 64];
#pragma unroll
  for (int q = 0; q < STAGE / 64; ++q) pv[q] = pp[min(lane + 64 * q, pend - p0 - 1)];
  int k = run_first[(int64_t)b * runs + run];
  k = k < 0 ? K : k;
  if (k >= K) return;

  // offsets window: win holds ob[kw + lane]
  int kw = k;
  int win = ob[min(kw + lane, K)];
#pragma unroll
  for (int q = 0; q < STAGE / 64; ++q)
    if (lane + 64 * q < pend - p0) lperm[wv][lane + 64 * q] = pv[q];
  auto off = [&](int kk) {
    if ((unsigned)(kk - kw) >= 64u) {            // outside the window (either side)
      kw = kk;
      win = ob[min(kw + lane, K)];
    }
    return __builtin_amdgcn_readlane(win, kk - kw);
  };
  // Segment list: lane i holds the (kk, end, count) of one owned segment.
  // fill() lists up to 64 segments starting at cluster kk (whose rows begin
  // at `start`) and returns how many; nxt receives where to continue (K: no
  // more).
  int sk = 0, se = 0, sc = 0;
  auto fill = [&](int kk, int& nxt) {
    int n = 0;
    while (kk < K && n < 64) {
      const int lo = off(kk);
      if (lo >= p1) {
        kk = K;
        break;
      }
      const int hi = off(kk + 1);
      if (hi > lo && (is_long(lo, hi) || lo >= p0)) {
        const int end = is_long(lo, hi) ? min(hi, p1) : hi;
        const int cnt = is_long(lo, hi) ? -(hi - lo) : hi - lo;   // negative: long
        sk = lane == n ? kk : sk;
        se = lane == n ? end : se;
        sc = lane == n ? cnt : sc;
        ++n;
      }
      ++kk;
    }
    nxt = kk;
    return n;
  };
  int knext;
  int nseg = fill(k, knext);
  if (nseg == 0) return;
  // first row: a long piece starts at max(lo, p0), a short segment at lo
  const int c0 = __builtin_amdgcn_readlane(sc, 0);
  const int lo0 = off(__builtin_amdgcn_readlane(sk, 0));
  const int s = c0 < 0 ? max(lo0, p0) : __builtin_amdgcn_readlane(se, 0) - c0;
  // last row + 1: the end of the last owned segment
  int E = __builtin_amdgcn_readlane(se, nseg - 1);
  for (int kk = knext; kk < K; ++kk) {           // only with more than 64 segments
    const int lo = off(kk);
    if (lo >= p1) break;
    const int hi = off(kk + 1);
    if (hi > lo && (is_long(lo, hi) || lo >= p0)) E = is_long(lo, hi) ? min(hi, p1) : hi;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // current segment: list entry si
  int si = 0;
  int jk = __builtin_amdgcn_readlane(sk, 0);
  int jend = __builtin_amdgcn_readlane(se, 0);
  int jcnt = __builtin_amdgcn_readlane(sc, 0);
  int jstart = s;
  // the current piece is the run's head piece (slot 0): a long segment that
  // started before the run; any later long piece starts inside it (slot 1)
  bool jhead = c0 < 0 && lo0 < p0;
  float acc[EV];
#pragma unroll
  for (int i = 0; i < EV; ++i) acc[i] = 0.f;

  // Loads are unconditional (a position past E reads a valid staged row and
  // gets weight 0), so the compiler can count them and keep the next batch in
  // flight while this one is summed.
  const int colc = colok ? col : 0;
  auto load = [&](int base, uint4* v) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = min(base + u * R + g, E - 1);
      const int64_t row = (int64_t)lperm[wv][p - p0] * d;
      if constexpr (VEC) {
        v[u] = *reinterpret_cast<const uint4*>(xb + (row + colc) * EB);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < EV; ++i) {
          const int64_t e = row + (colc + i < d ? colc + i : 0);
          uint32_t bits;
          if constexpr (DT == FK_F32) bits = reinterpret_cast<const uint32_t*>(xb)[e];
          else bits = reinterpret_cast<const uint16_t*>(xb)[e];
          if constexpr (DT == FK_F32) w[i] = bits;
          else w[i / 2] |= bits << (16 * (i & 1));
        }
        v[u] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < EV; ++i) acc[i] = group_sum<LPR>(acc[i]);
    if (g == 0 && colok) {
      if (jcnt > 0 && !acc_all) {                // short: the finished mean, straight into c
        float* row = cb + (int64_t)jk * d + col;
        const float inv = 1.0f / (float)jcnt;
        float nw[EV];
#pragma unroll
        for (int i = 0; i < EV; ++i) nw[i] = acc[i] * inv;
        if constexpr (VEC) {
          // whole 16-byte vectors: col is a multiple of EV and d of EV
          if (part) {
#pragma unroll
            for (int i = 0; i < EV; i += 4) {
              const float4 o = *reinterpret_cast<const float4*>(row + i);
              const float dl[4] = {nw[i] - o.x, nw[i + 1] - o.y, nw[i + 2] - o.z, nw[i + 3] - o.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) moved = fmaf(dl[e], dl[e], moved);
            }
          }
#pragma unroll
          for (int i = 0; i < EV; i += 4)
            *reinterpret_cast<float4*>(row + i) = make_float4(nw[i], nw[i + 1], nw[i + 2], nw[i + 3]);
        } else {
#pragma unroll
          for (int i = 0; i < EV; ++i) {
            if (col + i < d) {
              if (part) {
                const float dl = nw[i] - row[i];
                moved = fmaf(dl, dl, moved);
              }
              row[i] = nw[i];
            }
          }
        }
      } else if (acc_all) {                      // accumulating: every segment into sums
        float* row = sb + (int64_t)jk * d + col;
#pragma unroll
        for (int i = 0; i < EV; ++i)
          if (col + i < d) unsafeAtomicAdd(row + i, acc[i]);
      } else {                                   // a piece of a long segment: its slot
        float* row = pr + (jhead ? 0 : d) + col;
        if constexpr (VEC) {                     // d % 4 == 0: 16-byte aligned slots
#pragma unroll
          for (int i = 0; i < EV; i += 4)
            *reinterpret_cast<float4*>(row + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
        } else {
#pragma unroll
          for (int i = 0; i < EV; ++i)
            if (col + i < d) row[i] = acc[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < EV; ++i) acc[i] = 0.f;
  };
  // sum one batch of rows [base, base + BR)
  auto consume = [&](int base, const uint4* v) {
    const int bend = min(base + BR, E);
    for (;;) {
      const int r0 = max(jstart, base), r1 = min(jend, bend);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = base + u * R + g;
        const float m = (p >= r0 && p < r1) ? 1.f : 0.f;
        float f[EV];
        widen16<DT>(v[u], f);
#pragma unroll
        for (int i = 0; i < EV; ++i) acc[i] = fmaf(f[i], m, acc[i]);
      }
      if (jend > bend) return;                   // segment continues in the next batch
      flush();
      if (jend >= E) return;                     // owned range done
      ++si;
      if (si == nseg) {                          // refill the list (more than 64 segments)
        nseg = fill(knext, knext);
        si = 0;
      }
      jstart = jend;
      jhead = false;
      jk = __builtin_amdgcn_readlane(sk, si);
      jend = __builtin_amdgcn_readlane(se, si);
      jcnt = __builtin_amdgcn_readlane(sc, si);
      if (jstart >= bend) return;                // next segment starts in the next batch
    }
  };
  // two batches in flight: the loads of the batch after next are issued
  // before a batch is summed (past E they re-read a staged row and get
  // weight 0)
  uint4 va[U], vb[U];
  load(s, va);
  for (int base = s; base < E; base += 2 * BR) {
    load(base + BR, vb);
    __builtin_amdgcn_sched_barrier(0);
    consume(base, va);
    load(base + 2 * BR, va);
    __builtin_amdgcn_sched_barrier(0);
    if (base + BR < E) consume(base + BR, vb);
  }
  }();
  if (part) {                                    // every wave writes its slot, zero included
    moved = wave_sum(moved);
    if (lane == 0) part[(int64_t)b * part_stride + rem] = moved;
  }
}

// Q1 and Q2 rows of the long pieces (see LongPieces), once segreduce has
// stored them. q1blocks: block (b, j) sums the slot-0 pieces of runs
// 32j .. 32j+31 in run order into Q1 row j; q2blocks: block (b, i) sums Q1
// rows 32i .. 32i+31 in order into Q2 row i. Only full blocks are formed;
// problems without long clusters do nothing. Kernels of their own: their
// start sees every piece, with no device-wide fence.
__global__ __launch_bounds__(kThreads) void q1blocks_kernel(LongPieces lp, float* __restrict__ q1,
                                                            const int32_t* __restrict__ has_long,
                                                            int d) {
  const int b = blockIdx.x / lp.nq1, j = blockIdx.x % lp.nq1;
  if (!has_long[b] || (j + 1) * kQ1 > lp.runs) return;
  const float* pb = lp.pieces + (int64_t)b * lp.runs * 2 * d;
  float* out = q1 + ((int64_t)b * lp.nq1 + j) * d;
  for (int c = threadIdx.x; c < d; c += kThreads) {
    float t = 0.f;
#pragma unroll 8
    for (int r = 0; r < kQ1; ++r) t += pb[((int64_t)(j * kQ1 + r) * 2) * d + c];
    out[c] = t;
  }
}

__global__ __launch_bounds__(kThreads) void q2blocks_kernel(LongPieces lp, const float* __restrict__ q1,
                                                            float* __restrict__ q2,
                                                            const int32_t* __restrict__ has_long,
                                                            int d) {
  const int b = blockIdx.x / lp.nq2, i = blockIdx.x % lp.nq2;
  if (!has_long[b] || (i + 1) * kQ1 * kQ2 > lp.runs) return;
  const float* qb = q1 + (int64_t)b * lp.nq1 * d;
  float* out = q2 + ((int64_t)b * lp.nq2 + i) * d;
  for (int c = threadIdx.x; c < d; c += kThreads) {
    float t = 0.f;
#pragma unroll 8
    for (int r = 0; r < kQ2; ++r) t += qb[(int64_t)(i * kQ2 + r) * d + c];
    out[c] = t;
  }
}

// ---------------------------------------------------------------------------
// finalize, one thread per group of kFinVec consecutive elements of a
// problem's (K, d) centroid block: a long cluster's new value is the sum of
// its pieces (fixed order, LongPieces) divided by its count, and the block's
// squared moves go to its partial. Short clusters were finished by segreduce;
// empty clusters keep their centroid.
constexpr int kFinVec = 4;

template <bool SHIFT>
__global__ __launch_bounds__(kThreads) void finalize_kernel(
    LongPieces lp, const int32_t* __restrict__ offsets, float* __restrict__ c,
    float* __restrict__ part, int part_stride, const int32_t* __restrict__ has_long, int d, int K,
    int blocks_per_batch) {
  __shared__ float wsum[kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x / blocks_per_batch, j = blockIdx.x % blocks_per_batch;
  if (!has_long[b]) {                            // nothing to finish in this problem
    if (SHIFT && threadIdx.x == 0) part[(int64_t)b * part_stride + j] = 0.f;
    return;
  }
  const int64_t per = (int64_t)K * d;
  const int64_t e0 = ((int64_t)j * kThreads + threadIdx.x) * kFinVec;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  float* cb = c + (int64_t)b * per;
  float moved = 0.f;
  for (int64_t e = e0; e < e0 + kFinVec && e < per; ++e) {
    const int k = (int)(e / d);
    const int lo = ob[k], hi = ob[k + 1];
    if (!is_long(lo, hi)) continue;
    const float nw = long_sum(lp, b, d, lo, hi, e - (int64_t)k * d) / (float)(hi - lo);
    if constexpr (SHIFT) {
      const float dl = nw - cb[e];
      moved = fmaf(dl, dl, moved);
    }
    cb[e] = nw;
  }
  if constexpr (SHIFT) {
    moved = wave_sum(moved);
    if (lane == 0) wsum[wv] = moved;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
      part[(int64_t)b * part_stride + j] = t;
    }
  }
}

// Accumulating update over chunks of points (the host-streamed Lloyd loop):
// counts_run += counts of one chunk.
__global__ __launch_bounds__(kThreads) void add_counts_kernel(int32_t* __restrict__ run,
                                                              const int32_t* __restrict__ chunk,
                                                              int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    run[i] += chunk[i];
}

// After the last chunk: c = sums / count for non-empty clusters (empty ones
// keep c), one thread per element, blocks_per_batch blocks per problem
// striding over its (K, d) block; with SHIFT each block's squared moves go to
// part[b * blocks_per_batch + j].
template <bool SHIFT>
__global__ __launch_bounds__(kThreads) void finalize_sums_kernel(
    const float* __restrict__ sums, const int32_t* __restrict__ counts, float* __restrict__ c,
    float* __restrict__ part, int64_t per, int d, int blocks_per_batch) {
  __shared__ float wsum[kThreads / 64];
  const int b = blockIdx.x / blocks_per_batch, j = blockIdx.x % blocks_per_batch;
  const float* sb = sums + (int64_t)b * per;
  const int32_t* nb = counts + (int64_t)b * (per / d);
  float* cb = c + (int64_t)b * per;
  float moved = 0.f;
  for (int64_t e = (int64_t)j * kThreads + threadIdx.x; e < per;
       e += (int64_t)blocks_per_batch * kThreads) {
    const int n = nb[e / d];
    if (n > 0) {
      const float nw = sb[e] / (float)n;
      if constexpr (SHIFT) {
        const float dl = nw - cb[e];
        moved = fmaf(dl, dl, moved);
      }
      cb[e] = nw;
    }
  }
  if constexpr (SHIFT) {
    moved = wave_sum(moved);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = moved;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
      part[(int64_t)b * blocks_per_batch + j] = t;
    }
  }
}

// shift[b] = sum of the problem's finalize partials, in index order.
__global__ __launch_bounds__(kThreads) void shift_reduce_kernel(const float* __restrict__ part,
                                                                float* __restrict__ shift,
                                                                int parts_per_batch) {
  __shared__ float wsum[kThreads / 64];
  const int b = blockIdx.x;
  const float* p = part + (int64_t)b * parts_per_batch;
  float t = 0.f;
  for (int i = threadIdx.x; i < parts_per_batch; i += kThreads) t += p[i];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += wsum[w];
    shift[b] = s;
  }
}

// ---------------------------------------------------------------------------
template <int IPT>
hipError_t run_hist_scatter(const int32_t* ids, int32_t* counts, int32_t* cursor, int32_t* perm,
                            int64_t B, int64_t N, int64_t K, bool scatter, hipStream_t s) {
  constexpr int CH = kThreads * IPT;
  const int nchunks = (int)((N + CH - 1) / CH);
  const int nranges = (int)((K + kMaxLdsBins - 1) / kMaxLdsBins);
  const int64_t grid = B * nchunks * nranges;
  const int nb = K < kMaxLdsBins ? (int)K : kMaxLdsBins;
  const size_t lds = (size_t)nb * sizeof(int32_t);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // Bins above 64 KB of LDS need the per-kernel limit raised; a refusal shows
  // up as a launch error below.
  if (!scatter) {
    static bool attr = false;
    if (!attr && lds > 65536) {
      (void)hipFuncSetAttribute((const void*)hist_kernel<IPT>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                kMaxLdsBins * sizeof(int32_t));
      (void)hipGetLastError();
      attr = true;
    }
    hist_kernel<IPT><<<(unsigned)grid, kThreads, lds, s>>>(ids, counts, (int)N, (int)K, nchunks,
                                                           nranges);
  } else {
    static bool attr = false;
    if (!attr && lds > 65536) {
      (void)hipFuncSetAttribute((const void*)scatter_kernel<IPT>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                kMaxLdsBins * sizeof(int32_t));
      (void)hipGetLastError();
      attr = true;
    }
    scatter_kernel<IPT><<<(unsigned)grid, kThreads, lds, s>>>(ids, cursor, perm, (int)N, (int)K,
                                                              nchunks, nranges);
  }
  return hipGetLastError();
}

#define FK_CHECK(call)                   \
  do {                                   \
    hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

// Lanes per row slice: enough 16-byte vectors for the row, as a power of two,
// from 4 to 8 (a 128-byte slice, one cache line); wider rows are cut into
// column slices, each its own wave, so a problem with few points still fills
// the machine. 8 lanes beat 16 (more waves in flight, one line per row read).
template <int DT>
int seg_lanes(int64_t d) {
  constexpr int EV = DT == FK_F32 ? 4 : 8;
  const int64_t nvec = (d + EV - 1) / EV;
  int l = 4;
  while (l < 8 && l < nvec) l <<= 1;
  return l;
}

template <int DT>
int seg_slices_dt(int64_t d) {
  constexpr int EV = DT == FK_F32 ? 4 : 8;
  const int64_t span = (int64_t)seg_lanes<DT>(d) * EV;
  return (int)((d + span - 1) / span);
}

template <int DT, int LPR>
hipError_t run_segreduce(const void* x, const UpdateWs& ws, int64_t B, int64_t N, int64_t d,
                         int64_t K, float* sums, float* c, float* part, int part_stride,
                         bool acc_all, hipStream_t s) {
  constexpr int EB = DT == FK_F32 ? 4 : 2;
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int slices = seg_slices_dt<DT>(d);
  const int64_t total = B * runs * slices;
  const int64_t grid = (total + 3) / 4;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // vector path: 16-byte x rows and 16-byte-aligned rows of c
  const float* cc = acc_all ? sums : c;
  const bool vec = (d * EB) % 16 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)cc % 16) == 0;
  if (vec)
    segreduce_kernel<DT, LPR, true><<<(unsigned)grid, kThreads, 0, s>>>(
        x, ws.perm, ws.offsets, ws.run_first, sums, c, part, part_stride, ws.pieces, (int)N,
        (int)d, (int)K, runs, slices, total, acc_all);
  else
    segreduce_kernel<DT, LPR, false><<<(unsigned)grid, kThreads, 0, s>>>(
        x, ws.perm, ws.offsets, ws.run_first, sums, c, part, part_stride, ws.pieces, (int)N,
        (int)d, (int)K, runs, slices, total, acc_all);
  return hipGetLastError();
}

// part: per-wave squared moves of short clusters (null: no shift), wave w of
// problem b at part[b * part_stride + w].
// acc_all: every segment is added with atomics into sums (an accumulating
// pass over one chunk of points); c and part are not touched.
template <int DT>
hipError_t segreduce_dt(const void* x, const UpdateWs& ws, int64_t B, int64_t N, int64_t d,
                        int64_t K, float* sums, float* c, float* part, int part_stride,
                        bool acc_all, hipStream_t s) {
  switch (seg_lanes<DT>(d)) {
    case 4: return run_segreduce<DT, 4>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
    case 8: return run_segreduce<DT, 8>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
    default:
      return run_segreduce<DT, 16>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
  }
}

hipError_t segreduce_any(const void* x, int dt, const UpdateWs& ws, int64_t B, int64_t N,
                         int64_t d, int64_t K, float* sums, float* c, float* part,
                         int part_stride, bool acc_all, hipStream_t s) {
  if (dt == FK_F16)
    return segreduce_dt<FK_F16>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
  if (dt == FK_BF16)
    return segreduce_dt<FK_BF16>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
  return segreduce_dt<FK_F32>(x, ws, B, N, d, K, sums, c, part, part_stride, acc_all, s);
}

// column slices of a segreduce row (fp32 rows have the most)
int seg_slices(int dt, int64_t d) {
  if (dt == FK_F16) return seg_slices_dt<FK_F16>(d);
  if (dt == FK_BF16) return seg_slices_dt<FK_BF16>(d);
  return seg_slices_dt<FK_F32>(d);
}

// segreduce waves per problem (one per run and column slice)
int64_t seg_waves(int dt, int64_t N, int64_t d) {
  return (N + kSegRun - 1) / kSegRun * seg_slices(dt, d);
}

}  // namespace

// Chunks per problem for the split sort: about 512 blocks in all, at least
// 4096 ids per chunk, at most 256 chunks and 2^24 count-matrix entries;
// 0 when K needs more than one LDS range of bins.
int split_groups(int64_t B, int64_t N, int64_t K) {
  if (K > kMaxLdsBins || B <= 0 || N <= 0) return 0;
  int64_t g = (512 + B - 1) / B;
  const int64_t by_n = (N + 4095) / 4096;
  g = g < by_n ? g : by_n;
  g = g < 256 ? g : 256;
  const int64_t by_mem = ((int64_t)1 << 24) / (B * K);
  g = g < by_mem ? g : by_mem;
  return (int)(g < 1 ? 1 : g);
}

// finalize blocks per problem: one thread per kFinVec centroid elements
int64_t fin_blocks(int64_t K, int64_t d) {
  return (K * d + (int64_t)kThreads * kFinVec - 1) / ((int64_t)kThreads * kFinVec);
}

// How perm is built: in LDS per chunk of the split sort (chunks of at most
// kStableChunk ids), by radix passes over the whole problem (K <= 2^16), or
// by the atomic-cursor scatter (larger K).
enum PermPath { kPermDirect, kPermStable, kPermRadix, kPermAtomic };

// FK_FORCE_RADIX=1 (a test hook) takes the radix passes whenever K allows.
bool force_radix() {
  const char* v = getenv("FK_FORCE_RADIX");
  return v && v[0] == '1';
}

PermPath perm_path(int64_t B, int64_t N, int64_t K) {
  const int G = split_groups(B, N, K);
  if (G > 0 && (N + G - 1) / G <= kStableChunk && !(force_radix() && K <= 65536))
    return key_bits(K) <= kDirectKeyBits && direct_lds_bytes((N + G - 1) / G, K) <= kStableLdsMax
               ? kPermDirect
               : kPermStable;
  if (K <= 65536) return kPermRadix;
  return kPermAtomic;
}

int radix_passes(int64_t K) { return (key_bits(K) + 7) / 8; }

// The split sort's count matrix needs the grid kernels (colscan, offsets_runs).
bool big_count_matrix(int G, int64_t K) { return G > 0 && (int64_t)G * K > kFusedOffsetsMax; }

// Radix passes after a split sort with a large count matrix whose chunks are
// at most one hist2 step or a whole number of steps: hist2 counts the first
// pass's digits per step, and the radix chunks are those steps (the whole
// split chunk when it is shorter). Otherwise chunks of kRadixChunk.
static_assert(kRadixChunk == kSortThreads * kSortUnroll, "a radix chunk is one hist2 step");
bool radix_after_split(int64_t B, int64_t N, int64_t K) {
  const int64_t G = split_groups(B, N, K);
  if (perm_path(B, N, K) != kPermRadix || !big_count_matrix((int)G, K)) return false;
  const int64_t chunk = (N + G - 1) / G;
  return chunk <= kRadixChunk || chunk % kRadixChunk == 0;
}
int64_t radix_chunk_len(int64_t B, int64_t N, int64_t K) {
  if (!radix_after_split(B, N, K)) return kRadixChunk;
  const int64_t G = split_groups(B, N, K);
  const int64_t chunk = (N + G - 1) / G;
  return chunk < kRadixChunk ? chunk : kRadixChunk;
}

// Radix chunks per problem and their groups. After the split sort they are
// exactly hist2's digit rows, G chunks of `steps` each (trailing ones may be
// empty).
int64_t radix_chunks(int64_t B, int64_t N, int64_t K) {
  if (radix_after_split(B, N, K)) {
    const int64_t G = split_groups(B, N, K);
    const int64_t chunk = (N + G - 1) / G;
    return G * ((chunk + kRadixChunk - 1) / kRadixChunk);
  }
  return N > 0 ? (N + kRadixChunk - 1) / kRadixChunk : 1;
}
int64_t radix_rgroups(int64_t B, int64_t N, int64_t K) {
  return (radix_chunks(B, N, K) + kRadixRows - 1) / kRadixRows;
}

struct WsLayout {
  int64_t runs, nq1, nq2, slices, G, GR, RG;
  bool radix, two_sets, cursor, ktot;
};

WsLayout ws_layout(int64_t B, int64_t N, int64_t d, int64_t K) {
  WsLayout L;
  L.runs = (N + kSegRun - 1) / kSegRun;
  L.nq1 = (L.runs + kQ1 - 1) / kQ1;
  L.nq2 = (L.nq1 + kQ2 - 1) / kQ2;
  L.slices = seg_slices(FK_F32, d);              // the most of any element type
  L.G = split_groups(B, N, K);
  const PermPath pp = perm_path(B, N, K);
  L.radix = pp == kPermRadix;
  L.two_sets = L.radix && radix_passes(K) > 2;
  L.cursor = pp == kPermAtomic;
  L.ktot = big_count_matrix((int)L.G, K);          // colscan + offsets_runs
  L.GR = L.radix ? radix_chunks(B, N, K) : 0;
  L.RG = L.radix ? radix_rgroups(B, N, K) : 0;
  return L;
}

size_t update_ws_bytes(int64_t B, int64_t N, int64_t d, int64_t K) {
  const WsLayout L = ws_layout(B, N, d, K);
  size_t n = align256((size_t)B * L.runs * 2 * d * 4) + align256((size_t)B * L.nq1 * d * 4) +
             align256((size_t)B * L.nq2 * d * 4) +
             align256((size_t)B * (K + 1) * 4) + align256((size_t)B * N * 4) +
             align256((size_t)B * L.runs * 4) +
             align256((size_t)B * (seg_waves(FK_F32, N, d) + fin_blocks(K, d)) * 4) +
             align256((size_t)B * L.G * K * 4) + align256((size_t)B * 4);
  if (L.radix)
    n += (L.two_sets ? 4 : 2) * align256((size_t)B * N * 4) +
         align256((size_t)B * L.GR * kRadix * 4) +
         align256((size_t)radix_passes(K) * B * L.RG * kRadix * 4) +
         align256((size_t)B * L.RG * kRadix * 4);
  if (L.cursor) n += align256((size_t)B * K * 4);
  if (L.ktot) n += align256((size_t)B * ((K + kThreads - 1) / kThreads) * 4);
  return n;
}

UpdateWs carve_update_ws(void* base, int64_t B, int64_t N, int64_t d, int64_t K) {
  const WsLayout L = ws_layout(B, N, d, K);
  char* p = static_cast<char*>(base);
  UpdateWs w;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += align256(bytes);
    return q;
  };
  w.pieces = reinterpret_cast<float*>(take((size_t)B * L.runs * 2 * d * 4));
  w.q1 = reinterpret_cast<float*>(take((size_t)B * L.nq1 * d * 4));
  w.q2 = reinterpret_cast<float*>(take((size_t)B * L.nq2 * d * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((size_t)B * (K + 1) * 4));
  w.perm = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
  w.run_first = reinterpret_cast<int32_t*>(take((size_t)B * L.runs * 4));
  w.part = reinterpret_cast<float*>(take((size_t)B * (seg_waves(FK_F32, N, d) + fin_blocks(K, d)) * 4));
  w.hist = reinterpret_cast<int32_t*>(take((size_t)B * L.G * K * 4));
  w.has_long = reinterpret_cast<int32_t*>(take((size_t)B * 4));
  w.rkeys[0] = w.rkeys[1] = nullptr;
  w.ridx[0] = w.ridx[1] = nullptr;
  w.rhist = w.rcolsum = w.rgbase = nullptr;
  w.cursor = nullptr;
  if (L.radix) {
    w.rkeys[0] = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
    w.ridx[0] = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
    if (L.two_sets) {
      w.rkeys[1] = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
      w.ridx[1] = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
    }
    w.rhist = reinterpret_cast<int32_t*>(take((size_t)B * L.GR * kRadix * 4));
    w.rcolsum = reinterpret_cast<int32_t*>(take((size_t)radix_passes(K) * B * L.RG * kRadix * 4));
    w.rgbase = reinterpret_cast<int32_t*>(take((size_t)B * L.RG * kRadix * 4));
  }
  if (L.cursor) w.cursor = reinterpret_cast<int32_t*>(take((size_t)B * K * 4));
  w.ktot = L.ktot ? reinterpret_cast<int32_t*>(take((size_t)B * ((K + kThreads - 1) / kThreads) * 4))
                  : nullptr;
  w.runs = (int)L.runs;
  w.nq1 = (int)L.nq1;
  w.nq2 = (int)L.nq2;
  return w;
}

LongPieces long_pieces(const UpdateWs& ws) {
  LongPieces lp;
  lp.pieces = ws.pieces;
  lp.q1 = ws.q1;
  lp.q2 = ws.q2;
  lp.runs = ws.runs;
  lp.nq1 = ws.nq1;
  lp.nq2 = ws.nq2;
  lp.blocks = ws.runs > kPieceDirectRuns;
  return lp;
}

// perm by LSD radix passes (8 key bits each) over whole problems. After a
// split sort with a large count matrix (radix_after_split) the first pass's
// digit counts and group starts are already there (hist2, colscan,
// offsets_runs) and the later passes' group sums already cleared.
hipError_t run_radix(const int32_t* ids, int64_t B, int64_t N, int64_t K, const UpdateWs& ws,
                     hipStream_t s) {
  const int64_t G = radix_chunks(B, N, K), RG = radix_rgroups(B, N, K);
  const int64_t rc = radix_chunk_len(B, N, K);
  const bool first_done = radix_after_split(B, N, K);
  const int passes = radix_passes(K);
  if (B * G > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (!first_done) {
    const int64_t ncs = passes * B * RG * kRadix;
    int64_t zg = (ncs + kThreads - 1) / kThreads;
    zg = zg < 1 ? 1 : (zg > 4096 ? 4096 : zg);
    zero_kernel<<<(unsigned)zg, kThreads, 0, s>>>(ws.rcolsum, ncs);
    FK_CHECK(hipGetLastError());
  }
  // two passes, point indices in 24 bits: one packed word per point between them
  const bool pack = passes == 2 && N <= ((int64_t)1 << 24);
  const int32_t* kin = nullptr;
  const int32_t* xin = nullptr;
  for (int q = 0; q < passes; ++q) {
    const bool last = q == passes - 1;
    const bool pout = pack && q == 0, pin = pack && q == 1;
    int32_t* kout = last ? nullptr : ws.rkeys[q & 1];
    int32_t* xout = last ? ws.perm : (pout ? nullptr : ws.ridx[q & 1]);
    int32_t* cs = ws.rcolsum + (int64_t)q * B * RG * kRadix;
    const int shift = pin ? 24 : 8 * q;
    if (q > 0 || !first_done) {
      radix_hist_kernel<<<(unsigned)(B * G), kSortThreads, 0, s>>>(
          kin ? kin : ids, ws.rhist, cs, (int)N, (int)K, (int)G, (int)RG, shift, pin, (int)rc);
      FK_CHECK(hipGetLastError());
      radix_scan_kernel<<<(unsigned)B, kThreads, 0, s>>>(cs, ws.rgbase, (int)RG);
      FK_CHECK(hipGetLastError());
    }
    if (pout)
      radix_scatter_packed_kernel<true><<<(unsigned)(B * G), kSortThreads, 0, s>>>(
          ids, ws.rhist, ws.rgbase, kout, (int)N, (int)K, (int)G, (int)RG, (int)rc);
    else if (pin)
      radix_scatter_packed_kernel<false><<<(unsigned)(B * G), kSortThreads, 0, s>>>(
          kin, ws.rhist, ws.rgbase, xout, (int)N, (int)K, (int)G, (int)RG, (int)rc);
    else
      radix_scatter_kernel<<<(unsigned)(B * G), kSortThreads, 0, s>>>(
          ids, kin, xin, ws.rhist, ws.rgbase, kout, xout, (int)N, (int)K, (int)G, (int)RG, shift,
          (int)rc);
    FK_CHECK(hipGetLastError());
    kin = kout;
    xin = xout;
  }
  return hipSuccess;
}

// Counting sort of a batch's ids into per-cluster segments: counts, offsets,
// run starts, the long-cluster flag, perm.
hipError_t run_sort(const int32_t* ids, int dt, int64_t B, int64_t N, int64_t d, int64_t K,
                    int32_t* counts, const UpdateWs& ws, hipStream_t s) {
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int G = split_groups(B, N, K);
  const PermPath pp = perm_path(B, N, K);
  if (G > 0) {
    const int chunk = (int)((N + G - 1) / G);
    const size_t lds = (size_t)K * sizeof(int32_t);            // bins
    const size_t lds1 = (size_t)(K + 1) * sizeof(int32_t);     // offsets + total
    static bool attr = false;
    if (!attr && lds1 > 65536) {
      for (const void* f : {(const void*)hist2_kernel, (const void*)offsets_kernel})
        (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (kMaxLdsBins + 64) * sizeof(int32_t));
      (void)hipGetLastError();
      attr = true;
    }
    // radix passes after a large count matrix: hist2 also counts the first
    // pass's digits (chunks shared) and clears the later passes' group sums
    const bool fuse = radix_after_split(B, N, K);
    const int64_t GR = fuse ? radix_chunks(B, N, K) : 0;
    const int64_t RG = fuse ? radix_rgroups(B, N, K) : 0;
    int32_t* rdig = fuse ? ws.rhist : nullptr;
    int32_t* zero = fuse ? ws.rcolsum + B * RG * kRadix : nullptr;
    const int64_t nzero = fuse ? (radix_passes(K) - 1) * B * RG * kRadix : 0;
    hist2_kernel<<<(unsigned)(B * G), kSortThreads, lds, s>>>(ids, ws.hist, (int)N, (int)K, G,
                                                             chunk, rdig, zero, nzero);
    FK_CHECK(hipGetLastError());
    if ((int64_t)G * K <= kFusedOffsetsMax) {
      offsets_kernel<<<(unsigned)B, kSortThreads, lds1, s>>>(ws.hist, counts, ws.offsets,
                                                            ws.run_first, ws.has_long, (int)K,
                                                            G, runs);
      FK_CHECK(hipGetLastError());
    } else {
      const int kblocks = (int)((K + kThreads - 1) / kThreads);
      if (B * (kblocks + RG) > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
      colscan_kernel<<<(unsigned)(B * (kblocks + RG)), kThreads, 0, s>>>(
          ws.hist, counts, ws.ktot, (int)K, G, kblocks, (int)B, rdig, ws.rcolsum, (int)GR,
          (int)RG, pp != kPermRadix);
      FK_CHECK(hipGetLastError());
      offsets_runs_kernel<<<(unsigned)(B * kblocks + (fuse ? B : 0)), kThreads, 0, s>>>(
          counts, ws.ktot, ws.offsets, ws.run_first, ws.has_long, (int)K, runs, kblocks, (int)B,
          ws.rcolsum, ws.rgbase, (int)RG);
      FK_CHECK(hipGetLastError());
    }
    if (pp == kPermDirect) {
      const size_t dlds = direct_lds_bytes(chunk, K);
      static bool dattr = false;
      if (!dattr) {
        (void)hipFuncSetAttribute((const void*)scatter_direct_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kStableLdsMax);
        (void)hipGetLastError();
        dattr = true;
      }
      scatter_direct_kernel<<<(unsigned)(B * G), kSortThreads, dlds, s>>>(
          ids, ws.hist, ws.offsets, ws.perm, (int)N, (int)K, G, chunk);
      FK_CHECK(hipGetLastError());
      return hipSuccess;
    }
    if (pp == kPermStable) {
      const int kb = key_bits(K);
      const int passes = (kb + 7) / 8;
      const int db = (kb + passes - 1) / passes;
      const size_t slds = (size_t)2 * chunk * 4 + ((size_t)1 << db) * kWavesSort * 4;
      static bool sattr = false;
      if (!sattr) {
        (void)hipFuncSetAttribute((const void*)scatter_stable_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kStableLdsMax);
        (void)hipGetLastError();
        sattr = true;
      }
      scatter_stable_kernel<<<(unsigned)(B * G), kSortThreads, slds, s>>>(
          ids, ws.hist, ws.offsets, ws.perm, (int)N, (int)K, G, chunk, kb);
      FK_CHECK(hipGetLastError());
      return hipSuccess;
    }
    return run_radix(ids, B, N, K, ws, s);
  }
  int64_t g = (B * K + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
  zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts, B * K);
  FK_CHECK(hipGetLastError());
  FK_CHECK(run_hist_scatter<64>(ids, counts, nullptr, nullptr, B, N, K, false, s));
  scan_kernel<<<(unsigned)B, kSortThreads, 0, s>>>(counts, ws.offsets, ws.cursor, (int)K);
  FK_CHECK(hipGetLastError());
  const int pb = (int)((K + 255) / 256 < 256 ? (K + 255) / 256 : 256);   // blocks per problem
  prep_kernel<<<(unsigned)(B * pb), kThreads, 0, s>>>(ws.offsets, ws.run_first, ws.has_long,
                                                       (int)K, runs, pb);
  FK_CHECK(hipGetLastError());
  if (pp == kPermRadix) return run_radix(ids, B, N, K, ws, s);
  return run_hist_scatter<64>(ids, nullptr, ws.cursor, ws.perm, B, N, K, true, s);
}

hipError_t launch_update(const void* x, const int32_t* ids, int dt, int64_t B, int64_t N,
                         int64_t d, int64_t K, float* c, int32_t* counts, float* shift,
                         const UpdateWs& ws, hipStream_t s, bool defer) {
  if (B == 0) return hipSuccess;
  if (N == 0) {
    // no point: every cluster is empty and keeps its centroid
    int64_t g = (B * K + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts, B * K);
    FK_CHECK(hipGetLastError());
    if (shift) fill_f32_kernel<<<1, kThreads, 0, s>>>(shift, 0.f, B);
    return hipGetLastError();
  }
  const int64_t fb = fin_blocks(K, d);
  FK_CHECK(run_sort(ids, dt, B, N, d, K, counts, ws, s));
  // shift partials of a problem: its segreduce waves, then its finalize blocks
  const int64_t sw = seg_waves(dt, N, d);
  const int64_t pstride = sw + fb;
  if (pstride > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  float* spart = shift ? ws.part : nullptr;
  FK_CHECK(segreduce_any(x, dt, ws, B, N, d, K, nullptr, c, spart, (int)pstride, false, s));
  const int64_t grid = B * fb;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (B * ws.nq1 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const bool blocks = ws.runs > kPieceDirectRuns;   // else long sums add their pieces directly
  if (blocks && ws.runs >= kQ1) {                // some full Q1 block
    q1blocks_kernel<<<(unsigned)(B * ws.nq1), kThreads, 0, s>>>(long_pieces(ws), ws.q1,
                                                                ws.has_long, (int)d);
    FK_CHECK(hipGetLastError());
  }
  if (blocks && ws.runs >= kQ1 * kQ2) {          // some full Q2 block
    q2blocks_kernel<<<(unsigned)(B * ws.nq2), kThreads, 0, s>>>(long_pieces(ws), ws.q1, ws.q2,
                                                                ws.has_long, (int)d);
    FK_CHECK(hipGetLastError());
  }
  if (!shift) {                                  // the caller does not need the shift
    if (defer) return hipSuccess;                // the next norms pass finishes long clusters
    finalize_kernel<false><<<(unsigned)grid, kThreads, 0, s>>>(
        long_pieces(ws), ws.offsets, c, ws.part, 0, ws.has_long, (int)d, (int)K, (int)fb);
    return hipGetLastError();
  }
  finalize_kernel<true><<<(unsigned)grid, kThreads, 0, s>>>(
      long_pieces(ws), ws.offsets, c, ws.part + sw, (int)pstride, ws.has_long, (int)d, (int)K,
      (int)fb);
  FK_CHECK(hipGetLastError());
  shift_reduce_kernel<<<(unsigned)B, kThreads, 0, s>>>(ws.part, shift, (int)pstride);
  return hipGetLastError();
}

PendingFinish pending_finish(const UpdateWs& ws, int64_t K) {
  PendingFinish pf;
  pf.lp = long_pieces(ws);
  pf.offsets = ws.offsets;
  pf.has_long = ws.has_long;
  pf.K = K;
  return pf;
}

// The long clusters a deferred update left, when no norms pass follows.
hipError_t launch_finish(float* c, const UpdateWs& ws, int64_t B, int64_t d, int64_t K,
                         hipStream_t s) {
  const int64_t fb = fin_blocks(K, d);
  if (B * fb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  finalize_kernel<false><<<(unsigned)(B * fb), kThreads, 0, s>>>(
      long_pieces(ws), ws.offsets, c, ws.part, 0, ws.has_long, (int)d, (int)K, (int)fb);
  return hipGetLastError();
}

// Finalize blocks per problem of finalize_sums_kernel.
int64_t sums_fin_blocks(int64_t K, int64_t d) {
  const int64_t g = (K * d + kThreads - 1) / kThreads;
  return g < 64 ? (g < 1 ? 1 : g) : 64;
}

hipError_t launch_update_accumulate(const void* x, const int32_t* ids, int dt, int64_t B,
                                    int64_t N, int64_t d, int64_t K, float* sums_run,
                                    int32_t* counts_run, int32_t* counts_chunk,
                                    const UpdateWs& ws, hipStream_t s) {
  if (B == 0 || N == 0) return hipSuccess;
  FK_CHECK(run_sort(ids, dt, B, N, d, K, counts_chunk, ws, s));
  FK_CHECK(segreduce_any(x, dt, ws, B, N, d, K, sums_run, nullptr, nullptr, 0, true, s));
  int64_t g = (B * K + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
  add_counts_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts_run, counts_chunk, B * K);
  return hipGetLastError();
}

hipError_t launch_zero_sums(float* sums, int32_t* counts, int64_t B, int64_t K, int64_t d,
                            hipStream_t s) {
  int64_t g = (B * K * d + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
  zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(reinterpret_cast<int32_t*>(sums), B * K * d);
  FK_CHECK(hipGetLastError());
  g = (B * K + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
  zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts, B * K);
  return hipGetLastError();
}

hipError_t launch_finalize_sums(const float* sums, const int32_t* counts, float* c,
                                float* shift, float* part, int64_t B, int64_t K, int64_t d,
                                hipStream_t s) {
  const int64_t fb = sums_fin_blocks(K, d);
  if (B * fb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (!shift) {
    finalize_sums_kernel<false><<<(unsigned)(B * fb), kThreads, 0, s>>>(sums, counts, c, part,
                                                                       K * d, (int)d, (int)fb);
    return hipGetLastError();
  }
  finalize_sums_kernel<true><<<(unsigned)(B * fb), kThreads, 0, s>>>(sums, counts, c, part,
                                                                    K * d, (int)d, (int)fb);
  FK_CHECK(hipGetLastError());
  shift_reduce_kernel<<<(unsigned)B, kThreads, 0, s>>>(part, shift, (int)fb);
  return hipGetLastError();
}

}  // namespace fk
