// Sort-inverse centroid update for gfx950.
//
// The assignment vector is counting-sorted by cluster id into contiguous
// segments through an inverse permutation of point indices; the point matrix
// itself never moves. Each segment is then reduced on chip, and a cluster
// whose segment is longer than one run of sorted positions is summed in
// pieces, with one atomic add per element per piece instead of one scatter
// atomic per point (itinai.com summary, third paragraph; "Flash-KMeans：IO感知
// 的精确K-Means…", section "它攻克的两大瓶颈" and the update-contention panel of
// "交互式讲解"; "Flash-KMeans: Implementação Exata…", section "Sort-Inverse
// Update"; "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", Abstract).
//
// Terms. Sorted positions of a problem are cut into runs of kSegRun; the
// segment [lo, hi) of cluster k is short when it holds at most kSegRun
// positions, long otherwise.
//
// Steps:
//   sort      counts, offsets (exclusive prefix sum of counts), perm
//             (perm[offsets[id] + rank] = n) and, per run, the cluster that
//             holds its first position; long clusters get zeroed sums rows.
//             Split sort (K <= 32768): per-chunk LDS histograms into a count
//             matrix, column prefixes and offsets, then LDS-ranked scatter;
//             no global atomics. Larger K: per-range LDS histograms with one
//             global atomic per non-empty bin, scan, prep, scatter.
//   segreduce one wave per (run, column slice). A short segment is summed
//             whole by the wave whose run holds its first position (it may
//             read up to kSegRun - 1 positions past its run) and its mean
//             (sum / count) is written straight into c, the squared move into
//             the wave's shift partial. A long segment is summed piecewise,
//             one piece per run it touches, into its zeroed sums row with one
//             fp32 atomic per element: at most (number of long clusters +
//             number of runs) * d atomics per problem, none at all when every
//             cluster is short.
//   finalize  elementwise over (cluster, column) of long clusters:
//             c = sums / count, squared moves into the block's partial; with
//             a shift buffer, shift_reduce sums a problem's partials (its
//             segreduce waves', then its finalize blocks') in a fixed order
//             into shift[b].
// Empty clusters are never touched, so they keep their centroid. Ids outside
// [0, K) are skipped: they count nowhere and add to no cluster.
#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsBins = 32768;            // 128 KB of LDS bins per block
constexpr int kSortThreads = 1024;
constexpr int kSortUnroll = 16;               // ids in flight per thread in the sort kernels
constexpr int64_t kFusedOffsetsMax = 1 << 16; // G*K up to this: one offsets block per problem
constexpr size_t kSortedScatterLds = 96 * 1024;  // LDS budget of the sorted scatter
constexpr int kLongList = 1024;               // long clusters listed per problem by offsets

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }


// Runs whose first position lies in [lo, hi) start inside cluster k.
__device__ __forceinline__ void mark_runs(int32_t* rf, int k, int lo, int hi) {
  for (int64_t r = (lo + (int64_t)kSegRun - 1) / kSegRun; r * kSegRun < hi; ++r) rf[r] = k;
}

// A long cluster's sums row, zeroed by one thread before its pieces are added
// (rows start 16-byte aligned when d % 4 == 0: the buffer is 256-byte aligned).
__device__ __forceinline__ void zero_row(float* row, int d) {
  if (d % 4 == 0) {
    for (int j = 0; j < d; j += 4) *reinterpret_cast<float4*>(row + j) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int j = 0; j < d; ++j) row[j] = 0.f;
  }
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

// Exclusive prefix sum over the kSortThreads threads of a block; `total`
// receives the block sum. wtot: kSortThreads / 64 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int32_t* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
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

// ---------------------------------------------------------------------------
// Split sort (K <= kMaxLdsBins): each problem's ids are cut into G chunks, one
// block each.
//   hist2    block (b, g): LDS histogram of its chunk, stored as row g of the
//            problem's (G, K) count matrix H (no global atomics);
//   offsets  per problem: H's columns become exclusive prefix sums over g,
//            their totals are the counts, whose exclusive prefix sum gives
//            the segment offsets; also the run starts and zeroed sums rows of
//            long clusters (one block per problem when G*K is small;
//            colscan + scan + prep otherwise);
//   scatter2 block (b, g): LDS cursors offsets[k] + H[g][k], LDS ranks,
//            perm[cursor] = n.
__global__ __launch_bounds__(kSortThreads) void hist2_kernel(const int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ H, int N, int K,
                                                             int G, int chunk) {
  extern __shared__ int32_t bins[];
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  for (int i = t; i < K; i += kSortThreads) bins[i] = 0;
  __syncthreads();
  const int32_t* ib = ids + (int64_t)b * N;
  const int n0 = g * chunk, n1 = min(n0 + chunk, N);
  for (int m = n0; m < n1; m += kSortThreads * kSortUnroll) {
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int n = m + q * kSortThreads + t;
      kk[q] = n < n1 ? ib[n] : -1;
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q)
      if ((unsigned)kk[q] < (unsigned)K) atomicAdd(&bins[kk[q]], 1);
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

// offsets: G > 0: column prefixes of H and counts first, then offsets, run
// starts and zeroed long rows; G == 0: counts given, offsets only.
__global__ __launch_bounds__(kSortThreads) void offsets_kernel(
    int32_t* __restrict__ H, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ run_first, float* __restrict__ sums, int32_t* __restrict__ has_long,
    int K, int d, int G, int runs) {
  extern __shared__ int32_t cnt[];              // K + 1
  __shared__ int32_t wtot[kSortThreads / 64];
  __shared__ int32_t longs[kLongList];           // long clusters, zeroed by the whole block
  __shared__ int32_t nlong;
  const int b = blockIdx.x, t = threadIdx.x;
  if (t == 0) nlong = 0;
  int32_t* hb = H + (int64_t)b * G * K;
  int32_t* cb = counts + (int64_t)b * K;
  if (G > 0) {
    for (int k = t; k < K; k += kSortThreads) cnt[k] = column_prefix(hb, K, G, k);
  } else {
    for (int k0 = t; k0 < K; k0 += kSortThreads * 8) {   // 8 loads in flight per thread
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = k0 + q * kSortThreads < K ? cb[k0 + q * kSortThreads] : 0;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (k0 + q * kSortThreads < K) cnt[k0 + q * kSortThreads] = v[q];
    }
  }
  __syncthreads();
  const int per = (K + kSortThreads - 1) / kSortThreads;
  const int lo = min(t * per, K), hi = min(lo + per, K);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += cnt[i];
  int total;
  int run = block_exclusive_scan(s, wtot, total);
  int32_t* ob = offsets + (int64_t)b * (K + 1);
  int32_t* rf = run_first + (int64_t)b * runs;
  float* sb = sums ? sums + (int64_t)b * K * d : nullptr;   // null: no rows to zero
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    if (G > 0) cb[i] = c;
    cnt[i] = run;
    if (G > 0 && c > 0) mark_runs(rf, i, run, run + c);
    if (G > 0 && sb && is_long(run, run + c)) {
      const int q = atomicAdd(&nlong, 1);
      if (q < kLongList) longs[q] = i;
      else zero_row(sb + (int64_t)i * d, d);     // past the list: this thread alone
    }
    run += c;
  }
  if (t == 0) cnt[K] = total;
  __syncthreads();
  for (int k = t; k <= K; k += kSortThreads) ob[k] = cnt[k];   // coalesced
  if (G == 0) return;                            // run starts, rows, flag: prep_kernel
  if (t == 0) has_long[b] = nlong;
  for (int64_t r = (total + (int64_t)kSegRun - 1) / kSegRun + t; r < runs; r += kSortThreads)
    rf[r] = K;                                   // runs past the last valid position
  // the listed long clusters' sums rows, spread over the block
  if (!sb) return;
  const int nl = min(nlong, kLongList);
  if (d % 4 == 0) {
    const int nv = d / 4;
    for (int64_t e = t; e < (int64_t)nl * nv; e += kSortThreads) {
      const int k = longs[e / nv];
      *reinterpret_cast<float4*>(sb + (int64_t)k * d + (e % nv) * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    for (int64_t e = t; e < (int64_t)nl * d; e += kSortThreads) sb[(int64_t)longs[e / d] * d + e % d] = 0.f;
  }
}

// Large G*K: column prefixes on a grid, one thread per (problem, cluster).
__global__ __launch_bounds__(kThreads) void colscan_kernel(int32_t* __restrict__ H,
                                                           int32_t* __restrict__ counts, int K,
                                                           int G, int kblocks) {
  const int b = blockIdx.x / kblocks;
  const int k = (blockIdx.x % kblocks) * kThreads + threadIdx.x;
  if (k >= K) return;
  counts[(int64_t)b * K + k] = column_prefix(H + (int64_t)b * G * K, K, G, k);
}

__global__ __launch_bounds__(kSortThreads) void scatter2_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ H,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int N, int K, int G,
    int chunk) {
  extern __shared__ int32_t bins[];
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int32_t* hr = H + ((int64_t)b * G + g) * K;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  for (int i = t; i < K; i += kSortThreads) bins[i] = ob[i] + hr[i];
  __syncthreads();
  const int32_t* ib = ids + (int64_t)b * N;
  int32_t* pb = perm + (int64_t)b * N;
  const int n0 = g * chunk, n1 = min(n0 + chunk, N);
  for (int m = n0; m < n1; m += kSortThreads * kSortUnroll) {
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int n = m + q * kSortThreads + t;
      kk[q] = n < n1 ? ib[n] : -1;
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q)
      if ((unsigned)kk[q] < (unsigned)K) pb[atomicAdd(&bins[kk[q]], 1)] = m + q * kSortThreads + t;
  }
}

// scatter2, sorted form (when 2K + 2*chunk ints fit LDS): the chunk is
// counting-sorted in LDS first, so the perm stores of one cluster's piece go
// out as consecutive addresses instead of one scattered 4-byte store per
// point.
//   cur[k]  local cursor, from the chunk's exclusive prefix of cluster sizes
//   gof[k]  global position of the chunk's piece of cluster k minus its local
//           start: perm[gof[k] + p] = sidx[p] for local sorted position p
__global__ __launch_bounds__(kSortThreads) void scatter2s_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ H,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int N, int K, int G,
    int chunk) {
  extern __shared__ int32_t sm[];
  int32_t* cur = sm;
  int32_t* gof = sm + K;
  int32_t* skey = sm + 2 * K;
  int32_t* sidx = skey + chunk;
  __shared__ int32_t wtot[kSortThreads / 64];
  const int b = blockIdx.x / G, g = blockIdx.x % G, t = threadIdx.x;
  const int32_t* hr = H + ((int64_t)b * G + g) * K;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  const int32_t* ib = ids + (int64_t)b * N;
  const int n0 = g * chunk, n1 = min(n0 + chunk, N);
  for (int i = t; i < K; i += kSortThreads) cur[i] = 0;
  __syncthreads();
  for (int m = n0; m < n1; m += kSortThreads * kSortUnroll) {
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int n = m + q * kSortThreads + t;
      kk[q] = n < n1 ? ib[n] : -1;
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q)
      if ((unsigned)kk[q] < (unsigned)K) atomicAdd(&cur[kk[q]], 1);
  }
  __syncthreads();
  const int per = (K + kSortThreads - 1) / kSortThreads;
  const int lo = min(t * per, K), hi = min(lo + per, K);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += cur[i];
  int total;
  int run = block_exclusive_scan(sum, wtot, total);
  for (int i = lo; i < hi; ++i) {
    const int c = cur[i];
    cur[i] = run;
    gof[i] = ob[i] + hr[i] - run;
    run += c;
  }
  __syncthreads();
  for (int m = n0; m < n1; m += kSortThreads * kSortUnroll) {
    int kk[kSortUnroll];
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      const int n = m + q * kSortThreads + t;
      kk[q] = n < n1 ? ib[n] : -1;
    }
#pragma unroll
    for (int q = 0; q < kSortUnroll; ++q) {
      if ((unsigned)kk[q] < (unsigned)K) {
        const int p = atomicAdd(&cur[kk[q]], 1);
        skey[p] = kk[q];
        sidx[p] = m + q * kSortThreads + t;
      }
    }
  }
  __syncthreads();
  int32_t* pb = perm + (int64_t)b * N;
  for (int p = t; p < total; p += kSortThreads) pb[gof[skey[p]] + p] = sidx[p];
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
// cursor = offsets.
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
  int32_t* kb = cursor + (int64_t)b * K;
  for (int64_t i = lo; i < hi; ++i) {
    ob[i] = run;
    kb[i] = run;
    run += cb[i];
  }
  if (t == 0) ob[K] = total;
}

// prep: one wave per cluster marks the runs that start inside it and zeroes
// the sums row of a long cluster; runs past the last position get K.
__global__ __launch_bounds__(kThreads) void prep_kernel(const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ run_first,
                                                        float* __restrict__ sums,
                                                        int32_t* __restrict__ has_long, int K,
                                                        int d, int runs, int blocks_per_batch) {
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
    if (sums && is_long(lo, hi)) {
      float* row = sums + ((int64_t)b * K + k) * d;
      for (int i = lane; i < d; i += 64) row[i] = 0.f;
    }
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
// mean), added with atomics to its sums row for a piece of a long one.
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
    int N, int d, int K, int runs, int slices, int64_t total_waves, bool acc_all) {
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
  const int b = (int)(wid / per_batch);
  const int rem = (int)(wid % per_batch);
  const int run = rem / slices, slice = rem % slices;
  const int p0 = run * kSegRun;
  const int p1 = min(p0 + kSegRun, N);
  const int col = slice * SPAN + li * EV;        // my first column
  const bool colok = col < d;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  const char* xb = reinterpret_cast<const char*>(x) + (int64_t)b * N * d * EB;
  float* sb = sums + (int64_t)b * K * d;
  float* cb = c + (int64_t)b * K * d;
  float moved = 0.f;                             // squared moves of this wave's short clusters
  [&]() {

  int k = run_first[(int64_t)b * runs + run];
  k = k < 0 ? K : k;
  if (k >= K) return;
  const int pend = min(p0 + STAGE, N);
  for (int j = lane; j < pend - p0; j += 64) lperm[wv][j] = perm[(int64_t)b * N + p0 + j];

  // offsets window: win holds ob[kw + lane]
  int kw = k;
  int win = ob[min(kw + lane, K)];
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
  const int s = c0 < 0 ? max(off(__builtin_amdgcn_readlane(sk, 0)), p0)
                       : __builtin_amdgcn_readlane(se, 0) - c0;
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
      } else {                                   // a piece of a long segment, or any
        float* row = sb + (int64_t)jk * d + col;   // segment when accumulating
#pragma unroll
        for (int i = 0; i < EV; ++i)
          if (col + i < d) unsafeAtomicAdd(row + i, acc[i]);
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

// ---------------------------------------------------------------------------
// finalize, one thread per group of kFinVec consecutive elements of a
// problem's (K, d) centroid block: a non-empty cluster takes its new value
// from its sums row (already the mean for a short segment; divided by the
// count for a long one), and the block's squared moves go to its partial.
// Empty clusters keep their centroid.
constexpr int kFinVec = 4;

template <bool SHIFT>
__global__ __launch_bounds__(kThreads) void finalize_kernel(
    const float* __restrict__ sums, const int32_t* __restrict__ offsets, float* __restrict__ c,
    float* __restrict__ part, int part_stride, const int32_t* __restrict__ has_long, int d, int K,
    int blocks_per_batch, bool vec) {
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
  const float* sb = sums + (int64_t)b * per;
  float* cb = c + (int64_t)b * per;
  float moved = 0.f;
  if (e0 < per) {
    if (vec && e0 + kFinVec <= per) {         // vec: d % kFinVec == 0, c 16-byte aligned
      const int k = (int)(e0 / d);               // the kFinVec elements share a row
      const int lo = ob[k], hi = ob[k + 1];
      if (is_long(lo, hi)) {
        const float4 sv = *reinterpret_cast<const float4*>(sb + e0);
        const float cnt = (float)(hi - lo);
        float nw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) nw[i] = nw[i] / cnt;
        if constexpr (SHIFT) {
          const float4 cv = *reinterpret_cast<const float4*>(cb + e0);
          const float od[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float dl = nw[i] - od[i];
            moved = fmaf(dl, dl, moved);
          }
        }
        *reinterpret_cast<float4*>(cb + e0) = make_float4(nw[0], nw[1], nw[2], nw[3]);
      }
    } else {
      for (int64_t e = e0; e < e0 + kFinVec && e < per; ++e) {
        const int k = (int)(e / d);
        const int lo = ob[k], hi = ob[k + 1];
        if (!is_long(lo, hi)) continue;
        const float nw = sb[e] / (float)(hi - lo);
        if constexpr (SHIFT) {
          const float dl = nw - cb[e];
          moved = fmaf(dl, dl, moved);
        }
        cb[e] = nw;
      }
    }
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
  const bool vec = (d * EB) % 16 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)c % 16) == 0;
  if (vec)
    segreduce_kernel<DT, LPR, true><<<(unsigned)grid, kThreads, 0, s>>>(
        x, ws.perm, ws.offsets, ws.run_first, sums, c, part, part_stride, (int)N, (int)d,
        (int)K, runs, slices, total, acc_all);
  else
    segreduce_kernel<DT, LPR, false><<<(unsigned)grid, kThreads, 0, s>>>(
        x, ws.perm, ws.offsets, ws.run_first, sums, c, part, part_stride, (int)N, (int)d,
        (int)K, runs, slices, total, acc_all);
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

// segreduce waves per problem (one per run and column slice)
int64_t seg_waves(int dt, int64_t N, int64_t d) {
  const int64_t runs = (N + kSegRun - 1) / kSegRun;
  if (dt == FK_F16) return runs * seg_slices_dt<FK_F16>(d);
  if (dt == FK_BF16) return runs * seg_slices_dt<FK_BF16>(d);
  return runs * seg_slices_dt<FK_F32>(d);
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

size_t update_ws_bytes(int64_t B, int64_t N, int64_t d, int64_t K) {
  const int64_t runs = (N + kSegRun - 1) / kSegRun;
  return align256((size_t)B * K * d * 4) + align256((size_t)B * (K + 1) * 4) +
         align256((size_t)B * K * 4) + align256((size_t)B * N * 4) +
         align256((size_t)B * runs * 4) +
         align256((size_t)B * (seg_waves(FK_F32, N, d) + fin_blocks(K, d)) * 4) +
         align256((size_t)B * split_groups(B, N, K) * K * 4) + align256((size_t)B * 4);
}

UpdateWs carve_update_ws(void* base, int64_t B, int64_t N, int64_t d, int64_t K) {
  const int64_t runs = (N + kSegRun - 1) / kSegRun;
  char* p = static_cast<char*>(base);
  UpdateWs w;
  w.sums = reinterpret_cast<float*>(p);
  p += align256((size_t)B * K * d * 4);
  w.offsets = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * (K + 1) * 4);
  w.cursor = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.perm = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * N * 4);
  w.run_first = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * runs * 4);
  w.part = reinterpret_cast<float*>(p);
  p += align256((size_t)B * (seg_waves(FK_F32, N, d) + fin_blocks(K, d)) * 4);
  w.hist = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * split_groups(B, N, K) * K * 4);
  w.has_long = reinterpret_cast<int32_t*>(p);
  return w;
}

// Counting sort of a batch's ids into per-cluster segments: counts, offsets,
// run starts, perm. zsums: the sums rows of long clusters are zeroed there
// (null: left alone).
hipError_t run_sort(const int32_t* ids, int64_t B, int64_t N, int64_t d, int64_t K,
                    int32_t* counts, float* zsums, const UpdateWs& ws, hipStream_t s) {
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int G = split_groups(B, N, K);
  if (G > 0) {
    const int chunk = (int)((N + G - 1) / G);
    const size_t lds = (size_t)K * sizeof(int32_t);            // bins
    const size_t lds1 = (size_t)(K + 1) * sizeof(int32_t);     // offsets + total
    static bool attr = false;
    if (!attr && lds1 > 65536) {
      for (const void* f : {(const void*)hist2_kernel, (const void*)offsets_kernel,
                            (const void*)scatter2_kernel})
        (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (kMaxLdsBins + 64) * sizeof(int32_t));
      (void)hipGetLastError();
      attr = true;
    }
    hist2_kernel<<<(unsigned)(B * G), kSortThreads, lds, s>>>(ids, ws.hist, (int)N, (int)K, G,
                                                             chunk);
    FK_CHECK(hipGetLastError());
    if ((int64_t)G * K <= kFusedOffsetsMax) {
      offsets_kernel<<<(unsigned)B, kSortThreads, lds1, s>>>(ws.hist, counts, ws.offsets,
                                                            ws.run_first, zsums, ws.has_long,
                                                            (int)K, (int)d, G, runs);
      FK_CHECK(hipGetLastError());
    } else {
      const int kblocks = (int)((K + kThreads - 1) / kThreads);
      colscan_kernel<<<(unsigned)(B * kblocks), kThreads, 0, s>>>(ws.hist, counts, (int)K, G,
                                                                  kblocks);
      FK_CHECK(hipGetLastError());
      offsets_kernel<<<(unsigned)B, kSortThreads, lds1, s>>>(ws.hist, counts, ws.offsets,
                                                             ws.run_first, zsums, ws.has_long,
                                                             (int)K, (int)d, 0, runs);
      FK_CHECK(hipGetLastError());
      const int pb = (int)((K + 255) / 256 < 256 ? (K + 255) / 256 : 256);
      prep_kernel<<<(unsigned)(B * pb), kThreads, 0, s>>>(ws.offsets, ws.run_first, zsums,
                                                           ws.has_long, (int)K, (int)d, runs, pb);
      FK_CHECK(hipGetLastError());
    }
    // the sorted form pays off with enough chunks to fill the chip; with few,
    // its extra passes cost more than the scattered stores
    const size_t lds_sorted = (size_t)(2 * K + 2 * (int64_t)chunk) * sizeof(int32_t);
    if (lds_sorted <= kSortedScatterLds && B * G >= 256) {
      static bool sattr = false;
      if (!sattr && lds_sorted > 65536) {
        (void)hipFuncSetAttribute((const void*)scatter2s_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kSortedScatterLds);
        (void)hipGetLastError();
        sattr = true;
      }
      scatter2s_kernel<<<(unsigned)(B * G), kSortThreads, lds_sorted, s>>>(
          ids, ws.hist, ws.offsets, ws.perm, (int)N, (int)K, G, chunk);
    } else {
      scatter2_kernel<<<(unsigned)(B * G), kSortThreads, lds, s>>>(
          ids, ws.hist, ws.offsets, ws.perm, (int)N, (int)K, G, chunk);
    }
    FK_CHECK(hipGetLastError());
  } else {
    int64_t g = (B * K + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts, B * K);
    FK_CHECK(hipGetLastError());
    FK_CHECK(run_hist_scatter<64>(ids, counts, nullptr, nullptr, B, N, K, false, s));
    scan_kernel<<<(unsigned)B, kSortThreads, 0, s>>>(counts, ws.offsets, ws.cursor, (int)K);
    FK_CHECK(hipGetLastError());
    const int pb = (int)((K + 255) / 256 < 256 ? (K + 255) / 256 : 256);   // blocks per problem
    prep_kernel<<<(unsigned)(B * pb), kThreads, 0, s>>>(ws.offsets, ws.run_first, zsums,
                                                         ws.has_long, (int)K, (int)d, runs, pb);
    FK_CHECK(hipGetLastError());
    FK_CHECK(run_hist_scatter<64>(ids, nullptr, ws.cursor, ws.perm, B, N, K, true, s));
  }
  return hipSuccess;
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
  FK_CHECK(run_sort(ids, B, N, d, K, counts, ws.sums, ws, s));
  // shift partials of a problem: its segreduce waves, then its finalize blocks
  const int64_t sw = seg_waves(dt, N, d);
  const int64_t pstride = sw + fb;
  if (pstride > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  float* spart = shift ? ws.part : nullptr;
  FK_CHECK(segreduce_any(x, dt, ws, B, N, d, K, ws.sums, c, spart, (int)pstride, false, s));
  const int64_t grid = B * fb;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const bool fvec = d % kFinVec == 0 && ((uintptr_t)c % 16) == 0;
  if (!shift) {                                  // the caller does not need the shift
    if (defer) return hipSuccess;                // the next norms pass divides
    finalize_kernel<false><<<(unsigned)grid, kThreads, 0, s>>>(
        ws.sums, ws.offsets, c, ws.part, 0, ws.has_long, (int)d, (int)K, (int)fb, fvec);
    return hipGetLastError();
  }
  finalize_kernel<true><<<(unsigned)grid, kThreads, 0, s>>>(
      ws.sums, ws.offsets, c, ws.part + sw, (int)pstride, ws.has_long, (int)d, (int)K, (int)fb,
      fvec);
  FK_CHECK(hipGetLastError());
  shift_reduce_kernel<<<(unsigned)B, kThreads, 0, s>>>(ws.part, shift, (int)pstride);
  return hipGetLastError();
}

PendingFinish pending_finish(const UpdateWs& ws, int64_t K) {
  PendingFinish pf;
  pf.sums = ws.sums;
  pf.offsets = ws.offsets;
  pf.has_long = ws.has_long;
  pf.K = K;
  return pf;
}

// The division a deferred update left, when no norms pass follows.
hipError_t launch_finish(float* c, const UpdateWs& ws, int64_t B, int64_t d, int64_t K,
                         hipStream_t s) {
  const int64_t fb = fin_blocks(K, d);
  if (B * fb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const bool fvec = d % kFinVec == 0 && ((uintptr_t)c % 16) == 0;
  finalize_kernel<false><<<(unsigned)(B * fb), kThreads, 0, s>>>(
      ws.sums, ws.offsets, c, ws.part, 0, ws.has_long, (int)d, (int)K, (int)fb, fvec);
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
  FK_CHECK(run_sort(ids, B, N, d, K, counts_chunk, nullptr, ws, s));
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
