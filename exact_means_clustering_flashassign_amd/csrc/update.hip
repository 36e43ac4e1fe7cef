// Sort-inverse centroid update for gfx950.
//
// The assignment vector is counting-sorted by cluster id into contiguous
// segments through an inverse permutation of point indices; the point matrix
// itself never moves. Each segment is then reduced on chip and each block
// issues one atomic add per segment piece instead of one scatter atomic per
// point (itinai.com summary, third paragraph; "Flash-KMeans：IO感知的精确
// K-Means…", section "它攻克的两大瓶颈" and the update-contention panel of
// "交互式讲解"; "Flash-KMeans: Implementação Exata…", section "Sort-Inverse
// Update"; "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", Abstract).
//
// Steps (one launch each, all on the caller's stream):
//   zero      sums, counts and shift start at zero;
//   hist      counts[b,k]: per-block LDS histogram, one global atomic per
//             (block, non-empty bin);
//   scan      offsets[b,0..K] = exclusive prefix sum of counts; cursor = copy;
//   scatter   perm[b, offsets[id] + rank] = n: per-block LDS ranks, one
//             cursor atomic per (block, non-empty bin);
//   segreduce sums[b,k,:] = sum of x[b, perm[i], :] over segment k; each wave
//             owns a fixed run of sorted positions (balanced by position, not
//             by segment, so a hot cluster spreads over many waves); a segment
//             lying wholly inside the run is written with plain stores, a
//             piece of a longer segment with one fp32 atomic add per element;
//             at most (K + number of runs) * d atomics per problem;
//   finalize  c = sums / counts where counts > 0, else unchanged;
//             shift[b] += sum (c_new - c_old)^2.
#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsBins = 32768;     // 128 KB of LDS bins per block
constexpr int kSegRun = 256;           // sorted positions per wave in segreduce

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ sums, int64_t nsums,
                                                        int32_t* __restrict__ counts,
                                                        int64_t ncounts, float* __restrict__ shift,
                                                        int64_t B) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float4* s4 = reinterpret_cast<float4*>(sums);
  const int64_t n4 = nsums / 4;
  for (int64_t i = i0; i < n4; i += stride) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = n4 * 4 + i0; i < nsums; i += stride) sums[i] = 0.f;
  for (int64_t i = i0; i < ncounts; i += stride) counts[i] = 0;
  for (int64_t i = i0; i < B; i += stride) shift[i] = 0.f;
}

// ---------------------------------------------------------------------------
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
      if ((unsigned)k < (unsigned)nb) atomicAdd(&bins[k], 1);
    }
  }
  __syncthreads();
  int32_t* cb = counts + (int64_t)b * K + k0;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const int v = bins[i];
    if (v) atomicAdd(&cb[i], v);
  }
}

// ---------------------------------------------------------------------------
// scan: one block per problem; exclusive prefix sum of counts.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ cursor, int K) {
  __shared__ int32_t part[1024];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t per = ((int64_t)K + 1023) / 1024;
  const int64_t lo = t * per < K ? t * per : K;
  const int64_t hi = (t + 1) * per < K ? (t + 1) * per : K;
  const int32_t* cb = counts + (int64_t)b * K;
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += cb[i];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  int32_t* ob = offsets + (int64_t)b * (K + 1);
  int32_t* kb = cursor + (int64_t)b * K;
  for (int64_t i = lo; i < hi; ++i) {
    ob[i] = run;
    kb[i] = run;
    run += cb[i];
  }
  if (t == 1023) ob[K] = part[1023];
}

// ---------------------------------------------------------------------------
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
      if ((unsigned)k < (unsigned)nb) {
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
// segreduce: one wave per run of kSegRun sorted positions. Lane l owns
// dims [db + l*V, db + l*V + V) of the row; DT element type, V elements.
template <int DT>
struct RowLoad;
template <>
struct RowLoad<FK_F32> {
  static constexpr int bytes = 4;
  __device__ static __forceinline__ float get(const void* p, int64_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
};
template <>
struct RowLoad<FK_F16> {
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float get(const void* p, int64_t i) {
    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
};
template <>
struct RowLoad<FK_BF16> {
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float get(const void* p, int64_t i) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
};

// V elements starting at element index i of a row, widened to fp32; only the
// first `nvalid` are read (the rest are zero). VEC: when nvalid >= V the V
// elements are contiguous and aligned to V*bytes.
template <int DT, int V, bool VEC>
__device__ __forceinline__ void load_row(const void* x, int64_t i, int nvalid, float (&v)[V]) {
  if (VEC && nvalid >= V) {
    if constexpr (DT == FK_F32) {
      if constexpr (V == 1) {
        v[0] = reinterpret_cast<const float*>(x)[i];
      } else if constexpr (V == 2) {
        const float2 t = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(x) + i);
        v[0] = t.x; v[1] = t.y;
      } else {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
          const float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i + e);
          v[e] = t.x; v[e + 1] = t.y; v[e + 2] = t.z; v[e + 3] = t.w;
        }
      }
    } else {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + i;
      uint16_t h[V];
      if constexpr (V == 1) {
        h[0] = p[0];
      } else if constexpr (V == 2) {
        const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
        h[0] = (uint16_t)t; h[1] = (uint16_t)(t >> 16);
      } else if constexpr (V == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        h[0] = (uint16_t)t.x; h[1] = (uint16_t)(t.x >> 16);
        h[2] = (uint16_t)t.y; h[3] = (uint16_t)(t.y >> 16);
      } else {
#pragma unroll
        for (int e = 0; e < V; e += 8) {
          const uint4 t = *reinterpret_cast<const uint4*>(p + e);
          h[e + 0] = (uint16_t)t.x; h[e + 1] = (uint16_t)(t.x >> 16);
          h[e + 2] = (uint16_t)t.y; h[e + 3] = (uint16_t)(t.y >> 16);
          h[e + 4] = (uint16_t)t.z; h[e + 5] = (uint16_t)(t.z >> 16);
          h[e + 6] = (uint16_t)t.w; h[e + 7] = (uint16_t)(t.w >> 16);
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e)
        v[e] = (DT == FK_F16) ? f16_bits_to_f32(h[e]) : bf16_bits_to_f32(h[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = e < nvalid ? RowLoad<DT>::get(x, i + e) : 0.f;
  }
}

template <int DT, int V, bool VEC>
__global__ __launch_bounds__(kThreads) void segreduce_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, float* __restrict__ sums, int N, int d, int K,
    int runs_per_batch, int64_t total_runs) {
  constexpr int U = 8;   // rows in flight per lane
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (wid >= total_runs) return;
  const int b = (int)(wid / runs_per_batch);
  const int p0 = (int)(wid % runs_per_batch) * kSegRun;
  const int p1 = p0 + kSegRun < N ? p0 + kSegRun : N;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  const int32_t* pb = perm + (int64_t)b * N;
  const int64_t xoff = (int64_t)b * N * d;
  float* sb = sums + (int64_t)b * K * d;

  // cluster holding position p0: the last k with offsets[k] <= p0
  int lo = 0, hi = K;   // invariant: offsets[lo] <= p0 < offsets[hi+1]... search on [0,K)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(ob[mid]) <= p0) lo = mid; else hi = mid - 1;
  }
  const int k_first = lo;

  for (int db = 0; db < d; db += 64 * V) {
    const int col = db + lane * V;
    const bool ok = col < d;
    const int nvalid = d - col;
    int k = k_first;
    int seg_lo = __builtin_amdgcn_readfirstlane(ob[k]);
    while (seg_lo < p1) {
      const int seg_hi = __builtin_amdgcn_readfirstlane(ob[k + 1]);
      if (seg_hi > seg_lo) {
        const int a = seg_lo > p0 ? seg_lo : p0;
        const int e = seg_hi < p1 ? seg_hi : p1;
        float acc[V];
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] = 0.f;
        int i = a;
        for (; i + U <= e; i += U) {
          float v[U][V];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int n = __builtin_amdgcn_readfirstlane(pb[i + u]);
            load_row<DT, V, VEC>(x, xoff + (int64_t)n * d + col, nvalid, v[u]);
          }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < V; ++j) acc[j] += v[u][j];
        }
        for (; i < e; ++i) {
          float v[V];
          const int n = __builtin_amdgcn_readfirstlane(pb[i]);
          load_row<DT, V, VEC>(x, xoff + (int64_t)n * d + col, nvalid, v);
#pragma unroll
          for (int j = 0; j < V; ++j) acc[j] += v[j];
        }
        float* dst = sb + (int64_t)k * d + col;
        const bool whole = seg_lo >= p0 && seg_hi <= p1;
        if (ok) {
#pragma unroll
          for (int j = 0; j < V; ++j) {
            if (col + j < d) {
              if (whole) dst[j] = acc[j];
              else unsafeAtomicAdd(dst + j, acc[j]);
            }
          }
        }
      }
      ++k;
      if (k >= K) break;
      seg_lo = seg_hi;
    }
  }
}

// ---------------------------------------------------------------------------
// finalize: block (chunk of one problem's K*d elements, b).
constexpr int kFinPerThread = 4;
__global__ __launch_bounds__(kThreads) void finalize_kernel(const float* __restrict__ sums,
                                                            const int32_t* __restrict__ counts,
                                                            float* __restrict__ c,
                                                            float* __restrict__ shift, int64_t Kd,
                                                            int d, int K, int chunks_per_batch) {
  __shared__ float part[kThreads / 64];
  const int b = blockIdx.x / chunks_per_batch;
  const int64_t e0 = (int64_t)(blockIdx.x % chunks_per_batch) * kThreads * kFinPerThread;
  const float* sb = sums + (int64_t)b * Kd;
  const int32_t* nb = counts + (int64_t)b * K;
  float* cbp = c + (int64_t)b * Kd;
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < kFinPerThread; ++q) {
    const int64_t e = e0 + (int64_t)q * kThreads + threadIdx.x;
    if (e < Kd) {
      const int k = (int)(e / d);
      const int n = nb[k];
      if (n > 0) {
        const float old = cbp[e];
        const float nw = sb[e] / (float)n;
        cbp[e] = nw;
        const float dl = nw - old;
        acc = fmaf(dl, dl, acc);
      }
    }
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += part[w];
    if (s != 0.f) unsafeAtomicAdd(&shift[b], s);
  }
}

// ---------------------------------------------------------------------------
template <int IPT>
hipError_t run_hist_scatter(const int32_t* ids, int32_t* counts, int32_t* cursor, int32_t* perm,
                            const int32_t* offsets_unused, int64_t B, int64_t N, int64_t K,
                            bool scatter, hipStream_t s) {
  (void)offsets_unused;
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

template <int DT, int V>
hipError_t run_segreduce(const void* x, const int32_t* perm, const int32_t* offsets, float* sums,
                         int64_t B, int64_t N, int64_t d, int64_t K, hipStream_t s) {
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int64_t total = B * runs;
  const int64_t grid = (total + 3) / 4;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int eb = DT == FK_F32 ? 4 : 2;
  const bool vec = (d % V) == 0 && ((uintptr_t)x % (uintptr_t)(V * eb)) == 0;
  if (vec)
    segreduce_kernel<DT, V, true><<<(unsigned)grid, kThreads, 0, s>>>(
        x, perm, offsets, sums, (int)N, (int)d, (int)K, runs, total);
  else
    segreduce_kernel<DT, V, false><<<(unsigned)grid, kThreads, 0, s>>>(
        x, perm, offsets, sums, (int)N, (int)d, (int)K, runs, total);
  return hipGetLastError();
}

template <int DT>
hipError_t segreduce_dt(const void* x, const int32_t* perm, const int32_t* offsets, float* sums,
                        int64_t B, int64_t N, int64_t d, int64_t K, hipStream_t s) {
  if (d <= 64) return run_segreduce<DT, 1>(x, perm, offsets, sums, B, N, d, K, s);
  if (d <= 128) return run_segreduce<DT, 2>(x, perm, offsets, sums, B, N, d, K, s);
  if (d <= 256) return run_segreduce<DT, 4>(x, perm, offsets, sums, B, N, d, K, s);
  if (d <= 512) return run_segreduce<DT, 8>(x, perm, offsets, sums, B, N, d, K, s);
  return run_segreduce<DT, 16>(x, perm, offsets, sums, B, N, d, K, s);
}

#define FK_CHECK(call)                   \
  do {                                   \
    hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

}  // namespace

size_t update_ws_bytes(int64_t B, int64_t N, int64_t d, int64_t K) {
  return align256((size_t)B * K * d * 4) + align256((size_t)B * (K + 1) * 4) +
         align256((size_t)B * K * 4) + align256((size_t)B * N * 4);
}

UpdateWs carve_update_ws(void* base, int64_t B, int64_t N, int64_t d, int64_t K) {
  char* p = static_cast<char*>(base);
  UpdateWs w;
  w.sums = reinterpret_cast<float*>(p);
  p += align256((size_t)B * K * d * 4);
  w.offsets = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * (K + 1) * 4);
  w.cursor = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.perm = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_update(const void* x, const int32_t* ids, int dt, int64_t B, int64_t N,
                         int64_t d, int64_t K, float* c, int32_t* counts, float* shift,
                         const UpdateWs& ws, hipStream_t s, hipEvent_t) {
  if (B == 0) return hipSuccess;
  {
    const int64_t work = B * K * d / 4 + B * K;
    int64_t g = (work + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(ws.sums, B * K * d, counts, B * K, shift, B);
    FK_CHECK(hipGetLastError());
  }
  if (N > 0) {
    if (K <= 4096) {
      FK_CHECK(run_hist_scatter<16>(ids, counts, nullptr, nullptr, nullptr, B, N, K, false, s));
    } else {
      FK_CHECK(run_hist_scatter<64>(ids, counts, nullptr, nullptr, nullptr, B, N, K, false, s));
    }
    scan_kernel<<<(unsigned)B, 1024, 0, s>>>(counts, ws.offsets, ws.cursor, (int)K);
    FK_CHECK(hipGetLastError());
    if (K <= 4096) {
      FK_CHECK(run_hist_scatter<16>(ids, nullptr, ws.cursor, ws.perm, nullptr, B, N, K, true, s));
    } else {
      FK_CHECK(run_hist_scatter<64>(ids, nullptr, ws.cursor, ws.perm, nullptr, B, N, K, true, s));
    }
    if (dt == FK_F16)
      FK_CHECK(segreduce_dt<FK_F16>(x, ws.perm, ws.offsets, ws.sums, B, N, d, K, s));
    else if (dt == FK_BF16)
      FK_CHECK(segreduce_dt<FK_BF16>(x, ws.perm, ws.offsets, ws.sums, B, N, d, K, s));
    else
      FK_CHECK(segreduce_dt<FK_F32>(x, ws.perm, ws.offsets, ws.sums, B, N, d, K, s));
  }
  {
    const int64_t Kd = K * d;
    const int64_t per = (int64_t)kThreads * kFinPerThread;
    const int chunks = (int)((Kd + per - 1) / per);
    const int64_t grid = B * chunks;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    finalize_kernel<<<(unsigned)grid, kThreads, 0, s>>>(ws.sums, counts, c, shift, Kd, (int)d,
                                                        (int)K, chunks);
    FK_CHECK(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace fk
