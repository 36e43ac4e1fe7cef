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
//   zero      counts and shift start at zero;
//   hist      counts[b,k]: per-block LDS histogram, one global atomic per
//             (block, non-empty bin);
//   scan      offsets[b,0..K] = exclusive prefix sum of counts; cursor = copy;
//             the fp32 sums of clusters that straddle a run (below) are zeroed;
//   scatter   perm[b, offsets[id] + rank] = n: per-block LDS ranks, one
//             cursor atomic per (block, non-empty bin);
//   segreduce sums[b,k,:] = sum of x[b, perm[i], :] over segment k; each wave
//             owns a fixed run of sorted positions (balanced by position, not
//             by segment, so a hot cluster spreads over many waves); a segment
//             lying wholly inside the run is finished by that wave
//             (c = sum / count, its squared move added to the shift); a piece
//             of a longer segment is added to sums with one fp32 atomic per
//             element: at most (K + number of runs) * d atomics per problem;
//   finalize_split  c = sums / count for the straddling clusters;
//   shift_reduce    shift[b] = sum of the per-wave / per-block squared moves
//             (partials in the workspace, summed in a fixed order).
// Empty clusters are never touched, so they keep their centroid.
#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsBins = 32768;     // 128 KB of LDS bins per block
constexpr int kSegRun = 256;           // sorted positions per wave in segreduce

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void zero_kernel(int32_t* __restrict__ counts,
                                                        int64_t ncounts) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < ncounts; i += stride) counts[i] = 0;
}

__global__ __launch_bounds__(kThreads) void fill_f32_kernel(float* __restrict__ p, float v,
                                                            int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
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
// scan: one block per problem; exclusive prefix sum of counts. Also zeroes
// the fp32 sums of clusters whose segment straddles a segreduce run.
// A cluster's segment [lo, hi) of sorted positions straddles a segreduce run
// boundary: it is then summed piecewise with atomics and finished in
// finalize_split; otherwise one wave sums it and finishes it.
__device__ __forceinline__ bool straddles(int lo, int hi) {
  return hi > lo && lo / kSegRun != (hi - 1) / kSegRun;
}

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ cursor,
                                                    float* __restrict__ sums, int K, int d) {
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
  float* sbase = sums + (int64_t)b * K * d;
  for (int64_t i = lo; i < hi; ++i) {
    ob[i] = run;
    kb[i] = run;
    const int next = run + cb[i];
    if (straddles(run, next)) {      // its pieces are summed with atomics: start at zero
      float* row = sbase + i * d;
      if ((d & 3) == 0) {
        float4* r4 = reinterpret_cast<float4*>(row);
        for (int j = 0; j < d / 4; ++j) r4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        for (int j = 0; j < d; ++j) row[j] = 0.f;
      }
    }
    run = next;
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
// segreduce: one wave per run of kSegRun sorted positions.
//
// The wave stages its run of perm in LDS, then walks the segments that
// intersect the run. Rows are read as 16-byte vectors: LPR lanes cover one
// row (VPL vectors each), so a wave instruction reads 64/LPR rows and each
// lane keeps U row-iterations of loads in flight. At the end of a piece the
// row groups are summed with lane shuffles. A segment wholly inside the run
// is finished here: c = sum / count, and its squared move is added to the
// shift. A piece of a longer segment is added to `sums` with one fp32 atomic
// per element; finalize_split completes those clusters.
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

template <int DT>
__device__ __forceinline__ float load_elem(const void* x, int64_t i) {
  if constexpr (DT == FK_F32) return reinterpret_cast<const float*>(x)[i];
  else return Elem<DT>::widen(reinterpret_cast<const uint16_t*>(x)[i]);
}

template <int DT, int LPR, int VPL, bool VEC>
__global__ __launch_bounds__(kThreads) void segreduce_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, float* __restrict__ sums, float* __restrict__ c,
    float* __restrict__ moved_part, int N, int d, int K, int runs_per_batch, int64_t total_runs,
    int dbase, int parts_per_batch) {
  constexpr int R = 64 / LPR;                    // rows per wave instruction
  constexpr int EB = DT == FK_F32 ? 4 : 2;
  constexpr int EV = 16 / EB;                    // elements per 16-byte vector
  constexpr int NE = VPL * EV;                   // elements per lane
  constexpr int U = VPL >= 8 ? 1 : (VPL == 4 ? 2 : (VPL == 2 ? 4 : 8));
  __shared__ int32_t lperm[kThreads / 64][kSegRun];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane / LPR, li = lane % LPR;
  const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + wv;
  if (wid >= total_runs) return;                 // whole wave; no block barrier follows
  const int b = (int)(wid / runs_per_batch);
  const int p0 = (int)(wid % runs_per_batch) * kSegRun;
  const int p1 = p0 + kSegRun < N ? p0 + kSegRun : N;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  const int32_t* pb = perm + (int64_t)b * N;
  const int64_t xoff = (int64_t)b * N * d;
  float* sb = sums + (int64_t)b * K * d;
  float* cb = c + (int64_t)b * K * d;

  for (int j = lane; j < p1 - p0; j += 64) lperm[wv][j] = pb[p0 + j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // first cluster of the run: the last k with offsets[k] <= p0
  int lo = 0, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(ob[mid]) <= p0) lo = mid; else hi = mid - 1;
  }
  int k = lo;

  int col[VPL];                                  // first element of each of my vectors
#pragma unroll
  for (int q = 0; q < VPL; ++q) col[q] = dbase + (li + LPR * q) * EV;

  float moved = 0.f;
  int seg_lo = __builtin_amdgcn_readfirstlane(ob[k]);
  while (seg_lo < p1) {
    const int seg_hi = __builtin_amdgcn_readfirstlane(ob[k + 1]);
    if (seg_hi > seg_lo) {
      const int a = seg_lo > p0 ? seg_lo : p0;
      const int e = seg_hi < p1 ? seg_hi : p1;
      float acc[NE];
#pragma unroll
      for (int i = 0; i < NE; ++i) acc[i] = 0.f;
      for (int base = a; base < e; base += U * R) {
        int n[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = base + u * R + g;
          n[u] = p < e ? lperm[wv][p - p0] : -1;
        }
        if constexpr (VEC) {
          uint4 v[U][VPL];
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < VPL; ++q) {
              const bool ok = n[u] >= 0 && col[q] < d;
              const int64_t idx = xoff + (int64_t)(ok ? n[u] : 0) * d + (ok ? col[q] : 0);
              v[u][q] = ok ? *reinterpret_cast<const uint4*>(
                                 reinterpret_cast<const char*>(x) + idx * EB)
                           : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < VPL; ++q) {
              float f[EV];
              widen16<DT>(v[u][q], f);
#pragma unroll
              for (int i = 0; i < EV; ++i) acc[q * EV + i] += f[i];
            }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (n[u] < 0) continue;
            const int64_t row = xoff + (int64_t)n[u] * d;
#pragma unroll
            for (int q = 0; q < VPL; ++q)
#pragma unroll
              for (int i = 0; i < EV; ++i)
                if (col[q] + i < d) acc[q * EV + i] += load_elem<DT>(x, row + col[q] + i);
          }
        }
      }
      // sum the R row groups
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < NE; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
      const bool whole = seg_lo >= p0 && seg_hi <= p1;
      if (g == 0) {
        const float cnt = (float)(seg_hi - seg_lo);
#pragma unroll
        for (int q = 0; q < VPL; ++q)
#pragma unroll
          for (int i = 0; i < EV; ++i) {
            const int j = col[q] + i;
            if (j < d) {
              const int64_t o = (int64_t)k * d + j;
              if (whole) {
                const float nw = acc[q * EV + i] / cnt;
                const float dl = nw - cb[o];
                cb[o] = nw;
                moved = fmaf(dl, dl, moved);
              } else {
                unsafeAtomicAdd(sb + o, acc[q * EV + i]);
              }
            }
          }
      }
    }
    ++k;
    if (k >= K) break;
    seg_lo = seg_hi;
  }
  // this wave's share of the shift; several d passes accumulate in order
  moved = wave_sum(moved);
  if (lane == 0) {
    float* slot = moved_part + (int64_t)b * parts_per_batch + (wid % runs_per_batch);
    *slot = dbase == 0 ? moved : *slot + moved;
  }
}

// ---------------------------------------------------------------------------
// finalize_split: clusters whose segment straddles a run boundary. Block j of
// problem b scans rows j*4+w, j*4+w+4*fb, ... (w = wave); straddling rows get
// c = sums / count; the block's squared moves go to its partial slot.
constexpr int kFinBlocks = 64;   // blocks per problem (at most)

__global__ __launch_bounds__(kThreads) void finalize_split_kernel(
    const float* __restrict__ sums, const int32_t* __restrict__ offsets, float* __restrict__ c,
    float* __restrict__ moved_part, int d, int K, int fb, int parts_per_batch, int part0) {
  __shared__ float wsum[kThreads / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.x / fb, j = blockIdx.x % fb;
  const int32_t* ob = offsets + (int64_t)b * (K + 1);
  float moved = 0.f;
  for (int k = j * (kThreads / 64) + wv; k < K; k += fb * (kThreads / 64)) {
    const int lo = ob[k], hi = ob[k + 1];
    if (!straddles(lo, hi)) continue;
    const float cnt = (float)(hi - lo);
    const float* srow = sums + ((int64_t)b * K + k) * d;
    float* crow = c + ((int64_t)b * K + k) * d;
    for (int i = lane; i < d; i += 64) {
      const float nw = srow[i] / cnt;
      const float dl = nw - crow[i];
      crow[i] = nw;
      moved = fmaf(dl, dl, moved);
    }
  }
  moved = wave_sum(moved);
  if (lane == 0) wsum[wv] = moved;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
    moved_part[(int64_t)b * parts_per_batch + part0 + j] = t;
  }
}

// shift[b] = sum of the problem's partials (fixed order: deterministic).
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

template <int DT, int LPR, int VPL>
hipError_t run_segreduce(const void* x, const int32_t* perm, const int32_t* offsets, float* sums,
                         float* c, float* part, int parts, int64_t B, int64_t N, int64_t d,
                         int64_t K, hipStream_t s) {
  constexpr int EB = DT == FK_F32 ? 4 : 2;
  constexpr int span = LPR * VPL * (16 / EB);    // elements covered per pass
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int64_t total = B * runs;
  const int64_t grid = (total + 3) / 4;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const bool vec = (d * EB) % 16 == 0 && ((uintptr_t)x % 16) == 0;
  for (int64_t db = 0; db < d; db += span) {
    if (vec)
      segreduce_kernel<DT, LPR, VPL, true><<<(unsigned)grid, kThreads, 0, s>>>(
          x, perm, offsets, sums, c, part, (int)N, (int)d, (int)K, runs, total, (int)db, parts);
    else
      segreduce_kernel<DT, LPR, VPL, false><<<(unsigned)grid, kThreads, 0, s>>>(
          x, perm, offsets, sums, c, part, (int)N, (int)d, (int)K, runs, total, (int)db, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Lanes per row: enough 16-byte vectors to cover the row, as a power of two;
// rows wider than 64 vectors take VPL vectors per lane (several passes above
// 64*8 vectors).
template <int DT>
hipError_t segreduce_dt(const void* x, const int32_t* perm, const int32_t* offsets, float* sums,
                        float* c, float* part, int parts, int64_t B, int64_t N, int64_t d,
                        int64_t K, hipStream_t s) {
  constexpr int EV = DT == FK_F32 ? 4 : 8;
  const int64_t nvec = (d + EV - 1) / EV;
#define FK_SEG(L, V) \
  run_segreduce<DT, L, V>(x, perm, offsets, sums, c, part, parts, B, N, d, K, s)
  if (nvec <= 4) return FK_SEG(4, 1);
  if (nvec <= 8) return FK_SEG(8, 1);
  if (nvec <= 16) return FK_SEG(16, 1);
  if (nvec <= 32) return FK_SEG(32, 1);
  if (nvec <= 64) return FK_SEG(64, 1);
  if (nvec <= 128) return FK_SEG(64, 2);
  if (nvec <= 256) return FK_SEG(64, 4);
  return FK_SEG(64, 8);
#undef FK_SEG
}

#define FK_CHECK(call)                   \
  do {                                   \
    hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

}  // namespace

int fin_blocks(int64_t K) {
  const int64_t fb = (K + 63) / 64;
  return (int)(fb < kFinBlocks ? fb : kFinBlocks);
}

int64_t shift_parts(int64_t N, int64_t K) { return (N + kSegRun - 1) / kSegRun + fin_blocks(K); }

size_t update_ws_bytes(int64_t B, int64_t N, int64_t d, int64_t K) {
  return align256((size_t)B * K * d * 4) + align256((size_t)B * (K + 1) * 4) +
         align256((size_t)B * K * 4) + align256((size_t)B * N * 4) +
         align256((size_t)B * shift_parts(N, K) * 4);
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
  p += align256((size_t)B * N * 4);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

hipError_t launch_update(const void* x, const int32_t* ids, int dt, int64_t B, int64_t N,
                         int64_t d, int64_t K, float* c, int32_t* counts, float* shift,
                         const UpdateWs& ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int parts = (int)shift_parts(N, K);
  const int runs = (int)((N + kSegRun - 1) / kSegRun);
  const int fb = fin_blocks(K);
  {
    int64_t g = (B * K + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    zero_kernel<<<(unsigned)g, kThreads, 0, s>>>(counts, B * K);
    FK_CHECK(hipGetLastError());
  }
  if (N > 0) {
    if (K <= 4096)
      FK_CHECK(run_hist_scatter<16>(ids, counts, nullptr, nullptr, B, N, K, false, s));
    else
      FK_CHECK(run_hist_scatter<64>(ids, counts, nullptr, nullptr, B, N, K, false, s));
    scan_kernel<<<(unsigned)B, 1024, 0, s>>>(counts, ws.offsets, ws.cursor, ws.sums, (int)K,
                                             (int)d);
    FK_CHECK(hipGetLastError());
    if (K <= 4096)
      FK_CHECK(run_hist_scatter<16>(ids, nullptr, ws.cursor, ws.perm, B, N, K, true, s));
    else
      FK_CHECK(run_hist_scatter<64>(ids, nullptr, ws.cursor, ws.perm, B, N, K, true, s));
    if (dt == FK_F16)
      FK_CHECK(segreduce_dt<FK_F16>(x, ws.perm, ws.offsets, ws.sums, c, ws.part, parts, B, N, d,
                                    K, s));
    else if (dt == FK_BF16)
      FK_CHECK(segreduce_dt<FK_BF16>(x, ws.perm, ws.offsets, ws.sums, c, ws.part, parts, B, N,
                                     d, K, s));
    else
      FK_CHECK(segreduce_dt<FK_F32>(x, ws.perm, ws.offsets, ws.sums, c, ws.part, parts, B, N, d,
                                    K, s));
    const int64_t grid = B * fb;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    finalize_split_kernel<<<(unsigned)grid, kThreads, 0, s>>>(ws.sums, ws.offsets, c, ws.part,
                                                              (int)d, (int)K, fb, parts, runs);
    FK_CHECK(hipGetLastError());
  } else {
    // no point: every cluster is empty and keeps its centroid; zero the partials
    const int64_t n = B * parts;
    int64_t g = (n + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    fill_f32_kernel<<<(unsigned)g, kThreads, 0, s>>>(ws.part, 0.f, n);
    FK_CHECK(hipGetLastError());
  }
  shift_reduce_kernel<<<(unsigned)B, kThreads, 0, s>>>(ws.part, shift, parts);
  FK_CHECK(hipGetLastError());
  return hipSuccess;
}

}  // namespace fk
