// FlashAssign for large d (d > 512) on gfx950: outer K loop, inner D loop.
//
// Same contraction and argmax as the small-D path (score_k = x.c_k -
// ||c_k||^2 / 2, lowest k on ties; the distance matrix is never written), but
// a point's fragments no longer fit in registers for the whole K range, so the
// loop order flips: a block holds a (256 points x TK centroids) score block in
// accumulator registers and walks d in chunks ("Flash-KMeans: Fast and
// Memory-Efficient Exact K-Means", Abstract; "flash-kmeans and the return of
// exact K-Means on the GPU", section "The point of the kernel is that the
// distance matrix never exists").
//
// Block: 4 waves, one per SIMD (the 256 accumulator registers of a lane fill
// the AGPR file), 2 point fragments of 32 points per wave. TK = 256 centroids
// (8 row blocks of 32) when K > 128, else 128, so a problem with K <= 256
// reads each point row exactly once. Per d-chunk of 128 (8 MFMA k-steps,
// k-step outer, row block inner):
//   - as soon as a k-step is done for every row block, its point-fragment
//     registers are reloaded with the next chunk's columns, so each load has
//     most of a chunk to land;
//   - the next chunk's centroid rows are staged into the other LDS buffer in
//     NSUB/2 parts spread over the chunk (each fetched one part-interval
//     before it is stored), so only 16 registers hold staged data;
//   - one barrier per chunk.
// At the last chunk of a K tile the accumulators are scanned for each lane's
// best score and row, then reloaded with -||c||^2/2 of the next tile's rows.
#include <math.h>

#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kThreads = 256;              // 4 waves
constexpr int kWaves = 4;
constexpr int kNF = 2;                     // point fragments per wave
constexpr int kBN = kWaves * kNF * 32;     // points per block
constexpr int kDC = 128;                   // d-chunk
constexpr int kKS = kDC / 16;              // MFMA k-steps per chunk
constexpr int kPitch = kDC + 8;            // LDS row pitch (elements): +16 B against bank conflicts
constexpr int kVPR = kDC / 8;              // 16-byte vectors per chunk row

// Running argmax over one 32x32 accumulator: the lane holds rows
// 8*(r/4) + 4*half + r%4 of the block; the 4*half term is added at the merge.
// Rows are visited in increasing order with a strict '>', so the first
// (lowest) row wins among equal scores.
__device__ __forceinline__ void argmax_update(const floatx16_t& acc, int base, float& best,
                                              int& bidx) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = acc[r];
    const bool gt = v > best;
    best = gt ? v : best;
    bidx = gt ? base + 8 * (r >> 2) + (r & 3) : bidx;
  }
}

// FULL: VEC and d % kDC == 0, so every chunk column is real and loads need no
// guard; otherwise columns >= d read as zero.
template <int DT, int NSUB, bool VEC, bool FULL>
__global__ __launch_bounds__(kThreads) void assign_splitd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ c,
    const float* __restrict__ cnorm, int32_t* __restrict__ ids, int N, int d, int K,
    int blocks_per_batch, int grid) {
  constexpr int TK = NSUB * 32;                   // centroids per K tile
  constexpr int NPART = NSUB / 2;                 // staging parts per chunk
  constexpr int PROWS = TK / NPART;               // rows per staging part
  constexpr int NV = PROWS * kVPR / kThreads;     // vectors per thread per part
  static_assert(PROWS * kVPR % kThreads == 0, "staging split");
  static_assert(TK <= kThreads, "one norm per thread");
  constexpr int Q = NSUB * kKS;                   // (row block, k-step) pairs per chunk
  __shared__ __align__(16) uint16_t lds_c[2][TK * kPitch];
  __shared__ __align__(16) float lds_h[2][TK];    // -||c||^2/2 by K-tile parity

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, r32 = lane & 31;
  const int64_t logical = xcd_remap(blockIdx.x, grid);
  const int b = (int)(logical / blocks_per_batch);
  const int nblk = (int)(logical % blocks_per_batch) * kBN + wave * kNF * 32;
  const uint16_t* xb = x + (int64_t)b * N * d;
  const uint16_t* cb = c + (int64_t)b * K * d;
  const float* cnb = cnorm + (int64_t)b * K;

  // rows past N repeat row N-1; their results are never stored
  const uint16_t* xrow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) xrow[f] = xb + (int64_t)min(nblk + f * 32 + r32, N - 1) * d;

  const int nchunks = (d + kDC - 1) / kDC;
  const int ktiles = (K + TK - 1) / TK;
  const int steps = ktiles * nchunks;             // (K tile, d-chunk) pairs, K tile outer

  auto load_x = [&](int ch, uint4 (&xf)[kNF][kKS]) {
#pragma unroll
    for (int f = 0; f < kNF; ++f)
#pragma unroll
      for (int s = 0; s < kKS; ++s)
        xf[f][s] = FULL ? *reinterpret_cast<const uint4*>(xrow[f] + ch * kDC + s * 16 + half * 8)
                        : load8<VEC>(xrow[f], ch * kDC + s * 16 + half * 8, d);
  };

  // Centroid staging of step st, part h (rows h*PROWS .. h*PROWS+PROWS-1 of
  // its K tile). Rows past K repeat row K-1 and get -inf norms, so they never win.
  uint4 pre[NV];
  float pre_n = 0.f;
  auto fetch = [&](int st, int h) {
    const int kt = st / nchunks, ch = st - kt * nchunks;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = tid + kThreads * q;
      const int row = v / kVPR, col = ch * kDC + (v % kVPR) * 8;
      const int k = min(kt * TK + h * PROWS + row, K - 1);
      pre[q] = FULL ? *reinterpret_cast<const uint4*>(cb + (int64_t)k * d + col)
                    : load8<VEC>(cb + (int64_t)k * d, col, d);
    }
    if (h == 0) pre_n = cnb[min(kt * TK + (tid % TK), K - 1)];
  };
  auto stash = [&](int st, int buf, int h, bool fresh) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = tid + kThreads * q;
      const int row = v / kVPR, col = (v % kVPR) * 8;
      *reinterpret_cast<uint4*>(&lds_c[buf][(h * PROWS + row) * kPitch + col]) = pre[q];
    }
    const int kt = st / nchunks;
    // a K tile's norms are written with its first chunk (not by the repeat
    // past the last step); the other parity slot is the one being read
    if (fresh && h == 0 && st - kt * nchunks == 0 && tid < TK)
      lds_h[kt & 1][tid] = (kt * TK + tid < K) ? -0.5f * pre_n : -INFINITY;
  };

  floatx16_t acc[NSUB][kNF];
  float best[kNF];
  int bidx[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    best[f] = -INFINITY;
    bidx[f] = 0;
  }

  // A fragment of pair q: row block q % NSUB, k-step q / NSUB (k-step outer,
  // so each point fragment register is free once its k-step is done).
  auto read_a = [&](int buf, int q) -> uint4 {
    const int sub = q % NSUB, kk = q / NSUB;
    return *reinterpret_cast<const uint4*>(
        &lds_c[buf][(sub * 32 + r32) * kPitch + half * 8 + kk * 16]);
  };

  uint4 xf[kNF][kKS];
  load_x(0, xf);
  fetch(0, 0);
  stash(0, 0, 0, true);
#pragma unroll
  for (int h = 1; h < NPART; ++h) {
    fetch(0, h);
    stash(0, 0, h, true);
  }
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      floatx16_t ci;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 hv =
            *reinterpret_cast<const float4*>(&lds_h[kt & 1][sub * 32 + 8 * i + 4 * half]);
        ci[4 * i + 0] = hv.x;
        ci[4 * i + 1] = hv.y;
        ci[4 * i + 2] = hv.z;
        ci[4 * i + 3] = hv.w;
      }
#pragma unroll
      for (int f = 0; f < kNF; ++f) acc[sub][f] = ci;
    }
    for (int ch = 0; ch < nchunks; ++ch) {
      const int st = kt * nchunks + ch;
      const int buf = st & 1;
      // the next step's data; past the last step a harmless repeat of it,
      // stored into the idle buffer (never read)
      const int sn = st + 1 < steps ? st + 1 : st;
      const int chn = sn % nchunks;
      fetch(sn, 0);
      uint4 ar[4];
      ar[0] = read_a(buf, 0);
      ar[1] = read_a(buf, 1);
      ar[2] = read_a(buf, 2);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int sub = q % NSUB, kk = q / NSUB;
        if (q + 3 < Q) ar[(q + 3) % 4] = read_a(buf, q + 3);
        if (q > 0 && q % (Q / NPART) == 0) {   // part q*NPART/Q - 1 has had time to land
          stash(sn, buf ^ 1, q / (Q / NPART) - 1, sn != st);
          fetch(sn, q / (Q / NPART));
        }
#pragma unroll
        for (int f = 0; f < kNF; ++f)
          acc[sub][f] = Mfma<DT>::run(ar[q % 4], xf[f][kk], acc[sub][f]);
        if (sub == NSUB - 1) {
          // k-step kk is done for every row block: its point registers take
          // the next step's columns, most of a chunk ahead of their use
#pragma unroll
          for (int f = 0; f < kNF; ++f)
            xf[f][kk] = FULL ? *reinterpret_cast<const uint4*>(xrow[f] + chn * kDC + kk * 16 + half * 8)
                             : load8<VEC>(xrow[f], chn * kDC + kk * 16 + half * 8, d);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      stash(sn, buf ^ 1, NPART - 1, sn != st);
      __syncthreads();
    }
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int f = 0; f < kNF; ++f) argmax_update(acc[sub][f], kt * TK + sub * 32, best[f], bidx[f]);
  }

  int32_t* ib = ids + (int64_t)b * N;
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    const int idx = merge_halves(best[f], bidx[f], half);
    const int n = nblk + f * 32 + r32;
    if (half == 0 && n < N) ib[n] = idx;
  }
}

// 16-byte vector loads need rows of whole 8-element vectors and aligned bases.
bool vec_ok(const void* x, const void* c, int64_t d) {
  return d % 8 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)c % 16) == 0;
}

template <int DT, int NSUB>
hipError_t run_splitd(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                      int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  const int bpb = (int)((N + kBN - 1) / kBN);
  const int64_t grid = B * bpb;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* cp = (const uint16_t*)c;
  if (vec_ok(x, c, d) && d % kDC == 0)
    assign_splitd_kernel<DT, NSUB, true, true><<<(unsigned)grid, kThreads, 0, s>>>(
        xp, cp, cn, ids, (int)N, (int)d, (int)K, bpb, (int)grid);
  else if (vec_ok(x, c, d))
    assign_splitd_kernel<DT, NSUB, true, false><<<(unsigned)grid, kThreads, 0, s>>>(
        xp, cp, cn, ids, (int)N, (int)d, (int)K, bpb, (int)grid);
  else if constexpr (NSUB == 4)
    assign_splitd_kernel<DT, NSUB, false, false><<<(unsigned)grid, kThreads, 0, s>>>(
        xp, cp, cn, ids, (int)N, (int)d, (int)K, bpb, (int)grid);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

// K <= 128: one 128-row tile; otherwise 256-row tiles. Element-wise loads
// (unaligned or d % 8 != 0) keep 128-row tiles: with 256 the accumulators
// leave no registers for them.
template <int DT>
hipError_t splitd_dt(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                     int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  if (K <= 128 || !vec_ok(x, c, d)) return run_splitd<DT, 4>(x, c, cn, B, N, d, K, ids, s);
  return run_splitd<DT, 8>(x, c, cn, B, N, d, K, ids, s);
}

}  // namespace

hipError_t launch_assign_splitd(const void* x, const void* c_lp, const float* cnorm, int dt,
                                int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                                hipStream_t s) {
  if (B == 0 || N == 0) return hipSuccess;
  if (dt == FK_F16) return splitd_dt<FK_F16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  if (dt == FK_BF16) return splitd_dt<FK_BF16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  return hipErrorNotSupported;
}

}  // namespace fk
