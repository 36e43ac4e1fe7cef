// FlashAssign for large d (d > 512; fp32 d > 256) on gfx950: outer K loop,
// inner D loop.
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
    int blocks_per_batch, int total, int nblocks) {
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
  const int nchunks = (d + kDC - 1) / kDC;
  const int ktiles = (K + TK - 1) / TK;

  // point block v -> problem, this wave's first row and the lane's rows
  // (rows past N repeat row N-1; their results are never stored)
  auto locate = [&](int64_t v, int& pb, int& row0, const uint16_t* (&rows)[kNF]) {
    const int64_t logical = xcd_remap(v, total);
    pb = (int)(logical / blocks_per_batch);
    row0 = (int)(logical % blocks_per_batch) * kBN + wave * kNF * 32;
#pragma unroll
    for (int f = 0; f < kNF; ++f)
      rows[f] = x + ((int64_t)pb * N + min(row0 + f * 32 + r32, N - 1)) * d;
  };
  auto load_frag = [&](const uint16_t* row, int ch, int kk) -> uint4 {
    return FULL ? *reinterpret_cast<const uint4*>(row + ch * kDC + kk * 16 + half * 8)
                : load8<VEC>(row, ch * kDC + kk * 16 + half * 8, d);
  };

  // Centroid staging of (problem pb, K tile kt, chunk ch), part h (rows
  // h*PROWS .. h*PROWS+PROWS-1 of the tile). Rows past K repeat row K-1 and
  // get -inf norms, so they never win.
  uint4 pre[NV];
  float pre_n = 0.f;
  auto fetch = [&](int pb, int kt, int ch, int h) {
    const uint16_t* cb = c + (int64_t)pb * K * d;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = tid + kThreads * q;
      const int row = v / kVPR, col = ch * kDC + (v % kVPR) * 8;
      const int k = min(kt * TK + h * PROWS + row, K - 1);
      pre[q] = FULL ? *reinterpret_cast<const uint4*>(cb + (int64_t)k * d + col)
                    : load8<VEC>(cb + (int64_t)k * d, col, d);
    }
    if (h == 0) pre_n = cnorm[(int64_t)pb * K + min(kt * TK + (tid % TK), K - 1)];
  };
  // norm_slot >= 0: the staged chunk starts a K tile (kt) whose norms go to
  // lds_h[norm_slot]
  auto stash = [&](int buf, int h, int kt, int norm_slot) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = tid + kThreads * q;
      const int row = v / kVPR, col = (v % kVPR) * 8;
      *reinterpret_cast<uint4*>(&lds_c[buf][(h * PROWS + row) * kPitch + col]) = pre[q];
    }
    if (h == 0 && norm_slot >= 0 && tid < TK)
      lds_h[norm_slot][tid] = (kt * TK + tid < K) ? -0.5f * pre_n : -INFINITY;
  };

  floatx16_t acc[NSUB][kNF];
  float best[kNF];
  int bidx[kNF];

  // A fragment of pair q: row block q % NSUB, k-step q / NSUB (k-step outer,
  // so each point fragment register is free once its k-step is done).
  auto read_a = [&](int buf, int q) -> uint4 {
    const int sub = q % NSUB, kk = q / NSUB;
    return *reinterpret_cast<const uint4*>(
        &lds_c[buf][(sub * 32 + r32) * kPitch + half * 8 + kk * 16]);
  };

  // Persistent: point blocks v = blockIdx.x, + nblocks, ... (nblocks is a
  // multiple of 8, so each stays on this block's XCD). The step after the
  // last one of a point block is the next point block's first: its centroid
  // chunk and its point fragments load during the current block's last
  // chunk. Past the last point block the loads repeat the current step's
  // data, stored into the idle buffer that nothing reads.
  int64_t v = blockIdx.x;
  int pb, row0;
  const uint16_t* xrow[kNF];
  locate(v, pb, row0, xrow);
  int64_t vn = v + nblocks;
  int npb = pb, nrow0 = row0;
  const uint16_t* nxrow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) nxrow[f] = xrow[f];
  if (vn < total) locate(vn, npb, nrow0, nxrow);

  uint4 xf[kNF][kKS];
#pragma unroll
  for (int f = 0; f < kNF; ++f)
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) xf[f][kk] = load_frag(xrow[f], 0, kk);
#pragma unroll
  for (int h = 0; h < NPART; ++h) {
    fetch(pb, 0, 0, h);
    stash(0, h, 0, 0);
  }
  __syncthreads();
  int buf = 0, tc = 0;                            // tc: K tiles started by this block
  for (;;) {
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      best[f] = -INFINITY;
      bidx[f] = 0;
    }
    for (int kt = 0; kt < ktiles; ++kt) {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        floatx16_t ci;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 hv =
              *reinterpret_cast<const float4*>(&lds_h[tc & 1][sub * 32 + 8 * i + 4 * half]);
          ci[4 * i + 0] = hv.x;
          ci[4 * i + 1] = hv.y;
          ci[4 * i + 2] = hv.z;
          ci[4 * i + 3] = hv.w;
        }
#pragma unroll
        for (int f = 0; f < kNF; ++f) acc[sub][f] = ci;
      }
      for (int ch = 0; ch < nchunks; ++ch) {
        // the next step: (kt, ch+1), (kt+1, 0), the next point block's
        // (0, 0), or past the end a repeat of this one
        const bool in_tile = ch + 1 < nchunks;
        const bool in_block = in_tile || kt + 1 < ktiles;
        const bool to_next = !in_block && vn < total;
        const bool fresh = in_block || to_next;
        const int pbn = to_next ? npb : pb;
        const int ktn = in_tile ? kt : (in_block ? kt + 1 : (to_next ? 0 : kt));
        const int chn = in_tile ? ch + 1 : (fresh ? 0 : ch);
        const int slot = fresh && !in_tile ? (tc + 1) & 1 : -1;
        const uint16_t* rn[kNF];
#pragma unroll
        for (int f = 0; f < kNF; ++f) rn[f] = to_next ? nxrow[f] : xrow[f];
        fetch(pbn, ktn, chn, 0);
        uint4 ar[4];
        ar[0] = read_a(buf, 0);
        ar[1] = read_a(buf, 1);
        ar[2] = read_a(buf, 2);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const int sub = q % NSUB, kk = q / NSUB;
          if (q + 3 < Q) ar[(q + 3) % 4] = read_a(buf, q + 3);
          if (q > 0 && q % (Q / NPART) == 0) {   // part q*NPART/Q - 1 has had time to land
            stash(buf ^ 1, q / (Q / NPART) - 1, ktn, slot);
            fetch(pbn, ktn, chn, q / (Q / NPART));
          }
#pragma unroll
          for (int f = 0; f < kNF; ++f)
            acc[sub][f] = Mfma<DT>::run(ar[q % 4], xf[f][kk], acc[sub][f]);
          if (sub == NSUB - 1) {
            // k-step kk is done for every row block: its point registers take
            // the next step's columns, most of a chunk ahead of their use
#pragma unroll
            for (int f = 0; f < kNF; ++f) xf[f][kk] = load_frag(rn[f], chn, kk);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        stash(buf ^ 1, NPART - 1, ktn, slot);
        __syncthreads();
        buf ^= 1;
      }
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int f = 0; f < kNF; ++f) argmax_update(acc[sub][f], kt * TK + sub * 32, best[f], bidx[f]);
      ++tc;
    }
    int32_t* ib = ids + (int64_t)pb * N;
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const int idx = merge_halves(best[f], bidx[f], half);
      const int n = row0 + f * 32 + r32;
      if (half == 0 && n < N) ib[n] = idx;
    }
    if (vn >= total) break;
    v = vn;
    pb = npb;
    row0 = nrow0;
#pragma unroll
    for (int f = 0; f < kNF; ++f) xrow[f] = nxrow[f];
    vn = v + nblocks;
    if (vn < total) locate(vn, npb, nrow0, nxrow);
  }
}

// 16-byte vector loads need rows of whole 8-element vectors and aligned bases.
bool vec_ok(const void* x, const void* c, int64_t d) {
  return d % 8 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)c % 16) == 0;
}

// Blocks of kernel `kern` that fit on the current device at once, cached per
// device in `cache` (one cache per kernel instance; 0 = not yet queried).
template <typename Kern>
int resident_blocks(Kern kern, int threads, int (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <int DT, int NSUB, bool VEC, bool FULL>
hipError_t launch_splitd(const uint16_t* x, const uint16_t* c, const float* cn, int64_t total,
                         int bpb, int64_t N, int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  static int cache[64];
  auto kern = assign_splitd_kernel<DT, NSUB, VEC, FULL>;
  const int resident = resident_blocks(kern, kThreads, cache);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  // a multiple of 8 so each block's point blocks stay on its XCD
  int64_t nblocks = resident >= 8 ? resident / 8 * 8 : resident;
  if (nblocks > total) nblocks = total;
  kern<<<(unsigned)nblocks, kThreads, 0, s>>>(x, c, cn, ids, (int)N, (int)d, (int)K, bpb,
                                              (int)total, (int)nblocks);
  return hipGetLastError();
}

template <int DT, int NSUB>
hipError_t run_splitd(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                      int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  const int bpb = (int)((N + kBN - 1) / kBN);
  const int64_t total = B * bpb;
  if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* cp = (const uint16_t*)c;
  if (vec_ok(x, c, d) && d % kDC == 0)
    return launch_splitd<DT, NSUB, true, true>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if (vec_ok(x, c, d))
    return launch_splitd<DT, NSUB, true, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if constexpr (NSUB == 4)
    return launch_splitd<DT, NSUB, false, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  return hipErrorNotSupported;
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
  if (K < 1) return hipErrorInvalidValue;    // the point-block loop needs a tile
  if (dt == FK_F16) return splitd_dt<FK_F16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  if (dt == FK_BF16) return splitd_dt<FK_BF16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  // fp32: rows of 2d 16-bit units (every load and LDS copy moves bytes), four
  // v_mfma_f32_32x32x2_f32 per 16-byte k-step
  if (dt == FK_F32) return splitd_dt<FK_F32>(x, c_lp, cnorm, B, N, 2 * d, K, ids, s);
  return hipErrorNotSupported;
}

}  // namespace fk
