// FlashAssign for gfx950: fused point-centroid distance + online argmin.
//
// What is computed (per problem b and point n):
//   ids[b,n] = argmin_k  ||c_k||^2 - 2 x_n . c_k
// (scores equal to within the fp32 rounding may resolve to either centroid;
// see the slot code below)
// maximised here in the equivalent, exactly scaled form
//   score_k = x_n . c_k - ||c_k||^2 / 2.
// The B x N x K distance matrix is never written: point tiles and centroid
// tiles stream through on-chip memory and each point keeps a running
// (best score, best index) in registers ("flash-kmeans and the return of
// exact K-Means on the GPU", section "The point of the kernel is that the
// distance matrix never exists"; itinai.com summary, second paragraph;
// "Flash-KMeans: Implementação Exata de K-Means…", section "FlashAssign").
//
// Small-D path (d <= 512): a block owns WAVES waves x NF x 32 points whose
// fragments are loaded once into VGPRs; centroid tiles of TK rows are
// double-buffered through LDS. v_mfma_f32_32x32x16_{f16,bf16}: A = 32
// centroid rows from LDS, B = 32 points from registers, C-input = -||c||^2/2
// of those rows, so the accumulator is the score itself. Each lane holds 16
// centroid scores for one point; the running max stays in-lane across all
// tiles and one lane swap at the end merges the two lanes that share a point.
// The running max works on scores whose 4 low mantissa bits carry the row
// slot, so one v_max3 tree gives the maximum and where it is.
//
// fp32 inputs with d <= 256 run the same kernel on rows of 2d 16-bit units:
// every load and LDS copy moves bytes, so only the MFMA differs (four
// v_mfma_f32_32x32x2_f32 per 16-byte k-step, Mfma<FK_F32>).
//
// The split-D path (d > 512 units: fp16/bf16 d > 512, fp32 d > 256) lives in
// assign_splitd.hip.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "fk_internal.hpp"

namespace fk {
namespace {


// ===========================================================================
// small-D
// ===========================================================================
// Running argmax, per point fragment f, over the 16 scores a lane holds for
// one 32-row subtile (slot r = 0..15 holds row 8*(r/4) + 4*half + r%4 of the
// subtile). Each score's 4 low mantissa bits are replaced by 15 - r (one
// v_and_or_b32), so a single v_max3 tree yields the maximum and its slot:
//   m = max of the 16 coded scores;  if m > best: best = m, btile = subtile
// The code moves a score by less than 2^-19 of its magnitude, the size of
// the rounding of the fp32 accumulation over d products, so it only orders
// scores that agree to that precision; among those it prefers the lower row
// for positive scores and the higher row for negative ones. Across subtiles
// the strict '>' keeps the earlier subtile, and the two lane halves merge on
// (coded score, lowest row). Scores that must never win are -FLT_MAX (a
// finite value, so the code cannot turn it into a NaN).
struct Argmax {
  float best;
  int btile;
};

// Part `part` (0..7) of draining accumulator `acc` of subtile g into st.
// The work is split so it can be spread over the k-steps of the next
// subtile in even pieces: parts 0-6 code two or three scores each and fold
// them into the two partial maxima, part 7 compares. With 8 k-steps a
// subtile (d = 128) each k-step carries one part per fragment, so the VALU
// work under each pair of MFMAs stays the same size.
__device__ __forceinline__ void drain_part(const floatx16_t& acc, int part, int g, Argmax& st,
                                           float (&m)[2], bool& gt) {
  switch (part) {
    case 0:
      m[0] = vmax3(code_slot(acc[0], 0), code_slot(acc[1], 1), code_slot(acc[2], 2));
      break;
    case 1:
      m[1] = vmax3(code_slot(acc[3], 3), code_slot(acc[4], 4), code_slot(acc[5], 5));
      break;
    case 2:
      m[0] = vmax3(m[0], code_slot(acc[6], 6), code_slot(acc[7], 7));
      break;
    case 3:
      m[1] = vmax3(m[1], code_slot(acc[8], 8), code_slot(acc[9], 9));
      break;
    case 4:
      m[0] = vmax3(m[0], code_slot(acc[10], 10), code_slot(acc[11], 11));
      break;
    case 5:
      m[1] = vmax3(m[1], code_slot(acc[12], 12), code_slot(acc[13], 13));
      break;
    case 6: {
      const float c15 = code_slot(acc[15], 15);
      m[0] = vmax3(m[0], m[1], code_slot(acc[14], 14));
      m[0] = vmax3(m[0], c15, c15);
      break;
    }
    case 7:
      gt = m[0] > st.best;
      st.best = gt ? m[0] : st.best;
      st.btile = gt ? g : st.btile;
      break;
    default:
      break;
  }
}

// Row of the maximum, relative to the kernel's first row, for half `half`.
__device__ __forceinline__ int argmax_row(const Argmax& st, int half) {
  return st.btile * 32 + slot_row(slot_of(st.best)) + 4 * half;
}

// Persistent: a block walks point blocks v = blockIdx.x, + nblocks, ... of the
// virtual grid of `total` point blocks (each mapped through xcd_remap, and
// nblocks is a multiple of 8, so every point block a block takes shares its
// XCD's L2 with the ones it would have had as a plain launch). During the
// last centroid tile of one point block the block already stages tile 0 of
// the next and (8-wave blocks) loads the first half of the next block's
// point fragments into spare registers; the other half loads while the last
// argmax drains, so consecutive point blocks run back to back.
// FULL: d == 16*KS, so every column of a row is real and loads need no
// column guard; otherwise columns >= d read as zero.
template <int DT, int KS, int NF, int TK, int WAVES, bool VEC, bool FULL, bool RING>
__global__ __launch_bounds__(WAVES * 64) void assign_smalld_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ c,
    const float* __restrict__ cnorm, int32_t* __restrict__ ids, int N, int d, int K,
    int blocks_per_batch, int total, int nblocks) {
  constexpr int NT = WAVES * 64;         // threads per block
  constexpr int DP = KS * 16;            // padded dimension
  constexpr int PITCH = DP + 8;          // LDS row pitch (elements): +16 B against bank conflicts
  constexpr int NSUB = TK / 32;          // MFMA row blocks per tile
  constexpr int BN = WAVES * NF * 32;    // points per block
  constexpr int VPR = DP / 8;            // 16-byte vectors per centroid row
  constexpr int NV = (TK * VPR + NT - 1) / NT;   // vectors per thread per tile
  static_assert(NSUB % 2 == 0, "accumulator sets alternate by subtile");
  static_assert(TK <= NT, "one norm per thread");
  // k-steps of the next point block prefetched into registers during a
  // point block's last tile (8-wave blocks with whole rows only)
  constexpr int XP = (FULL && WAVES == 8) ? KS / 2 : 0;
  // RING: four tile buffers staged two tiles ahead, one barrier per two
  // tiles (needs at least two tiles per point block); else double buffering
  constexpr int NBUF = RING ? 4 : 2;
  __shared__ __align__(16) uint16_t lds_c[NBUF][TK * PITCH];
  __shared__ __align__(16) float lds_h[NBUF][NT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int half = lane >> 5, r32 = lane & 31;
  const int ntiles = (K + TK - 1) / TK;

  // Tail: when the last round of point blocks would leave at least half of
  // the blocks idle (r = total % nblocks, 0 < 2r <= nblocks), its r point
  // blocks become 2r half blocks: in each, the waves of one half do the
  // MFMA work for their rows and the other waves only help stage tiles, so
  // that round takes about half as long.
  const uint32_t rtail = (uint32_t)(total % nblocks);
  const bool split = WAVES == 8 && rtail > 0 && 2 * rtail <= (uint32_t)nblocks;
  const uint32_t nfull = split ? (uint32_t)total - rtail : (uint32_t)total;
  const uint32_t nitems = split ? (uint32_t)total + rtail : (uint32_t)total;
  // item v -> problem, this wave's first row, and whether the wave works on it
  auto locate = [&](uint32_t v, int& pb, int& row0, bool& act) {
    int64_t logical = 0;
    act = true;
    if (v < nfull) {
      logical = xcd_remap(v, nfull);
    } else {
      const int64_t hr = xcd_remap(v - nfull, 2 * rtail);
      logical = nfull + hr / 2;
      act = wave / (WAVES / 2) == (int)(hr % 2);
    }
    pb = __builtin_amdgcn_readfirstlane((int)(logical / blocks_per_batch));
    row0 = __builtin_amdgcn_readfirstlane((int)(logical % blocks_per_batch) * BN + wave * NF * 32);
  };
  // the lane's point row of fragment f; rows past N repeat row N-1 (their
  // results are never stored)
  auto point_row = [&](int pb, int row0, int f) -> const uint16_t* {
    return x + ((int64_t)pb * N + min(row0 + f * 32 + r32, N - 1)) * d;
  };
  auto load_frag = [&](const uint16_t* row, int s) -> uint4 {
    return FULL ? *reinterpret_cast<const uint4*>(row + s * 16 + half * 8)
                : load8<VEC>(row, s * 16 + half * 8, d);
  };

  // Tile loads: rows past K repeat row K-1 and get the never-winning norm term
  // (kNeverWins, finite so that the slot code stays a number), so they never
  // win. Loads and stores are unconditional (tile indices clamp, every
  // thread owns an lds_h slot) so one tile iteration is a single basic block
  // the scheduler can interleave.
  // Buffer resources over at most `cap` whole rows from base (the rows one
  // load instruction covers: a point fragment's 32, or a staging load's
  // NT / VPR): rows at or past the end of the data read as zero (a raw
  // buffer's range check) instead of being clamped, and the per-lane offsets
  // are constants of the kernel, so the loads cost no per-load 64-bit
  // address registers.
  auto rows_rsrc = [&](const void* base, int rows_left, int row_bytes, int cap) {
    const int n = min(max(rows_left, 0), cap) * row_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), 0,
                                             __builtin_amdgcn_readfirstlane(n), kRawBufferWord3);
  };
  uint4 pre[NV];
  float pre_n = 0.f;
  auto fetch = [&](int pb, int t) {
    const uint16_t* cb = c + (int64_t)pb * K * d;
    if constexpr (FULL && TK * VPR % NT == 0 && NT % VPR == 0) {
      const uint32_t cvo = (uint32_t)((tid / VPR) * d + (tid % VPR) * 8) * 2;
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int r0 = t * TK + q * (NT / VPR);
        pre[q] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       rows_rsrc(cb + (int64_t)r0 * d, K - r0, d * 2, NT / VPR), cvo, 0, 0));
      }
    } else {
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int v = tid + NT * q;
        if (TK * VPR % NT == 0 || v < TK * VPR) {
          const int row = v / VPR, col = (v % VPR) * 8;
          const int k = min(t * TK + row, K - 1);
          pre[q] = FULL ? *reinterpret_cast<const uint4*>(cb + (int64_t)k * d + col)
                        : load8<VEC>(cb + (int64_t)k * d, col, d);
        }
      }
    }
    pre_n = cnorm[(int64_t)pb * K + min(t * TK + (tid % TK), K - 1)];
  };
  auto stash = [&](int t, int buf) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = tid + NT * q;
      if (TK * VPR % NT == 0 || v < TK * VPR) {
        const int row = v / VPR, col = (v % VPR) * 8;
        *reinterpret_cast<uint4*>(&lds_c[buf][row * PITCH + col]) = pre[q];
      }
    }
    lds_h[buf][tid] = (t * TK + tid < K) ? -0.5f * pre_n : kNeverWins;
  };

  // LDS operands of a step, read ahead of use: A fragments two k-steps ahead
  // (ring of three), C inputs (-||c||^2/2 of the lane's rows) one subtile
  // ahead (two sets, alternating by subtile).
  constexpr int STEPS = NSUB * KS;              // k-steps per tile
  constexpr int PARTS = 8 * NF;                 // drain parts per subtile
  constexpr int PPS = (PARTS + KS - 1) / KS;    // drain parts per k-step
  auto read_a = [&](int buf, int q) -> uint4 {
    const int sub = q / KS, kk = q % KS;
    return *reinterpret_cast<const uint4*>(
        &lds_c[buf][(sub * 32 + r32) * PITCH + half * 8 + kk * 16]);
  };
  auto read_c = [&](int buf, int sub, floatx16_t& ci) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 hv =
          *reinterpret_cast<const float4*>(&lds_h[buf][sub * 32 + 8 * i + 4 * half]);
      ci[4 * i + 0] = hv.x;
      ci[4 * i + 1] = hv.y;
      ci[4 * i + 2] = hv.z;
      ci[4 * i + 3] = hv.w;
    }
  };

  uint4 xf[NF][KS];
  Argmax st[NF];
  // Two accumulator sets alternate by subtile: while the MFMAs of subtile g
  // fill one set, the argmax of subtile g-1 drains the other, spread over the
  // k-steps, so VALU work issues in the shadow of the matrix core. The first
  // drain of a point block is of an all-kNeverWins set standing for subtile -1.
  floatx16_t acc[2][NF];

  // The switch to the next point block: its first XP k-steps are loaded
  // into spare registers at the start of the current block's last tile, a
  // whole tile ahead of use, so at the switch only the remaining k-steps
  // come from HBM, and those are first needed XP k-steps into the new
  // block's first subtile.
  const uint32_t xvo = (uint32_t)(r32 * d + half * 8) * 2;   // lane's bytes within a fragment
  auto frag_rsrc = [&](int pb, int row0, int f) {
    return rows_rsrc(x + ((int64_t)pb * N + row0 + f * 32) * d, N - (row0 + f * 32), d * 2, 32);
  };
  uint4 xn[NF][XP > 0 ? XP : 1];
  auto prefetch_x = [&](int pb, int row0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const auto rs = frag_rsrc(pb, row0, f);
#pragma unroll
      for (int s = 0; s < XP; ++s)
        xn[f][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, xvo + s * 32, 0, 0));
    }
  };

  // One centroid tile from LDS buffer buf.
  auto tile = [&](int buf, int t) {
    floatx16_t ci;
    uint4 ar[3];
    read_c(buf, 0, ci);
    ar[0] = read_a(buf, 0);
    ar[1] = read_a(buf, 1 % STEPS);
    float m[NF][2];
    bool gt[NF];
#pragma unroll
    for (int q = 0; q < STEPS; ++q) {
      const int sub = q / KS, kk = q % KS;
      const int g = t * NSUB + sub;          // subtile index within the point block
      floatx16_t (&cur)[NF] = acc[sub & 1];
      const floatx16_t (&prev)[NF] = acc[(sub + 1) & 1];
      if (q + 2 < STEPS) ar[(q + 2) % 3] = read_a(buf, q + 2);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        cur[f] = Mfma<DT>::run(ar[q % 3], xf[f][kk], kk == 0 ? ci : cur[f]);
      if (kk == 0 && sub + 1 < NSUB) read_c(buf, sub + 1, ci);
#pragma unroll
      for (int p = kk * PPS; p < (kk + 1) * PPS && p < PARTS; ++p)
        drain_part(prev[p % NF], p / NF, g - 1, st[p % NF], m[p % NF], gt[p % NF]);
      // keep program order across steps: the reads above stay ahead of use
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto reset = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      st[f].best = -INFINITY;
      st[f].btile = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][f][r] = kNeverWins;
    }
  };
  auto load_block = [&](int pb, int row0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint16_t* row = point_row(pb, row0, f);
#pragma unroll
      for (int s = 0; s < KS; ++s) xf[f][s] = load_frag(row, s);
    }
  };
  auto load_block_next = [&](int pb, int row0) {
    if constexpr (XP > 0) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const auto rs = frag_rsrc(pb, row0, f);
#pragma unroll
        for (int s = XP; s < KS; ++s)
          xf[f][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, xvo + s * 32, 0, 0));
#pragma unroll
        for (int s = 0; s < XP; ++s) xf[f][s] = xn[f][s];
      }
    } else {
      load_block(pb, row0);
    }
  };

  // item indices stay below 2 * total < 2^32
  uint32_t v = blockIdx.x;
  int pb, row0;
  bool act;
  locate(v, pb, row0, act);
  // the next point block, or this one again past the end (its loads and
  // tile-0 stage are then harmless repeats that nothing reads)
  uint32_t vn = v + (uint32_t)nblocks;
  int npb = pb, nrow0 = row0;
  bool nact = act;
  if (vn < nitems) locate(vn, npb, nrow0, nact);
  load_block(pb, row0);
  fetch(pb, 0);
  stash(0, 0);
  if constexpr (RING) {
    fetch(pb, 1);
    stash(1, 1);
  }
  reset();
  __syncthreads();
  int buf = 0, t = 0;
  uint32_t it = 0;   // tiles done by the block
  for (;;) {
    // one centroid tile; the tile staged meanwhile is the next one (RING:
    // the one after next) in the stream of this point block's tiles followed
    // by the next point block's
    const bool last = t == ntiles - 1;
    const int ahead = t + (RING ? 2 : 1);
    const bool in_next = ahead >= ntiles;
    const int ft = in_next ? ahead - ntiles : ahead;
    fetch(in_next ? npb : pb, ft);
    if (XP > 0 && last) prefetch_x(npb, nrow0);
    // the MFMA phase at raised wave priority: where the two waves of a SIMD
    // are out of step, the one still in its tile issues ahead of the one
    // staging and about to wait at the barrier
    __builtin_amdgcn_s_setprio(1);
    if (act) tile(buf, t);
    __builtin_amdgcn_s_setprio(0);
    stash(ft, RING ? (buf + 2) & 3 : buf ^ 1);
    if (last) {
      // the next point block's fragments first (the rest of its k-steps
      // load while this one's final subtile drains), then this one's ids
      int32_t* ib = ids + (int64_t)pb * N;
      const int g = ntiles * NSUB - 1;       // the last subtile, still in acc[1]
      float m[NF][2];
      bool gt[NF];
      load_block_next(npb, nrow0);
#pragma unroll
      for (int p = 0; p < 8 * NF; ++p)
        drain_part(acc[1][p % NF], p / NF, g, st[p % NF], m[p % NF], gt[p % NF]);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int idx = merge_halves(st[f].best, argmax_row(st[f], half) - 4 * half, half);
        const int n = row0 + f * 32 + r32;
        if (act && half == 0 && n < N) ib[n] = min(max(idx, 0), K - 1);
      }
      reset();
    }
    // RING: a buffer is restaged two tiles after it was read, and the
    // barrier after every odd tile separates each such read from the write
    // and each write from its read
    if (!RING || (it & 1)) __syncthreads();
    ++it;
    buf = RING ? (buf + 1) & 3 : buf ^ 1;
    if (!last) {
      ++t;
      continue;
    }
    if (vn >= nitems) break;
    v = vn;
    pb = npb;
    row0 = nrow0;
    act = nact;
    vn = v + (uint32_t)nblocks;
    if (vn < nitems) locate(vn, npb, nrow0, nact);
    t = 0;
  }
}

// ===========================================================================
// dispatch
// ===========================================================================
// 16-byte vector loads need rows of whole 8-element vectors and aligned bases.
bool vec_ok(const void* x, const void* c, int64_t d) {
  return d % 8 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)c % 16) == 0;
}

// Blocks of kernel `kern` that fit on the current device at once (resident
// blocks per CU times the CU count), cached per device in `cache` (one cache
// per kernel instance; 0 = not yet queried).
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

template <int DT, int KS, int NF, int TK, int WAVES, bool VEC, bool FULL, bool RING>
hipError_t launch_smalld(const uint16_t* x, const uint16_t* c, const float* cn, int64_t total,
                         int bpb, int64_t N, int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  static int cache[64];
  auto kern = assign_smalld_kernel<DT, KS, NF, TK, WAVES, VEC, FULL, RING>;
  const int resident = resident_blocks(kern, WAVES * 64, cache);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  // a multiple of 8 so each block's point blocks stay on its XCD
  int64_t nblocks = resident >= 8 ? resident / 8 * 8 : resident;
  if (nblocks > total) nblocks = total;
  return launch_timed(kern, dim3((unsigned)nblocks), dim3(WAVES * 64), s, x, c, cn, ids, (int)N,
                      (int)d, (int)K, bpb, (int)total, (int)nblocks);
}

template <int DT, int KS, int NF, int TK, int WAVES>
hipError_t run_smalld(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                      int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  constexpr int BN = WAVES * NF * 32;
  const int bpb = (int)((N + BN - 1) / BN);
  const int64_t total = B * bpb;
  if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* cp = (const uint16_t*)c;
  if constexpr (TK == 128 && WAVES == 8) {   // the ring needs two tiles per point block
    if (vec_ok(x, c, d) && d == 16 * KS && K > TK)
      return launch_smalld<DT, KS, NF, TK, WAVES, true, true, true>(xp, cp, cn, total, bpb, N, d, K,
                                                                     ids, s);
  }
  if (vec_ok(x, c, d) && d == 16 * KS)
    return launch_smalld<DT, KS, NF, TK, WAVES, true, true, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if (vec_ok(x, c, d))
    return launch_smalld<DT, KS, NF, TK, WAVES, true, false, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  return launch_smalld<DT, KS, NF, TK, WAVES, false, false, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
}

// Tile candidates for rows of up to 128 16-bit units (k-steps KS, two point
// fragments per wave): 8-wave blocks with 128-row centroid tiles (a ring of
// four tile buffers once a point block has two tiles or more), 4-wave blocks
// with 128-row tiles, 4-wave blocks with 64-row tiles. Eight waves share each
// staged tile among 512 points, half the staging work per MFMA of four; four
// waves make twice as many point blocks, which fills the GPU when there are
// few points.
enum SmallTile { kTile8w128 = 0, kTile4w128 = 1, kTile4w64 = 2, kSmallTiles = 3 };
const char* const kSmallTileNames[kSmallTiles] = {"8w128", "4w128", "4w64"};

template <int DT, int KS>
hipError_t run_small_tile(int tile, const void* x, const void* c, const float* cn, int64_t B,
                          int64_t N, int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  if (tile == kTile4w128) return run_smalld<DT, KS, 2, 128, 4>(x, c, cn, B, N, d, K, ids, s);
  if (tile == kTile4w64) return run_smalld<DT, KS, 2, 64, 4>(x, c, cn, B, N, d, K, ids, s);
  return run_smalld<DT, KS, 2, 128, 8>(x, c, cn, B, N, d, K, ids, s);
}

// The tile a problem shape gets (rows of `units` 16-bit units, units <= 128),
// read off the timing sweep of every candidate over d in {32, 64, 128}, K in
// {64 .. 4096} and 16K .. 2.4M points (bench.py --tile-sweep):
//   - 128-unit rows: 64-row tiles for K <= 64 (a 128-row tile would be half
//     padding: 2-12% faster); else 8-wave blocks once their 512-point blocks
//     cover every CU; with fewer points, 4-wave blocks with 128-row tiles
//     (twice the blocks: up to 1.4x faster at 16K-64K points);
//   - 64-unit rows: 64-row tiles for K < 256; above, 128-row 4-wave tiles,
//     8-wave blocks only for K >= 1024 with 512-point blocks on at least
//     twice the CUs (within 5% of each other there);
//   - 32-unit rows: 64-row tiles for K < 256, 128-row 4-wave tiles above
//     (up to 1.3x at K = 4096).
// FK_TILE=<name> forces a candidate.
int small_tile(int64_t units, int64_t K, int64_t B, int64_t N) {
  if (const char* e = getenv("FK_TILE")) {
    for (int i = 0; i < kSmallTiles; ++i)
      if (strcmp(e, kSmallTileNames[i]) == 0) return i;
  }
  const int64_t blocks8 = B * ((N + 511) / 512);    // point blocks of the 8-wave tile
  const int64_t cus = device_cus() > 0 ? device_cus() : 256;
  if (units > 64) return K <= 64 ? kTile4w64 : (blocks8 >= cus ? kTile8w128 : kTile4w128);
  if (K < 256) return kTile4w64;
  if (units > 32 && K >= 1024 && blocks8 >= 2 * cus) return kTile8w128;
  return kTile4w128;
}

// Shapes per d: k-steps KS (16 elements each), point fragments NF per wave,
// tile rows TK, waves per block; rows of up to 128 units take the tile the
// table above picks.
template <int DT>
hipError_t smalld_dt(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                     int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  if (d <= 128) {
    const int tile = small_tile(d, K, B, N);
    if (d <= 32) return run_small_tile<DT, 2>(tile, x, c, cn, B, N, d, K, ids, s);
    if (d <= 64) return run_small_tile<DT, 4>(tile, x, c, cn, B, N, d, K, ids, s);
    return run_small_tile<DT, 8>(tile, x, c, cn, B, N, d, K, ids, s);
  }
  if (d <= 256) return run_smalld<DT, 16, 2, 64, 4>(x, c, cn, B, N, d, K, ids, s);
  if (d <= 512) return run_smalld<DT, 32, 1, 64, 4>(x, c, cn, B, N, d, K, ids, s);
  return hipErrorNotSupported;
}

}  // namespace

int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0 &&
      hipDeviceGetAttribute(&cache[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cache[dev] = 0;
  return cache[dev];
}

// The small-D tiles fit LDS for every d <= 512 16-bit units (largest:
// 2 x 32 x 520 x 2 B); an fp32 row of d elements is 2d units.
bool smalld_supported(int dt, int64_t d) {
  return ((dt == FK_F16 || dt == FK_BF16) && d <= 512) || (dt == FK_F32 && d <= 256);
}

hipError_t launch_assign_smalld(const void* x, const void* c_lp, const float* cnorm, int dt,
                                int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                                hipStream_t s) {
  if (B == 0 || N == 0) return hipSuccess;
  if (K < 1) return hipErrorInvalidValue;    // the point-block loop needs a tile
  if (dt == FK_F16) return smalld_dt<FK_F16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  if (dt == FK_BF16) return smalld_dt<FK_BF16>(x, c_lp, cnorm, B, N, d, K, ids, s);
  if (dt == FK_F32 && d <= 256)     // rows of 2d 16-bit units
    return smalld_dt<FK_F32>(x, c_lp, cnorm, B, N, 2 * d, K, ids, s);
  return hipErrorNotSupported;
}

}  // namespace fk
