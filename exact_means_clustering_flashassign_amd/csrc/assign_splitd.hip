// FlashAssign for large d (d > 512; fp32 d > 256) on gfx950: outer K loop,
// inner D loop.
//
// Same contraction and argmax as the small-D path (score_k = x.c_k -
// ||c_k||^2 / 2; the distance matrix is never written; the register-staged
// kernel keeps the lowest k on exact ties, the LDS-staged one orders scores
// that agree to the fp32 rounding by a slot code, as small-D does), but
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
#include <stdlib.h>
#include <string.h>

#include <type_traits>

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

// The LDS-staged kernel's argmax over one K tile, slot-coded as in the
// small-D path: each accumulator's 16 scores x.c - ||c||^2/2 (one fma on the
// accumulator and the staged norm) get their slot in the 4 low mantissa bits,
// one v_max3 tree gives the lane's best of the 16 and its slot, and a strict
// '>' against the running best keeps the earlier row block. The code moves a
// score by less than 2^-19 of its magnitude, so it only orders scores that
// agree to the fp32 rounding of the accumulation; among those the row is
// either one. GUARD: the tile runs past K, and rows at or past K (zero rows
// and zero norms in LDS) are set to a score that never wins.
template <int NSUB, bool GUARD>
__device__ __forceinline__ void drain_tile_coded(const floatx16_t (&acc)[NSUB][kNF],
                                                 const float* __restrict__ hrow, int left0,
                                                 int base, float (&best)[kNF], int (&bt)[kNF]) {
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    float hv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(hrow + sub * 32 + 8 * i);
      hv[4 * i + 0] = v.x;
      hv[4 * i + 1] = v.y;
      hv[4 * i + 2] = v.z;
      hv[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      float sc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // -0.5 * ||c||^2 is exact, so the fma rounds once, as the sum did
        const float v = __builtin_fmaf(hv[r], -0.5f, acc[sub][f][r]);
        sc[r] = code_slot(GUARD && sub * 32 + 8 * (r >> 2) + (r & 3) >= left0 ? kNeverWins : v, r);
      }
      float m0 = vmax3(sc[0], sc[1], sc[2]);
      float m1 = vmax3(sc[3], sc[4], sc[5]);
      m0 = vmax3(m0, sc[6], sc[7]);
      m1 = vmax3(m1, sc[8], sc[9]);
      m0 = vmax3(m0, sc[10], sc[11]);
      m1 = vmax3(m1, sc[12], sc[13]);
      m0 = vmax3(m0, m1, sc[14]);
      m0 = vmax3(m0, sc[15], sc[15]);
      const bool gt = m0 > best[f];
      best[f] = gt ? m0 : best[f];
      bt[f] = gt ? base + sub * 32 : bt[f];
    }
    __builtin_amdgcn_sched_barrier(0);
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

// ---------------------------------------------------------------------------
// Direct-to-LDS staging, for whole rows (16-byte aligned, d a multiple of
// 128). Same tiles, accumulators and argmax as above, but both operands go
// from memory straight into LDS with 16-byte buffer loads that write LDS,
// and both MFMA operands are read from LDS:
//   - d-chunks of 64 (4 k-steps); a staged load writes 64 consecutive
//     16-byte slots, i.e. whole rows, so the point rows stream in whole
//     cache lines (a register load of an MFMA fragment touches 32 rows at 32
//     bytes each, and those partial-line requests, not HBM, were the limit);
//   - centroid chunks are double-buffered and shared by the block; each wave
//     stages its own 64 point rows into a ring of four half-chunk slots (two
//     k-steps each), refilled as soon as the wave has read a slot, so a
//     point load has about 1.5 chunks to land;
//   - a wave's memory loads retire in issue order: each chunk issues the next
//     chunk's centroid loads first, and just before the chunk's closing
//     barrier the wave waits until only the point loads issued after them
//     are outstanding.
// Rows are stored unpadded (a staged load fills whole rows) with their
// 16-byte units permuted by an XOR of the row index, so the fragment reads
// (consecutive rows, one unit) fall on distinct banks. Every slot and buffer
// is its own LDS array and the chunk loop is unrolled by two, so each read
// names its array at compile time and the compiler's wait before a read
// covers only the loads into that array.
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate: at most vm vector-memory and lgkm LDS/scalar
// operations outstanding (expcnt not waited on).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

constexpr int kLC = 64;                         // d-chunk of the LDS-staged kernel
constexpr int kLKS = kLC / 16;                  // k-steps per chunk
constexpr int kCRowB = kLC * 2;                 // bytes of a staged centroid row (128)
constexpr int kXRowB = kLC;                     // bytes of a staged half-chunk point row (64)
constexpr int kWaveRows = kNF * 32;             // point rows per wave
constexpr int kXSlotB = kWaveRows * kXRowB;     // bytes of one wave's half-chunk slot (4 KB)

// unit permutations: centroid row r keeps unit u (of 8) at u ^ cperm(r),
// point row r keeps unit u (of 4) at u ^ xperm(r)
__device__ __forceinline__ int cperm(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int xperm(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <int DT, int NSUB>
__global__ __launch_bounds__(kThreads) void assign_splitd_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ c,
    const float* __restrict__ cnorm, int32_t* __restrict__ ids, int N, int d, int K,
    int blocks_per_batch, int total, int nblocks) {
  constexpr int TK = NSUB * 32;                   // centroids per K tile
  constexpr int CTILEB = TK * kCRowB;             // bytes of a staged centroid chunk
  constexpr int RPW = TK / kWaves;                // centroid rows staged per wave
  constexpr int NCL = RPW / 8;                    // centroid loads per thread (8 rows each)
  constexpr int NXL = kWaveRows / 16;             // point loads per half-chunk (16 rows each)
  constexpr int Q = NSUB * kLKS;                  // (row block, k-step) pairs per chunk
  static_assert(RPW % 8 == 0 && TK <= kThreads, "staging split");
  __shared__ __align__(256) unsigned char cs0[CTILEB];
  __shared__ __align__(256) unsigned char cs1[CTILEB];
  __shared__ __align__(256) unsigned char xs0[kWaves * kXSlotB];   // even chunks, k-steps 0-1
  __shared__ __align__(256) unsigned char xs1[kWaves * kXSlotB];   // even chunks, k-steps 2-3
  __shared__ __align__(256) unsigned char xs2[kWaves * kXSlotB];   // odd chunks, k-steps 0-1
  __shared__ __align__(256) unsigned char xs3[kWaves * kXSlotB];   // odd chunks, k-steps 2-3
  __shared__ __align__(16) float lds_h[2][kWaves * 64];   // ||c||^2 by K-tile parity

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, r32 = lane & 31;
  const int nchunks = d / kLC;                    // even
  const int ktiles = (K + TK - 1) / TK;
  const int T = ktiles * nchunks;                 // chunks per point block
  const uint32_t rowb = (uint32_t)d * 2;          // bytes per row in HBM

  // point block v -> problem, first row, and the rotation of its d-chunk
  // order: blocks running at the same time read different column slices of
  // their rows, so their requests spread over the memory channels instead of
  // all hitting the few that hold one slice
  auto locate = [&](int64_t v, int& pb, int& row0, int& rot) {
    const int64_t logical = xcd_remap(v, total);
    pb = __builtin_amdgcn_readfirstlane((int)(logical / blocks_per_batch));
    row0 = __builtin_amdgcn_readfirstlane((int)(logical % blocks_per_batch) * kBN);
    rot = __builtin_amdgcn_readfirstlane((int)(logical % nchunks));
  };

  // Centroid chunk t of (problem pb) into dst: load j of wave w fills rows
  // w*RPW + 8j .. +7; lane l writes slot l % 8 of row 8j + l / 8, i.e. unit
  // (l % 8) ^ cperm(row). Rows past K lie past the buffer's range and read as
  // zero, as do their norms; the argmax of a tile that runs past K masks
  // them, so they never win.
  // Loads jlo .. jhi-1 of the chunk (and, with norm, the norms' load), so a
  // chunk's staging can be issued a few loads at a time between its MFMAs.
  auto stage_c = [&](unsigned char* dst, float* hdst, int pb, int rot, int t, int jlo, int jhi,
                     bool norm) {
    const int kt = t / nchunks;
    int ch = t - kt * nchunks + rot;
    ch = ch >= nchunks ? ch - nchunks : ch;
    const int rows = min(K - kt * TK, TK);
    const uint16_t* tb = c + ((int64_t)pb * K + (int64_t)kt * TK) * d;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(tb), 0, __builtin_amdgcn_readfirstlane(rows * (int)rowb), kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < NCL; ++j) {
      if (j < jlo || j >= jhi) continue;
      const int row = wave * RPW + 8 * j + (lane >> 3);
      const uint32_t voff = (uint32_t)row * rowb + (uint32_t)(ch * kCRowB) +
                            (uint32_t)(((lane & 7) ^ cperm(row)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void_t*)(dst + (wave * RPW + 8 * j) * kCRowB), 16, voff, 0, 0, 0);
    }
    // ||c||^2 of rows kt*TK + wave*64 + lane into hdst (64 per wave, so
    // every wave issues the same loads; rows past K read as zero and rows
    // past the tile are never used). Every chunk stages the norms of its
    // successor's K tile into the slot of the next tile, which only the next
    // tile's start reads.
    if (norm) {
      const auto rn = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(cnorm + (int64_t)pb * K), 0, __builtin_amdgcn_readfirstlane(K * 4),
          kRawBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rn, (lds_void_t*)(hdst + wave * 64), 4, (uint32_t)(kt * TK + lane) * 4 + wave * 256, 0,
          0, 0);
    }
  };
  // Half hh (k-steps 2hh, 2hh+1) of point chunk t of the wave's 64 rows
  // (from row0 + wave*64) into the wave's part of slot array dst: load j
  // fills rows 16j .. 16j+15; lane l writes slot l % 4 of row 16j + l / 4,
  // i.e. unit (l % 4) ^ xperm(row). Rows past N read as zero (their ids are
  // never stored).
  auto stage_x = [&](unsigned char* dst, int pb, int row0, int rot, int t, int hh, int jlo,
                     int jhi) {
    int ch = t % nchunks + rot;
    ch = ch >= nchunks ? ch - nchunks : ch;
    const int r0 = row0 + wave * kWaveRows;
    const uint16_t* xb = x + ((int64_t)pb * N + r0) * d;
    const int rows = min(max(N - r0, 0), kWaveRows);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(xb), 0, __builtin_amdgcn_readfirstlane(rows * (int)rowb), kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < NXL; ++j) {
      if (j < jlo || j >= jhi) continue;
      const int row = 16 * j + (lane >> 2);
      const uint32_t voff = (uint32_t)row * rowb + (uint32_t)(ch * kCRowB + hh * kXRowB) +
                            (uint32_t)(((lane & 3) ^ xperm(row)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void_t*)(dst + wave * kXSlotB + 16 * j * kXRowB), 16, voff, 0, 0, 0);
    }
  };

  // A fragment of (row block sub, k-step kk): lane (r32, half) reads unit
  // 2kk + half of centroid row sub*32 + r32, at byte
  // sub*32*128 + (a_lane[sub & 1] ^ (kk * 32)).
  const uint32_t a_lane0 = (uint32_t)r32 * kCRowB + (uint32_t)((half ^ cperm(r32)) * 16);
  const uint32_t a_lane1 = (uint32_t)r32 * kCRowB + (uint32_t)((half ^ cperm(32 + r32)) * 16);
  auto read_a = [&](const unsigned char* buf, int q) -> uint4 {
    const int sub = q % NSUB, kk = q / NSUB;
    return *reinterpret_cast<const uint4*>(
        buf + (((sub & 1 ? a_lane1 : a_lane0) ^ (uint32_t)(kk << 5)) +
               (uint32_t)(sub * 32 * kCRowB)));
  };
  // B fragment f of k-step kk (within its half-chunk slot): lane (r32, half)
  // reads unit 2(kk % 2) + half of the wave's point row f*32 + r32.
  const uint32_t b_lane = (uint32_t)wave * kXSlotB + (uint32_t)r32 * kXRowB +
                          (uint32_t)((half ^ xperm(r32)) * 16);
  auto read_b = [&](const unsigned char* slot, int f, int kk) -> uint4 {
    return *reinterpret_cast<const uint4*>(
        slot + ((b_lane ^ (uint32_t)((kk & 1) << 5)) + (uint32_t)(f * 32 * kXRowB)));
  };

  floatx16_t acc[NSUB][kNF];
  float best[kNF];
  int bidx[kNF];

  int64_t v = blockIdx.x;
  int pb, row0, rot;
  locate(v, pb, row0, rot);
  int64_t vn = v + nblocks;
  int npb = pb, nrow0 = row0, nrot = rot;
  if (vn < total) locate(vn, npb, nrow0, nrot);
  bool has_next = vn < total;

  // prologue: centroid chunk 0, point chunk 0 (both halves), point chunk 1's
  // first half (a chunk issues its successor's second half and the first
  // half of the chunk after that)
  stage_c(cs0, lds_h[0], pb, rot, 0, 0, NCL, true);
  stage_x(xs0, pb, row0, rot, 0, 0, 0, NXL);
  stage_x(xs1, pb, row0, rot, 0, 1, 0, NXL);
  stage_x(xs2, pb, row0, rot, 1, 0, 0, NXL);       // every point block has T >= 2 chunks
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  __syncthreads();

  int tc = 0;                                     // K tiles started by this block
  for (;;) {
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      best[f] = -INFINITY;
      bidx[f] = 0;
    }
    for (int kt = 0; kt < ktiles; ++kt) {
      // accumulators start at zero; the argmax adds -||c||^2/2 of the rows
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int f = 0; f < kNF; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[sub][f][r] = 0.f;
      // Chunk t of the current point block, of parity P (every K tile has
      // an even number of chunks, so the parity loop, unrolled, names every
      // buffer at compile time): read centroids from cs[P] and points from
      // xs[2P], xs[2P+1]; meanwhile stage the next step's centroid chunk and
      // second point half, and the step after next's first point half. Past
      // the last point block the staging repeats data that nothing reads.
      for (int ch = 0; ch < nchunks; ch += 2) {
#pragma unroll
        for (int P = 0; P < 2; ++P) {
          const int t = kt * nchunks + ch + P;
          const unsigned char* cc = P ? cs1 : cs0;
          unsigned char* cn = P ? cs0 : cs1;
          const unsigned char* xh0 = P ? xs2 : xs0;
          const unsigned char* xh1 = P ? xs3 : xs1;
          unsigned char* xn1 = P ? xs1 : xs3;        // step + 1, second half
          // step + 1 and step + 2: (point block, chunk)
          const bool s1_in = t + 1 < T, s1_nx = !s1_in && has_next;
          const int s1_pb = s1_nx ? npb : pb;
          const int s1_row0 = s1_nx ? nrow0 : row0;
          const int s1_rot = s1_nx ? nrot : rot;
          const int s1_t = s1_in ? t + 1 : (has_next ? 0 : t);
          const bool s2_in = t + 2 < T, s2_nx = !s2_in && has_next;
          const int s2_pb = s2_nx ? npb : pb;
          const int s2_row0 = s2_nx ? nrow0 : row0;
          const int s2_rot = s2_nx ? nrot : rot;
          const int s2_t = s2_in ? t + 2 : (has_next ? t + 2 - T : t);
          // The staging of this chunk is issued one load per (row block,
          // k-step) pair, between the MFMAs, so the four waves do not queue
          // all their loads at the address unit at once after the barrier:
          //   q in [0, NCL):               step + 1's centroid rows (load q;
          //                                the norms with load 0),
          //   q in [NSUB, NSUB + NXL):     step + 1's second point half,
          //   q in [2NSUB, 2NSUB + NXL):   step + 2's first point half (k-steps
          //                                0-1 are done: their slot is free).
          // (NCL == NSUB and NXL <= NSUB, so the three ranges are disjoint.)
          static_assert(NCL == NSUB && NXL <= NSUB, "staging issue order");
          uint4 ar[4], br[2][kNF];
          ar[0] = read_a(cc, 0);
          ar[1] = read_a(cc, 1);
          ar[2] = read_a(cc, 2);
#pragma unroll
          for (int f = 0; f < kNF; ++f) br[0][f] = read_b(xh0, f, 0);
#pragma unroll
          for (int q = 0; q < Q; ++q) {
            const int sub = q % NSUB, kk = q / NSUB;
            if (sub == 0 && kk + 1 == 2) {
              // this chunk's second point half was staged during the
              // previous chunk; the loads issued since (the first half of
              // the next chunk, then, in this chunk, the next chunk's
              // centroids and norms) may still be in flight
              asm volatile("" ::: "memory");
              __builtin_amdgcn_s_waitcnt(waitcnt_imm(NXL + NCL + 1, 15));
              asm volatile("" ::: "memory");
            }
            if (sub == 0 && kk + 1 < kLKS) {           // the next k-step's point fragments
#pragma unroll
              for (int f = 0; f < kNF; ++f)
                br[(kk + 1) & 1][f] = read_b(kk + 1 < 2 ? xh0 : xh1, f, kk + 1);
            }
            if (q + 3 < Q) ar[(q + 3) % 4] = read_a(cc, q + 3);
#pragma unroll
            for (int f = 0; f < kNF; ++f)
              acc[sub][f] = Mfma<DT>::run(ar[q % 4], br[kk & 1][f], acc[sub][f]);
            __builtin_amdgcn_sched_barrier(0);
            if (q < NCL)
              stage_c(cn, lds_h[(tc + 1) & 1], s1_pb, s1_rot, s1_t, q, q + 1, q == 0);
            else if (q >= NSUB && q < NSUB + NXL)
              stage_x(xn1, s1_pb, s1_row0, s1_rot, s1_t, 1, q - NSUB, q - NSUB + 1);
            else if (q >= 2 * NSUB && q < 2 * NSUB + NXL)
              stage_x(P ? xs2 : xs0, s2_pb, s2_row0, s2_rot, s2_t, 0, q - 2 * NSUB,
                      q - 2 * NSUB + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
          // This wave's centroid and norm loads have landed once at most the
          // 2 * NXL point loads issued after them are outstanding. The
          // barrier has no memory fence (a fence would also wait for those
          // point loads); the empty asm statements keep the compiler from
          // moving LDS accesses across it.
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * NXL, 0));
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
        }
      }
      // scores x.c - ||c||^2/2, then the running argmax (rows of the lane
      // relative to the tile: sub*32 + 8i + 4*half + j; those at or past
      // K - kt*TK never win)
      {
        const float* hrow = &lds_h[tc & 1][4 * half];
        const int left0 = K - kt * TK - 4 * half;
        if (kt * TK + TK <= K)
          drain_tile_coded<NSUB, false>(acc, hrow, left0, kt * TK, best, bidx);
        else
          drain_tile_coded<NSUB, true>(acc, hrow, left0, kt * TK, best, bidx);
      }
      ++tc;
    }
    int32_t* ib = ids + (int64_t)pb * N;
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const int idx = merge_halves(best[f], bidx[f] + slot_row(slot_of(best[f])), half);
      const int n = row0 + wave * kWaveRows + f * 32 + r32;
      if (half == 0 && n < N) ib[n] = idx;
    }
    if (!has_next) {
      // the repeated staging loads of the last chunks still write LDS: let
      // them land before the block ends
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      break;
    }
    v = vn;
    pb = npb;
    row0 = nrow0;
    rot = nrot;
    vn = v + nblocks;
    has_next = vn < total;
    if (has_next) locate(vn, npb, nrow0, nrot);
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
  return launch_timed(kern, dim3((unsigned)nblocks), dim3(kThreads), s, x, c, cn, ids, (int)N,
                      (int)d, (int)K, bpb, (int)total, (int)nblocks);
}

template <int DT, int NSUB>
hipError_t launch_splitd_lds(const uint16_t* x, const uint16_t* c, const float* cn, int64_t total,
                             int bpb, int64_t N, int64_t d, int64_t K, int32_t* ids,
                             hipStream_t s) {
  static int cache[64];
  auto kern = assign_splitd_lds_kernel<DT, NSUB>;
  const int resident = resident_blocks(kern, kThreads, cache);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  int64_t nblocks = resident >= 8 ? resident / 8 * 8 : resident;
  if (nblocks > total) nblocks = total;
  return launch_timed(kern, dim3((unsigned)nblocks), dim3(kThreads), s, x, c, cn, ids, (int)N,
                      (int)d, (int)K, bpb, (int)total, (int)nblocks);
}

// Split-D tile candidates: the centroid tile (256 or 128 rows) and the
// staging (straight into LDS, for whole rows with d a multiple of 128; else
// through registers). FK_TILE=<name> forces one (where it applies);
// FK_SPLITD_REGISTER_STAGING=1 keeps whole-row problems on register staging.
enum SplitTile { kSplitLds8 = 0, kSplitLds4 = 1, kSplitReg8 = 2, kSplitReg4 = 3, kSplitTiles = 4 };
const char* const kSplitTileNames[kSplitTiles] = {"lds8", "lds4", "reg8", "reg4"};

// The staging and tile rows a problem gets, read off the timing sweep of
// the four candidates over d in {768, 1024}, K in {64, 256, 1000} and 16K ..
// 262K points (bench.py --tile-sweep): 128-row tiles for K <= 128 (one tile:
// up to 1.4x faster), 256-row tiles above (x is read once for K <= 256); LDS
// staging wherever the rows allow it (whole 16-byte-aligned rows of a
// multiple of 128 units: up to 1.3x faster at 262K points, 2-16% at 16K),
// register staging for other rows. FK_TILE or FK_SPLITD_REGISTER_STAGING
// override.
void split_tile(int64_t K, bool& lds, bool& rows128) {
  rows128 = K <= 128;
  lds = true;
  if (const char* e = getenv("FK_TILE")) {
    for (int i = 0; i < kSplitTiles; ++i)
      if (strcmp(e, kSplitTileNames[i]) == 0) {
        lds = i == kSplitLds8 || i == kSplitLds4;
        rows128 = i == kSplitLds4 || i == kSplitReg4;
        return;
      }
  }
  const char* r = getenv("FK_SPLITD_REGISTER_STAGING");
  if (r && r[0] == '1') lds = false;
}

template <int DT, int NSUB>
hipError_t run_splitd(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                      int64_t d, int64_t K, int32_t* ids, bool lds, hipStream_t s) {
  const int bpb = (int)((N + kBN - 1) / kBN);
  const int64_t total = B * bpb;
  if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* cp = (const uint16_t*)c;
  if (lds && vec_ok(x, c, d) && d % (2 * kLC) == 0)
    return launch_splitd_lds<DT, NSUB>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if (vec_ok(x, c, d) && d % kDC == 0)
    return launch_splitd<DT, NSUB, true, true>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if (vec_ok(x, c, d))
    return launch_splitd<DT, NSUB, true, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  if constexpr (NSUB == 4)
    return launch_splitd<DT, NSUB, false, false>(xp, cp, cn, total, bpb, N, d, K, ids, s);
  return hipErrorNotSupported;
}

// Element-wise loads (unaligned or d % 8 != 0) keep 128-row tiles: with 256
// the accumulators leave no registers for them.
template <int DT>
hipError_t splitd_dt(const void* x, const void* c, const float* cn, int64_t B, int64_t N,
                     int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  bool lds, rows128;
  split_tile(K, lds, rows128);
  if (rows128 || !vec_ok(x, c, d)) return run_splitd<DT, 4>(x, c, cn, B, N, d, K, ids, lds, s);
  return run_splitd<DT, 8>(x, c, cn, B, N, d, K, ids, lds, s);
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
