// Internal declarations shared by the libfkmeans translation units.
// Device helpers (element types, rounding, wave reductions) and the host-side
// launchers each kernel file exports to the API layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "../../include/fkmeans.h"

namespace fk {

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Widening of one stored 16-bit element (raw bits) to fp32 -- exact.
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Rounding fp32 -> 16-bit storage, nearest-even. fp16 uses the hardware
// convert (default round-to-nearest-even mode); bf16 adds half an ulp minus
// one plus the kept lsb, so exact halves go to the even neighbour.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 v = (_Float16)f;
  return __builtin_bit_cast(uint16_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int DT> struct Elem;
template <> struct Elem<FK_F16> {
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float widen(uint16_t h) { return f16_bits_to_f32(h); }
  __device__ static __forceinline__ uint16_t narrow(float f) { return f32_to_f16_bits(f); }
};
template <> struct Elem<FK_BF16> {
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float widen(uint16_t h) { return bf16_bits_to_f32(h); }
  __device__ static __forceinline__ uint16_t narrow(float f) { return f32_to_bf16_bits(f); }
};

// Word 3 of a raw (unformatted, stride 0) buffer resource.
constexpr int kRawBufferWord3 = 0x00020000;

// A pointer the caller knows to be the same in every lane, moved to scalar
// registers (a buffer resource must be scalar).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 32x32x16 MFMA with fp32 accumulate; A rows = centroids, B cols = points.
template <int DT> struct Mfma;
template <> struct Mfma<FK_F16> {
  __device__ static __forceinline__ floatx16_t run(uint4 a, uint4 b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                 __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<FK_BF16> {
  __device__ static __forceinline__ floatx16_t run(uint4 a, uint4 b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
// fp32: the 16 bytes a lane holds per k-step are 4 floats, k-elements
// half*4 .. half*4+3 of an 8-wide k-step; four v_mfma_f32_32x32x2_f32 take
// element j of every lane in turn (half 0 and half 1 give the two k of one
// MFMA), so A and B, loaded with the same byte layout, pair up k for k.
template <> struct Mfma<FK_F32> {
  __device__ static __forceinline__ floatx16_t run(uint4 a, uint4 b, floatx16_t c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a.x),
                                             __builtin_bit_cast(float, b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a.y),
                                             __builtin_bit_cast(float, b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a.z),
                                             __builtin_bit_cast(float, b.z), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a.w),
                                                __builtin_bit_cast(float, b.w), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// MFMA tile helpers (v_mfma_f32_32x32x16: lane = point column r32 + 32*half,
// holding k-elements half*8 .. half*8+7 of each 16-wide k-step)
// ---------------------------------------------------------------------------
// 16-byte load of 8 stored elements starting at col; elements at or past
// limit read as zero. VEC: the row base is 16-byte aligned and limit % 8 == 0.
template <bool VEC>
__device__ __forceinline__ uint4 load8(const uint16_t* row, int col, int limit) {
  if (VEC) {
    if (col < limit) return *reinterpret_cast<const uint4*>(row + col);
    return make_uint4(0, 0, 0, 0);
  } else {
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (col + i < limit) ? row[col + i] : (uint16_t)0;
    uint4 v;
    v.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    v.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    v.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    v.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    return v;
  }
}

// Slot-coded scores for a running argmax over the 16 scores a lane holds of
// one 32-row MFMA output (slot r = 0..15 is row 8*(r/4) + 4*half + r%4): the
// 4 low mantissa bits of each score are replaced by 15 - r, so a max over
// coded scores also says where the maximum is. The code changes a score by
// less than 2^-19 of its size; scores that agree to that precision are
// ordered by it (lower row first when positive, higher row when negative).
// Scores that must never win are kNeverWins, a finite value (a code on -inf
// would make a NaN).
constexpr float kNeverWins = -3.40282346638528859812e+38f;   // -FLT_MAX

__device__ __forceinline__ float code_slot(float score, int r) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, score) & ~0xFu) | (uint32_t)(15 - r));
}
__device__ __forceinline__ int slot_of(float coded) {
  return 15 - (int)(__builtin_bit_cast(uint32_t, coded) & 0xFu);
}
// Row (within the 32-row block, without the 4*half term) of slot r.
__device__ __forceinline__ int slot_row(int r) { return 8 * (r >> 2) + (r & 3); }

// v_max3_f32 of three finite scores. The compiler turns a two-operand fmaxf
// of MFMA results into canonicalising maxes; this keeps the tree at one
// instruction per two new scores (the kernels that use it build with
// -fno-honor-nans; inputs are finite by contract).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The two lanes (half 0 and half 1) that hold the same point each carry the
// best score and row over their 16 rows of every 32-row block; half 1's rows
// sit 4 above half 0's. Returns the winning row, lowest row on equal scores.
__device__ __forceinline__ int merge_halves(float best, int bidx, int half) {
  int idx = bidx + 4 * half;
  const float ob = __shfl_xor(best, 32, 64);
  const int oi = __shfl_xor(idx, 32, 64);
  if (ob > best || (ob == best && oi < idx)) idx = oi;
  return idx;
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block id -> logical tile so that each XCD (blocks are dealt round-robin to
// the 8 XCDs) works on a contiguous range of tiles and keeps them in its L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t grid) {
  const int64_t q = grid / 8, r = grid % 8;
  const int64_t xcd = bid % 8, slot = bid / 8;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// ---------------------------------------------------------------------------
// segments of the sort-inverse update
// ---------------------------------------------------------------------------
constexpr int kSegRun = 256;   // sorted positions per segment-reduce run

// A segment longer than one run is reduced in pieces (one per run it
// touches, see LongPieces); shorter ones are reduced whole and written as
// their mean.
__device__ __forceinline__ bool is_long(int lo, int hi) { return hi - lo > kSegRun; }

// Pieces of long segments, reduced in a fixed order. The segment-reduce wave
// of run r writes at most two pieces: slot 0, the piece of the long segment
// that covers the run's first position and started before it (its "head"),
// and slot 1, the piece of a long segment that starts inside the run (at
// most one can: it then covers the rest of the run). Q1 row j holds the sum
// of the slot-0 pieces of runs 32j .. 32j+31 in run order, Q2 row i the sum
// of Q1 rows 32i .. 32i+31 in order; each exists only for full blocks. A long
// cluster with positions [lo, hi) then sums to
//   slot1[lo/256] + (slot0 of runs lo/256+1 .. (hi-1)/256, in run order)
// where whole aligned blocks of 32 (1024) runs are taken from Q1 (Q2) when a
// problem has more than kPieceDirectRuns runs (else every piece is added in
// run order). The order depends only on lo, hi and the problem size, so the
// result does not depend on how the GPU schedules its waves.
constexpr int kQ1 = 32;     // runs per Q1 block
constexpr int kQ2 = 32;     // Q1 blocks per Q2 block

struct LongPieces {
  const float* pieces = nullptr;   // (B, runs, 2, d)
  const float* q1 = nullptr;       // (B, nq1, d)
  const float* q2 = nullptr;       // (B, nq2, d)
  int runs = 0, nq1 = 0, nq2 = 0;
  bool blocks = true;              // Q1/Q2 sums exist (runs > kPieceDirectRuns)
};

// Up to this many runs per problem, no Q1/Q2 sums are formed (two launches
// less): a long segment's pieces are added one by one, at most this many.
constexpr int kPieceDirectRuns = 1024;

// Column c of the sum of long segment [lo, hi) of problem b.
__device__ __forceinline__ float long_sum(const LongPieces& lp, int64_t b, int64_t d, int lo,
                                          int hi, int64_t c) {
  const int rlo = lo / kSegRun, e = (hi - 1) / kSegRun + 1;
  const float* pb = lp.pieces + (int64_t)b * lp.runs * 2 * d + c;
  const float* q1 = lp.q1 + (int64_t)b * lp.nq1 * d + c;
  const float* q2 = lp.q2 + (int64_t)b * lp.nq2 * d + c;
  float t = 0.f;
  int r = rlo + 1;
  if (!lp.blocks) {
    for (; r < e; ++r) t += pb[(int64_t)r * 2 * d];
    return pb[((int64_t)rlo * 2 + 1) * d] + t;
  }
  for (; r < e && (r % kQ1) != 0; ++r) t += pb[(int64_t)r * 2 * d];
  for (; r + kQ1 <= e && (r % (kQ1 * kQ2)) != 0; r += kQ1) t += q1[(int64_t)(r / kQ1) * d];
  for (; r + kQ1 * kQ2 <= e; r += kQ1 * kQ2) t += q2[(int64_t)(r / (kQ1 * kQ2)) * d];
  for (; r + kQ1 <= e; r += kQ1) t += q1[(int64_t)(r / kQ1) * d];
  for (; r < e; ++r) t += pb[(int64_t)r * 2 * d];
  return pb[((int64_t)rlo * 2 + 1) * d] + t;
}

// An update whose long clusters are still in pieces (their sum and the
// division by the count are left to the next pass over the centroids).
// offsets null: nothing pending.
struct PendingFinish {
  LongPieces lp;
  const int32_t* offsets = nullptr;     // (B,K+1)
  const int32_t* has_long = nullptr;    // (B)
  int64_t K = 0;
};

// For centroid row `row` (= b*K + k): its long segment [lo, hi) when the row
// is pending, else hi == lo.
__device__ __forceinline__ void pending_segment(const PendingFinish& pf, int64_t row, int& lo,
                                                int& hi) {
  lo = hi = 0;
  if (!pf.offsets) return;
  const int64_t b = row / pf.K, k = row - b * pf.K;
  if (!pf.has_long[b]) return;
  const int32_t* ob = pf.offsets + b * (pf.K + 1);
  const int l = ob[k], h = ob[k + 1];
  if (is_long(l, h)) lo = l, hi = h;
}

// ---------------------------------------------------------------------------
// Timed launches: events that the next launch_timed stamps with that kernel's
// own start and end (hipExtLaunchKernel), so timing a phase adds no packets
// to the stream. Set by the caller's trace, taken by one launch (per thread).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

template <typename... P, typename... A>
hipError_t launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one value per kernel parameter");
  LaunchEvents& le = launch_events();
  if (!le.start && !le.stop) {
    kernel<<<grid, block, 0, s>>>(static_cast<P>(args)...);
    return hipGetLastError();
  }
  const LaunchEvents ev = le;
  le = LaunchEvents();
  std::tuple<P...> vals{static_cast<P>(args)...};
  void* argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&](auto&... v) {
    size_t i = 0;
    ((argv[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s,
                            ev.start, ev.stop, 0);
}

// ---------------------------------------------------------------------------
// launchers (host); each returns hipSuccess or the launch error
// ---------------------------------------------------------------------------
// pf: an update to finish first (its long clusters' rows of c are divided
// and written back, so c must then be writable).
hipError_t launch_norms(const float* c, void* c_lp, float* cnorm, int dt, int64_t rows,
                        int64_t d, hipStream_t s, const PendingFinish& pf = PendingFinish());
hipError_t launch_widen(const void* src, float* dst, int dt, int64_t count, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t count, hipStream_t s);

// Assignment paths. Each returns hipErrorNotSupported when it cannot run the shape.
// Compute units of the current device (cached per device; 0 if unknown).
int device_cus();
bool smalld_supported(int dt, int64_t d);
hipError_t launch_assign_smalld(const void* x, const void* c_lp, const float* cnorm, int dt,
                                int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                                hipStream_t s);
hipError_t launch_assign_splitd(const void* x, const void* c_lp, const float* cnorm, int dt,
                                int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                                hipStream_t s);

// Sort-inverse update; workspace carved by the API layer.
struct UpdateWs {
  float* pieces;        // (B,runs,2,d) fp32 pieces of long segments (see LongPieces)
  float* q1;            // (B,nq1,d) sums of 32 consecutive slot-0 pieces
  float* q2;            // (B,nq2,d) sums of 32 consecutive Q1 rows
  int32_t* offsets;     // (B,K+1) segment starts
  int32_t* perm;        // (B,N) point index per sorted position
  int32_t* run_first;   // (B,runs) cluster holding each run's first position
  float* part;          // (B, finalize blocks) partial squared moves
  int32_t* hist;        // (B, G, K) per-chunk counts of the split sort
  int32_t* has_long;    // (B) nonzero when the problem has a long cluster
  int32_t* rkeys[2];    // (B,N) keys between radix passes (large chunks / large K)
  int32_t* ridx[2];     // (B,N) point indices between radix passes
  int32_t* rhist;       // (B, radix chunks, 256) digit counts of one radix pass
  int32_t* rcolsum;     // (passes, B, chunk groups, 256) digit counts per group of chunks
  int32_t* rgbase;      // (B, chunk groups, 256) first output position per group and digit
  int32_t* cursor;      // (B,K) scatter cursors (K above 2^16 only)
  int32_t* ktot;        // (B, K / 256 blocks) cluster counts per block of 256 (large G*K only)
  int runs, nq1, nq2;
};
size_t update_ws_bytes(int64_t B, int64_t N, int64_t d, int64_t K);
UpdateWs carve_update_ws(void* base, int64_t B, int64_t N, int64_t d, int64_t K);
// shift may be null: the new centroids are written and no shift is computed.
// defer (only with shift == null): the long clusters' division is left to
// the next norms pass (see pending_finish) or to launch_finish.
hipError_t launch_update(const void* x, const int32_t* ids, int dt, int64_t B, int64_t N,
                         int64_t d, int64_t K, float* c, int32_t* counts, float* shift,
                         const UpdateWs& ws, hipStream_t s, bool defer = false);
PendingFinish pending_finish(const UpdateWs& ws, int64_t K);
LongPieces long_pieces(const UpdateWs& ws);
hipError_t launch_finish(float* c, const UpdateWs& ws, int64_t B, int64_t d, int64_t K,
                         hipStream_t s);

// Accumulating update for points that arrive in chunks: the sorted segments
// of one chunk are added into sums_run with atomics and its counts into
// counts_run (counts_chunk: scratch of B*K ints); ws sized for the chunk.
hipError_t launch_update_accumulate(const void* x, const int32_t* ids, int dt, int64_t B,
                                    int64_t N, int64_t d, int64_t K, float* sums_run,
                                    int32_t* counts_run, int32_t* counts_chunk,
                                    const UpdateWs& ws, hipStream_t s);
hipError_t launch_zero_sums(float* sums, int32_t* counts, int64_t B, int64_t K, int64_t d,
                            hipStream_t s);
// c = sums / counts for non-empty clusters; shift (nullable) from part, which
// holds B * sums_fin_blocks(K, d) floats.
int64_t sums_fin_blocks(int64_t K, int64_t d);
hipError_t launch_finalize_sums(const float* sums, const int32_t* counts, float* c,
                                float* shift, float* part, int64_t B, int64_t K, int64_t d,
                                hipStream_t s);

}  // namespace fk
