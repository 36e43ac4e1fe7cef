// Centroid precompute and small element-wise kernels.
//
// norms: a group of lanes per centroid row (16-byte loads when d % 4 == 0,
// else one wave per row). Each lane rounds its share of the fp32 master row
// to the element type (nearest-even), stores the rounded copy that the
// assignment reads, and accumulates the square of the *rounded* value in
// fp32; a reduction over the group gives ||c_lp||^2. The assignment then measures the
// true distance to the centroid it actually uses. The ||c||^2 term is the
// only centroid-side quantity the fused distance needs besides x.c
// ("Flash-KMeans：IO感知的精确K-Means…", section "它攻克的两大瓶颈").
#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kWaves = 4;

// Every norms kernel first finishes a deferred update (pf): a long cluster's
// row is the sum of its pieces (fixed order, see LongPieces) divided by its
// count, written back to c.
template <int DT>
__global__ __launch_bounds__(256) void norms_kernel(float* __restrict__ c,
                                                    uint16_t* __restrict__ c_lp,
                                                    float* __restrict__ cnorm, int64_t rows,
                                                    int64_t d, PendingFinish pf) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  int lo, hi;
  pending_segment(pf, row, lo, hi);
  const int64_t b = pf.offsets ? row / pf.K : 0;
  uint16_t* dst = c_lp + row * d;
  float acc = 0.f;
  for (int64_t j = lane; j < d; j += 64) {
    float v = c[row * d + j];
    if (hi > lo) {
      v = long_sum(pf.lp, b, d, lo, hi, j) / (float)(hi - lo);
      c[row * d + j] = v;
    }
    const uint16_t h = Elem<DT>::narrow(v);
    dst[j] = h;
    const float r = Elem<DT>::widen(h);
    acc = fmaf(r, r, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) cnorm[row] = acc;
}

// Vector form (d % 4 == 0, 16-byte aligned c, 8-byte aligned c_lp): LPR lanes
// per row, 4 elements per lane per step, so one wave covers 64/LPR rows; the
// row's squares are summed over its lane group.
template <int DT, int LPR>
__global__ __launch_bounds__(256) void norms_vec_kernel(float* __restrict__ c,
                                                        uint16_t* __restrict__ c_lp,
                                                        float* __restrict__ cnorm, int64_t rows,
                                                        int d, PendingFinish pf) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, li = lane % LPR;
  const int64_t row = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool ok = row < rows;
  float acc = 0.f;
  if (ok) {
    int lo, hi;
    pending_segment(pf, row, lo, hi);
    const int64_t b = pf.offsets ? row / pf.K : 0;
    const float cnt = (float)(hi - lo);
    uint16_t* dst = c_lp + row * d;
    for (int j = li * 4; j < d; j += LPR * 4) {
      float4 v;
      if (hi > lo) {
        v = make_float4(long_sum(pf.lp, b, d, lo, hi, j) / cnt,
                        long_sum(pf.lp, b, d, lo, hi, j + 1) / cnt,
                        long_sum(pf.lp, b, d, lo, hi, j + 2) / cnt,
                        long_sum(pf.lp, b, d, lo, hi, j + 3) / cnt);
        *reinterpret_cast<float4*>(c + row * d + j) = v;
      } else {
        v = *reinterpret_cast<const float4*>(c + row * d + j);
      }
      const uint16_t h[4] = {Elem<DT>::narrow(v.x), Elem<DT>::narrow(v.y), Elem<DT>::narrow(v.z),
                             Elem<DT>::narrow(v.w)};
      *reinterpret_cast<uint2*>(dst + j) =
          make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = Elem<DT>::widen(h[i]);
        acc = fmaf(r, r, acc);
      }
    }
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && li == 0) cnorm[row] = acc;
}

template <int DT, int LPR>
hipError_t run_norms_vec(float* c, uint16_t* c_lp, float* cnorm, int64_t rows, int64_t d,
                         const PendingFinish& pf, hipStream_t s) {
  constexpr int RPB = kWaves * (64 / LPR);       // rows per block
  const int64_t grid = (rows + RPB - 1) / RPB;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_timed(norms_vec_kernel<DT, LPR>, dim3((unsigned)grid), dim3(256), s, c, c_lp, cnorm,
                      rows, (int)d, pf);
}

// lanes per row: the vectors of a row, rounded up to a power of two in [4, 64]
template <int DT>
hipError_t norms_vec_dt(float* c, uint16_t* c_lp, float* cnorm, int64_t rows, int64_t d,
                        const PendingFinish& pf, hipStream_t s) {
  const int64_t nv = d / 4;
  if (nv <= 4) return run_norms_vec<DT, 4>(c, c_lp, cnorm, rows, d, pf, s);
  if (nv <= 8) return run_norms_vec<DT, 8>(c, c_lp, cnorm, rows, d, pf, s);
  if (nv <= 16) return run_norms_vec<DT, 16>(c, c_lp, cnorm, rows, d, pf, s);
  if (nv <= 32) return run_norms_vec<DT, 32>(c, c_lp, cnorm, rows, d, pf, s);
  return run_norms_vec<DT, 64>(c, c_lp, cnorm, rows, d, pf, s);
}

__global__ __launch_bounds__(256) void norms_f32_kernel(float* __restrict__ c,
                                                        float* __restrict__ c_lp,
                                                        float* __restrict__ cnorm,
                                                        int64_t rows, int64_t d,
                                                        PendingFinish pf) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  int lo, hi;
  pending_segment(pf, row, lo, hi);
  const int64_t b = pf.offsets ? row / pf.K : 0;
  float* dst = c_lp + row * d;
  float acc = 0.f;
  for (int64_t j = lane; j < d; j += 64) {
    float r = c[row * d + j];
    if (hi > lo) {
      r = long_sum(pf.lp, b, d, lo, hi, j) / (float)(hi - lo);
      c[row * d + j] = r;
    }
    dst[j] = r;
    acc = fmaf(r, r, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) cnorm[row] = acc;
}

template <int DT>
__global__ __launch_bounds__(256) void widen_kernel(const uint16_t* __restrict__ src,
                                                    float* __restrict__ dst, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    dst[i] = Elem<DT>::widen(src[i]);
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src,
                                                       float* __restrict__ dst, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int32_t v,
                                                       int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    p[i] = v;
}

unsigned grid_for(int64_t count) {
  int64_t g = (count + 255) / 256;
  if (g > 8192) g = 8192;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_norms(const float* c_in, void* c_lp, float* cnorm, int dt, int64_t rows,
                        int64_t d, hipStream_t s, const PendingFinish& pf) {
  if (rows == 0) return hipSuccess;
  // written only when an update is pending (pf.offsets), on the caller's own buffer
  float* c = const_cast<float*>(c_in);
  const bool vec = d % 4 == 0 && d <= 0x7FFFFFFF && ((uintptr_t)c % 16) == 0 &&
                   ((uintptr_t)c_lp % 8) == 0;
  if (vec && dt == FK_F16)
    return norms_vec_dt<FK_F16>(c, (uint16_t*)c_lp, cnorm, rows, d, pf, s);
  if (vec && dt == FK_BF16)
    return norms_vec_dt<FK_BF16>(c, (uint16_t*)c_lp, cnorm, rows, d, pf, s);
  const unsigned grid = (unsigned)((rows + kWaves - 1) / kWaves);
  if (dt == FK_F16)
    return launch_timed(norms_kernel<FK_F16>, dim3(grid), dim3(256), s, c, (uint16_t*)c_lp, cnorm,
                        rows, d, pf);
  if (dt == FK_BF16)
    return launch_timed(norms_kernel<FK_BF16>, dim3(grid), dim3(256), s, c, (uint16_t*)c_lp, cnorm,
                        rows, d, pf);
  return launch_timed(norms_f32_kernel, dim3(grid), dim3(256), s, c, (float*)c_lp, cnorm, rows, d,
                      pf);
}

hipError_t launch_widen(const void* src, float* dst, int dt, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  if (dt == FK_F16)
    widen_kernel<FK_F16><<<grid_for(count), 256, 0, s>>>((const uint16_t*)src, dst, count);
  else if (dt == FK_BF16)
    widen_kernel<FK_BF16><<<grid_for(count), 256, 0, s>>>((const uint16_t*)src, dst, count);
  else
    copy_f32_kernel<<<grid_for(count), 256, 0, s>>>((const float*)src, dst, count);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  fill_i32_kernel<<<grid_for(count), 256, 0, s>>>(p, v, count);
  return hipGetLastError();
}

}  // namespace fk
