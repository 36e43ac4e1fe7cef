// Centroid precompute and small element-wise kernels.
//
// norms: one wave per centroid row. Each lane rounds its share of the fp32
// master row to the element type (nearest-even), stores the rounded copy that
// the assignment reads, and accumulates the square of the *rounded* value in
// fp32; a wave reduction gives ||c_lp||^2. The assignment then measures the
// true distance to the centroid it actually uses. The ||c||^2 term is the
// only centroid-side quantity the fused distance needs besides x.c
// ("Flash-KMeans：IO感知的精确K-Means…", section "它攻克的两大瓶颈").
#include "fk_internal.hpp"

namespace fk {
namespace {

constexpr int kWaves = 4;

template <int DT>
__global__ __launch_bounds__(256) void norms_kernel(const float* __restrict__ c,
                                                    uint16_t* __restrict__ c_lp,
                                                    float* __restrict__ cnorm, int64_t rows,
                                                    int64_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* src = c + row * d;
  uint16_t* dst = c_lp + row * d;
  float acc = 0.f;
  for (int64_t j = lane; j < d; j += 64) {
    const uint16_t h = Elem<DT>::narrow(src[j]);
    dst[j] = h;
    const float r = Elem<DT>::widen(h);
    acc = fmaf(r, r, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) cnorm[row] = acc;
}

__global__ __launch_bounds__(256) void norms_f32_kernel(const float* __restrict__ c,
                                                        float* __restrict__ c_lp,
                                                        float* __restrict__ cnorm,
                                                        int64_t rows, int64_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* src = c + row * d;
  float* dst = c_lp + row * d;
  float acc = 0.f;
  for (int64_t j = lane; j < d; j += 64) {
    const float r = src[j];
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

hipError_t launch_norms(const float* c, void* c_lp, float* cnorm, int dt, int64_t rows,
                        int64_t d, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + kWaves - 1) / kWaves);
  if (dt == FK_F16)
    norms_kernel<FK_F16><<<grid, 256, 0, s>>>(c, (uint16_t*)c_lp, cnorm, rows, d);
  else if (dt == FK_BF16)
    norms_kernel<FK_BF16><<<grid, 256, 0, s>>>(c, (uint16_t*)c_lp, cnorm, rows, d);
  else
    norms_f32_kernel<<<grid, 256, 0, s>>>(c, (float*)c_lp, cnorm, rows, d);
  return hipGetLastError();
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
