// libfkbaseline: the standard assign (materialised distance matrix + argmin)
// and the standard update (scatter atomics), for contrast with FlashAssign
// and the sort-inverse update. The pages describe both as the formulations
// the method replaces (itinai.com summary, the paragraphs on the first and
// second bottleneck; "Flash-KMeans: Implementação Exata ...", section on
// conventional assignment; "Flash-KMeans：IO感知的精确K-Means ...", update
// section). The GEMM is rocBLAS, as a library GEMM would be in a standard
// implementation; the argmin, scatter and divide kernels are plain HIP.
// Nothing here is shared with libfkmeans.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include "../../include/fkmeans_baselines.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
  if (dt == FK_F32) return reinterpret_cast<const float*>(p)[i];
  const uint16_t h = reinterpret_cast<const uint16_t*>(p)[i];
  if (dt == FK_F16) return (float)__builtin_bit_cast(_Float16, h);
  return __builtin_bit_cast(float, (uint32_t)h << 16);   // bf16
}

// One wave per point row: min over k of cnorm[k] + dist[n,k], lowest k on
// ties (each lane scans increasing k; the wave keeps the lower index on
// equal values).
__global__ __launch_bounds__(kThreads) void argmin_rows_kernel(const float* __restrict__ dist,
                                                               const float* __restrict__ cnorm,
                                                               int32_t* __restrict__ ids,
                                                               int64_t rows, int N, int K,
                                                               bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t b = row / N;
  const float* dr = dist + row * K;
  const float* cn = cnorm + b * K;
  float best = INFINITY;
  int bidx = 0;
  if (vec) {                   // K % 4 == 0 and 16-byte aligned bases: 16-byte loads
    for (int k = 4 * lane; k < K; k += 256) {
      const float4 dv = *reinterpret_cast<const float4*>(dr + k);
      const float4 cv = *reinterpret_cast<const float4*>(cn + k);
      const float v[4] = {cv.x + dv.x, cv.y + dv.y, cv.z + dv.z, cv.w + dv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (v[i] < best) {
          best = v[i];
          bidx = k + i;
        }
      }
    }
  } else {
    for (int k = lane; k < K; k += 64) {
      const float v = cn[k] + dr[k];
      if (v < best) {
        best = v;
        bidx = k;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(bidx, off, 64);
    if (ov < best || (ov == best && oi < bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (lane == 0) ids[row] = bidx;
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ s, int64_t ns,
                                                        int32_t* __restrict__ c, int64_t nc) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < ns; i += stride) s[i] = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nc; i += stride) c[i] = 0;
}

// One thread per element of x: one fp32 atomic add into its cluster's sums
// (hardware float atomic), and one count per point.
__global__ __launch_bounds__(kThreads) void scatter_add_kernel(const void* __restrict__ x,
                                                               const int32_t* __restrict__ ids,
                                                               float* __restrict__ sums,
                                                               int32_t* __restrict__ counts,
                                                               int dt, int64_t total, int N, int d,
                                                               int K) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const int64_t pt = e / d;                  // b * N + n
    const int j = (int)(e - pt * d);
    const int64_t b = pt / N;
    const int k = ids[pt];
    if ((unsigned)k >= (unsigned)K) continue;  // out of contract: ignored
    unsafeAtomicAdd(&sums[(b * K + k) * d + j], load_elem(x, e, dt));
    if (j == 0) atomicAdd(&counts[b * K + k], 1);
  }
}

__global__ __launch_bounds__(kThreads) void divide_kernel(const float* __restrict__ sums,
                                                          const int32_t* __restrict__ counts,
                                                          float* __restrict__ c, int64_t total,
                                                          int d) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const int n = counts[e / d];
    if (n > 0) c[e] = sums[e] / (float)n;
  }
}

// MFMA peak probe: every wave issues v_mfma_f32_32x32x16_f16 back to back on
// operands drawn from a counter-based hash (values in [-1, 1), different per
// lane and per operand), kPeakChains independent accumulator chains so no
// MFMA waits for the previous one's result, rotating through four A and two B
// operands; one loop iteration is 4 rounds of kPeakChains MFMAs.
// Lane 0 of each block records the shader-clock counter (s_memtime) and the
// constant-rate counter (s_memrealtime) at its start and end, so the host can
// tell the clock the loop ran at; every wave writes the sum of its
// accumulators so nothing is optimised away.
typedef _Float16 fkb_half8 __attribute__((ext_vector_type(8)));
typedef float fkb_floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t hash32(uint32_t v) {
  v ^= v >> 16;
  v *= 0x7feb352dU;
  v ^= v >> 15;
  v *= 0x846ca68bU;
  v ^= v >> 16;
  return v;
}

__device__ __forceinline__ fkb_half8 random_half8(uint32_t seed) {
  fkb_half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t r = hash32(seed * 8u + (uint32_t)i);
    h[i] = (_Float16)((float)(r >> 8) * (1.0f / 8388608.0f) - 1.0f);
  }
  return h;
}

constexpr int kPeakChains = 8;

__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(float* __restrict__ out,
                                                             long long* __restrict__ stamps,
                                                             int iters, uint32_t seed) {
  const uint32_t gl = (uint32_t)(blockIdx.x * kThreads + threadIdx.x);
  long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = (long long)__builtin_amdgcn_s_memtime();
    r0 = (long long)__builtin_amdgcn_s_memrealtime();
  }
  fkb_half8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = random_half8(hash32(seed ^ (gl * 16u + (uint32_t)i)));
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = random_half8(hash32(~seed ^ (gl * 16u + (uint32_t)i)));
  fkb_floatx16 acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(c + r) & 3], b[c & 1], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[gl] = s;
  if (threadIdx.x == 0) {
    const long long t1 = (long long)__builtin_amdgcn_s_memtime();
    const long long r1 = (long long)__builtin_amdgcn_s_memrealtime();
    stamps[4 * blockIdx.x + 0] = t0;
    stamps[4 * blockIdx.x + 1] = t1;
    stamps[4 * blockIdx.x + 2] = r0;
    stamps[4 * blockIdx.x + 3] = r1;
  }
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

rocblas_handle handle_for_device() {
  static rocblas_handle handles[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!handles[dev] && rocblas_create_handle(&handles[dev]) != rocblas_status_success)
    handles[dev] = nullptr;
  return handles[dev];
}

bool sizes_ok(int64_t B, int64_t N, int64_t d, int64_t K) {
  const int64_t lim = 0x7FFFFFFF;
  return B > 0 && N > 0 && d > 0 && K > 0 && B < lim && N < lim && d < lim && K < lim;
}

}  // namespace

extern "C" fk_status_t fkb_assign_materialized(const void* x, const void* c_lp,
                                               const float* cnorm, fk_dtype_t dt, int64_t B,
                                               int64_t N, int64_t d, int64_t K, float* dist,
                                               int32_t* ids, hipStream_t stream) {
  if (!sizes_ok(B, N, d, K) || !x || !c_lp || !cnorm || !dist || !ids) return FK_ERR_INVALID;
  rocblas_datatype in_t;
  if (dt == FK_F32) in_t = rocblas_datatype_f32_r;
  else if (dt == FK_F16) in_t = rocblas_datatype_f16_r;
  else if (dt == FK_BF16) in_t = rocblas_datatype_bf16_r;
  else return FK_ERR_INVALID;
  rocblas_handle h = handle_for_device();
  if (!h || rocblas_set_stream(h, stream) != rocblas_status_success) return FK_ERR_HIP;
  // Row-major dist (N,K) of problem b is the column-major K x N product
  // c_lp_b (K x d) * x_b^T: A = c_lp as column-major d x K, transposed;
  // B = x as column-major d x N.
  const float alpha = -2.f, beta = 0.f;
  const rocblas_status st = rocblas_gemm_strided_batched_ex(
      h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)K, (rocblas_int)N,
      (rocblas_int)d, &alpha, c_lp, in_t, (rocblas_int)d, (rocblas_stride)(K * d), x, in_t,
      (rocblas_int)d, (rocblas_stride)(N * d), &beta, dist, rocblas_datatype_f32_r,
      (rocblas_int)K, (rocblas_stride)(N * K), dist, rocblas_datatype_f32_r, (rocblas_int)K,
      (rocblas_stride)(N * K), (rocblas_int)B, rocblas_datatype_f32_r, rocblas_gemm_algo_standard,
      0, 0);
  if (st != rocblas_status_success) return FK_ERR_HIP;
  const int64_t rows = B * N;
  const int64_t blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7FFFFFFF) return FK_ERR_INVALID;
  const bool vec = K % 4 == 0 && (uintptr_t)dist % 16 == 0 && (uintptr_t)cnorm % 16 == 0;
  argmin_rows_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(dist, cnorm, ids, rows, (int)N,
                                                                 (int)K, vec);
  return hipGetLastError() == hipSuccess ? FK_OK : FK_ERR_HIP;
}

extern "C" fk_status_t fkb_update_atomic(const void* x, const int32_t* ids, fk_dtype_t dt,
                                         int64_t B, int64_t N, int64_t d, int64_t K, float* c,
                                         int32_t* counts, float* sums, hipStream_t stream) {
  if (!sizes_ok(B, N, d, K) || !x || !ids || !c || !counts || !sums) return FK_ERR_INVALID;
  if (dt != FK_F32 && dt != FK_F16 && dt != FK_BF16) return FK_ERR_INVALID;
  const int64_t kd = B * K * d, total = B * N * d;
  zero_kernel<<<grid_for(kd), kThreads, 0, stream>>>(sums, kd, counts, B * K);
  if (hipGetLastError() != hipSuccess) return FK_ERR_HIP;
  scatter_add_kernel<<<grid_for(total), kThreads, 0, stream>>>(x, ids, sums, counts, (int)dt,
                                                               total, (int)N, (int)d, (int)K);
  if (hipGetLastError() != hipSuccess) return FK_ERR_HIP;
  divide_kernel<<<grid_for(kd), kThreads, 0, stream>>>(sums, counts, c, kd, (int)d);
  return hipGetLastError() == hipSuccess ? FK_OK : FK_ERR_HIP;
}

extern "C" fk_status_t fkb_mfma_peak(int64_t blocks, int32_t iters, uint32_t seed, float* out,
                                     long long* stamps, hipStream_t stream) {
  if (blocks < 1 || blocks > 0x7FFFFFFF || iters < 1 || !out || !stamps) return FK_ERR_INVALID;
  mfma_peak_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(out, stamps, iters, seed);
  return hipGetLastError() == hipSuccess ? FK_OK : FK_ERR_HIP;
}

extern "C" int32_t fkb_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return 0;
  return khz;
}
