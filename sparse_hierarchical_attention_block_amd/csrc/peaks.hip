// peaks.hip -- measurement helpers: the HBM streaming rate and the bf16 MFMA
// rate this GPU actually attains, so that the kernels' roofline fractions can
// be stated against both the nominal peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense
// bf16) and what a plain kernel reaches on the same part in the same run.
//
//   peak_stream_kernel  grid-stride 16-byte loads over a buffer; mode 0 also
//                       stores every vector to a second buffer (a copy), modes
//                       1 and 2 only fold the loaded words into one value per
//                       thread (a read stream; mode 2 with the non-temporal
//                       cache policy of decode's K/V loads, mode 1 with loads
//                       that allocate in the caches, which evicts them)
//   peak_mfma_kernel    back-to-back v_mfma_f32_32x32x16_bf16 on eight
//                       independent accumulators held in registers; no memory
//                       traffic inside the loop
#include <hip/hip_runtime.h>

#include "dash.h"
#include "device_common.hpp"

namespace dash {
namespace {

constexpr int kPeakThreads = 256;
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kPeakThreads) void peak_stream_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t n16, int mode) {
  const int64_t stride = (int64_t)gridDim.x * kPeakThreads;
  int64_t i = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  if (mode == 0) {
    for (; i + 3 * stride < n16; i += 4 * stride) {
      const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                  e = src[i + 3 * stride];
      dst[i] = a;
      dst[i + stride] = b;
      dst[i + 2 * stride] = c;
      dst[i + 3 * stride] = e;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
  } else {
    // eight loads in flight per thread before any is consumed
    const bool nt = mode == 2;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 7 * stride < n16; i += 8 * stride) {
      u32x4 r[8];
      if (nt) {
#pragma unroll
        for (int m = 0; m < 8; ++m) r[m] = __builtin_nontemporal_load(src + i + m * stride);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) r[m] = src[i + m * stride];
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) acc ^= r[m];
    }
    for (; i < n16; i += stride) acc ^= src[i];
    // one store per thread keeps the loads live; the destination holds
    // gridDim.x * kPeakThreads vectors
    dst[(int64_t)blockIdx.x * kPeakThreads + threadIdx.x] = acc;
  }
}

__global__ __launch_bounds__(kPeakThreads) void peak_mfma_kernel(int64_t iters,
                                                                 float* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16 c[kMfmaChains];
  for (int j = 0; j < kMfmaChains; ++j)
    for (int e = 0; e < 16; ++e) c[j][e] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) c[j] = mfma32(a, b, c[j]);
  }
  float s = 0.0f;
  for (int j = 0; j < kMfmaChains; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  s = wave_sum(s);
  if (lane == 0) sink[((int64_t)blockIdx.x * kPeakThreads + threadIdx.x) / kWave] = s;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

}  // namespace
}  // namespace dash

extern "C" {

dash_status dash_peak_stream_grid(int64_t* threads) {
  if (!threads) return DASH_ERR_INVALID_ARG;
  const int cus = dash::device_cus();
  if (cus <= 0) return DASH_ERR_HIP;
  *threads = (int64_t)cus * 8 * dash::kPeakThreads;
  return DASH_OK;
}

dash_status dash_peak_stream(const void* src, void* dst, int64_t bytes, int32_t mode,
                             void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 != 0 || mode < 0 || mode > 2)
    return DASH_ERR_INVALID_ARG;
  if (((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0) return DASH_ERR_INVALID_ARG;
  const int cus = dash::device_cus();
  if (cus <= 0) return DASH_ERR_HIP;
  const int grid = cus * 8;
  hipLaunchKernelGGL(dash::peak_stream_kernel, dim3(grid), dim3(dash::kPeakThreads), 0,
                     (hipStream_t)stream, (const dash::u32x4*)src, (dash::u32x4*)dst, bytes / 16,
                     (int)mode);
  return hipGetLastError() == hipSuccess ? DASH_OK : DASH_ERR_HIP;
}

dash_status dash_peak_mfma_grid(int64_t* waves) {
  if (!waves) return DASH_ERR_INVALID_ARG;
  const int cus = dash::device_cus();
  if (cus <= 0) return DASH_ERR_HIP;
  *waves = (int64_t)cus * 4 * (dash::kPeakThreads / dash::kWave);
  return DASH_OK;
}

dash_status dash_peak_mfma(int64_t iters, float* sink, double* flops, void* stream) {
  if (iters < 1 || !sink || !flops) return DASH_ERR_INVALID_ARG;
  const int cus = dash::device_cus();
  if (cus <= 0) return DASH_ERR_HIP;
  const int grid = cus * 4;
  const double waves = (double)grid * (dash::kPeakThreads / dash::kWave);
  *flops = waves * (double)iters * dash::kMfmaChains * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(dash::peak_mfma_kernel, dim3(grid), dim3(dash::kPeakThreads), 0,
                     (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? DASH_OK : DASH_ERR_HIP;
}

}  // extern "C"
