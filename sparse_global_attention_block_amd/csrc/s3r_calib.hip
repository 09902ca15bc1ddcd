// Measured ceilings for the roofline figures: a streaming copy (the HBM bandwidth a plain
// kernel reaches on this chip) and a loop of independent 16x16x32 bf16 matrix products (the
// matrix-core rate a kernel reaches with nothing else to do). Neither is part of the attention;
// the benchmark divides each kernel's achieved rate by these as well as by the vendor peaks.
#include "../../include/speed3r.h"
#include "s3r_common.hpp"

namespace s3r {

constexpr int kCopyUnroll = 4;     // 16-byte loads in flight per thread
constexpr int kMfmaChains = 8;     // independent accumulators per wave

__global__ __launch_bounds__(256) void calib_copy_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256 * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x; base < n16;
       base += stride) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n16) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n16) dst[i] = v[u];
    }
  }
}

__global__ __launch_bounds__(256) void calib_mfma_kernel(float* sink, int iters) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds to a constant
  const float x = 0x1p-10f * (float)((tid & 7) + 1);
  const bf16x8 a = pack8(x, -x, x, x, -x, x, x, -x);
  const bf16x8 b = pack8(x, x, -x, x, x, -x, x, x);
  floatx4 c[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) c[j] = mfma16(a, b, c[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  sink[(int64_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace s3r

using namespace s3r;

extern "C" {

s3r_status speed3r_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16))
    return S3R_ERR_INVALID_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t wg = (n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  if (wg > 256 * 16) wg = 256 * 16;
  hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)wg), dim3(256), 0, stream,
                     (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError() == hipSuccess ? S3R_OK : S3R_ERR_HIP;
}

int64_t speed3r_calib_mfma_flops(int32_t work_groups, int32_t iters) {
  if (work_groups < 1 || iters < 1) return -1;
  return (int64_t)work_groups * 4 * iters * kMfmaChains * (16 * 16 * 32 * 2);
}

s3r_status speed3r_calib_mfma(float* sink, int32_t work_groups, int32_t iters,
                              hipStream_t stream) {
  if (!sink || ((uintptr_t)sink % 4) || work_groups < 1 || iters < 1) return S3R_ERR_INVALID_ARG;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)work_groups), dim3(256), 0, stream, sink,
                     iters);
  return hipGetLastError() == hipSuccess ? S3R_OK : S3R_ERR_HIP;
}

}  // extern "C"
