// Measurement helper: the f16 MFMA issue rate the chip sustains at the clock it holds
// under matrix load, for reporting achievable peaks beside the datasheet ones.  Each
// wave keeps four independent 32x32x16 f16 MFMA accumulation chains busy and touches
// memory only once, at the end (so the result is not optimized away).
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(256) void k_mfma_peak(int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int64_t iters, int32_t n_blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(n_blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace nvfp4
