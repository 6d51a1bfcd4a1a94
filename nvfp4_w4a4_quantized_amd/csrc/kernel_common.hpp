// Device helpers shared by the GEMM and GEMV kernels: segment lookup, the epilogue
// (per-segment global scales, GDN gates, output cast), synchronization and
// waitcnt helpers, exact scale-pair conversion.
#pragma once

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

__device__ __forceinline__ int seg_of_col(const SegTable& seg, int64_t n) {
  int s = 0;
  while (s + 1 < seg.n && n >= seg.end[s]) ++s;
  return s;
}

__device__ __forceinline__ float softplus_f32(float z) {
  return __builtin_fmaxf(z, 0.0f) + log1pf(expf(-__builtin_fabsf(z)));
}

// 1/(1+e^-z), evaluated as e^z/(1+e^z) for z < 0 so that e^-z never overflows: for
// z below about -87.3 the result is an fp32 subnormal rather than 0.
__device__ __forceinline__ float sigmoid_f32(float z) {
  const float e = expf(-__builtin_fabsf(z));
  const float r = 1.0f / (1.0f + e);
  return z >= 0.0f ? r : e * r;
}

// Workgroup barrier that waits for this wave's LDS traffic only.  __syncthreads()
// would also wait for every outstanding global load (vmcnt(0)); kernels that keep a
// weight stream in flight across a barrier use this instead.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Output kinds of the epilogue (a template parameter, so that every accumulator
// index stays a compile-time constant).
enum : int { EPI_F32 = 0, EPI_BF16 = 1, EPI_GATE = 2 };

template <int EPI>
__device__ __forceinline__ float col_alpha(const GemmArgs& a, int64_t n, float ga) {
  return ga * a.w_seg_gscale[seg_of_col(a.seg, n)];
}

// Epilogue for one output element: alpha scaling, optional gate (Eq. 1), store.
template <int EPI>
__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, float acc, float alpha) {
  float v = acc * alpha;
  if constexpr (EPI == EPI_GATE) {
    const int64_t H = a.gate.n_heads;
    if (n < H) {
      const float z = v + a.gate.dt_bias[n];
      v = -expf(a.gate.A_log[n]) * softplus_f32(z);
    } else {
      v = sigmoid_f32(v);
    }
  }
  if constexpr (EPI == EPI_BF16) {
    reinterpret_cast<uint16_t*>(a.y)[m * a.ldy + n] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<float*>(a.y)[m * a.ldy + n] = v;
  }
}

// Epilogue with per-row and per-column factors: y = (acc * fp32(alpha * col)) * row,
// every product rounded once (alpha * col is folded into the caller's alpha).
template <int EPI>
__device__ __forceinline__ void store_out_rc(const GemmArgs& a, int64_t m, int64_t n, float acc, float alpha_col,
                                             float row) {
  static_assert(EPI != EPI_GATE, "no gate epilogue with row/column factors");
  const float v = (acc * alpha_col) * row;
  if constexpr (EPI == EPI_BF16) {
    reinterpret_cast<uint16_t*>(a.y)[m * a.ldy + n] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<float*>(a.y)[m * a.ldy + n] = v;
  }
}

__device__ __forceinline__ float dpp_swap_adjacent(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_barrier" ::: "memory");
}


// s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// E4M3 scale bytes of blocks (2h, 2h+1) -> f16 pair {s0, s1} (exact)
__device__ __forceinline__ f16x2 scale_pair_f16(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ f16x2 bcast(f16x2 p, int hi) {
  f16x2 r;
  if (hi) { r[0] = p[1]; r[1] = p[1]; } else { r[0] = p[0]; r[1] = p[0]; }
  return r;
}

// Raise a kernel's dynamic-LDS limit beyond the 64 KiB default, once per process:
// a function-local static is initialised exactly once even when several host
// threads make their first call together (C++11), and every later call returns the
// status of that one hipFuncSetAttribute.
template <auto Kernel>
hipError_t lds_limit_once(int bytes) {
  static const hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e;
}

#define SCHED_MFMA_VALU(n_mfma, n_valu)                          \
  _Pragma("unroll") for (int _i = 0; _i < (n_mfma); ++_i) {     \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
    __builtin_amdgcn_sched_group_barrier(0x002, (n_valu), 0);    \
  }


}  // namespace
}  // namespace nvfp4
