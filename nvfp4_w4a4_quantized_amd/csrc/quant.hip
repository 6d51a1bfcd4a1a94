// Activation quantization and weight packing kernels (HBM-bound).
//
// Layout: each lane owns 8 consecutive elements of a row (one 16-byte bf16 load or
// two fp32 loads); lanes 2j and 2j+1 together hold one 16-element block, so the
// block amax needs one DPP swap.  A wave covers 512 consecutive elements of a row:
// 1 KiB of bf16 in, 256 B of codes and 32 B of scales out, all coalesced.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float dpp_swap_adjacent(float v) {
  // quad_perm [1,0,3,2]: exchange with the neighbouring lane
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <InType T>
__device__ __forceinline__ void load8(const void* base, int64_t elem_off, float v[8]) {
  if constexpr (T == InType::BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + elem_off;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

__device__ __forceinline__ int seg_of(const SegTable& seg, int64_t row) {
  int s = 0;
  while (s + 1 < seg.n && row >= seg.end[s]) ++s;
  return s;
}

// Each wave walks "segments" of 64 chunks (512 elements) of one row, QU segments per
// iteration with all their loads issued before any is used (4 x 16 bytes in flight
// per lane).  The per-segment scale constants (global scale and fp32(1/(6g))) are
// computed once per workgroup into LDS.
constexpr int QU = 4;

template <InType T>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const void* __restrict__ x, int64_t rows,
                                                         int64_t K, int64_t ld,
                                                         const float* __restrict__ gvec, SegTable seg,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  __shared__ ScaleConsts sc_lds[kMaxSeg];
  if ((int)threadIdx.x < seg.n) sc_lds[threadIdx.x] = scale_consts(gvec[threadIdx.x]);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t chunks = (uint32_t)(K >> 3);
  const uint32_t segs_per_row = (chunks + 63u) >> 6;
  const uint64_t total = (uint64_t)rows * segs_per_row;
  const uint64_t stride = (uint64_t)gridDim.x * kWaves * QU;
  for (uint64_t base = ((uint64_t)blockIdx.x * kWaves + wave) * QU; base < total; base += stride) {
    float v[QU][8];
    uint64_t row[QU];
    uint32_t chunk[QU];
    bool valid[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const uint64_t sgi = base + u;
      row[u] = sgi / segs_per_row;
      chunk[u] = (uint32_t)(sgi - row[u] * segs_per_row) * 64u + lane;
      valid[u] = sgi < total && chunk[u] < chunks;
      if (valid[u]) {
        load8<T>(x, (int64_t)row[u] * ld + (int64_t)chunk[u] * 8, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      float a = __builtin_fabsf(v[u][0]);
#pragma unroll
      for (int i = 1; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[u][i]));
      a = __builtin_fmaxf(a, dpp_swap_adjacent(a));
      const ScaleConsts sc = sc_lds[seg_of(seg, (int64_t)(valid[u] ? row[u] : 0))];
      const uint32_t sb = block_scale_byte(a, sc);
      const uint32_t w = quant8(v[u], sb, sc.g);
      if (valid[u]) {
        const int64_t col = (int64_t)chunk[u] * 8;
        *reinterpret_cast<uint32_t*>(codes + (int64_t)row[u] * (K >> 1) + (col >> 1)) = w;
        if ((lane & 1) == 0) scales[(int64_t)row[u] * (K >> 4) + (col >> 4)] = (uint8_t)sb;
      }
    }
  }
}

// amax over rows x K, then atomicMax of fp32(amax/2688) into *out (which the caller
// zeroed).  g is monotone in amax, so the max of the per-workgroup g is the g of
// the global amax.
template <InType T>
__global__ __launch_bounds__(kThreads) void k_amax_gscale(const void* __restrict__ x, int64_t rows,
                                                          int64_t K, int64_t ld, float* out) {
  __shared__ float red[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t chunks = (uint32_t)(K >> 3);
  const uint32_t segs_per_row = (chunks + 63u) >> 6;
  const uint64_t total = (uint64_t)rows * segs_per_row;
  float a = 0.0f;
  for (uint64_t sgi = (uint64_t)blockIdx.x * kWaves + wave; sgi < total;
       sgi += (uint64_t)gridDim.x * kWaves) {
    const uint64_t row = sgi / segs_per_row;
    const uint32_t chunk = (uint32_t)(sgi - row * segs_per_row) * 64u + lane;
    if (chunk < chunks) {
      float v[8];
      load8<T>(x, (int64_t)row * ld + (int64_t)chunk * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  if (lane == 0) red[wave] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = __builtin_fmaxf(m, red[i]);
    atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(global_scale_from_amax(m)));
  }
}

__global__ void k_fill(float* dst, int n, SegTable vals, int use_vals) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = use_vals ? vals.scale[i] : 0.0f;
}

__global__ void k_copy_scalar(const float* src, float* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

int grid_for(uint64_t segments) {
  uint64_t g = (segments + kWaves - 1) / kWaves;
  const uint64_t cap = 256ull * 16ull;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_fill(float* dst, int n, const SegTable* vals, hipStream_t s) {
  SegTable v{};
  if (vals) v = *vals;
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(kMaxSeg), 0, s, dst, n, v, vals ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_copy_scalar(const float* src, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_scalar, dim3(1), dim3(64), 0, s, src, dst);
  return hipGetLastError();
}

hipError_t launch_amax_gscale(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                              float* gscale_out, hipStream_t s) {
  const uint64_t segs = (uint64_t)rows * (uint64_t)((K / 8 + 63) / 64);
  const int grid = grid_for(segs);
  if (t == InType::BF16)
    hipLaunchKernelGGL(k_amax_gscale<InType::BF16>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gscale_out);
  else
    hipLaunchKernelGGL(k_amax_gscale<InType::F32>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gscale_out);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                             const float* gvec, const SegTable& seg, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
  const uint64_t segs = (uint64_t)rows * (uint64_t)((K / 8 + 63) / 64);
  const int grid = grid_for((segs + QU - 1) / QU);
  if (t == InType::BF16)
    hipLaunchKernelGGL(k_quant_rows<InType::BF16>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gvec, seg,
                       codes, scales);
  else
    hipLaunchKernelGGL(k_quant_rows<InType::F32>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gvec, seg,
                       codes, scales);
  return hipGetLastError();
}

}  // namespace nvfp4
