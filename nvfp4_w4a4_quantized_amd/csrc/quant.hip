// Activation quantization and weight packing kernels (HBM-bound).
//
// Layout: each lane owns one 16-element block of a row; a wave covers 1024
// consecutive elements of a row: 2 KiB of bf16 in, 512 B of codes and 64 B of
// scales out, all contiguous.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int seg_of(const SegTable& seg, int64_t row) {
  int s = 0;
  while (s + 1 < seg.n && row >= seg.end[s]) ++s;
  return s;
}

// Quantization: one lane = one 16-element block (two 16-byte bf16 loads or four
// fp32 loads), so the block amax needs no cross-lane step and the block scale is
// computed once per block.  One wave = a "segment" of 64 consecutive blocks (1024
// elements) of one row; QU segments per iteration with all their loads issued
// (non-temporal: x is read once) before any is used.  Segment -> (row, block)
// bookkeeping is wave-uniform and runs on the scalar unit.  The per-segment scale
// constants (global scale and fp32(1/(6g))) are computed once per workgroup into LDS.
constexpr int QU = 4;

template <InType T> struct Blk16;
template <> struct Blk16<InType::BF16> { u32x4 a, b; };
template <> struct Blk16<InType::F32> { f32x4 a, b, c, d; };

template <InType T>
__device__ __forceinline__ void load_blk16(const void* base, int64_t elem_off, Blk16<T>& r) {
  if constexpr (T == InType::BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem_off);
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
    r.c = __builtin_nontemporal_load(p + 2);
    r.d = __builtin_nontemporal_load(p + 3);
  }
}

template <InType T>
__device__ __forceinline__ void unpack_blk16(const Blk16<T>& r, float v[16]) {
  if constexpr (T == InType::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r.a[i] << 16);
      v[2 * i + 1] = __uint_as_float(r.a[i] & 0xFFFF0000u);
      v[8 + 2 * i] = __uint_as_float(r.b[i] << 16);
      v[8 + 2 * i + 1] = __uint_as_float(r.b[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = r.a[i];
      v[4 + i] = r.b[i];
      v[8 + i] = r.c[i];
      v[12 + i] = r.d[i];
    }
  }
}

template <InType T>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const void* __restrict__ x, int64_t rows,
                                                         int64_t K, int64_t ld,
                                                         const float* __restrict__ gvec, SegTable seg,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         float* __restrict__ gcopy) {
  __shared__ ScaleConsts sc_lds[kMaxSeg];
  if ((int)threadIdx.x < seg.n) sc_lds[threadIdx.x] = scale_consts(gvec[threadIdx.x]);
  if (gcopy != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *gcopy = gvec[0];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t bpr = (uint32_t)(K >> 4);            // blocks per row
  const uint32_t spr = (bpr + 63u) >> 6;              // segments per row
  const uint64_t total = (uint64_t)rows * spr;
  const uint64_t stride = (uint64_t)gridDim.x * kWaves * QU;
  for (uint64_t base = ((uint64_t)blockIdx.x * kWaves + wave) * QU; base < total; base += stride) {
    // scalar: (row, segment) of the first of the QU segments, then step through
    uint64_t row0 = base / spr;
    uint32_t sg0 = (uint32_t)(base - row0 * spr);
    Blk16<T> raw[QU];
    int64_t row[QU];
    uint32_t blk[QU];
    bool valid[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      row[u] = (int64_t)row0;
      blk[u] = sg0 * 64u + lane;
      valid[u] = (base + u) < total && blk[u] < bpr;
      if (valid[u]) load_blk16<T>(x, row[u] * ld + (int64_t)blk[u] * 16, raw[u]);
      else raw[u] = Blk16<T>{};
      if (++sg0 == spr) { sg0 = 0; ++row0; }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      float v[16];
      unpack_blk16<T>(raw[u], v);
      const float a = amax_abs<16>(v);
      const ScaleConsts sc = sc_lds[seg.n > 1 ? seg_of(seg, row[u] < rows ? row[u] : 0) : 0];
      const uint32_t sb = block_scale_byte(a, sc);
      uint32_t w[2];
      quant16(v, sb, sc.g, w);
      if (valid[u]) {
        *reinterpret_cast<uint2*>(codes + row[u] * (K >> 1) + (int64_t)blk[u] * 8) = uint2{w[0], w[1]};
        scales[row[u] * (K >> 4) + blk[u]] = (uint8_t)sb;
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t bpr = (uint32_t)(K >> 4);
  const uint32_t spr = (bpr + 63u) >> 6;
  const uint64_t total = (uint64_t)rows * spr;
  const uint64_t stride = (uint64_t)gridDim.x * kWaves * QU;
  float a = 0.0f;
  for (uint64_t base = ((uint64_t)blockIdx.x * kWaves + wave) * QU; base < total; base += stride) {
    uint64_t row0 = base / spr;
    uint32_t sg0 = (uint32_t)(base - row0 * spr);
    Blk16<T> raw[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const uint32_t blk = sg0 * 64u + lane;
      if ((base + u) < total && blk < bpr) load_blk16<T>(x, (int64_t)row0 * ld + (int64_t)blk * 16, raw[u]);
      else raw[u] = Blk16<T>{};
      if (++sg0 == spr) { sg0 = 0; ++row0; }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      float v[16];
      unpack_blk16<T>(raw[u], v);
#pragma unroll
      for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
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


// Workgroups for `items` wave-iterations of a grid-stride kernel: at most 2048
// workgroups (8 per compute unit), and the waves evenly loaded (the same number of
// iterations each, give or take one), so that no last round runs with a few waves
// only: 10240 iterations (8192 rows of 5120) run as 5120 waves of two, not 8192
// waves of which 2048 run a second one.
uint64_t grid_for(uint64_t items) {
  const uint64_t max_waves = 2048ull * kWaves;
  const uint64_t per_wave = items > max_waves ? (items + max_waves - 1) / max_waves : 1;
  const uint64_t waves = (items + per_wave - 1) / per_wave;
  uint64_t g = (waves + kWaves - 1) / kWaves;
  if (g < 1) g = 1;
  return g;
}

}  // namespace

hipError_t launch_fill(float* dst, int n, const SegTable* vals, hipStream_t s) {
  SegTable v{};
  if (vals) v = *vals;
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(kMaxSeg), 0, s, dst, n, v, vals ? 1 : 0);
  return hipGetLastError();
}


hipError_t launch_amax_gscale(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                              float* gscale_out, hipStream_t s) {
  const uint64_t items = ((uint64_t)rows * (uint64_t)((K / 16 + 63) / 64) + QU - 1) / QU;
  const unsigned grid = (unsigned)grid_for(items);
  if (t == InType::BF16) {
    hipLaunchKernelGGL(k_amax_gscale<InType::BF16>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld,
                       gscale_out);
  } else {
    hipLaunchKernelGGL(k_amax_gscale<InType::F32>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld,
                       gscale_out);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                             const float* gvec, const SegTable& seg, uint8_t* codes, uint8_t* scales,
                             float* gcopy, hipStream_t s) {
  const uint64_t items = ((uint64_t)rows * (uint64_t)((K / 16 + 63) / 64) + QU - 1) / QU;
  const unsigned grid = (unsigned)grid_for(items);
  if (t == InType::BF16) {
    hipLaunchKernelGGL(k_quant_rows<InType::BF16>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gvec,
                       seg, codes, scales, gcopy);
  } else {
    hipLaunchKernelGGL(k_quant_rows<InType::F32>, dim3(grid), dim3(kThreads), 0, s, x, rows, K, ld, gvec,
                       seg, codes, scales, gcopy);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
