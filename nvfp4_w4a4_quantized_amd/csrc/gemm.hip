// Block-scaled W4A4 GEMM kernels for gfx950.
//
// Operands stay packed (4-bit codes + E4M3 block scales) in HBM and LDS.  Each lane
// decodes its MFMA operand in registers: 8 codes (one dword) -> f16 e2m1 values by the
// hardware fp4 conversion, times the block scale as f16 (exact: the product has <= 6
// significant bits and lies in [2^-10, 2688]).  f16 x f16 products are exact in
// fp32; MFMA accumulates in fp32.  The epilogue multiplies column n by
// g_a * g_w[segment(n)] (the per-segment global-scale repair for fused GEMMs over
// per-module-calibrated weights: "Why Gated DeltaNet Survives 4-Bit Quantization"
// review page, strengths paragraph / the paper's section 6) and optionally applies
// the GDN gates of Eq. 1 (same page, mechanism step 2).
//
// K-permutation.  A lane loads 16 contiguous bytes (32 elements) of its row; MFMA
// step t uses dword t of them.  Both operands use the same permutation of k, so the
// sum over k is unchanged, and every 8-element group a lane feeds to one MFMA lies
// inside one 16-element scale block.
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

__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

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

// ---------------------------------------------------------------------------------
// Tiled GEMM: 128 x 128 output tile per workgroup, BK = 64, 4 waves of 64 x 64,
// MFMA 32x32x16 f16.  Packed tiles are staged through LDS (codes 4 KiB + scales
// 512 B per operand per K step) with a register prefetch of the next step.
// ---------------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TBK = 64;

struct TileRegs {
  u32x4 ca, cw;     // 16 bytes of codes for A and W
  uint32_t sc;      // 4 scale bytes (A for threads < 128, W otherwise)
};

template <bool ALIGNED>
__device__ __forceinline__ u32x4 load_codes16(const uint8_t* base, int64_t row, int64_t rows, int64_t K,
                                              int64_t k0, int h) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (row >= rows) return r;
  const int64_t kk = k0 + 32 * h;             // first element of this half
  const uint8_t* p = base + row * (K >> 1) + (kk >> 1);
  if constexpr (ALIGNED) {
    r = *reinterpret_cast<const u32x4*>(p);
  } else {
    // K % 64 != 0: load 8 bytes (16 elements) at a time, only inside the row
    if (kk < K) {
      const uint2 lo = *reinterpret_cast<const uint2*>(p);
      r[0] = lo.x; r[1] = lo.y;
    }
    if (kk + 16 < K) {
      const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
      r[2] = hi.x; r[3] = hi.y;
    }
  }
  return r;
}

template <bool ALIGNED>
__device__ __forceinline__ uint32_t load_scales4(const uint8_t* base, int64_t row, int64_t rows, int64_t K,
                                                 int64_t k0) {
  if (row >= rows) return 0u;
  const int64_t kb = K >> 4;
  const uint8_t* p = base + row * kb + (k0 >> 4);
  if constexpr (ALIGNED) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else {
    uint32_t r = 0;
    for (int j = 0; j < 4; ++j)
      if ((k0 >> 4) + j < kb) r |= (uint32_t)p[j] << (8 * j);
    return r;
  }
}

template <bool ALIGNED, int EPI>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs a) {
  __shared__ u32x4 lds_ca[2][TBM];
  __shared__ u32x4 lds_cw[2][TBN];
  __shared__ uint32_t lds_sa[TBM];
  __shared__ uint32_t lds_sw[TBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;

  // tile order: groups of 8 row-tiles sweep the column tiles (L2 reuse of W)
  const int64_t tiles_m = (a.M + TBM - 1) / TBM;
  const int64_t tiles_n = (a.N + TBN - 1) / TBN;
  const int64_t pid = blockIdx.x;
  const int64_t group = 8;
  const int64_t per_group = group * tiles_n;
  const int64_t gid = pid / per_group;
  const int64_t first_m = gid * group;
  const int64_t gsize = (tiles_m - first_m) < group ? (tiles_m - first_m) : group;
  const int64_t bm = first_m + (pid % per_group) % gsize;
  const int64_t bn = (pid % per_group) / gsize;
  const int64_t m0 = bm * TBM, n0 = bn * TBN;

  // loader roles: thread -> (row, half) for codes; threads < 128 load A scales, others W
  const int lrow = tid >> 1, lh = tid & 1;
  const int srow = tid & 127;
  const bool s_is_a = tid < 128;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto gload = [&](int64_t k0) {
    TileRegs t;
    t.ca = load_codes16<ALIGNED>(a.a_codes, m0 + lrow, a.M, a.K, k0, lh);
    t.cw = load_codes16<ALIGNED>(a.w_codes, n0 + lrow, a.N, a.K, k0, lh);
    t.sc = s_is_a ? load_scales4<ALIGNED>(a.a_scales, m0 + srow, a.M, a.K, k0)
                  : load_scales4<ALIGNED>(a.w_scales, n0 + srow, a.N, a.K, k0);
    return t;
  };

  TileRegs cur = gload(0);
  for (int64_t k0 = 0; k0 < a.K; k0 += TBK) {
    lds_ca[lh][lrow] = cur.ca;
    lds_cw[lh][lrow] = cur.cw;
    if (s_is_a) lds_sa[srow] = cur.sc; else lds_sw[srow] = cur.sc;
    __syncthreads();
    if (k0 + TBK < a.K) cur = gload(k0 + TBK);

    f16x8 A[2][4], B[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + li;
      const u32x4 c = lds_ca[h][r];
      const uint32_t s = lds_sa[r] >> (16 * h);
      const f16x2 s0 = scale_f16x2(s & 0xFFu), s1 = scale_f16x2((s >> 8) & 0xFFu);
      A[i][0] = decode8_f16(c[0], s0);
      A[i][1] = decode8_f16(c[1], s0);
      A[i][2] = decode8_f16(c[2], s1);
      A[i][3] = decode8_f16(c[3], s1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn * 64 + j * 32 + li;
      const u32x4 c = lds_cw[h][r];
      const uint32_t s = lds_sw[r] >> (16 * h);
      const f16x2 s0 = scale_f16x2(s & 0xFFu), s1 = scale_f16x2((s >> 8) & 0xFFu);
      B[j][0] = decode8_f16(c[0], s0);
      B[j][1] = decode8_f16(c[1], s0);
      B[j][2] = decode8_f16(c[2], s1);
      B[j][3] = decode8_f16(c[3], s1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][t], B[j][t], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  const float ga = *a.a_gscale;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + li;
    const bool n_ok = n < a.N;
    const float alpha = n_ok ? col_alpha<EPI>(a, n, ga) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (n_ok && m < a.M) store_out<EPI>(a, m, n, acc[i][j][r], alpha);
      }
  }
}

// ---------------------------------------------------------------------------------
// Fused decode GEMV (M <= 8).  One workgroup = 64 weight rows, 8 waves: wave w takes
// rows 16*(w&3) .. +15 and half of K.  Prologue: the workgroup quantizes all of x
// (M x K) into LDS as f16 dequantized values (e2m1 * s), using the same exact
// quantizer as the stand-alone kernel.  Main loop: MFMA 16x16x32 f16 with the 16
// weight rows as the A operand and the M tokens (padded to 16 columns) as B.
// ---------------------------------------------------------------------------------
constexpr int GV_ROWS = 64;
constexpr int GV_THREADS = 512;

__device__ __forceinline__ float dpp_swap_adjacent(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <InType T>
__device__ __forceinline__ void gv_load8(const void* base, int64_t off, float v[8]) {
  if constexpr (T == InType::BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + off;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = x0[i]; v[4 + i] = x1[i]; }
  }
}

template <InType T>
__global__ __launch_bounds__(GV_THREADS) void k_gemv_fused(GemvArgs p) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];   // [M][K] f16
  __shared__ float red_g[GV_THREADS / 64];
  __shared__ f32x4 red_acc[4][64];
  const GemmArgs& a = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t M = a.M, K = a.K, N = a.N;
  const uint32_t chunks_per_row = (uint32_t)(K >> 3);
  const uint32_t total_chunks = (uint32_t)M * chunks_per_row;
  const uint32_t iters = (total_chunks + GV_THREADS - 1) / GV_THREADS;

  // ---- global scale (dynamic mode: amax over the whole of x)
  float g;
  if (p.gscale_in) {
    g = *p.gscale_in;
  } else {
    float am = 0.0f;
    for (uint32_t it = 0; it < iters; ++it) {
      const uint32_t c = it * GV_THREADS + tid;
      if (c < total_chunks) {
        const uint32_t row = c / chunks_per_row;
        const uint32_t col = (c - row * chunks_per_row) * 8u;
        float v[8];
        gv_load8<T>(p.x, (int64_t)row * p.ldx + col, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(v[i]));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red_g[wave] = am;
    __syncthreads();
    am = red_g[0];
#pragma unroll
    for (int i = 1; i < GV_THREADS / 64; ++i) am = __builtin_fmaxf(am, red_g[i]);
    g = global_scale_from_amax(am);
  }
  if (blockIdx.x == 0 && tid == 0 && p.gscale_out) *p.gscale_out = g;

  // ---- quantize x into LDS (f16 of e2m1 * s); workgroup 0 also writes the codes
  const bool write_codes = blockIdx.x == 0 && p.a_codes_out != nullptr;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t c = it * GV_THREADS + tid;
    const bool valid = c < total_chunks;
    uint32_t row = 0, col = 0;
    float v[8];
    if (valid) {
      row = c / chunks_per_row;
      col = (c - row * chunks_per_row) * 8u;
      gv_load8<T>(p.x, (int64_t)row * p.ldx + col, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float am = __builtin_fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(v[i]));
    am = __builtin_fmaxf(am, dpp_swap_adjacent(am));
    const uint32_t sb = block_scale_byte(am, g);
    const uint32_t w = quant8(v, sb, g);
    if (valid) {
      const f16x8 d = decode8_f16(w, scale_f16x2(sb));
      *reinterpret_cast<f16x8*>(xs + (int64_t)row * K + col) = d;
      if (write_codes) {
        *reinterpret_cast<uint32_t*>(p.a_codes_out + (int64_t)row * (K >> 1) + (col >> 1)) = w;
        if ((tid & 1) == 0) p.a_scales_out[(int64_t)row * (K >> 4) + (col >> 4)] = (uint8_t)sb;
      }
    }
  }
  __syncthreads();

  // ---- main loop
  const int sub = wave & 3, khalf = wave >> 2;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t wrow = (int64_t)blockIdx.x * GV_ROWS + sub * 16 + r16;   // weight row of this lane
  const bool row_ok = wrow < N;
  const int64_t n_chunks = K >> 7;                                      // 128 elements per chunk
  const int64_t c_begin = khalf ? n_chunks / 2 : 0;
  const int64_t c_end = khalf ? n_chunks : n_chunks / 2;
  const uint8_t* wc = a.w_codes + (row_ok ? wrow : 0) * (K >> 1);
  const uint8_t* wsc = a.w_scales + (row_ok ? wrow : 0) * (K >> 4);
  const int xtok = r16 % (int)M;
  const _Float16* xrow = xs + (int64_t)xtok * K;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t c = c_begin; c < c_end; ++c) {
    const u32x4 codes = row_ok ? *reinterpret_cast<const u32x4*>(wc + c * 64 + 16 * q) : u32x4{0u, 0u, 0u, 0u};
    const uint32_t s2 = row_ok ? *reinterpret_cast<const uint16_t*>(wsc + c * 8 + 2 * q) : 0u;
    const f16x2 s0 = scale_f16x2(s2 & 0xFFu), s1 = scale_f16x2(s2 >> 8);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x8 wa = decode8_f16(codes[t], t < 2 ? s0 : s1);
      const f16x8 xb = *reinterpret_cast<const f16x8*>(xrow + c * 128 + 32 * q + 8 * t);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, acc, 0, 0, 0);
    }
  }
  if (khalf) red_acc[sub][lane] = acc;
  __syncthreads();
  if (!khalf) {
    const f32x4 o = red_acc[sub][lane];
    const float ga = g;
    const int tok = r16;               // D column = token
    if (tok < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = (int64_t)blockIdx.x * GV_ROWS + sub * 16 + 4 * q + r;
        if (n < N) {
          const float alpha = ga * a.w_seg_gscale[seg_of_col(a.seg, n)];
          if (a.gate.n_heads > 0) store_out<EPI_GATE>(a, tok, n, acc[r] + o[r], alpha);
          else if (a.y_type == OutType::BF16) store_out<EPI_BF16>(a, tok, n, acc[r] + o[r], alpha);
          else store_out<EPI_F32>(a, tok, n, acc[r] + o[r], alpha);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Large-tile GEMM for prefill shapes: 256 x 256 output tile per workgroup, BK = 64,
// 4 waves of 128 x 128 (4 x 4 MFMA 32x32x16 f16, 256 fp32 accumulators per lane in
// AGPRs, so one wave per SIMD).  Decode work per wave grows with (128 + 128) while
// MFMA work grows with 128 x 128.
//
// Data movement: packed tiles (codes 16 KiB + scales 2 KiB per K step) go from HBM
// straight into a 4-stage LDS ring with gfx950's direct-to-LDS loads (no staging
// registers, no ds_write); the loads of K step k+3 are issued while step k computes.
// Before the barrier that publishes stage k+1 each wave waits only for its own loads
// of that stage (vmcnt), so two later stages stay in flight.
//
// Software pipeline inside a K step (4 MFMA steps of K = 16): while the 16 MFMAs of
// step t run, the lane decodes the operands of step t+1 (interleaved 1 MFMA : 4 VALU
// by sched_group_barrier).  The barrier sits before the last MFMA step, so the next
// K step's LDS reads and its step-0 decode run under those MFMAs.
// Requires K % 64 == 0 and K >= 192 (three K steps).
// ---------------------------------------------------------------------------------
constexpr int GBM = 256, GBN = 256, GBK = 64;

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each with its
// own L2), so workgroup id p runs on XCD p % 8.  When the tile count divides by 8,
// XCD x is given the contiguous logical tiles [x*T/8, (x+1)*T/8); logical tiles are
// ordered in groups of 4 row tiles sweeping the column tiles.  The ~32 workgroups
// an XCD runs at once then cover a 4 x 8 block of tiles: 12 operand tiles per K
// step come through its L2 instead of 33 with a plain row-group order.
__device__ __forceinline__ void big_tile_of(int64_t M, int64_t N, int64_t pid, int64_t* bm, int64_t* bn) {
  const int64_t tiles_m = (M + GBM - 1) / GBM;
  const int64_t tiles_n = (N + GBN - 1) / GBN;
  const int64_t num = tiles_m * tiles_n;
  const int64_t logical = (num % 8 == 0) ? (pid % 8) * (num / 8) + pid / 8 : pid;
  const int64_t group = 4;
  const int64_t per_group = group * tiles_n;
  const int64_t first_m = (logical / per_group) * group;
  const int64_t gsize = (tiles_m - first_m) < group ? (tiles_m - first_m) : group;
  *bm = first_m + (logical % per_group) % gsize;
  *bn = (logical % per_group) / gsize;
}
constexpr int GST = 4;                                  // LDS stages
constexpr int ST_A = 0, ST_W = 8192, ST_SA = 16384, ST_SW = 17408, ST_BYTES = 18432;

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

#define SCHED_MFMA_VALU(n_mfma, n_valu)                          \
  _Pragma("unroll") for (int _i = 0; _i < (n_mfma); ++_i) {     \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
    __builtin_amdgcn_sched_group_barrier(0x002, (n_valu), 0);    \
  }

template <int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_big(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GST * ST_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;

  int64_t bm, bn;
  big_tile_of(a.M, a.N, blockIdx.x, &bm, &bn);
  const int64_t m0 = bm * GBM, n0 = bn * GBN;
  const int64_t K = a.K;
  const int64_t kh = K >> 1, kb = K >> 4;

  // LDS stage layout: codes [row][32 B] (both halves of the row's 64 elements), the
  // two 16-byte halves of row r stored in swapped order when bit 2 xor bit 3 of r is
  // set, which makes the per-lane 16-byte reads below conflict-free; scales [row][4 B].
  // Load roles (per wave, per K step): 2 x 32 rows of A codes and of W codes (lanes
  // 2j and 2j+1 fetch the two halves of one row: 32 contiguous bytes), 64 rows of A
  // and of W scales.  Rows past M or N are clamped to the last row (in bounds; their
  // outputs are never stored).
  const uint8_t* ga_c[2];
  const uint8_t* gw_c[2];
  uint32_t lo_c[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r0 = 32 * (2 * wave + q);
    const int row = r0 + (lane >> 1);
    const int hl = (lane & 1) ^ (((row >> 2) ^ (row >> 3)) & 1);      // logical half of this slot
    const int64_t ra = min<int64_t>(m0 + row, a.M - 1);
    const int64_t rw = min<int64_t>(n0 + row, a.N - 1);
    ga_c[q] = a.a_codes + ra * kh + 16 * hl;
    gw_c[q] = a.w_codes + rw * kh + 16 * hl;
    lo_c[q] = (uint32_t)(r0 * 32);
  }
  const uint8_t* ga_s = a.a_scales + min<int64_t>(m0 + 64 * wave + lane, a.M - 1) * kb;
  const uint8_t* gw_s = a.w_scales + min<int64_t>(n0 + 64 * wave + lane, a.N - 1) * kb;
  const uint32_t lo_s = (uint32_t)(64 * wave * 4);
  auto issue = [&](int st, int64_t k0) {
    uint8_t* base = smem + st * ST_BYTES;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __builtin_amdgcn_global_load_lds(ga_c[q] + (k0 >> 1), base + ST_A + lo_c[q], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(gw_c[q] + (k0 >> 1), base + ST_W + lo_c[q], 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(ga_s + (k0 >> 4), base + ST_SA + lo_s, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(gw_s + (k0 >> 4), base + ST_SW + lo_s, 4, 0, 0);
  };

  u32x4 ca[4], cw[4];          // packed codes of this lane's rows for the current K step
  f16x2 pa[4], pw[4];          // scale pairs {block 2h, block 2h+1}
  auto lread = [&](int st) {
    const uint8_t* base = smem + st * ST_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + li;
      ca[i] = *reinterpret_cast<const u32x4*>(base + ST_A + r * 32 + 16 * (h ^ (((r >> 2) ^ (r >> 3)) & 1)));
      pa[i] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(base + ST_SA + r * 4 + 2 * h));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + li;
      cw[j] = *reinterpret_cast<const u32x4*>(base + ST_W + r * 32 + 16 * (h ^ (((r >> 2) ^ (r >> 3)) & 1)));
      pw[j] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(base + ST_SW + r * 4 + 2 * h));
    }
  };
  f16x8 A0[4], B0[4], A1[4], B1[4];
  auto decode = [&](int t, f16x8 A[4], f16x8 B[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] = decode8_f16(ca[i][t], bcast(pa[i], t >> 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) B[j] = decode8_f16(cw[j][t], bcast(pw[j], t >> 1));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mfma_step = [&](const f16x8 A[4], const f16x8 B[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
  };

  // One K step.  LOAD: issue the loads of tile k+3; NEXT: publish and read tile k+1
  // during the last MFMA step; VM: loads allowed in flight when tile k+1 is needed.
  const int64_t nk = K / GBK;
  auto kstep = [&]<bool LOAD, bool NEXT, int VM>(int64_t kt) {
    // step 0 MFMAs | decode step 1, loads of tile k+3
    mfma_step(A0, B0);
    decode(1, A1, B1);
    if constexpr (LOAD) {
      issue((int)((kt + 3) & 3), (kt + 3) * GBK);
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      SCHED_MFMA_VALU(10, 4)
    } else {
      SCHED_MFMA_VALU(16, 4)
    }
    // step 1 MFMAs | decode step 2
    mfma_step(A1, B1);
    decode(2, A0, B0);
    SCHED_MFMA_VALU(16, 4)
    // step 2 MFMAs | decode step 3
    mfma_step(A0, B0);
    decode(3, A1, B1);
    SCHED_MFMA_VALU(16, 4)
    if constexpr (NEXT) {
      wait_vmcnt<VM>();                 // this wave's loads of tile k+1 have landed
      wg_barrier();                     // ... and every other wave's
      lread((int)((kt + 1) & 3));
      mfma_step(A1, B1);
      decode(0, A0, B0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      SCHED_MFMA_VALU(12, 6)
    } else {
      mfma_step(A1, B1);
    }
  };

  issue(0, 0);
  issue(1, GBK);
  issue(2, 2 * GBK);
  wait_vmcnt<12>();
  wg_barrier();
  lread(0);
  decode(0, A0, B0);
  int64_t kt = 0;
  for (; kt + 3 < nk; ++kt) kstep.template operator()<true, true, 12>(kt);
  kstep.template operator()<false, true, 6>(kt);       // kt = nk - 3
  ++kt;
  kstep.template operator()<false, true, 0>(kt);       // kt = nk - 2
  ++kt;
  kstep.template operator()<false, false, 0>(kt);      // kt = nk - 1

  const float ga = *a.a_gscale;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + j * 32 + li;
    const bool n_ok = n < a.N;
    const float alpha = n_ok ? col_alpha<EPI>(a, n, ga) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (n_ok && m < a.M) store_out<EPI>(a, m, n, acc[i][j][r], alpha);
      }
  }
}

// ---------------------------------------------------------------------------------
// Two-waves-per-SIMD variant of the large-tile GEMM: the same 256 x 256 tile, LDS
// ring and K-step pipeline, but 8 waves of 128 x 64 (4 x 2 MFMA 32x32x16 tiles,
// 128 accumulators per lane), so that one wave's waits and decode overlap the other
// wave's MFMAs on the same SIMD.
// ---------------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_big8(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GST * ST_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, li = lane & 31;

  int64_t bm, bn;
  big_tile_of(a.M, a.N, blockIdx.x, &bm, &bn);
  const int64_t m0 = bm * GBM, n0 = bn * GBN;
  const int64_t K = a.K;
  const int64_t kh = K >> 1, kb = K >> 4;

  // loads per wave and K step: 32 rows of A codes, 32 rows of W codes (rows 32*wave ..),
  // and 64 rows of scales (waves 0-3: A, waves 4-7: W)
  const int crow = 32 * wave + (lane >> 1);
  const int hl = (lane & 1) ^ (((crow >> 2) ^ (crow >> 3)) & 1);
  const uint8_t* ga_c = a.a_codes + min<int64_t>(m0 + crow, a.M - 1) * kh + 16 * hl;
  const uint8_t* gw_c = a.w_codes + min<int64_t>(n0 + crow, a.N - 1) * kh + 16 * hl;
  const uint32_t lo_c = (uint32_t)(32 * wave * 32);
  const bool s_is_a = wave < 4;
  const int srow = 64 * (wave & 3) + lane;
  const uint8_t* g_s = s_is_a ? a.a_scales + min<int64_t>(m0 + srow, a.M - 1) * kb
                              : a.w_scales + min<int64_t>(n0 + srow, a.N - 1) * kb;
  const uint32_t lo_s = (uint32_t)((s_is_a ? ST_SA : ST_SW) + 64 * (wave & 3) * 4);

  auto issue = [&](int st, int64_t k0) {
    uint8_t* base = smem + st * ST_BYTES;
    __builtin_amdgcn_global_load_lds(ga_c + (k0 >> 1), base + ST_A + lo_c, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gw_c + (k0 >> 1), base + ST_W + lo_c, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(g_s + (k0 >> 4), base + lo_s, 4, 0, 0);
  };

  u32x4 ca[4], cw[2];
  f16x2 pa[4], pw[2];
  auto lread = [&](int st) {
    const uint8_t* base = smem + st * ST_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + li;
      ca[i] = *reinterpret_cast<const u32x4*>(base + ST_A + r * 32 + 16 * (h ^ (((r >> 2) ^ (r >> 3)) & 1)));
      pa[i] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(base + ST_SA + r * 4 + 2 * h));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn * 64 + j * 32 + li;
      cw[j] = *reinterpret_cast<const u32x4*>(base + ST_W + r * 32 + 16 * (h ^ (((r >> 2) ^ (r >> 3)) & 1)));
      pw[j] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(base + ST_SW + r * 4 + 2 * h));
    }
  };
  f16x8 A0[4], B0[2], A1[4], B1[2];
  auto decode = [&](int t, f16x8 A[4], f16x8 B[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] = decode8_f16(ca[i][t], bcast(pa[i], t >> 1));
#pragma unroll
    for (int j = 0; j < 2; ++j) B[j] = decode8_f16(cw[j][t], bcast(pw[j], t >> 1));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mfma_step = [&](const f16x8 A[4], const f16x8 B[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
  };

  const int64_t nk = K / GBK;
  auto kstep = [&]<bool LOAD, bool NEXT, int VM>(int64_t kt) {
    mfma_step(A0, B0);
    decode(1, A1, B1);
    if constexpr (LOAD) {
      issue((int)((kt + 3) & 3), (kt + 3) * GBK);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      SCHED_MFMA_VALU(5, 6)
    } else {
      SCHED_MFMA_VALU(8, 6)
    }
    mfma_step(A1, B1);
    decode(2, A0, B0);
    SCHED_MFMA_VALU(8, 6)
    mfma_step(A0, B0);
    decode(3, A1, B1);
    SCHED_MFMA_VALU(8, 6)
    if constexpr (NEXT) {
      wait_vmcnt<VM>();
      wg_barrier();
      lread((int)((kt + 1) & 3));
      mfma_step(A1, B1);
      decode(0, A0, B0);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      SCHED_MFMA_VALU(5, 10)
    } else {
      mfma_step(A1, B1);
    }
  };

  issue(0, 0);
  issue(1, GBK);
  issue(2, 2 * GBK);
  wait_vmcnt<6>();
  wg_barrier();
  lread(0);
  decode(0, A0, B0);
  int64_t kt = 0;
  for (; kt + 3 < nk; ++kt) kstep.template operator()<true, true, 6>(kt);
  kstep.template operator()<false, true, 3>(kt);
  ++kt;
  kstep.template operator()<false, true, 0>(kt);
  ++kt;
  kstep.template operator()<false, false, 0>(kt);

  const float ga = *a.a_gscale;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + li;
    const bool n_ok = n < a.N;
    const float alpha = n_ok ? col_alpha<EPI>(a, n, ga) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (n_ok && m < a.M) store_out<EPI>(a, m, n, acc[i][j][r], alpha);
      }
  }
}

// ---------------------------------------------------------------------------------
// Fused decode GEMV, streaming version (M <= 8, K % 512 == 0, K <= 8192).
// Workgroup = 512 threads = 64 weight rows: wave w takes rows 16*(w&3) .. +15 and
// half w>>2 of K.  In a wave, lane (q = lane>>4, r = lane&15) feeds the MFMA with
// row r; its 16-byte code load i covers elements 128 i + 32 q .. +31 of the wave's
// half, so the 4 lanes of a row read 64 contiguous bytes per load instruction
// (coalesced).  Order of work: (1) issue this thread's loads of x, (2) issue every
// load of the weight stream (scales first, then codes, in consumption order), (3)
// quantize x into LDS while the weight stream is in flight (x loads were issued
// first, so waiting for them does not wait for the weight; the barrier after this
// step waits for LDS traffic only), (4) consume the weight in arrival order: exact
// fp4 x E4M3 -> f16 decode, MFMA 16x16x32 with the tokens as B, four independent
// accumulators, (5) add the two K halves through LDS, epilogue.
// LDS holds x as f16 (e2m1 * s), token t at t * (2K + 16) bytes: the 4 lane groups x
// M tokens then read distinct banks.
// ---------------------------------------------------------------------------------
constexpr int GS_THREADS = 512;
constexpr int GS_ROWS = 64;
constexpr int GS_NLMAX = 32;       // 16-byte code loads per lane: K / 256 <= 32
constexpr int GS_XMAX = 10;        // x chunks (8 elements) per thread: M * K / 4096 <= 10

__host__ __device__ constexpr int64_t gs_token_stride(int64_t K) { return 2 * K + 16; }

// x chunk as loaded: bf16 stays packed (4 dwords) until it is quantized
template <InType T> struct XRaw;
template <> struct XRaw<InType::BF16> { u32x4 q; };
template <> struct XRaw<InType::F32> { f32x4 a, b; };

template <InType T>
__device__ __forceinline__ void xraw_load(const void* base, int64_t off, XRaw<T>& r) {
  if constexpr (T == InType::BF16) {
    r.q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + off);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + off;
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
  }
}

template <InType T>
__device__ __forceinline__ void xraw_unpack(const XRaw<T>& r, float v[8]) {
  if constexpr (T == InType::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r.q[i] << 16);
      v[2 * i + 1] = __uint_as_float(r.q[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = r.a[i]; v[4 + i] = r.b[i]; }
  }
}

template <InType T, int NL>
__global__ __launch_bounds__(GS_THREADS, 1) void k_gemv_stream(GemvArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t gs_lds[];
  __shared__ float red_g[GS_THREADS / 64];
  __shared__ f32x4 red_acc[4][64];
  const GemmArgs& a = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t M = a.M, K = a.K, N = a.N;
  const int64_t TS = gs_token_stride(K);

  // (1) x loads: chunk c = i * 512 + tid, 8 elements each
  const uint32_t cpr = (uint32_t)(K >> 3);         // chunks per row
  const uint32_t total_chunks = (uint32_t)M * cpr;
  XRaw<T> xr[GS_XMAX];
#pragma unroll
  for (int i = 0; i < GS_XMAX; ++i) {
    const uint32_t c = (uint32_t)i * GS_THREADS + tid;
    if (c < total_chunks) {
      const uint32_t row = c / cpr, col = (c - row * cpr) * 8u;
      xraw_load<T>(p.x, (int64_t)row * p.ldx + col, xr[i]);
    } else {
      xr[i] = XRaw<T>{};
    }
  }

  // (2) the weight stream of this lane: row n, eighth e = 4 * khalf + q
  const int rg = wave & 3, khalf = wave >> 2;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t n = (int64_t)blockIdx.x * GS_ROWS + rg * 16 + r16;
  const int64_t nc = n < N ? n : N - 1;                          // clamped: in bounds, never stored
  const int64_t kbase = khalf * (K >> 1);                        // first element of this half
  const uint8_t* wc = a.w_codes + nc * (K >> 1) + (kbase >> 1) + 16 * q;
  const uint8_t* wsc = a.w_scales + nc * (K >> 4) + (kbase >> 4) + 4 * (q >> 1);
  u32x4 codes[NL];                                // NL = K / 256 code loads per lane
  uint32_t sw[NL];                                // scale bytes of load i: (8 i + 2 q, +1)
  // scales first: loads complete in issue order, and load i needs its scale dword
#pragma unroll
  for (int i = 0; i < NL; ++i) sw[i] = *reinterpret_cast<const uint32_t*>(wsc + 8 * i);
#pragma unroll
  for (int i = 0; i < NL; ++i) codes[i] = *reinterpret_cast<const u32x4*>(wc + 64 * i);

  // (3) global scale and x quantization into LDS
  float g;
  if (p.gscale_in) {
    g = *p.gscale_in;
  } else {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < GS_XMAX; ++i) {
      float v[8];
      xraw_unpack<T>(xr[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red_g[wave] = am;
    lds_sync();
    am = red_g[0];
#pragma unroll
    for (int i = 1; i < GS_THREADS / 64; ++i) am = __builtin_fmaxf(am, red_g[i]);
    g = global_scale_from_amax(am);
  }
  const ScaleConsts sc = scale_consts(g);
  // activation codes for the optional outputs, stored after the main loop: a global
  // store before the LDS barrier would make the compiler drain vmcnt, i.e. wait for
  // the whole weight stream
  uint32_t wq[GS_XMAX], sq[GS_XMAX];
#pragma unroll
  for (int i = 0; i < GS_XMAX; ++i) {
    wq[i] = 0u;
    sq[i] = 0u;
    const uint32_t c = (uint32_t)i * GS_THREADS + tid;
    if ((uint32_t)i * GS_THREADS >= total_chunks) break;          // uniform across the workgroup
    float xv[8];
    xraw_unpack<T>(xr[i], xv);
    float am = __builtin_fabsf(xv[0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(xv[e]));
    am = __builtin_fmaxf(am, dpp_swap_adjacent(am));
    const uint32_t sb = block_scale_byte(am, sc);
    const uint32_t w = quant8(xv, sb, g);
    if (c < total_chunks) {
      const uint32_t row = c / cpr, col = (c - row * cpr) * 8u;
      const f16x8 d = decode8_f16(w, scale_f16x2(sb));
      *reinterpret_cast<f16x8*>(gs_lds + row * TS + 2 * (int64_t)col) = d;
      wq[i] = w;
      sq[i] = sb;
    }
  }
  lds_sync();

  // (4) main loop over this lane's eighth of K
  const int xtok = r16 % (int)M;
  const uint8_t* xrow = gs_lds + xtok * TS + 2 * kbase + 64 * q;
  // four independent accumulators (one per MFMA step of a 16-byte code load) keep
  // the MFMAs out of a single dependency chain
  f32x4 acc4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const f16x2 sp = scale_pair_f16(sw[i] >> (16 * (q & 1)));     // {block 8i+2q, 8i+2q+1}
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x8 wa = decode8_f16(codes[i][t], bcast(sp, t >> 1));
      const f16x8 xb = *reinterpret_cast<const f16x8*>(xrow + 2 * (128 * i + 8 * t));
      acc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, acc4[t], 0, 0, 0);
    }
  }
  const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);

  if (blockIdx.x == 0) {
    if (tid == 0 && p.gscale_out) *p.gscale_out = g;
    if (p.a_codes_out != nullptr) {
#pragma unroll
      for (int i = 0; i < GS_XMAX; ++i) {
        const uint32_t c = (uint32_t)i * GS_THREADS + tid;
        if (c < total_chunks) {
          const uint32_t row = c / cpr, col = (c - row * cpr) * 8u;
          *reinterpret_cast<uint32_t*>(p.a_codes_out + (int64_t)row * (K >> 1) + (col >> 1)) = wq[i];
          if ((tid & 1) == 0) p.a_scales_out[(int64_t)row * (K >> 4) + (col >> 4)] = (uint8_t)sq[i];
        }
      }
    }
  }

  // (5) combine the two K halves, epilogue
  if (khalf) red_acc[rg][lane] = acc;
  __syncthreads();
  if (!khalf) {
    const f32x4 o = red_acc[rg][lane];
    const int tok = r16;                                   // D column = token
    if (tok < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t nn = (int64_t)blockIdx.x * GS_ROWS + rg * 16 + 4 * q + r;
        if (nn < N) {
          const float alpha = g * a.w_seg_gscale[seg_of_col(a.seg, nn)];
          if (a.gate.n_heads > 0) store_out<EPI_GATE>(a, tok, nn, acc[r] + o[r], alpha);
          else if (a.y_type == OutType::BF16) store_out<EPI_BF16>(a, tok, nn, acc[r] + o[r], alpha);
          else store_out<EPI_F32>(a, tok, nn, acc[r] + o[r], alpha);
        }
      }
    }
  }
}

}  // namespace

template <int EPI>
static hipError_t launch_gemm_epi(const GemmArgs& a, hipStream_t s) {
  if (EPI != EPI_GATE && a.K % GBK == 0 && a.K >= 3 * GBK && a.M >= 512 && a.N >= 512) {
    const int64_t big_tiles = ((a.M + GBM - 1) / GBM) * ((a.N + GBN - 1) / GBN);
    if constexpr (EPI != EPI_GATE) {
      hipLaunchKernelGGL(k_gemm_big<EPI>, dim3((unsigned)big_tiles), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  const int64_t tiles = ((a.M + TBM - 1) / TBM) * ((a.N + TBN - 1) / TBN);
  if (a.K % 64 == 0)
    hipLaunchKernelGGL((k_gemm_tiled<true, EPI>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_tiled<false, EPI>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t s) {
  if (a.gate.n_heads > 0) return launch_gemm_epi<EPI_GATE>(a, s);
  if (a.y_type == OutType::BF16) return launch_gemm_epi<EPI_BF16>(a, s);
  return launch_gemm_epi<EPI_F32>(a, s);
}

size_t gemv_lds_bytes(int64_t M, int64_t K) { return (size_t)M * (size_t)K * 2; }

template <InType T, int NL>
static hipError_t launch_stream(const GemvArgs& p, unsigned grid, size_t lds, hipStream_t s) {
  // allow dynamic LDS beyond the 64 KiB default (set once per instantiation)
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_stream<T, NL>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv_stream<T, NL>), dim3(grid), dim3(GS_THREADS), lds, s, p);
  return hipGetLastError();
}

bool gemv_stream_fits(int64_t M, int64_t K, InType t) {
  const int64_t chunks_per_thread = (M * K / 8 + GS_THREADS - 1) / GS_THREADS;
  return M <= 8 && K % 512 == 0 && K >= 512 && K / 256 <= GS_NLMAX && chunks_per_thread <= GS_XMAX &&
         (t == InType::BF16 || chunks_per_thread <= 5) && M * gs_token_stride(K) <= 128 * 1024;
}

hipError_t launch_gemv_fused(const GemvArgs& p, hipStream_t s) {
  if (gemv_stream_fits(p.g.M, p.g.K, p.x_type)) {
    const unsigned grid = (unsigned)((p.g.N + GS_ROWS - 1) / GS_ROWS);
    const size_t lds = (size_t)p.g.M * (size_t)gs_token_stride(p.g.K);
    switch ((int)(p.g.K / 256)) {
#define NVFP4_GS_CASE(nl)                                                                  \
  case nl:                                                                                 \
    return p.x_type == InType::BF16 ? launch_stream<InType::BF16, nl>(p, grid, lds, s)    \
                                    : launch_stream<InType::F32, nl>(p, grid, lds, s);
      NVFP4_GS_CASE(2) NVFP4_GS_CASE(4) NVFP4_GS_CASE(6) NVFP4_GS_CASE(8) NVFP4_GS_CASE(10)
      NVFP4_GS_CASE(12) NVFP4_GS_CASE(14) NVFP4_GS_CASE(16) NVFP4_GS_CASE(18) NVFP4_GS_CASE(20)
      NVFP4_GS_CASE(22) NVFP4_GS_CASE(24) NVFP4_GS_CASE(26) NVFP4_GS_CASE(28) NVFP4_GS_CASE(30)
      NVFP4_GS_CASE(32)
#undef NVFP4_GS_CASE
      default: break;
    }
  }
  const unsigned grid = (unsigned)((p.g.N + GV_ROWS - 1) / GV_ROWS);
  const size_t lds = gemv_lds_bytes(p.g.M, p.g.K);
  if (p.x_type == InType::BF16)
    hipLaunchKernelGGL(k_gemv_fused<InType::BF16>, dim3(grid), dim3(GV_THREADS), lds, s, p);
  else
    hipLaunchKernelGGL(k_gemv_fused<InType::F32>, dim3(grid), dim3(GV_THREADS), lds, s, p);
  return hipGetLastError();
}

}  // namespace nvfp4
