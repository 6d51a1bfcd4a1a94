// Fused decode GEMV kernels (M <= 8 tokens): quantize x, stream the packed weight,
// exact fp4 x E4M3 -> f16 decode, MFMA with fp32 accumulation, per-segment epilogue.
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

// ---------------------------------------------------------------------------------
// Fused decode GEMV (M <= 8).  One workgroup = 64 weight rows, 8 waves: wave w takes
// rows 16*(w&3) .. +15 and half of K.  Prologue: the workgroup quantizes all of x
// (M x K) into LDS as f16 dequantized values (e2m1 * s), using the same exact
// quantizer as the stand-alone kernel.  Main loop: MFMA 16x16x32 f16 with the 16
// weight rows as the A operand and the M tokens (padded to 16 columns) as B.
// ---------------------------------------------------------------------------------
constexpr int GV_ROWS = 64;
constexpr int GV_THREADS = 512;


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
// LDS bytes of the workgroup's weight scales: 64 rows x K/16 bytes, filled by
// ceil(K / 2048) direct-to-LDS load instructions of 512 x 16 bytes
__host__ __device__ constexpr int64_t gs_scale_bytes(int64_t K) { return ((K + 2047) / 2048) * 8192; }
__host__ __device__ constexpr int64_t gs_lds_bytes(int64_t M, int64_t K) {
  return M * gs_token_stride(K) + gs_scale_bytes(K);
}

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

template <InType T, int NL, int NA>
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
  const int64_t kb = K >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * GS_ROWS;
  uint8_t* const sc_lds = gs_lds + M * TS;                      // [64 rows][K/16] scale bytes

  // (0) the workgroup's weight scales (64 contiguous rows of K/16 bytes) straight into
  // LDS: 16-byte units u = j * 512 + tid.  Units past the last row clamp their source
  // (in bounds; those rows are never stored).  Issued first, so that waiting for any
  // later load also waits for them.
  {
    const int64_t last = (min<int64_t>(N, n0 + GS_ROWS) - n0) * kb - 16;
#pragma unroll
    for (int j = 0; j < (NL + 7) / 8; ++j) {
      const int64_t u = (int64_t)j * GS_THREADS + tid;
      __builtin_amdgcn_global_load_lds(a.w_scales + n0 * kb + min<int64_t>(16 * u, last),
                                       sc_lds + j * 8192 + wave * 1024, 16, 0, 0);
    }
    asm volatile("" ::: "memory");
  }

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
  const u32x4* wc = reinterpret_cast<const u32x4*>(a.w_codes + nc * (K >> 1) + (kbase >> 1) + 16 * q);
  u32x4 codes[NL];                                // NL = K / 256 code loads per lane
  // the first NA code loads now (non-temporal: the weight is streamed once), the rest
  // from inside the main loop, NA loads ahead of their use
#pragma unroll
  for (int i = 0; i < NA; ++i) codes[i] = __builtin_nontemporal_load(wc + 4 * i);

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
  wait_vmcnt<NA>();        // the scale loads (issued before everything else) have landed
  lds_sync();

  // (4) main loop over this lane's eighth of K
  const int xtok = r16 % (int)M;
  const uint8_t* xrow = gs_lds + xtok * TS + 2 * kbase + 64 * q;
  // four independent accumulators (one per MFMA step of a 16-byte code load) keep
  // the MFMAs out of a single dependency chain
  f32x4 acc4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* srow = sc_lds + (rg * 16 + r16) * kb + (kbase >> 4) + 2 * q;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (i + NA < NL) codes[i + NA] = __builtin_nontemporal_load(wc + 4 * (i + NA));
    const f16x2 sp = scale_pair_f16(*reinterpret_cast<const uint16_t*>(srow + 8 * i));   // {block 8i+2q, +1}
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

size_t gemv_lds_bytes(int64_t M, int64_t K) { return (size_t)M * (size_t)K * 2; }

// Code loads issued before the x quantization (the rest stream in from the main
// loop, that many loads ahead).  Measured at 4 x 16384 x 5120: a quarter beats
// issuing them all up front (17.6 vs 19.8 us per call back to back), since a wave
// blocked on issuing loads cannot quantize x meanwhile.
#ifndef NVFP4_GEMV_AHEAD
#define NVFP4_GEMV_AHEAD(nl) ((nl) / 4)
#endif

template <InType T, int NL>
static hipError_t launch_stream(const GemvArgs& p, unsigned grid, size_t lds, hipStream_t s) {
  constexpr int NA = NVFP4_GEMV_AHEAD(NL);
  // allow dynamic LDS beyond the 64 KiB default (set once per instantiation)
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_stream<T, NL, NA>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 152 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv_stream<T, NL, NA>), dim3(grid), dim3(GS_THREADS), lds, s, p);
  return hipGetLastError();
}

bool gemv_stream_fits(int64_t M, int64_t K, InType t) {
  const int64_t chunks_per_thread = (M * K / 8 + GS_THREADS - 1) / GS_THREADS;
  return M <= 8 && K % 512 == 0 && K >= 512 && K / 256 <= GS_NLMAX && chunks_per_thread <= GS_XMAX &&
         (t == InType::BF16 || chunks_per_thread <= 5) && gs_lds_bytes(M, K) <= 152 * 1024;
}

hipError_t launch_gemv_fused(const GemvArgs& p, hipStream_t s) {
  if (gemv_stream_fits(p.g.M, p.g.K, p.x_type)) {
    const unsigned grid = (unsigned)((p.g.N + GS_ROWS - 1) / GS_ROWS);
    const size_t lds = (size_t)gs_lds_bytes(p.g.M, p.g.K);
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
