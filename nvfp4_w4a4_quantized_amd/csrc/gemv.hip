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

  // (0) the calibrated global scale, loaded before anything else: vmcnt counts loads
  // in issue order, so waiting for it then waits for no other load.  The load is
  // unconditional (from an always-valid address in dynamic mode, result unused there).
  const float g_in = *(p.gscale_in ? p.gscale_in : a.w_seg_gscale);
  asm volatile("" ::: "memory");

  // (1) x loads first (the quantization waits for them, and vmcnt counts in issue
  // order): chunk c = i * 512 + tid, 8 elements each.  Chunks past the end load
  // the last chunk again (unconditional loads: no branch, so the compiler never has
  // to wait for a load to merge control flow); only chunks < total are used.  The row
  // of a chunk is found by comparisons (M <= 8), not by a division.
  const uint32_t cpr = (uint32_t)(K >> 3);         // chunks per row
  const uint32_t total_chunks = (uint32_t)M * cpr;
  auto chunk_row = [&](uint32_t c) {
    uint32_t row = 0;
#pragma unroll
    for (int r = 1; r < 8; ++r) row += (r < M && c >= (uint32_t)r * cpr) ? 1u : 0u;
    return row;
  };
  XRaw<T> xr[GS_XMAX];
#pragma unroll
  for (int i = 0; i < GS_XMAX; ++i) {
    if ((uint32_t)i * GS_THREADS < total_chunks) {                // uniform across the workgroup
      const uint32_t c = min((uint32_t)i * GS_THREADS + tid, total_chunks - 1);
      const uint32_t row = chunk_row(c), col = (c - row * cpr) * 8u;
      xraw_load<T>(p.x, (int64_t)row * p.ldx + col, xr[i]);
    }
  }

  // (2a) the workgroup's weight scales (64 contiguous rows of K/16 bytes) straight into
  // LDS: 16-byte units u = j * 512 + tid.  Units past the last row clamp their source
  // (in bounds; those rows are never stored).  Issued after x and before the codes:
  // the x quantization waits for x only, and waiting for any code also waits for them.
  asm volatile("" ::: "memory");                                 // keep the x loads first
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

  // (2b) the weight stream of this lane: row n, eighth e = 4 * khalf + q
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
    g = g_in;
  } else {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < GS_XMAX; ++i) {
      if ((uint32_t)i * GS_THREADS < total_chunks) {              // chunks that were loaded
        float v[8];
        xraw_unpack<T>(xr[i], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
      }
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
    if ((uint32_t)i * GS_THREADS < total_chunks) {                // uniform across the workgroup
      float xv[8];
      xraw_unpack<T>(xr[i], xv);
      float am = __builtin_fabsf(xv[0]);
#pragma unroll
      for (int e = 1; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(xv[e]));
      am = __builtin_fmaxf(am, dpp_swap_adjacent(am));
      const uint32_t sb = block_scale_byte(am, sc);
      const uint32_t w = quant8(xv, sb, g);
      if (c < total_chunks) {
        const uint32_t row = chunk_row(c), col = (c - row * cpr) * 8u;
        const f16x8 d = decode8_f16(w, scale_f16x2(sb));
        *reinterpret_cast<f16x8*>(gs_lds + row * TS + 2 * (int64_t)col) = d;
        wq[i] = w;
        sq[i] = sb;
      }
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
    __builtin_amdgcn_sched_barrier(0);    // keep the load here: the scheduler would sink it to its use
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
          const uint32_t row = chunk_row(c), col = (c - row * cpr) * 8u;
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


// ---------------------------------------------------------------------------------
// Fused decode GEMV, two wave roles (M <= 8, K % 1024 == 0).  Workgroup = 1024
// threads = 64 weight rows.
//  * stream waves 0-7: wave w takes rows 16*(w&3) .. +15 and half w>>2 of K, with the
//    lane layout of k_gemv_stream.  Once x has landed they issue the first NA code
//    loads of their stream (non-temporal: read once), wait for the quantized x, then
//    consume the stream in arrival order (MFMA 16x16x32, tokens as B) issuing each
//    further load NA ahead.  (x is loaded first by every workgroup: issued behind
//    the stream it would be queued behind it.)
//  * x waves 8-15: bring x and the workgroup's weight scales into LDS (direct-to-LDS
//    loads), (dynamic mode) reduce the amax, and quantize x in LDS, in place, to f16
//    e2m1 * s.  fp32 x is staged in a region of its own and quantized from there.
// A wave that issues more loads than the memory system takes stalls at issue, and the
// quantization is VALU work: with the roles apart, the x waves quantize while the
// stream waves wait on their loads.  The two K halves are added through LDS.
// ---------------------------------------------------------------------------------
constexpr int GW_THREADS = 1024;
constexpr int GW_STREAM = 512;     // threads of the stream waves
constexpr int GW_XT = 512;         // threads of the x waves
// dynamic LDS limit: 160 KiB per workgroup minus the kernel's static LDS (4 KiB + 32 B)
constexpr int GW_LDS_MAX = 152 * 1024;

// LDS bytes of the workgroup's weight scales: 64 rows x K/16 bytes, filled by
// ceil(K / 2048) direct-to-LDS load instructions of 512 x 16 bytes
__host__ __device__ constexpr int64_t gw_scale_bytes(int64_t K) { return ((K + 2047) / 2048) * 8192; }
// LDS bytes: x as f16 (bf16 input is staged in place there), the weight scales, and
// for fp32 input a staging region of M x K x 4 bytes
__host__ __device__ constexpr int64_t gw_lds_bytes(int64_t M, int64_t K, bool f32_in) {
  return M * gs_token_stride(K) + gw_scale_bytes(K) + (f32_in ? M * K * 4 : 0);
}

template <InType T, int NL, int NA>
__global__ __launch_bounds__(GW_THREADS, 1) void k_gemv_ws(GemvArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t gw_lds[];
  __shared__ float red_g[8];
  __shared__ f32x4 red_acc[4][64];
  const GemmArgs& a = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t M = a.M, K = a.K, N = a.N;
  const int64_t TS = gs_token_stride(K);
  const int64_t kb = K >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * GS_ROWS;
  uint8_t* const sc_lds = gw_lds + M * TS;                      // [64 rows][K/16] scale bytes
  const bool dynamic = (p.gscale_in == nullptr);
  // calibrated global scale (a scalar load; from an always-valid address in dynamic
  // mode, where the value is unused)
  const float g_in = *(dynamic ? a.w_seg_gscale : p.gscale_in);

  if (wave < 8) {
    // ---- stream wave ----
    const int rg = wave & 3, khalf = wave >> 2;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t kbase = khalf * (K >> 1);                      // first element of this half
    const int64_t nrow = n0 + rg * 16 + r16;
    const u32x4* wc = reinterpret_cast<const u32x4*>(a.w_codes + (nrow < N ? nrow : N - 1) * (K >> 1) +
                                                     (kbase >> 1) + 16 * q);   // row clamped: in bounds, never stored
    u32x4 codes[NL];
    lds_sync();                                                  // barrier X (x issued)
#pragma unroll
    for (int i = 0; i < NA; ++i) codes[i] = __builtin_nontemporal_load(wc + 4 * i);
    if (dynamic) lds_sync();                                     // barrier A (amax partials)
    lds_sync();                                                  // barrier B (x and scales in LDS)

    const int xtok = r16 % (int)M;
    const uint8_t* xrow = gw_lds + xtok * TS + 2 * kbase + 64 * q;
    const uint8_t* srow = sc_lds + (rg * 16 + r16) * kb + (kbase >> 4) + 2 * q;
    f32x4 acc4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (i + NA < NL) codes[i + NA] = __builtin_nontemporal_load(wc + 4 * (i + NA));
      __builtin_amdgcn_sched_barrier(0);    // keep the load here: the scheduler would sink it to its use
      const f16x2 sp = scale_pair_f16(*reinterpret_cast<const uint16_t*>(srow + 8 * i));   // {block 8i+2q, +1}
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x8 wa = decode8_f16(codes[i][t], bcast(sp, t >> 1));
        const f16x8 xb = *reinterpret_cast<const f16x8*>(xrow + 2 * (128 * i + 8 * t));
        acc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, acc4[t], 0, 0, 0);
      }
    }
    const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    if (khalf) red_acc[rg][lane] = acc;
    __syncthreads();                                             // barrier C
    if (!khalf) {
      float g = g_in;
      if (dynamic) {
        float am = red_g[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) am = __builtin_fmaxf(am, red_g[i]);
        g = global_scale_from_amax(am);
      }
      const f32x4 o = red_acc[rg][lane];
      const int tok = r16;                                       // D column = token
      if (tok < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t nn = n0 + rg * 16 + 4 * q + r;
          if (nn < N) {
            const float alpha = g * a.w_seg_gscale[seg_of_col(a.seg, nn)];
            if (a.gate.n_heads > 0) store_out<EPI_GATE>(a, tok, nn, acc[r] + o[r], alpha);
            else if (a.y_type == OutType::BF16) store_out<EPI_BF16>(a, tok, nn, acc[r] + o[r], alpha);
            else store_out<EPI_F32>(a, tok, nn, acc[r] + o[r], alpha);
          }
        }
      }
    }
    return;
  }

  // ---- x wave ----  Thread xt handles the 16-element blocks b = i * 512 + xt; x wave v
  // owns, for each i, the 64 consecutive blocks [i * 512 + 64 v, +64) (K % 1024 == 0:
  // a multiple of 64 blocks per row, so never split across rows) and brings exactly
  // those into LDS itself, so waiting for its own loads is all the synchronisation it
  // needs.  One lane quantizes one whole block: no cross-lane step.
  const int xt = tid - GW_STREAM;                                // 0 .. 511
  const int xw = wave - 8;
  const uint32_t bpr = (uint32_t)(K >> 4);                       // blocks per row
  const uint32_t total = (uint32_t)M * bpr;
  const int niter = (int)((total + GW_XT - 1) / GW_XT);
  constexpr int BB = (T == InType::BF16) ? 32 : 64;              // bytes per block as stored
  uint8_t* const xstage = (T == InType::BF16) ? gw_lds : sc_lds + gw_scale_bytes(K);
  const int64_t sstride = (T == InType::BF16) ? TS : K * 4;      // staging bytes per token row
  // row and block column of this wave's first block of step i (wave-uniform: the
  // division runs on the scalar unit)
  auto wave_block = [&](int i, uint32_t& row, uint32_t& bc) {
    const uint32_t b0 = __builtin_amdgcn_readfirstlane((uint32_t)i * GW_XT + 64u * (uint32_t)xw);
    row = b0 / bpr;
    bc = b0 - row * bpr;
  };
  auto wave_has = [&](int i) { return (uint32_t)i * GW_XT + 64u * (uint32_t)xw < total; };
  for (int i = 0; i < niter; ++i) {
    if (wave_has(i)) {
      uint32_t row, bc;
      wave_block(i, row, bc);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(p.x) + ((int64_t)row * p.ldx + bc * 16u) * (BB / 16);
      uint8_t* dst = xstage + (int64_t)row * sstride + (int64_t)bc * BB;
#pragma unroll
      for (int h = 0; h < BB / 16; ++h)
        __builtin_amdgcn_global_load_lds(src + 1024 * h + 16 * lane, dst + 1024 * h, 16, 0, 0);
    }
  }
  // the weight scales (64 contiguous rows of K/16 bytes): 16-byte units
  // u = j * 512 + xt at LDS offset 16 u; units past the last row clamp their source
  // (in bounds; those rows are never stored)
  {
    const int64_t last = (min<int64_t>(N, n0 + GS_ROWS) - n0) * kb - 16;
    const int nj = (int)((K + 2047) / 2048);
    for (int j = 0; j < nj; ++j) {
      const int64_t u = (int64_t)j * GW_XT + xt;
      __builtin_amdgcn_global_load_lds(a.w_scales + n0 * kb + min<int64_t>(16 * u, last),
                                       sc_lds + j * 8192 + xw * 1024, 16, 0, 0);
    }
  }
  // Both issued before the stream: once the stream waves issue their loads, a load
  // issued here would wait in the same queue behind them.
  lds_sync();                                                    // barrier X: the stream starts now
  wait_vmcnt<0>();                                               // this wave's x and scales are in LDS

  // this lane's block of step i: staging offset, f16 offset, row, block column
  auto lane_block = [&](int i, int64_t& soff, int64_t& xoff, uint32_t& row, uint32_t& bc) {
    wave_block(i, row, bc);
    bc += (uint32_t)lane;
    soff = (int64_t)row * sstride + (int64_t)bc * BB;
    xoff = (int64_t)row * TS + (int64_t)bc * 32;
  };
  auto load_block = [&](int64_t soff, float v[16]) {
    const uint8_t* sp = xstage + soff;
    if constexpr (T == InType::BF16) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 q4 = *reinterpret_cast<const u32x4*>(sp + 16 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * hh + 2 * e] = __uint_as_float(q4[e] << 16);
          v[8 * hh + 2 * e + 1] = __uint_as_float(q4[e] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(sp + 16 * qq);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * qq + e] = f[e];
      }
    }
  };
  float g = g_in;
  if (dynamic) {
    float am = 0.0f;
    for (int i = 0; i < niter; ++i) {
      if (wave_has(i)) {
        int64_t soff, xoff;
        uint32_t row, bc;
        lane_block(i, soff, xoff, row, bc);
        float v[16];
        load_block(soff, v);
#pragma unroll
        for (int e = 0; e < 16; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red_g[xw] = am;
    lds_sync();                                                  // barrier A
    am = red_g[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) am = __builtin_fmaxf(am, red_g[i]);
    g = global_scale_from_amax(am);
  }
  const ScaleConsts sc = scale_consts(g);
  const bool codes_out = (blockIdx.x == 0) && (p.a_codes_out != nullptr);
#pragma unroll 1
  for (int i = 0; i < niter; ++i) {
    if (wave_has(i)) {
      int64_t soff, xoff;
      uint32_t row, bc;
      lane_block(i, soff, xoff, row, bc);
      float xv[16];
      load_block(soff, xv);
      float am = __builtin_fabsf(xv[0]);
#pragma unroll
      for (int e = 1; e < 16; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(xv[e]));
      const uint32_t sb = block_scale_byte(am, sc);
      uint32_t w[2];
      quant16(xv, sb, g, w);
      const f16x2 s2 = scale_f16x2(sb);
      *reinterpret_cast<f16x8*>(gw_lds + xoff) = decode8_f16(w[0], s2);
      *reinterpret_cast<f16x8*>(gw_lds + xoff + 16) = decode8_f16(w[1], s2);
      if (codes_out) {
        *reinterpret_cast<u32x2*>(p.a_codes_out + (int64_t)row * (K >> 1) + bc * 8u) = u32x2{w[0], w[1]};
        p.a_scales_out[(int64_t)row * (K >> 4) + bc] = (uint8_t)sb;
      }
    }
  }
  if (blockIdx.x == 0 && xt == 0 && p.gscale_out) *p.gscale_out = g;
  lds_sync();                                                    // barrier B
  __syncthreads();                                               // barrier C
}


// ---------------------------------------------------------------------------------
// Fused decode GEMV for M <= 4 tokens, K % 512 == 0, 2 <= K / 512 <= 16 (the decode
// shape 4 x 16384 x 5120 among them).  Workgroup = 64 weight rows, one wave per
// 512-element K slice.  MFMA 4x4x4 f16 (16 blocks): block b = lane >> 2 takes the
// slice's K positions 32 b .. 32 b + 31; A lane (b, i = lane & 3) = weight row i of
// the current group of four rows, B lane (b, j = lane & 3) = token j, so four tokens
// fill the B columns with no padding.  Lane layout of this instruction (measured on
// the GPU with one-hot operands): A[i][k] of block b in lane 4 b + i, element k;
// B[k][j] in lane 4 b + j, element k; D[i][j] in lane 4 b + j, register i.
//  * weight: load r (0..15) brings rows 4 r .. 4 r + 3: lane (b, i) reads the 16
//    bytes of row 4 r + i at chunk b of the slice, so each instruction reads four
//    rows' 256 bytes as whole cache lines (the 16-rows-by-64-bytes pattern of the
//    other decode kernels reads half lines and streams about 25% slower).
//  * x: lane (b, j) loads token j's 32 elements of chunk b, quantizes them in the lane
//    (two whole 16-element blocks, the exact quantizer of the stand-alone kernel) and
//    keeps them as f16 e2m1 * s for all 16 row groups: no LDS and, with a calibrated
//    scale, no barrier before the stream is consumed.
//  * weight scales: the slice's 32 bytes of each of the 64 rows go to LDS by two
//    direct-to-LDS loads per wave, read by the same wave only.
//  * end: a butterfly over the 16 blocks (lane bits 5, 4, 3, 2) leaves lane (b, j)
//    with rows 4 b .. 4 b + 3 of token j; the slices are added through LDS in slice
//    order; epilogue.
// ---------------------------------------------------------------------------------
constexpr int G4_RG = 16;                // groups of four weight rows per workgroup (64 rows)
// Weight loads in flight per lane in the main loop, and how many of them are issued
// before the x quantization.  Measured at 4 x 16384 x 5120: loads issued ahead of the
// quantization stall the wave at issue once the memory system stops taking them, and
// the quantization waits behind them (8 ahead: 14.0 us, 12: 15.0, 16: 19.7; 2-6 ahead
// of the quantization with 8 in the loop are within noise of each other).
constexpr int G4_NA = 8;
constexpr int G4_NA0 = 4;
constexpr int G4_MAXW = 16;              // K / 512 <= 16

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int64_t g4_lds_bytes(int nw, int rg) { return (int64_t)nw * 4 * rg * (32 + 16) + 64; }

template <InType T> struct G4X;                       // 32 elements of one token
template <> struct G4X<InType::BF16> { u32x4 q[4]; };
template <> struct G4X<InType::F32> { f32x4 q[8]; };

template <InType T>
__device__ __forceinline__ void g4x_load(const void* base, int64_t elem_off, G4X<T>& r) {
  if constexpr (T == InType::BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = p[i];
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.q[i] = p[i];
  }
}

template <InType T>
__device__ __forceinline__ void g4x_unpack(const G4X<T>& r, float v[32]) {
  if constexpr (T == InType::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * i + 2 * e] = __uint_as_float(r.q[i][e] << 16);
        v[8 * i + 2 * e + 1] = __uint_as_float(r.q[i][e] & 0xFFFF0000u);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = r.q[i][e];
  }
}

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 v, int m) {
  f32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = __shfl_xor(v[c], m);
  return r;
}

// One butterfly step over lane bit `bit`: of the 2h row-group accumulators in[],
// lanes with the bit clear keep the first h and add their partner's, lanes with the
// bit set keep the second h.
template <int H>
__device__ __forceinline__ void g4_fold(const f32x4* in, f32x4* out, int lane, int bit) {
  const bool hi = (lane & bit) != 0;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const f32x4 mine = hi ? in[H + k] : in[k];
    const f32x4 give = hi ? in[k] : in[H + k];
    out[k] = mine + shfl_xor4(give, bit);
  }
}

// The same step over lane bit 5 (bit 4) by v_permlane32_swap (v_permlane16_swap): the
// swap of the upper half of in[k] with the lower half of in[H + k] (of the odd 16-lane
// rows of in[k] with the even rows of in[H + k]) leaves every lane holding its own kept
// value and its partner's in the two results, with no LDS round trip.
template <int H>
__device__ __forceinline__ void g4_fold_swap32(const f32x4* in, f32x4* out) {
#pragma unroll
  for (int k = 0; k < H; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(in[k][c]), __float_as_uint(in[H + k][c]), false, false);
      out[k][c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <int H>
__device__ __forceinline__ void g4_fold_swap16(const f32x4* in, f32x4* out) {
#pragma unroll
  for (int k = 0; k < H; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(in[k][c]), __float_as_uint(in[H + k][c]), false, false);
      out[k][c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <InType T, int EPI>
__global__ __launch_bounds__(64 * G4_MAXW) void k_gemv_k4(GemvArgs p) {
  constexpr int RG = G4_RG;                                      // groups of four weight rows
  constexpr int ROWS = 4 * RG;                                   // weight rows per workgroup
  static_assert(G4_NA0 >= 1 && G4_NA0 <= RG && G4_NA >= G4_NA0, "load look-ahead");
  extern __shared__ __attribute__((aligned(16))) uint8_t g4_lds[];
  const GemmArgs& a = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;                                        // K slice
  const int nw = (int)(a.K >> 9);
  const int64_t M = a.M, K = a.K, N = a.N;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int b = lane >> 2, i4 = lane & 3;
  uint8_t* const sc_lds = g4_lds + w * (32 * ROWS);             // [ROWS rows][32 scale bytes]
  float* const part = reinterpret_cast<float*>(g4_lds + nw * 32 * ROWS);   // [nw][ROWS rows][4 tokens]
  float* const red = part + nw * 4 * ROWS;                       // [nw] amax of each slice
  const bool dynamic = (p.gscale_in == nullptr);
  // calibrated global scale (from an always-valid address in dynamic mode, unused there)
  const float g_in = *(dynamic ? a.w_seg_gscale : p.gscale_in);
  // the epilogue operands of this thread's output row (threads t < 4 ROWS take row
  // t % ROWS in the last step), loaded now so that the tail has no memory round trip
  const int64_t n_ep = min<int64_t>(n0 + (tid % ROWS), N - 1);
  const float w_seg_g = a.w_seg_gscale[seg_of_col(a.seg, n_ep)];
  float ep_alog = 0.0f, ep_db = 0.0f;
  if constexpr (EPI == EPI_GATE) {
    const int64_t nh = n_ep < a.gate.n_heads ? n_ep : 0;
    ep_alog = a.gate.A_log[nh];
    ep_db = a.gate.dt_bias[nh];
  }

  // (1) x: token j = i4, elements 512 w + 32 b .. +31; tokens past M re-read token 0
  // (in bounds) and are zeroed below
  const int64_t kx = 512 * (int64_t)w + 32 * b;
  G4X<T> xr;
  g4x_load<T>(p.x, (i4 < M ? i4 : 0) * p.ldx + kx, xr);
  asm volatile("" ::: "memory");
  // (2) the slice's weight scales: row r's 32 bytes at sc_lds + 32 r; load h covers
  // rows 32 h .. 32 h + 31 (rows past N clamp their source: in bounds, never stored)
  {
    const int64_t kb = K >> 4;
#pragma unroll
    for (int h = 0; h < RG / 8; ++h) {
      const int64_t row = min<int64_t>(n0 + 32 * h + (lane >> 1), N - 1);
      __builtin_amdgcn_global_load_lds(a.w_scales + row * kb + 32 * w + 16 * (lane & 1), sc_lds + 1024 * h, 16, 0, 0);
    }
  }
  asm volatile("" ::: "memory");
  // (3) the weight stream: load r = row 4 r + i4, chunk b of the slice
  const int64_t kh = K >> 1;
  const uint8_t* const wbase = a.w_codes + 256 * (int64_t)w + 16 * b;
  auto wptr = [&](int r) {
    const int64_t row = min<int64_t>(n0 + 4 * r + i4, N - 1);
    return reinterpret_cast<const u32x4*>(wbase + row * kh);
  };
  u32x4 codes[RG];
#pragma unroll
  for (int r = 0; r < G4_NA0; ++r) codes[r] = __builtin_nontemporal_load(wptr(r));

  // (4) global scale and the quantization of the lane's two blocks of x
  wait_vmcnt<G4_NA0 + RG / 8>();                                 // x has landed
  float v[32];
  g4x_unpack<T>(xr, v);
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = (i4 < M) ? v[e] : 0.0f;
  float g = g_in;
  if (dynamic) {
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red[w] = am;
    lds_sync();
    am = red[0];
    for (int k = 1; k < nw; ++k) am = __builtin_fmaxf(am, red[k]);
    g = global_scale_from_amax(am);
  }
  const ScaleConsts sc = scale_consts(g);
  uint32_t sb[2], qw[4];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float am = amax_abs<16>(v + 16 * blk);
    sb[blk] = block_scale_byte(am, sc);
    quant16(v + 16 * blk, sb[blk], g, qw + 2 * blk);
  }
  // B operand of step t (0..7): the lane's elements 4 t .. 4 t + 3
  f16x4 xb[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f16x8 dd = decode8_f16(qw[d], scale_f16x2(sb[d >> 1]));
    xb[2 * d] = f16x4{dd[0], dd[1], dd[2], dd[3]};
    xb[2 * d + 1] = f16x4{dd[4], dd[5], dd[6], dd[7]};
  }
  wait_vmcnt<G4_NA0>();                                          // the scale loads have landed

  // (5) main loop: row group r, MFMA steps t = 0..7 (elements 4 t .. 4 t + 3 of the
  // lane's 32; block 2 b for t < 4, 2 b + 1 after)
  f32x4 acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    // loads up to r + G4_NA - 1 in flight (at r = 0 the ones not issued before the
    // quantization, then one per row group)
    constexpr int lo0 = G4_NA0;
#pragma unroll
    for (int k = (r == 0 ? lo0 : min(RG, max(G4_NA0, r - 1 + G4_NA))); k < min(RG, max(G4_NA0, r + G4_NA)); ++k)
      codes[k] = __builtin_nontemporal_load(wptr(k));
    __builtin_amdgcn_sched_barrier(0);    // keep the loads here: the scheduler would sink them to their use
    const f16x2 sp = scale_pair_f16(*reinterpret_cast<const uint16_t*>(sc_lds + 32 * (4 * r + i4) + 2 * b));
#pragma unroll
    for (int d = 0; d < 4; ++d) {                                // dword d: steps 2 d, 2 d + 1
      const f16x2 s2 = bcast(sp, d >> 1);
      const uint32_t dw = codes[r][d];
      const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 0) * s2;
      const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 1) * s2;
      const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 2) * s2;
      const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 3) * s2;
      acc[r] = __builtin_amdgcn_mfma_f32_4x4x4f16(f16x4{p0[0], p0[1], p1[0], p1[1]}, xb[2 * d], acc[r], 0, 0, 0);
      acc[r] = __builtin_amdgcn_mfma_f32_4x4x4f16(f16x4{p2[0], p2[1], p3[0], p3[1]}, xb[2 * d + 1], acc[r], 0, 0, 0);
    }
  }

  // (6) the optional outputs of workgroup 0 (after the stream: a store before it would
  // make the compiler wait for the stream's loads)
  if (blockIdx.x == 0) {
    if (tid == 0 && p.gscale_out) *p.gscale_out = g;
    if (p.a_codes_out != nullptr && i4 < M) {
      *reinterpret_cast<u32x4*>(p.a_codes_out + i4 * (K >> 1) + 256 * w + 16 * b) = u32x4{qw[0], qw[1], qw[2], qw[3]};
      *reinterpret_cast<uint16_t*>(p.a_scales_out + i4 * (K >> 4) + 32 * w + 2 * b) = (uint16_t)(sb[0] | (sb[1] << 8));
    }
  }

  // (7) sum over the 16 blocks: lane (b, j) ends with row group b of token j,
  // register i = row 4 b + i
  f32x4 h8[8], h4[4], h2[2], h1[1];
  g4_fold_swap32<8>(acc, h8);
  g4_fold_swap16<4>(h8, h4);
  g4_fold<2>(h4, h2, lane, 8);
  g4_fold<1>(h2, h1, lane, 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w * 4 * ROWS + (4 * b + i) * 4 + i4] = h1[0][i];
  lds_sync();

  // (8) add the slices in order, epilogue (the store_out arithmetic with the operands
  // loaded at the start): thread t -> row t % ROWS (the same for every t of a thread,
  // as the block size is a multiple of ROWS), token t / ROWS
  for (int t = tid; t < 4 * ROWS; t += 64 * nw) {
    const int rr = t % ROWS, j = t / ROWS;
    const int64_t n = n0 + rr;
    if (j < M && n < N) {
      float s = part[rr * 4 + j];
      for (int k = 1; k < nw; ++k) s += part[k * 4 * ROWS + rr * 4 + j];
      float v = s * (g * w_seg_g);
      if constexpr (EPI == EPI_GATE) {
        v = n < a.gate.n_heads ? -expf(ep_alog) * softplus_f32(v + ep_db) : sigmoid_f32(v);
      }
      if constexpr (EPI == EPI_BF16) {
        reinterpret_cast<uint16_t*>(a.y)[j * a.ldy + n] = (uint16_t)f32_to_bf16_bits(v);
      } else {
        reinterpret_cast<float*>(a.y)[j * a.ldy + n] = v;
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
  const hipError_t e = lds_limit_once<&k_gemv_stream<T, NL, NA>>(152 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemv_stream<T, NL, NA>), dim3(grid), dim3(GS_THREADS), lds, s, p);
  return hipGetLastError();
}

// Code loads each stream wave of k_gemv_ws keeps in flight (issued before the x
// barrier, then one per step).  Measured at 4 x 16384 x 5120: 10-14 of 20 are within
// noise of each other; 8 and 20 are slower.
#ifndef NVFP4_GEMV_WS_AHEAD
#define NVFP4_GEMV_WS_AHEAD(nl) ((nl) / 2)
#endif

template <InType T, int NL>
static hipError_t launch_ws(const GemvArgs& p, unsigned grid, size_t lds, hipStream_t s) {
  constexpr int NA = NVFP4_GEMV_WS_AHEAD(NL);
  const hipError_t e = lds_limit_once<&k_gemv_ws<T, NL, NA>>(GW_LDS_MAX);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemv_ws<T, NL, NA>), dim3(grid), dim3(GW_THREADS), lds, s, p);
  return hipGetLastError();
}

static bool gemv_ws_fits(int64_t M, int64_t K, InType t) {
  return M <= 8 && K % 1024 == 0 && K / 256 <= GS_NLMAX &&
         gw_lds_bytes(M, K, t == InType::F32) <= GW_LDS_MAX;
}

bool gemv_stream_fits(int64_t M, int64_t K, InType t) {
  const int64_t chunks_per_thread = (M * K / 8 + GS_THREADS - 1) / GS_THREADS;
  return M <= 8 && K % 512 == 0 && K >= 512 && K / 256 <= GS_NLMAX && chunks_per_thread <= GS_XMAX &&
         (t == InType::BF16 || chunks_per_thread <= 5) && gs_lds_bytes(M, K) <= 152 * 1024;
}

static bool gemv_k4_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= 4 && K % 512 == 0 && K / 512 >= 2 && K / 512 <= G4_MAXW;
}

template <InType T>
static hipError_t launch_k4(const GemvArgs& p, hipStream_t s) {
  const int nw = (int)(p.g.K / 512);
  const unsigned grid = (unsigned)((p.g.N + 4 * G4_RG - 1) / (4 * G4_RG));
  const size_t lds = (size_t)g4_lds_bytes(nw, G4_RG);
  if (p.g.gate.n_heads > 0)
    hipLaunchKernelGGL((k_gemv_k4<T, EPI_GATE>), dim3(grid), dim3(64 * nw), lds, s, p);
  else if (p.g.y_type == OutType::BF16)
    hipLaunchKernelGGL((k_gemv_k4<T, EPI_BF16>), dim3(grid), dim3(64 * nw), lds, s, p);
  else
    hipLaunchKernelGGL((k_gemv_k4<T, EPI_F32>), dim3(grid), dim3(64 * nw), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv_fused(const GemvArgs& p, hipStream_t s) {
  if (gemv_k4_fits(p.g.M, p.g.K))
    return p.x_type == InType::BF16 ? launch_k4<InType::BF16>(p, s) : launch_k4<InType::F32>(p, s);
  if (gemv_ws_fits(p.g.M, p.g.K, p.x_type)) {
    const unsigned grid = (unsigned)((p.g.N + GS_ROWS - 1) / GS_ROWS);
    const size_t lds = (size_t)gw_lds_bytes(p.g.M, p.g.K, p.x_type == InType::F32);
    switch ((int)(p.g.K / 256)) {
#define NVFP4_GW_CASE(nl)                                                                  \
  case nl:                                                                                 \
    return p.x_type == InType::BF16 ? launch_ws<InType::BF16, nl>(p, grid, lds, s)        \
                                    : launch_ws<InType::F32, nl>(p, grid, lds, s);
      NVFP4_GW_CASE(4) NVFP4_GW_CASE(8) NVFP4_GW_CASE(12) NVFP4_GW_CASE(16)        // K % 1024 == 0
      NVFP4_GW_CASE(20) NVFP4_GW_CASE(24) NVFP4_GW_CASE(28) NVFP4_GW_CASE(32)
#undef NVFP4_GW_CASE
      default: break;
    }
  }
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
