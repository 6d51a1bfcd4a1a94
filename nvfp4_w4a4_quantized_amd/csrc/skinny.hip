// Fused W4A4 linear for skinny N (N <= 128, K % 256 == 0): x (bf16 or fp32) is read
// once, quantized to NVFP4 in registers and fed straight into the block-scaled
// GEMM against the packed weight, with the per-segment / GDN-gate epilogue.  The
// activation codes never go through HBM (unless the caller asks for them).
//
// This is the shape of the GDN gate projections a, b (N = 2 x 48 heads) in "Why
// Gated DeltaNet Survives 4-Bit Quantization" (review page, mechanism step 2, Eq. 1):
// a tall activation times a tiny weight, bound by the single read of x.
//
// Workgroup = 512 threads (8 waves, two per SIMD) = 128 tokens; wave w owns tokens
// 16w .. 16w+15.  Lane (q = lane >> 4, rr = lane & 15) owns token rr and, in every
// 128-element unit of K, the four octets 32t + 8q .. 32t + 8q + 7 (t = 0..3): load
// instruction t then reads 64 contiguous bytes of each of the wave's 16 token rows (a
// lane holding 32 contiguous elements would spread every instruction over twice as many
// cache lines: 15% slower on the GDN gates shape).  Octet t of lanes q and q ^ 1 (16
// lanes apart) is one 16-element block: its amax takes one v_permlane16_swap; of the
// pair's four scale bytes (the stand-alone quantizer's arithmetic) the lane with q even
// derives those of octets 0 and 1, its partner those of 2 and 3, and two more swaps give
// both lanes all four (sharing the work: 137 vs 143 us on the GDN gates shape).
// Octet t is MFMA 16x16x32 f16 step t (K positions 32t + 8q ..); the weight operand is
// read at the same positions, so the sum over k is unchanged.
//
// The weight (N x K packed, a few hundred KiB: L2-resident) is decoded exactly to
// f16 (e2m1 x E4M3 scale) 256 K-elements at a time into a double-buffered LDS tile
// shared by the workgroup; row stride 2 x 256 + 16 bytes keeps the per-lane 16-byte
// reads of 32 consecutive rows on distinct banks.  x units are loaded R - 1
// units ahead of their use, with ordinary loads (the non-temporal form was 3% slower
// on the GDN gates shape).
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

constexpr int SK_THREADS = 512;                     // 8 waves, two per SIMD
constexpr int SK_TM = 128;                          // tokens per workgroup (16 per wave)
constexpr int SK_KC = 256;                          // K elements per decoded weight chunk
constexpr int SK_ROWB = 2 * SK_KC + 16;             // LDS bytes per decoded weight row

template <InType T> struct XUnit;                   // 32 elements of one token
template <> struct XUnit<InType::BF16> { u32x4 q[4]; };
template <> struct XUnit<InType::F32> { f32x4 q[8]; };

// The lane's four octets of a unit: elem_off = the unit's first element + 8q; octet t
// is 32t elements further.
template <InType T>
__device__ __forceinline__ void xunit_load(const void* base, int64_t elem_off, XUnit<T>& r) {
  if constexpr (T == InType::BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = p[4 * i];
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.q[2 * i] = p[8 * i];
      r.q[2 * i + 1] = p[8 * i + 1];
    }
  }
}

template <InType T>
__device__ __forceinline__ void xunit_unpack(const XUnit<T>& r, float v[32]) {
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

// Weight chunk staging: NT*16 rows x 32 octets (8 elements) per chunk, NT octets per
// thread; octet index o = e * 512 + tid -> row o >> 5, octet o & 31.  Loads are
// unconditional (rows past N re-read row N - 1; wchunk_store zeroes them): with no
// load under a branch, the compiler counts the loads in flight exactly and never
// has to drain the x stream.
template <int NT>
struct WStage {
  uint32_t code[NT];
  uint32_t scale[NT];
};

template <int NT>
__device__ __forceinline__ void wchunk_load(const GemmArgs& a, int64_t c, WStage<NT>& w) {
  const int64_t kh = a.K >> 1, kb = a.K >> 4;
#pragma unroll
  for (int e = 0; e < NT; ++e) {
    const int o = e * SK_THREADS + (int)threadIdx.x;
    const int64_t row = min<int64_t>(o >> 5, a.N - 1);
    const int oct = o & 31;
    w.code[e] = *reinterpret_cast<const uint32_t*>(a.w_codes + row * kh + c * (SK_KC / 2) + oct * 4);
    w.scale[e] = a.w_scales[row * kb + c * (SK_KC / 16) + (oct >> 1)];
  }
}

template <int NT>
__device__ __forceinline__ void wchunk_store(uint8_t* buf, const WStage<NT>& w, int64_t N) {
#pragma unroll
  for (int e = 0; e < NT; ++e) {
    const int o = e * SK_THREADS + (int)threadIdx.x;
    const bool live = (o >> 5) < N;
    const f16x8 d = decode8_f16(live ? w.code[e] : 0u, scale_f16x2(live ? w.scale[e] : 0u));
    *reinterpret_cast<f16x8*>(buf + (o >> 5) * SK_ROWB + (o & 31) * 16) = d;
  }
}

// No load or store of the main loop sits under a data-dependent branch (vmcnt counts
// both on gfx950): the compiler then knows exactly how many are in flight and only
// waits for the unit it is about to use.
template <InType T, int NT, int EPI, bool CODES>
__global__ __launch_bounds__(SK_THREADS, 1) void k_linear_skinny(GemvArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sk_lds[];   // 2 x NT*16 rows x SK_ROWB
  constexpr int R = (T == InType::BF16) ? 4 : 2;                     // x units in the register ring
  constexpr int WBUF = NT * 16 * SK_ROWB;
  const GemmArgs& a = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4, rr = lane & 15;
  const int64_t M = a.M, K = a.K;
  const int64_t m0 = (int64_t)blockIdx.x * SK_TM;
  const int64_t tok = m0 + wave * 16 + rr;
  const int64_t trow = tok < M ? tok : M - 1;                        // clamped: in bounds, never stored
  // Global scale: the caller's, or (gscale_in NULL: dynamic mode with every token in
  // this one workgroup) fp32(amax / 2688) of x taken here, 8 elements per step.
  float g;
  if (p.gscale_in != nullptr) {
    g = *p.gscale_in;
  } else {
    __shared__ float red_am[SK_THREADS / 64];
    const int64_t per_row = K / 8, n8 = M * per_row;
    float am = 0.0f;
    for (int64_t i = tid; i < n8; i += SK_THREADS) {
      const int64_t rr8 = i / per_row, c8 = (i - rr8 * per_row) * 8;
      if constexpr (T == InType::BF16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) + rr8 * p.ldx + c8);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w[e] << 16)),
                                                   __builtin_fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
      } else {
        const f32x4* xp = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.x) + rr8 * p.ldx + c8);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x4 w = xp[hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(w[e]));
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red_am[wave] = am;
    __syncthreads();
    am = red_am[0];
#pragma unroll
    for (int i = 1; i < SK_THREADS / 64; ++i) am = __builtin_fmaxf(am, red_am[i]);
    g = global_scale_from_amax(am);
  }
  const ScaleConsts sc = scale_consts(g);
  if (blockIdx.x == 0 && tid == 0 && p.gscale_out != nullptr) *p.gscale_out = g;

  const int64_t nu = K / 128;                                        // 128-element units
  const int64_t xoff = trow * p.ldx + 8 * q;
  XUnit<T> xr[R];
#pragma unroll
  for (int i = 0; i < R - 1; ++i) xunit_load<T>(p.x, xoff + 128 * min<int64_t>(i, nu - 1), xr[i]);

  // Weight chunks: the raw chunk c + 2 is loaded at the start of chunk c (into stage
  // c & 1) and decoded into LDS buffer (c + 1) & 1 during chunk c, so that the wait
  // for its loads leaves the x loads of about four units in flight.
  const int64_t nc = K / SK_KC;
  WStage<NT> ws[2];
  wchunk_load<NT>(a, 0, ws[0]);
  wchunk_load<NT>(a, min<int64_t>(1, nc - 1), ws[1]);
  wchunk_store<NT>(sk_lds, ws[0], a.N);

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // per-column epilogue constants, loaded once up front (all loads issued together)
  float alpha[NT], neg_ea[NT], db[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t n = min<int64_t>(16 * j + rr, a.N - 1);
    alpha[j] = g * a.w_seg_gscale[seg_of_col(a.seg, n)];
    if constexpr (EPI == EPI_GATE) {
      const int64_t nh = n < a.gate.n_heads ? n : 0;
      neg_ea[j] = a.gate.A_log[nh];
      db[j] = a.gate.dt_bias[nh];
    }
  }

  // B operand: weight row 16 j + rr, chunk column 128 (u % 2) + 32 t + 8 q
  const uint32_t bbase = (uint32_t)(rr * SK_ROWB + 16 * q);

  // two chunks (four 128-element units) per iteration, so that every ring and stage
  // index below is a compile-time constant (u0 % 4 == 0; nu is even)
  for (int64_t u0 = 0; u0 < nu; u0 += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t u = u0 + r;
      if (r == 2 && u >= nu) break;                                  // uniform
      const int64_t c = u >> 1;                                      // weight chunk
      const int cp = r >> 1;                                         // c & 1
      if (r % 2 == 0) {
        // chunk boundary: chunk c was decoded into buffer c & 1 during chunk c - 1
        // (chunk 0: before the loop); the barrier publishes it and ends every wave's
        // reads of buffer (c+1) & 1.  It waits for LDS traffic only: the x stream stays
        // in flight across it.  Stage chunk c + 2 (the last chunk again at the end).
        lds_sync();
        wchunk_load<NT>(a, min<int64_t>(c + 2, nc - 1), ws[cp]);
      }
      // keep R - 1 units of x in flight (past the end: re-read the last unit)
      xunit_load<T>(p.x, xoff + 128 * min<int64_t>(u + R - 1, nu - 1), xr[(r + R - 1) % R]);

      // quantize the lane's four octets (block 2t + (q >> 1) of unit u, half q & 1)
      float v[32];
      xunit_unpack<T>(xr[r % R], v);
      uint32_t sb[4], w[4];
      float am[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        am[t] = amax_abs<8>(v + 8 * t);
        // the other half of the block is in lane ^ 16: the swap of am with itself leaves
        // both halves' maxima in the two results of either lane
        const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(am[t]), __float_as_uint(am[t]), false, false);
        asm volatile("v_max_f32 %0, %1, %2" : "=v"(am[t]) : "v"(pr[0]), "v"(pr[1]));
      }
      // the pair shares its four blocks' scales: the lane with q even derives those of
      // octets 0 and 1, its partner those of octets 2 and 3, and one swap per pair of
      // scale bytes hands every lane all four (result 0 = the even lane's, 1 = the odd's)
      {
        const bool odd = (q & 1) != 0;
        const uint32_t s0 = block_scale_byte(odd ? am[2] : am[0], sc);
        const uint32_t s1 = block_scale_byte(odd ? am[3] : am[1], sc);
        const auto p0 = __builtin_amdgcn_permlane16_swap(s0, s0, false, false);
        const auto p1 = __builtin_amdgcn_permlane16_swap(s1, s1, false, false);
        sb[0] = p0[0];
        sb[2] = p0[1];
        sb[1] = p1[0];
        sb[3] = p1[1];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = quant8(v + 8 * t, sb[t], g);
      if constexpr (CODES) {
        // lanes past M quantized row M - 1 (trow) and store the same bytes there
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          *reinterpret_cast<uint32_t*>(p.a_codes_out + trow * (K >> 1) + u * 64 + 16 * t + 4 * q) = w[t];
          if ((q & 1) == 0) p.a_scales_out[trow * (K >> 4) + u * 8 + 2 * t + (q >> 1)] = (uint8_t)sb[t];
        }
      }
      // MFMA 16x16x32 steps: A = the lane's octet t, B = weight rows 16 j + rr at the
      // same K positions
      const uint8_t* bl = sk_lds + cp * WBUF + bbase + 256 * (r & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // all of this step's weight reads first, the decode of A under them
        f16x8 B[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) B[j] = *reinterpret_cast<const f16x8*>(bl + j * 16 * SK_ROWB + 64 * t);
        const f16x8 A = decode8_f16(w[t], scale_f16x2(sb[t]));
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[j], acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);     // the NT LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);      // the A decode
        __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);     // the NT MFMAs
      }
      if (r % 2 == 1) {
        // decode the next weight chunk into the other buffer (free since the last barrier)
        if (c + 1 < nc) wchunk_store<NT>(sk_lds + (cp ^ 1) * WBUF, ws[cp ^ 1], a.N);
      }
    }
  }

  // D (16 x 16) of tile j: lane (q, rr) holds tokens 4q .. 4q+3 of the wave, column 16 j + rr
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t n = 16 * j + rr;
    const bool n_ok = n < a.N;
    if constexpr (EPI == EPI_GATE) {
      // Eq. 1: g = -exp(A_log) softplus(a + dt_bias) for the a-heads, beta = sigmoid(b)
      const bool is_a = n < a.gate.n_heads;
      const float nea = -expf(neg_ea[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wave * 16 + 4 * q + i;
        const float v = acc[j][i] * alpha[j];
        const float o = is_a ? nea * softplus_f32(v + db[j]) : sigmoid_f32(v);
        if (n_ok && m < M) reinterpret_cast<float*>(a.y)[m * a.ldy + n] = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wave * 16 + 4 * q + i;
        if (n_ok && m < M) store_out<EPI>(a, m, n, acc[j][i], alpha[j]);
      }
    }
  }
}

template <InType T, int NT, int EPI, bool CODES>
hipError_t launch_ntc(const GemvArgs& p, hipStream_t s) {
  const size_t lds = 2 * (size_t)NT * 16 * SK_ROWB;
  const hipError_t e = lds_limit_once<&k_linear_skinny<T, NT, EPI, CODES>>((int)lds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((p.g.M + SK_TM - 1) / SK_TM);
  hipLaunchKernelGGL((k_linear_skinny<T, NT, EPI, CODES>), dim3(grid), dim3(SK_THREADS), lds, s, p);
  return hipGetLastError();
}

template <InType T, int NT, int EPI>
hipError_t launch_nt(const GemvArgs& p, hipStream_t s) {
  return p.a_codes_out != nullptr ? launch_ntc<T, NT, EPI, true>(p, s) : launch_ntc<T, NT, EPI, false>(p, s);
}

// NT = number of 16-column weight tiles, rounded up to an even count
template <InType T, int EPI>
hipError_t launch_t(const GemvArgs& p, hipStream_t s) {
  switch ((int)((p.g.N + 31) / 32)) {
    case 1: return launch_nt<T, 2, EPI>(p, s);
    case 2: return launch_nt<T, 4, EPI>(p, s);
    case 3: return launch_nt<T, 6, EPI>(p, s);
    default: return launch_nt<T, 8, EPI>(p, s);
  }
}

template <InType T>
hipError_t launch_epi(const GemvArgs& p, hipStream_t s) {
  if (p.g.gate.n_heads > 0) return launch_t<T, EPI_GATE>(p, s);
  if (p.g.y_type == OutType::BF16) return launch_t<T, EPI_BF16>(p, s);
  return launch_t<T, EPI_F32>(p, s);
}

}  // namespace

bool linear_skinny_fits(int64_t M, int64_t N, int64_t K) {
  return N >= 1 && N <= 128 && K % SK_KC == 0 && K > 0 && M >= 1;
}

hipError_t launch_linear_skinny(const GemvArgs& p, hipStream_t s) {
  // in-kernel dynamic scale only when one workgroup holds every token
  if (p.gscale_in == nullptr && p.g.M > SK_TM) return hipErrorInvalidValue;
  return p.x_type == InType::BF16 ? launch_epi<InType::BF16>(p, s) : launch_epi<InType::F32>(p, s);
}

int64_t linear_skinny_tokens_per_wg() { return SK_TM; }

}  // namespace nvfp4
