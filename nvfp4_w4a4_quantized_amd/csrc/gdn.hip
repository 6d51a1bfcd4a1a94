// The consumer of the GDN gate outputs: alpha = e^g and the gated delta rule.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
// Recurrent Half of a Hybrid 27B LLM" (review page): background section, Eq. 2 (per
// head, the state S [d_k x d_v] decays by alpha_t and is written along k_t with
// strength beta_t, replacing its prediction S_{t-1}^T k_t by v_t; o_t = S_t^T q_t /
// sqrt(d_k)); mechanism step 2, Eq. 1 (alpha_t = e^{g_t}, beta_t = sigmoid(b_t):
// the [g | beta] row the fused gate epilogue writes); the spec list (K = V = 128).
//
// Column j of the state evolves on its own: s_j <- alpha s_j + beta (v_j - s_j.k) k,
// and o_j = s_j.q / sqrt(d_k).  One wave = one value head x 4 state columns; lane
// (c = lane / 16, r = lane % 16) holds rows 8 r .. 8 r + 7 of column c in registers.
// Per token the lane takes its 8 elements of k_t and q_t, forms its part of s.k,
// the 16 lanes of the column sum their parts (two quad DPP steps and two mirrors),
// every lane updates its 8 elements, and the same reduction gives o.  The token chain
// is sequential; the chip is filled by heads x column groups (1536 waves for 48 heads
// of 128 columns, one or two per SIMD), so each wave's chain is short.  Keys, queries and values
// of token pairs go straight from memory into a per-wave LDS ring of NS pair slots
// (direct-to-LDS buffer loads, NS - 1 pairs ahead of use, no registers held for
// them, waited for with an explicit count).  The gates of the next 64 tokens are
// loaded into LDS the same way; at each 64-token block every lane takes one token's
// [g | beta], computes alpha = e^g, and the token loop reads them with lane reads.
// Waves of one head run on one XCD, so q_t and k_t come from that XCD's L2.
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

constexpr int GD_DK = 128;               // key dimension (state rows)
constexpr int GD_LPC = 16;               // lanes per state column
constexpr int GD_ROWS = GD_DK / GD_LPC;  // state rows per lane
constexpr int GD_CPW = 64 / GD_LPC;      // state columns per wave
constexpr int GD_NS = 8;                 // LDS slots of token pairs (a power of two)
constexpr int GD_SLOT = 2112;            // bytes per slot: k 2 x 512, q 2 x 512, v 2 x GD_CPW x 4
constexpr int GD_GATES = GD_NS * GD_SLOT;   // then 2 x [g 64 | beta 64] floats

struct GdnArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* gates;
  const float* state_in;
  float* state_out;
  float* o;
  int64_t T, ldq, ldk, ldv, ldg, ldo;
  int32_t n_k_heads, n_v_heads, d_v;
};

// sum over the GD_LPC consecutive lanes of a column (every one of them gets the sum):
// quad exchanges, then the mirror within 8 lanes, then within 16
__device__ __forceinline__ float sum_col(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // 7 - lane
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // 15 - lane
  return x;
}

// Direct-to-LDS buffer loads: lane l's bytes land at lds + size * l.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// One token of the recurrence on this lane's GD_ROWS state elements (k, q: the
// token's slices; v: the column's value).
__device__ __forceinline__ float gdn_token(float S[GD_ROWS], const f32x4 kq[GD_ROWS / 4],
                                           const f32x4 qq[GD_ROWS / 4], float vt, float alpha, float beta) {
  // prediction s.k (this lane's part, two chains), summed over the column's lanes
  float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
  for (int i = 0; i < GD_ROWS / 4; ++i) {
    d0 = __builtin_fmaf(S[4 * i], kq[i][0], d0);
    d1 = __builtin_fmaf(S[4 * i + 1], kq[i][1], d1);
    d0 = __builtin_fmaf(S[4 * i + 2], kq[i][2], d0);
    d1 = __builtin_fmaf(S[4 * i + 3], kq[i][3], d1);
  }
  const float d = sum_col(d0 + d1);
  const float u = beta * (vt - d);                               // beta (v - S^T k)
  float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int i = 0; i < GD_ROWS / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S[4 * i + e] = __builtin_fmaf(u, kq[i][e], alpha * S[4 * i + e]);   // alpha S + k u
      if (e & 1) o1 = __builtin_fmaf(S[4 * i + e], qq[i][e], o1);
      else o0 = __builtin_fmaf(S[4 * i + e], qq[i][e], o0);
    }
  return sum_col(o0 + o1) * 0.08838834764831845f;                // S^T q / sqrt(128)
}

__global__ __launch_bounds__(64) void k_gdn_delta(GdnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GD_NS * GD_SLOT + 2 * 2 * 64 * 4];
  const int lane = threadIdx.x;
  const int c = lane / GD_LPC, r = lane % GD_LPC;
  const int ncg = a.d_v / GD_CPW;                                // column groups per head
  const int nblk = gridDim.x;
  // blocks b, b + 8, b + 16, ... run on one XCD: give them consecutive (head, group)
  const int L = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int h = L / ncg, cg = L % ncg;
  const int kh = h / (a.n_v_heads / a.n_k_heads);
  const int col = cg * GD_CPW + c;
  const int64_t voff = (int64_t)h * a.d_v + col;
  const int64_t T = a.T;

  float S[GD_ROWS];
  const size_t sbase = ((size_t)h * GD_DK + GD_ROWS * r) * a.d_v + col;
#pragma unroll
  for (int i = 0; i < GD_ROWS; ++i) S[i] = a.state_in ? a.state_in[sbase + (size_t)i * a.d_v] : 0.0f;
  // The state enters the token loop through an empty asm: the loop then uses no
  // register written by a memory load outside it, so the compiler keeps the loads in
  // flight at the loop entry instead of draining them there.
#pragma unroll
  for (int i = 0; i < GD_ROWS; ++i) asm volatile("" : "+v"(S[i]));

  // Pair slot layout: k_t, k_t+1 of the key head (lane l loads 16 bytes of token
  // t + l / 32), q_t, q_t+1 likewise, then v of this wave's GD_CPW columns for both
  // tokens (lanes 0 .. 2 GD_CPW - 1).  Tokens past T re-read token T - 1; byte extents
  // (< 2^31, checked on the host) bound every access.
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.k), (short)0,
                                                                      (int)(T * a.ldk * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.q), (short)0,
                                                                      (int)(T * a.ldq * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.v), (short)0,
                                                                      (int)(T * a.ldv * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.gates), (short)0,
                                                                      (int)(T * a.ldg * 4), 0x00020000);
  const int second = lane >> 5;                                  // k/q lanes of the pair's second token
  const uint32_t off_kq = (uint32_t)((kh * GD_DK + 4 * (lane & 31)) * 4);
  const int vsecond = (lane / GD_CPW) & 1;                       // v lanes GD_CPW .. 2 GD_CPW - 1
  const uint32_t off_v = (uint32_t)((h * a.d_v + cg * GD_CPW + (lane % GD_CPW)) * 4);
  // 3 loads per pair, issued unconditionally
  auto issue = [&](int64_t t) {                                  // t: the pair's first token
    uint8_t* base = lds + (int)((t >> 1) & (GD_NS - 1)) * GD_SLOT;
    const int64_t t0 = t < T ? t : T - 1;
    const int64_t tk = (second ? t + 1 : t) < T ? (second ? t + 1 : t) : T - 1;
    const int64_t tv = (vsecond ? t + 1 : t) < T ? (vsecond ? t + 1 : t) : T - 1;
    load_lds16(rk, base, off_kq + (uint32_t)((tk - t0) * a.ldk * 4), (int)(t0 * a.ldk * 4));
    load_lds16(rq, base + 1024, off_kq + (uint32_t)((tk - t0) * a.ldq * 4), (int)(t0 * a.ldq * 4));
    if (lane < 2 * GD_CPW)
      load_lds4(rv, base + 2048, off_v + (uint32_t)((tv - t0) * a.ldv * 4), (int)(t0 * a.ldv * 4));
  };
  // gates of the 64 tokens from tb: lane l loads g and beta of token tb + l
  auto issue_gates = [&](int64_t tb) {
    uint8_t* gb = lds + GD_GATES + (int)((tb >> 6) & 1) * 512;
    const int64_t tg = tb + lane < T ? tb + lane : T - 1;
    const uint32_t off = (uint32_t)(tg * a.ldg * 4);
    load_lds4(rg, gb, off + (uint32_t)(h * 4), 0);
    load_lds4(rg, gb + 256, off + (uint32_t)((a.n_v_heads + h) * 4), 0);
  };
  issue_gates(0);
#pragma unroll
  for (int i = 0; i < GD_NS - 1; ++i) issue(2 * i);

  for (int64_t tb = 0; tb < T; tb += 64) {
    // this block's gates landed before the previous block's last wait (or the first one)
    if (tb == 0) wait_vmcnt<3 * (GD_NS - 1)>();
    const float* gb = reinterpret_cast<const float*>(lds + GD_GATES + (int)((tb >> 6) & 1) * 512);
    const bool lane_live = tb + lane < T;
    // tokens past T (the last block's tail) leave the state exactly as it is:
    // alpha = 1 and beta = 0 there, and nothing is stored
    const float alpha_l = lane_live ? expf(gb[lane]) : 1.0f;
    const float beta_l = lane_live ? gb[64 + lane] : 0.0f;
    issue_gates(tb + 64);
    for (int j = 0; j < 64; j += 2) {
      const int64_t t = tb + j;
      issue(t + 2 * (GD_NS - 1));                                // into the slot the last pair used
      // this pair's slot: 3 loads per pair, GD_NS - 1 pairs' worth issued after it
      // (gate loads and o stores in between only make the wait longer, never shorter)
      wait_vmcnt<3 * (GD_NS - 1)>();
      const uint8_t* slot = lds + (int)((t >> 1) & (GD_NS - 1)) * GD_SLOT;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        f32x4 kq[GD_ROWS / 4], qq[GD_ROWS / 4];
#pragma unroll
        for (int i = 0; i < GD_ROWS / 4; ++i) {
          kq[i] = *reinterpret_cast<const f32x4*>(slot + 512 * p + 4 * GD_ROWS * r + 16 * i);
          qq[i] = *reinterpret_cast<const f32x4*>(slot + 1024 + 512 * p + 4 * GD_ROWS * r + 16 * i);
        }
        const float vt = *reinterpret_cast<const float*>(slot + 2048 + 4 * GD_CPW * p + 4 * c);
        const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha_l), j + p));
        const float beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(beta_l), j + p));
        const float o = gdn_token(S, kq, qq, vt, alpha, beta);
        if (r == 0 && t + p < T) a.o[(t + p) * a.ldo + voff] = o;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < GD_ROWS; ++i) a.state_out[sbase + (size_t)i * a.d_v] = S[i];
}

}  // namespace

bool gdn_shape_ok(int32_t d_k, int32_t d_v) { return d_k == GD_DK && d_v >= 8 && d_v % 8 == 0; }
static_assert(8 % GD_CPW == 0, "a multiple of 8 columns must split into whole column groups");

hipError_t launch_gdn_delta(const float* q, int64_t ldq, const float* k, int64_t ldk, const float* v, int64_t ldv,
                            const float* gates, int64_t ldg, int64_t T, int32_t n_k_heads, int32_t n_v_heads,
                            int32_t d_v, const float* state_in, float* state_out, float* o, int64_t ldo,
                            hipStream_t s) {
  GdnArgs a{q, k, v, gates, state_in, state_out, o, T, ldq, ldk, ldv, ldg, ldo, n_k_heads, n_v_heads, d_v};
  const unsigned grid = (unsigned)(n_v_heads * (d_v / GD_CPW));
  hipLaunchKernelGGL(k_gdn_delta, dim3(grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvfp4
