// Device-side NVFP4 format routines for gfx950 (CDNA4).
//
// NVFP4 = E2M1 4-bit values, one E4M3 scale per 16-element block, one FP32 global
// scale per tensor ("Why Gated DeltaNet Survives 4-Bit Quantization" review page,
// background section / Key Numbers); the block maximum sets the block scale
// (same page, mechanism step 1).
//
// Exactness.  The block scale is E4M3-RNE of t = amax_block / (6 g) and each code is
// E2M1-RNE of |x| / (s g), both of the *exact* quotient.
//  * Block scale: fast path t' = amax * fp32(1/(6g)) in fp32 (|t' - t| <= 2 ulp) rounded
//    to E4M3 with integer arithmetic.  Every E4M3 midpoint has <= 5 significant bits
//    (its low 19 mantissa bits are zero); when t' is within 8 ulps of such a value v,
//    the side of v on which the exact t lies is the sign of amax - 6 v g, which one fma
//    gives exactly (6 v has <= 7 significant bits, so -(6 v) is exact and the fma rounds
//    amax - 6 v g once, which keeps its sign; g >= 2^-100 keeps every term far above
//    the subnormal range).  Subnormal scales and extreme global scales take one
//    float64 division instead (exact there: midpoints have <= 5 significant bits, a
//    non-zero gap is >= ~2^-32 relative, the division error <= 2^-53).
//  * Codes: two fp32 quotients lo = |x| rcp(s g) (1 - 2^-19) and hi = |x| rcp(s g)
//    (1 + 2^-19) bracket the exact q = |x| / (s g) strictly; both go through the
//    hardware E2M1 RNE conversion (v_cvt_scalef32_pk_fp4_f32: exact RNE with
//    saturation at 6, the sign of the input kept, power-of-two scale 1.0).  Equal codes
//    are the code of q.  Different codes mean that a midpoint m lies inside the
//    bracket, and the sign of |x| - m s g, again one exactly-signed fma (m s has <= 7
//    significant bits), picks the code.  Blocks whose s g is outside [2^-100, 2^120]
//    are redone in float64 (the product s g is exact there).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E4M3 (OCP FN) byte -> fp32.  gfx950's fp8 conversion implements OCP E4M3FN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// fp32 global scale from an amax: fp32(amax / 2688).  The float64 quotient is
// rounded to fp32 without double rounding (amax/2688 = amax/21 * 2^-7 is either
// exact or has a period-6 binary expansion, which never sits on an fp32 midpoint).
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  return (float)((double)amax / 2688.0);
}

// E4M3 byte of a float64 block-scale quotient t >= 0 (t within 2^-53 relative of
// the exact quotient, which is never that close to an E4M3 midpoint unless equal
// to it): round-to-nearest-even, saturated at 448.
__device__ __forceinline__ uint32_t e4m3_byte_of_quotient(double t) {
  if (t >= 448.0) return 0x7Eu;                    // saturate at the largest finite value
  if (t <= 0x1p-10) return 0u;                      // nearer to 0 than to 2^-9 (tie -> even 0)
  if (t < 0x1p-6) {                                 // subnormal range: multiples of 2^-9
    return (uint32_t)__builtin_rint(t * 512.0);     // RNE; 8 lands on byte 0x08 = 2^-6
  }
  uint64_t bits = (uint64_t)__double_as_longlong(t);
  bits += ((1ull << 48) - 1ull) + ((bits >> 49) & 1ull);   // RNE to 3 mantissa bits
  const int e = (int)((bits >> 52) & 0x7FF) - 1023;          // -6 .. 8
  const uint32_t m3 = (uint32_t)((bits >> 49) & 7ull);
  return ((uint32_t)(e + 7) << 3) | m3;                      // <= 0x7E because t < 448
}

// Exact E4M3 block-scale byte for block amax a >= 0 under global scale g >= 0, by
// float64 division (the reference path).  Inlined on purpose: a call would make the
// compiler wait for every outstanding memory operation (vmcnt(0)) at the call site.
__device__ __forceinline__ uint32_t block_scale_byte_exact(float a, float g) {
  if (!(a > 0.0f) || !(g > 0.0f)) return 0u;
  return e4m3_byte_of_quotient((double)a / (6.0 * (double)g));
}

// Per-tensor constants of the fast block-scale path.
struct ScaleConsts {
  float g;        // global scale
  float inv6g;    // fp32(1 / (6 g)), 0 when g == 0
};

__device__ __forceinline__ ScaleConsts scale_consts(float g) {
  ScaleConsts c;
  c.g = g;
  c.inv6g = (g > 0.0f) ? (float)(1.0 / (6.0 * (double)g)) : 0.0f;
  return c;
}

// E4M3 byte of t near a 5-significant-bit value, decided exactly (normal E4M3 range,
// t < 448).  v = t' rounded to 5 significant bits.  If v has only 4 (an E4M3 value),
// t rounds to v.  Otherwise v is the midpoint of two E4M3 neighbours and the sign of
// a - 6 v g (one fma: 6 v has <= 7 significant bits, so 6 v * g + a is rounded once
// and keeps its sign) says on which side of v the exact t = a / (6 g) lies; a tie goes
// to the neighbour with the even mantissa.
__device__ __forceinline__ uint32_t e4m3_byte_near(float a, float g, uint32_t tb) {
  const uint32_t vb = (tb + 0x40000u) & 0xFFF80000u;
  uint32_t chosen = vb;
  if ((vb >> 19) & 1u) {
    const float v = __uint_as_float(vb);
    const float r = __builtin_fmaf(-(6.0f * v), g, a);
    const uint32_t downb = vb & ~0x80000u, upb = downb + 0x100000u;
    chosen = (r > 0.0f) ? upb : ((r < 0.0f) ? downb : (((downb >> 20) & 1u) ? upb : downb));
  }
  const uint32_t byte = (chosen >> 20) - (120u << 3);
  return (__uint_as_float(chosen) < 448.0f) ? byte : 0x7Eu;
}

// Exact E4M3 block-scale byte.  The fast path is branch-free (selects only).  When
// t' is within 8 ulps of a 5-significant-bit value (which every E4M3 midpoint is),
// the byte is decided exactly by e4m3_byte_near in the normal E4M3 range and by the
// float64 reference outside it (subnormal scales, extreme global scales: rare).
// a == 0 or g == 0 gives t == 0 -> byte 0.
__device__ __forceinline__ uint32_t block_scale_byte(float a, const ScaleConsts& c) {
  const float t = a * c.inv6g;
  const uint32_t tb = __float_as_uint(t);
  const uint32_t b = tb + 0x7FFFFu + ((tb >> 20) & 1u);           // RNE to 3 mantissa bits
  uint32_t r = (b >> 20) - (120u << 3);                          // ((exp - 120) << 3) | m3
  const uint32_t sub = (uint32_t)__builtin_rintf(t * 512.0f);    // subnormal E4M3: multiples of 2^-9
  r = (t < 0x1p-6f) ? sub : r;
  r = (t < 448.0f) ? r : 0x7Eu;                                  // saturate at 448
  r = (t <= 0x1p-10f) ? 0u : r;                                  // nearer to 0 (tie -> even 0)
  const uint32_t key = (tb + 8u) & 0x7FFFFu;                     // near a 5-bit value?
  const bool extreme = !(t < 0x1p100f) || (t < 0x1p-100f && t != 0.0f) || !(c.g >= 0x1p-100f);
  if (key <= 16u || extreme) {
    if (!extreme && t >= 0x1p-5f && t < 448.0f) r = e4m3_byte_near(a, c.g, tb);
    else r = block_scale_byte_exact(a, c.g);
  }
  return r;
}

__device__ __forceinline__ uint32_t block_scale_byte(float a, float g) {
  return block_scale_byte(a, scale_consts(g));
}

// Exact E2M1 code of x under h = s * g (float64, exact product), h > 0.  Inlined for
// the same reason as block_scale_byte_exact.
__device__ __forceinline__ uint32_t e2m1_code_exact(float x, double h) {
  const double a = __builtin_fabs((double)x);
  uint32_t c = (a > 0.25 * h) + (a >= 0.75 * h) + (a > 1.25 * h) + (a >= 1.75 * h) +
               (a > 2.5 * h) + (a >= 3.5 * h) + (a > 5.0 * h);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Per-block constants of the code computation.  rl and rh bracket 1 / (s g):
// rl = rcp(s g) (1 - 2^-19) and rh = rcp(s g) (1 + 2^-19), each rounded once, so that
// for every x, fl(|x| rl) < |x| / (s g) < fl(|x| rh) (the rounding of s g, of rcp
// (<= 1 ulp) and of the two products add up to less than 5 * 2^-24 relative).
struct BlockConsts {
  float s;        // decoded block scale
  float s4;       // s / 4 (exact)
  float rl, rh;   // the bracket; 0 for a zero block: codes keep only the sign
  bool fast_ok;   // zero block, or s g in [2^-100, 2^120]: 1/(s g) is normal and the
                  // exact-sign fma below stays clear of the subnormal range
};

__device__ __forceinline__ BlockConsts block_consts(uint32_t sb, float g) {
  BlockConsts b;
  b.s = e4m3_to_f32(sb);
  b.s4 = 0.25f * b.s;
  const float h32 = b.s * g;
  const bool zero = (sb == 0u) || !(g > 0.0f);
  b.fast_ok = zero || (h32 >= 0x1p-100f && h32 <= 0x1p120f);
  const float r = zero ? 0.0f : __builtin_amdgcn_rcpf(h32);
  b.rl = r * (1.0f - 0x1p-19f);
  b.rh = r * (1.0f + 0x1p-19f);
  return b;
}

// Largest magnitude of N finite values (N >= 3) by v_max3_f32 with |.| source
// modifiers: (N - 1) / 2 instructions.  Written out because fmaxf on values the
// compiler cannot prove canonical (activations unpacked with integer operations) gets
// an extra canonicalizing max per element.
template <int N>
__device__ __forceinline__ float amax_abs(const float* v) {
  static_assert(N >= 3, "at least three values");
  float m;
  asm volatile("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
#pragma unroll
  for (int i = 3; i + 1 < N; i += 2)
    asm volatile("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(m) : "v"(v[i]), "v"(v[i + 1]));
  if constexpr (N % 2 == 0) asm volatile("v_max_f32 %0, %0, |%1|" : "+v"(m) : "v"(v[N - 1]));
  return m;
}

// 8 values -> 8 E2M1 codes by the hardware RNE conversion (element 0 in the low
// nibble; saturation at 6, the sign of each value kept)
__device__ __forceinline__ uint32_t cvt8_fp4(const float* y) {
  uint32_t x = 0;
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[0], y[1], 1.0f, 0);
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[2], y[3], 1.0f, 1);
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[4], y[5], 1.0f, 2);
  x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[6], y[7], 1.0f, 3);
  return x;
}

// Codes of n consecutive values v[0..n) of one block (n = 8 or 16) into w[n/8]
// (element 0 in the low nibble of w[0]).  The codes of the bracket ends lo = |x| rl
// and hi = |x| rh are computed for every element; where they agree, every value in
// between, the exact quotient q = |x| / (s g) included, has that code (RNE is
// monotone).  Where they differ, the bracket (2^-18 wide, relative) holds exactly one
// E2M1 midpoint m, between the codes dn and dn + 1: the sign of |x| - m s g, from one
// fma (m s has <= 7 significant bits, so -(m s) is exact and m s * g + |x| is rounded
// once and keeps its sign), says on which side q lies; an exact tie goes to the even
// code.  The positions holding such an element in any lane of the wave are found as
// one wave-uniform mask (the OR of the element masks of the lanes that have one);
// at each flagged position the decision is taken branch-free for all lanes.  Blocks whose s g or 1/(s g) is not a
// normal fp32 value (extreme scales) are recomputed in float64; the empty asm makes
// s opaque there, so the compiler cannot hoist the float64 product into the common
// path.
template <int NV>
__device__ __forceinline__ void quant_block(const float v[NV], const BlockConsts& b, float g, uint32_t w[NV / 8]) {
  uint32_t diff = 0, wh[NV / 8];
#pragma unroll
  for (int d = 0; d < NV / 8; ++d) {
    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = v[8 * d + e] * b.rl;
      hi[e] = v[8 * d + e] * b.rh;
    }
    w[d] = cvt8_fp4(lo);
    wh[d] = cvt8_fp4(hi);
    diff |= w[d] ^ wh[d];
  }
  if (!b.fast_ok) {
    float sv = b.s;
    asm volatile("" : "+v"(sv));
    const double h = (double)sv * (double)g;                  // exact
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t c = e2m1_code_exact(v[i], h);
      w[i / 8] = (w[i / 8] & ~(0xFu << (4 * (i % 8)))) | (c << (4 * (i % 8)));
    }
  } else if (uint64_t lanes = __builtin_amdgcn_ballot_w64(diff != 0u)) {
    // element mask of this lane: bit 4e (word 0) / 4e + 1 (word 1) set where the
    // bracket codes of element e / 8 + e differ; OR-ed over the few lanes that have
    // any (one readlane each), so that untaken positions cost only a scalar test
    uint32_t m = 0;
#pragma unroll
    for (int d = 0; d < NV / 8; ++d) {
      const uint32_t x = w[d] ^ wh[d];
      m |= ((x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x11111111u) << d;
    }
    uint32_t all = 0;
    while (lanes) {
      all |= __builtin_amdgcn_readlane(m, __builtin_ctzll(lanes));
      lanes &= lanes - 1;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int d = i / 8, sh = 4 * (i % 8);
      if (all & (1u << (sh + d))) {                            // wave-uniform
        const uint32_t dn = (w[d] >> sh) & 7u;
        // midpoint between codes dn and dn + 1, times 4: 1 3 5 7 10 14 20 (dn = 0 .. 6)
        const uint32_t m4 = __builtin_amdgcn_perm(0x00140E0Au, 0x07050301u, dn) & 0xFFu;
        const float r = __builtin_fmaf(-((float)m4 * b.s4), g, __builtin_fabsf(v[i]));
        const uint32_t take_up = ((uint32_t)(r > 0.0f) | ((uint32_t)(r == 0.0f) & dn)) & 1u;
        // where the bracket codes differ they are dn and dn + 1 with the same sign (lo and
        // hi are x times positive factors): taking the upper one is swapping in hi's
        // nibble; where they agree the xor is zero and nothing changes
        w[d] ^= take_up != 0u ? ((w[d] ^ wh[d]) & (0xFu << sh)) : 0u;
      }
    }
  }
}

// Quantize the 8 consecutive values v[0..7] of one block (block scale byte sb,
// global scale g).  Returns the 8 codes packed, element 0 in the low nibble.
__device__ __forceinline__ uint32_t quant8(const float v[8], uint32_t sb, float g) {
  uint32_t w[1];
  quant_block<8>(v, block_consts(sb, g), g, w);
  return w[0];
}

// Quantize the 16 values of one block: codes of elements 0-7 in w[0], 8-15 in w[1].
__device__ __forceinline__ void quant16(const float v[16], uint32_t sb, float g, uint32_t w[2]) {
  quant_block<16>(v, block_consts(sb, g), g, w);
}

// 8 packed codes (one dword) + E4M3 scale byte -> 8 f16 values e2m1 * s (exact:
// <= 6 significant bits, magnitude in [2^-10, 2688]).
__device__ __forceinline__ f16x8 decode8_f16(uint32_t w, f16x2 s2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ f16x2 scale_f16x2(uint32_t sbyte) {
  const _Float16 s = (_Float16)e4m3_to_f32(sbyte);   // every E4M3 value is exact in f16
  f16x2 r = {s, s};
  return r;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace nvfp4
