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
//    to E4M3 with integer arithmetic.  Every E4M3 midpoint (and every other value with
//    <= 4 significant bits) has its low 19 mantissa bits zero; a t' within 8 ulps of
//    such a value is redone exactly: one float64 division, whose result never crosses
//    or lands on an E4M3 midpoint unless the exact quotient does (midpoints have <= 5
//    significant bits, 6g <= 27, amax <= 24: a non-zero gap is >= ~2^-32 relative,
//    the division error <= 2^-53).
//  * Codes: y = x * rcp(s g) in fp32 (|y - r| <= 3 ulp(y)) converted by the hardware
//    E2M1 RNE conversion (v_cvt_scalef32_pk_fp4_f32: exact RNE with saturation at 6,
//    the sign of x kept, power-of-two scale 1.0).  A code can only be wrong if a
//    midpoint lies within that distance; every midpoint has its low 21 mantissa bits
//    zero, and any y within 16 ulps of such a value is redone exactly in float64
//    (mu * s * g is exact there).  Rare on real data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Exact E4M3 block-scale byte for block amax a >= 0 under global scale g >= 0, by
// float64 division (the reference path).  Inlined on purpose: a call would make the
// compiler wait for every outstanding memory operation (vmcnt(0)) at the call site.
__device__ __forceinline__ uint32_t block_scale_byte_exact(float a, float g) {
  if (!(a > 0.0f) || !(g > 0.0f)) return 0u;
  const double t = (double)a / (6.0 * (double)g);
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

// E4M3 RNE (saturating) of an fp32 t >= 0 with integer arithmetic.
__device__ __forceinline__ uint32_t e4m3_rne_from_f32(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0x1p-6f) {                                   // subnormal E4M3: multiples of 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);      // exact scaling; RNE; 8 -> 0x08
  }
  uint32_t b = __float_as_uint(t);
  b += 0x7FFFFu + ((b >> 20) & 1u);                    // RNE to 3 mantissa bits
  return ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
}

// Exact E4M3 block-scale byte (fast path with an exact fallback near midpoints).
__device__ __forceinline__ uint32_t block_scale_byte(float a, const ScaleConsts& c) {
  const float t = a * c.inv6g;
  const uint32_t key = (__float_as_uint(t) + 8u) & 0x7FFFFu;     // near a <= 4-bit value?
  if (key <= 16u || !(t < 0x1p100f) || (t < 0x1p-100f && t != 0.0f)) return block_scale_byte_exact(a, c.g);
  if (!(a > 0.0f) || !(c.g > 0.0f)) return 0u;
  if (t <= 0x1p-10f) return 0u;
  return e4m3_rne_from_f32(t);
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

// Quantize the 8 consecutive values v[0..7] of one block (block scale byte sb,
// global scale g).  Returns the 8 codes packed, element 0 in the low nibble.
__device__ __forceinline__ uint32_t quant8(const float v[8], uint32_t sb, float g) {
  const float s = e4m3_to_f32(sb);
  const float h32 = s * g;
  const bool zero = (sb == 0u) || !(g > 0.0f);
  // fast path valid while s g and 1/(s g) are normal fp32 values
  const bool fast_ok = zero || (h32 >= 0x1p-120f && h32 <= 0x1p120f);
  const float rh = zero ? 0.0f : __builtin_amdgcn_rcpf(h32);   // <= 1 ulp; 0 keeps only the sign
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = v[i] * rh;
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  // key(y) = low 21 mantissa bits of y + 16, moved to the top: < 33 << 11 iff y is
  // within 16 ulps of a value whose low 21 mantissa bits are zero
  uint32_t k = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t k0 = (__float_as_uint(y[i]) << 11) + (16u << 11);
    const uint32_t k1 = (__float_as_uint(y[i + 1]) << 11) + (16u << 11);
    k = min(k, min(k0, k1));
  }
  if (!zero && (k < (33u << 11) || !fast_ok)) {
    const double h = (double)s * (double)g;                   // exact
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = e2m1_code_exact(v[i], h);
      w = (w & ~(0xFu << (4 * i))) | (c << (4 * i));
    }
  }
  return w;
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
