// Re-encoding of a multi-scale fused NVFP4 weight onto one shared global scale
// ("Why Gated DeltaNet Survives 4-Bit Quantization" review page, strengths
// paragraph / the paper's section 6: the fused-GEMM global-scale mismatch and its
// repair; this is the re-encoding form of the repair, the per-segment epilogue of
// the GEMM kernels the other).
//
// One lane = four consecutive 16-element blocks of a row (one when K/16 is not a
// multiple of 4).  A block's values are x = e2m1 * s * g_seg
// (exact in float64: <= 2 + 4 + 24 significant bits).  Its largest magnitude is
// e2m1(largest magnitude code) * s * g_seg, so the new block scale is the E4M3 RNE
// of that over 6 g_shared (float64 quotient, exact decision).  Every element with
// the same magnitude code has the same value, so the new codes come from an
// 8-entry table: new magnitude of old magnitude c = E2M1 RNE of
// e2m1(c) * s * g_seg / (s' g_shared), decided by float64 comparisons with the
// midpoints (both sides exact), and the 16 nibbles are mapped through it with two
// byte permutes per dword; signs are kept.
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

// E2M1 magnitude code of a / h (a >= 0, h > 0, both exact float64 values): RNE
// onto {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even code, saturated at 6
__device__ __forceinline__ uint32_t e2m1_mag_exact(double a, double h) {
  return (uint32_t)(a > 0.25 * h) + (uint32_t)(a >= 0.75 * h) + (uint32_t)(a > 1.25 * h) +
         (uint32_t)(a >= 1.75 * h) + (uint32_t)(a > 2.5 * h) + (uint32_t)(a >= 3.5 * h) + (uint32_t)(a > 5.0 * h);
}

__device__ __forceinline__ double e2m1_mag_value(uint32_t c) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  const double lo = (c & 1u) ? 1.5 : 1.0;
  const uint32_t e = (c >> 1) & 3u;
  return e == 0 ? 0.5 * (double)(c & 1u) : lo * (double)(1u << (e - 1));
}

// magnitudes (bits 0-2 of each nibble) of 8 codes -> new magnitudes via the table
// lut = {lo: new[0..3], hi: new[4..7]} (one byte each), signs kept
__device__ __forceinline__ uint32_t remap8(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  const uint32_t ev = __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u);
  const uint32_t od = __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u);
  return (w & 0x88888888u) | ev | (od << 4);
}

// Re-encode one block (codes w, scale byte sb, segment scale gs) under gsh; returns
// the new scale byte and rewrites w.
__device__ __forceinline__ uint32_t requant_block(u32x2& w, uint32_t sb, float gs, float gsh) {
  uint32_t cmax = 0;                                                   // largest magnitude code
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cmax = max(cmax, (w[0] >> (4 * i)) & 7u);
    cmax = max(cmax, (w[1] >> (4 * i)) & 7u);
  }
  const double sgs = (double)e4m3_to_f32(sb) * (double)gs;            // exact: 4 + 24 bits
  const double amax = e2m1_mag_value(cmax) * sgs;                     // exact
  const uint32_t nb = (amax > 0.0 && gsh > 0.0f) ? e4m3_byte_of_quotient(amax / (6.0 * (double)gsh)) : 0u;
  const double h = (double)e4m3_to_f32(nb) * (double)gsh;             // exact
  // Every code is kept when rho = s g_seg / (s' g_shared) lies in [7/8, 7/6): for each
  // E2M1 value v, v rho stays strictly between the midpoints around v or, at
  // rho = 7/8 (v = 2, 4), lands on a tie that goes to v's even code.  8 sgs, 7 h and
  // 6 sgs are exact, so the test is exact.  This holds for every normal-scale block
  // re-encoded under a larger shared scale (the re-rounded scale moves rho <= 1/16).
  if (nb != 0u && 8.0 * sgs >= 7.0 * h && 6.0 * sgs < 7.0 * h) return nb;
  uint32_t lut_lo = 0, lut_hi = 0;
  if (nb != 0u) {
#pragma unroll
    for (uint32_t c = 1; c < 8; ++c) {
      const uint32_t m = e2m1_mag_exact(e2m1_mag_value(c) * sgs, h);
      if (c < 4) lut_lo |= m << (8 * c); else lut_hi |= m << (8 * (c - 4));
    }
  }
  w = u32x2{remap8(w[0], lut_lo, lut_hi), remap8(w[1], lut_lo, lut_hi)};
  return nb;
}

// One lane = BPL consecutive blocks of one row (kb % BPL == 0): BPL * 8 bytes of
// codes and BPL scale bytes, read and written with vector accesses; the four-block
// form writes non-temporally (the re-encoded weight is not read back soon: 23.2 ->
// 20.2 us on the 16384 x 5120 weight).  Group indices
// fit 32 bits (checked on the host).
template <int BPL>
__global__ __launch_bounds__(256) void k_requantize(const uint8_t* codes, const uint8_t* scales, uint32_t groups,
                                                    uint32_t groups_per_row, SegTable seg, const float* seg_gscale,
                                                    const float* gscale_shared, uint8_t* codes_out,
                                                    uint8_t* scales_out, float* gscale_out) {
  float gsh;
  if (gscale_shared) {
    gsh = *gscale_shared;
  } else {
    gsh = seg_gscale[0];
    for (int i = 1; i < seg.n; ++i) gsh = __builtin_fmaxf(gsh, seg_gscale[i]);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale_out = gsh;
  for (uint32_t q = blockIdx.x * blockDim.x + threadIdx.x; q < groups; q += gridDim.x * blockDim.x) {
    const uint32_t row = q / groups_per_row;
    const float gs = seg_gscale[seg_of_col(seg, row)];
    const int64_t b0 = (int64_t)q * BPL;                               // first block
    if constexpr (BPL == 4) {
      const u32x4 c01 = *reinterpret_cast<const u32x4*>(codes + 8 * b0);
      const u32x4 c23 = *reinterpret_cast<const u32x4*>(codes + 8 * b0 + 16);
      const uint32_t s4 = *reinterpret_cast<const uint32_t*>(scales + b0);
      u32x2 w[4] = {u32x2{c01[0], c01[1]}, u32x2{c01[2], c01[3]}, u32x2{c23[0], c23[1]}, u32x2{c23[2], c23[3]}};
      uint32_t ns = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) ns |= requant_block(w[j], (s4 >> (8 * j)) & 0xFFu, gs, gsh) << (8 * j);
      __builtin_nontemporal_store(u32x4{w[0][0], w[0][1], w[1][0], w[1][1]}, reinterpret_cast<u32x4*>(codes_out + 8 * b0));
      __builtin_nontemporal_store(u32x4{w[2][0], w[2][1], w[3][0], w[3][1]}, reinterpret_cast<u32x4*>(codes_out + 8 * b0 + 16));
      __builtin_nontemporal_store(ns, reinterpret_cast<uint32_t*>(scales_out + b0));
    } else {
      u32x2 w = *reinterpret_cast<const u32x2*>(codes + 8 * b0);
      const uint32_t nb = requant_block(w, scales[b0], gs, gsh);
      *reinterpret_cast<u32x2*>(codes_out + 8 * b0) = w;
      scales_out[b0] = (uint8_t)nb;
    }
  }
}

}  // namespace

hipError_t launch_requantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, const SegTable& seg,
                             const float* seg_gscale, const float* gscale_shared, uint8_t* codes_out,
                             uint8_t* scales_out, float* gscale_out, hipStream_t s) {
  const int64_t kb = K / 16;
  const bool four = kb % 4 == 0;                  // 4 blocks per lane (16-byte aligned rows)
  const int64_t groups = N * (four ? kb / 4 : kb);
  if (groups >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int64_t want = (groups + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (four)
    hipLaunchKernelGGL(k_requantize<4>, dim3(grid), dim3(256), 0, s, codes, scales, (uint32_t)groups,
                       (uint32_t)(kb / 4), seg, seg_gscale, gscale_shared, codes_out, scales_out, gscale_out);
  else
    hipLaunchKernelGGL(k_requantize<1>, dim3(grid), dim3(256), 0, s, codes, scales, (uint32_t)groups, (uint32_t)kb,
                       seg, seg_gscale, gscale_shared, codes_out, scales_out, gscale_out);
  return hipGetLastError();
}

}  // namespace nvfp4
