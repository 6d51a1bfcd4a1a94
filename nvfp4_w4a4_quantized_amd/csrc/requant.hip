// Re-encoding of a multi-scale fused NVFP4 weight onto one shared global scale
// ("Why Gated DeltaNet Survives 4-Bit Quantization" review page, strengths
// paragraph / the paper's section 6: the fused-GEMM global-scale mismatch and its
// repair; this is the re-encoding form of the repair, the per-segment epilogue of
// the GEMM kernels the other).
//
// One lane = one 16-element block.  The block's values are x = e2m1 * s * g_seg
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

__global__ __launch_bounds__(256) void k_requantize(const uint8_t* codes, const uint8_t* scales,
                                                    int64_t N, int64_t K, SegTable seg, const float* seg_gscale,
                                                    const float* gscale_shared, uint8_t* codes_out,
                                                    uint8_t* scales_out, float* gscale_out) {
  const int64_t kb = K >> 4;
  const int64_t nblk = N * kb;
  float gsh;
  if (gscale_shared) {
    gsh = *gscale_shared;
  } else {
    gsh = seg_gscale[0];
    for (int i = 1; i < seg.n; ++i) gsh = __builtin_fmaxf(gsh, seg_gscale[i]);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale_out = gsh;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / kb;
    const u32x2 w = *reinterpret_cast<const u32x2*>(codes + 8 * b);    // row-major: block b at byte 8 b
    const uint32_t sb = scales[b];
    const float gs = seg_gscale[seg_of_col(seg, row)];
    // largest magnitude code of the block
    uint32_t cmax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cmax = max(cmax, (w[0] >> (4 * i)) & 7u);
      cmax = max(cmax, (w[1] >> (4 * i)) & 7u);
    }
    const double sgs = (double)e4m3_to_f32(sb) * (double)gs;            // exact: 4 + 24 bits
    const double amax = e2m1_mag_value(cmax) * sgs;                     // exact
    const uint32_t nb = (amax > 0.0 && gsh > 0.0f) ? e4m3_byte_of_quotient(amax / (6.0 * (double)gsh)) : 0u;
    const double h = (double)e4m3_to_f32(nb) * (double)gsh;             // exact
    uint32_t lut_lo = 0, lut_hi = 0;
    if (nb != 0u) {
#pragma unroll
      for (uint32_t c = 1; c < 8; ++c) {
        const uint32_t m = e2m1_mag_exact(e2m1_mag_value(c) * sgs, h);
        if (c < 4) lut_lo |= m << (8 * c); else lut_hi |= m << (8 * (c - 4));
      }
    }
    *reinterpret_cast<u32x2*>(codes_out + 8 * b) = u32x2{remap8(w[0], lut_lo, lut_hi), remap8(w[1], lut_lo, lut_hi)};
    scales_out[b] = (uint8_t)nb;
  }
}

}  // namespace

hipError_t launch_requantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, const SegTable& seg,
                             const float* seg_gscale, const float* gscale_shared, uint8_t* codes_out,
                             uint8_t* scales_out, float* gscale_out, hipStream_t s) {
  const int64_t nblk = N * (K / 16);
  const int64_t want = (nblk + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_requantize, dim3(grid), dim3(256), 0, s, codes, scales, N, K, seg, seg_gscale, gscale_shared,
                     codes_out, scales_out, gscale_out);
  return hipGetLastError();
}

}  // namespace nvfp4
