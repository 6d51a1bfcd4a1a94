// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMaxSeg = 64;
constexpr int kMaxDevices = 64;
// Size of the fixed workspace of nvfp4_w4a4_linear_noalloc: activation codes
// (M * K / 2 bytes) at offset 0, scale bytes (M * K / 16) at the next 256-byte
// boundary.
constexpr int64_t kNoallocScratchBytes = int64_t(32) << 20;

// Segment table passed to kernels by value.  end[i] = one past the last row
// (output column) of segment i; scale[i] = host-given calibrated scale (static mode).
struct SegTable {
  int32_t n;
  int32_t pad;
  int64_t end[kMaxSeg];
  float scale[kMaxSeg];
};

struct GateArgs {
  int32_t n_heads;         // 0 = no gate epilogue
  const float* A_log;
  const float* dt_bias;
};

enum class InType : int { F32 = 0, BF16 = 1 };
enum class OutType : int { F32 = 0, BF16 = 1 };

// quant.hip
hipError_t launch_fill(float* dst, int n, const SegTable* vals_or_null, hipStream_t s);
hipError_t launch_amax_gscale(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                              float* gscale_out, hipStream_t s);
// Quantize rows x K with the global scale gvec[segment(row)]; when gcopy is not
// NULL, gvec[0] is also copied there (the static-mode scale handed back).
hipError_t launch_quant_rows(const void* x, InType t, int64_t rows, int64_t K, int64_t ld,
                             const float* gvec, const SegTable& seg,
                             uint8_t* codes, uint8_t* scales, float* gcopy, hipStream_t s);

// gemm.hip
struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gscale;
  int64_t M, N, K;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_seg_gscale;
  SegTable seg;
  GateArgs gate;
  void* y;
  OutType y_type;
  int64_t ldy;
  // optional per-row (m) and per-column (n) fp32 output factors (the rotated front
  // end's bias corrections); NULL = none.  Supported by launch_gemm_tiled only.
  const float* row_scale;
  const float* col_scale;
};
hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t s);

// Fused decode GEMV (M <= 8): quantizes x itself, optionally writes the codes.
struct GemvArgs {
  const void* x;
  InType x_type;
  int64_t ldx;
  const float* gscale_in;      // NULL = dynamic
  float* gscale_out;
  uint8_t* a_codes_out;        // optional
  uint8_t* a_scales_out;       // optional
  GemmArgs g;                  // a_codes/a_scales/a_gscale unused
};
hipError_t launch_gemv_fused(const GemvArgs& a, hipStream_t s);
// Whether the streaming decode GEMV handles this shape (else the LDS-f16 fallback).
bool gemv_stream_fits(int64_t M, int64_t K, InType t);

// skinny.hip: fused quantize + GEMM for N <= 128 (x read once).  gscale_in is a
// device pointer to the activation global scale (the caller runs the amax pass first
// in dynamic mode), or NULL when M <= linear_skinny_tokens_per_wg() (one workgroup:
// the kernel takes the amax of x itself); gscale_out (optional) receives the scale
// used; a_codes_out / a_scales_out optional.
bool linear_skinny_fits(int64_t M, int64_t N, int64_t K);
int64_t linear_skinny_tokens_per_wg();
hipError_t launch_linear_skinny(const GemvArgs& a, hipStream_t s);

// requant.hip: re-encode a packed weight [N][K] with per-segment global scales
// (device seg_gscale) onto one shared scale (device gscale_shared, or NULL: the
// largest segment scale); in place allowed; the shared scale goes to gscale_out.
hipError_t launch_requantize(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, const SegTable& seg,
                             const float* seg_gscale, const float* gscale_shared, uint8_t* codes_out,
                             uint8_t* scales_out, float* gscale_out, hipStream_t s);

// mx.hip: MXFP4 quantizer (K % 32 == 0) and GEMM on the scaled FP4 MFMA (K % 128 == 0)
hipError_t launch_mx_quant(const void* x, InType t, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, hipStream_t s);
hipError_t launch_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, bool bf16_out,
                          int64_t ldy, hipStream_t s);

// gdn.hip: the gated delta-rule recurrence (d_k = 128, d_v % 8 == 0) over T tokens,
// alpha = e^g and beta read from the gate rows [g | beta] (ldg >= 2 n_v_heads).
bool gdn_shape_ok(int32_t d_k, int32_t d_v);
hipError_t launch_gdn_delta(const float* q, int64_t ldq, const float* k, int64_t ldk, const float* v, int64_t ldv,
                            const float* gates, int64_t ldg, int64_t T, int32_t n_k_heads, int32_t n_v_heads,
                            int32_t d_v, const float* state_in, float* state_out, float* o, int64_t ldo,
                            hipStream_t s);

// probe.hip: n_blocks workgroups of 4 waves, each wave 4 x iters MFMA 32x32x16 f16;
// out receives n_blocks * 256 floats.
hipError_t launch_mfma_peak(int64_t iters, int32_t n_blocks, float* out, hipStream_t s);

// soloq.hip: rotate rows (K = k * 512, k in {1, 2, 4, 8, 10}), quantize them to
// NVFP4 with per-segment global scales (dynamic: from the rotated rows; else the host
// values in seg.scale), write the bias-correction factor of every row and, when
// z_out is not NULL, the rotated rows in fp32.
bool rotate_shape_ok(int64_t K, int32_t h);
hipError_t launch_rotate_quant(const void* x, InType t, int64_t rows, int64_t K, int64_t ldx, const int32_t* perm,
                               const int8_t* signs, const float* Q, const SegTable& seg, bool dynamic,
                               uint8_t* codes, uint8_t* scales, float* seg_gscale_out, float* cbc, float* z_out,
                               hipStream_t s);

// noalloc.hip: this device's copy of the fixed workspace (kNoallocScratchBytes),
// looked up once per device with that device current.
hipError_t noalloc_scratch(void** ptr);

}  // namespace nvfp4
