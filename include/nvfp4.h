/*
 * nvfp4.h - C ABI of the NVFP4 W4A4 linear layer for AMD MI355X (gfx950).
 *
 * The layer (sources: "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4
 * for the Recurrent Half of a Hybrid 27B LLM", review page):
 *   - NVFP4 tensor = 4-bit E2M1 values + one E4M3 scale per 16-element block +
 *     one FP32 global scale per tensor (background section, the paper's section 1;
 *     Key Numbers list).
 *   - the block maximum sets the block scale (mechanism step 1, the paper's
 *     sections 2 and 5.1).
 *   - modules calibrated separately but served as one fused GEMM keep one global
 *     scale per module; the GEMM epilogue applies each segment's own scale
 *     (strengths paragraph, the paper's section 6; the paper's abstract).
 *   - GDN gates g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b)
 *     (mechanism step 2, Eq. 1).
 *
 * Numerics (identical for every entry point and every kernel variant):
 *   global scale (dynamic mode)  g = fp32(amax / 2688), 2688 = 6 * 448
 *   block scale  s = E4M3(t), t = amax_block / (6 g) exactly, round-to-nearest-even,
 *                saturated at 448; byte 0x00 for a zero block, g == 0 or t <= 2^-10
 *   element code RNE of |x| / (s g) (exact quotient) onto {0,.5,1,1.5,2,3,4,6},
 *                saturated at 6, ties to the even code; bit 3 = sign bit of x
 *   packing      codes [rows][K/2] bytes, low nibble = even element;
 *                scales [rows][K/16] E4M3 (OCP FN) bytes, row-major, unswizzled
 *   GEMM         y[m,n] = sum_k (e2m1*s_a)(e2m1*s_w) accumulated in fp32, times
 *                g_a * g_w[segment(n)], rounded once to the output dtype (RNE)
 *
 * Conventions for every function:
 *   - Returns NVFP4_OK (0) when the work was enqueued on `stream`, else an error
 *     code; nvfp4_last_error() then gives a message (thread-local).
 *   - Arguments are validated on the host before anything is enqueued; nothing
 *     synchronizes.  No exception, abort or exit crosses the ABI.
 *   - The caller owns every buffer.  The library allocates and frees no user
 *     memory and keeps no state between calls.
 *   - "device" pointers point to memory of the current HIP device; "host"
 *     pointers are read during the call only.  `stream` is a hipStream_t (NULL =
 *     the null stream).
 *   - Inputs containing NaN or Inf are outside the contract (results unspecified).
 *   - Errors: NVFP4_ERR_INVALID_ARG (null pointer, size <= 0, K % 16 != 0,
 *     ld < K, bad segment table, gate shape mismatch, distinct segment scales
 *     where one scale is required), NVFP4_ERR_UNSUPPORTED
 *     (dtype or alignment outside the supported set), NVFP4_ERR_DEVICE (current
 *     device is not gfx950), NVFP4_ERR_HIP (a HIP launch error).
 *   - Alignment: x, w, y and the packed buffers must be 16-byte aligned, and
 *     ldx/ldw/ldy must keep every row 16-byte aligned (NVFP4_ERR_UNSUPPORTED
 *     otherwise).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

#define NVFP4_ABI_VERSION 1
#define NVFP4_MAX_SEGMENTS 64

enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,
  NVFP4_ERR_UNSUPPORTED = 2,
  NVFP4_ERR_HIP = 3,
  NVFP4_ERR_DEVICE = 4
};

enum nvfp4_dtype {
  NVFP4_DTYPE_F32 = 0,
  NVFP4_DTYPE_BF16 = 1
};

/* GDN gate epilogue parameters (Eq. 1 of the review page, mechanism step 2).
 * The GEMM must have N == 2 * n_heads: columns [0, n_heads) are the a-heads,
 * [n_heads, 2 n_heads) the b-heads.  Output row m = [g_0..g_{H-1} | beta_0..beta_{H-1}],
 * fp32.  A_log and dt_bias are device arrays of n_heads fp32. */
typedef struct nvfp4_gate_params {
  int32_t n_heads;
  const float* A_log;
  const float* dt_bias;
} nvfp4_gate_params;

/* ABI version of the loaded library (NVFP4_ABI_VERSION). */
NVFP4_API int32_t nvfp4_abi_version(void);

/* Message of the last error on this thread ("" if none).  Valid until the next call. */
NVFP4_API const char* nvfp4_last_error(void);

/*
 * Activation quantization (the first stage of the layer).
 *   x         device, [M rows][ldx elements], dtype x_dtype (F32 or BF16)
 *   gscale_in device, 1 fp32: calibrated global scale (static mode), or NULL:
 *             dynamic mode, g = fp32(amax(x) / 2688) computed on the device
 *             (dynamic-mode scales from the tensor itself: "SoloQ" page,
 *             usage/assumptions section)
 *   codes     device, [M][K/2] bytes (output)
 *   scales    device, [M][K/16] bytes (output)
 *   gscale_out device, 1 fp32 (output): the global scale used (a copy of
 *             *gscale_in in static mode).  In dynamic mode it is also the
 *             reduction target, so it must not alias x.
 */
NVFP4_API int32_t nvfp4_quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* gscale_in, uint8_t* codes, uint8_t* scales,
                           float* gscale_out, void* stream);

/*
 * Offline weight packing with one global scale per fused-output segment (module).
 *   w             device, [N rows][ldw elements], F32 or BF16; row n is output column n
 *   n_seg, seg_end host, n_seg (1..NVFP4_MAX_SEGMENTS) strictly increasing row ends,
 *                 seg_end[n_seg-1] == N; segment i covers rows [seg_end[i-1], seg_end[i])
 *   seg_gscale_in host, n_seg fp32 calibrated scales (finite, >= 0), or NULL:
 *                 each segment gets fp32(amax(segment) / 2688)
 *   codes, scales device outputs as for nvfp4_quantize_act ([N][K/2], [N][K/16])
 *   seg_gscale_out device, n_seg fp32 (output): the scales used
 */
NVFP4_API int32_t nvfp4_pack_weight(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw,
                          int32_t n_seg, const int64_t* seg_end, const float* seg_gscale_in,
                          uint8_t* codes, uint8_t* scales, float* seg_gscale_out, void* stream);

/*
 * Block-scaled W4A4 GEMM with the per-segment global-scale epilogue
 * (the repair for fused GEMMs over per-module-calibrated weights) and an
 * optional GDN gate epilogue.
 *   a_codes, a_scales device, quantized activations [M][K/2], [M][K/16]
 *   a_gscale          device, 1 fp32
 *   w_codes, w_scales device, packed weight [N][K/2], [N][K/16]
 *   n_seg, seg_end    host segment table over N (as for nvfp4_pack_weight)
 *   w_seg_gscale      device, n_seg fp32
 *   gate              host struct or NULL; non-NULL requires N == 2 * gate->n_heads
 *                     and y_dtype == F32
 *   y                 device, [M][ldy] of y_dtype (F32 or BF16), output
 */
NVFP4_API int32_t nvfp4_w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        int64_t M, int64_t N, int64_t K,
                        const uint8_t* w_codes, const uint8_t* w_scales,
                        int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                        const nvfp4_gate_params* gate,
                        void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * The whole layer in one call: activation quantization + GEMM + epilogues, i.e. the
 * two stages of the layer ("Why Gated DeltaNet Survives 4-Bit Quantization" review
 * page: background section for the NVFP4 activations, strengths paragraph / the
 * paper's section 6 for the per-segment scales, mechanism step 2, Eq. 1 for the
 * gates).  Fusing the activation quantization into the GEMM addresses the
 * small-batch quantization overhead the page names for decode (limitations, the
 * paper's section 9).
 * Results equal nvfp4_quantize_act followed by nvfp4_w4a4_gemm.  Decode shapes
 * (M <= 8) and skinny shapes (N <= 128 with K a multiple of 256) run fused
 * kernels that quantize x in registers and never write the activation codes to
 * memory unless asked (in dynamic mode the skinny path first reads x once for
 * its amax: in a separate pass when M > 128, inside the one launch when M <= 128);
 * other shapes run the two stages and then need a_codes_out and
 * a_scales_out as the place to put the quantized activations.
 *   x, x_dtype, M, K, ldx, gscale_in   as for nvfp4_quantize_act
 *   gscale_out     device, 1 fp32 (output): the activation global scale used
 *   N, w_*, n_seg, seg_end, w_seg_gscale, gate, y, y_dtype, ldy  as for nvfp4_w4a4_gemm
 *   a_codes_out, a_scales_out  device [M][K/2], [M][K/16] or NULL.  When given,
 *                  they receive the activation codes and scales on every path.
 */
NVFP4_API int32_t nvfp4_w4a4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                          const float* gscale_in, float* gscale_out,
                          int64_t N, const uint8_t* w_codes, const uint8_t* w_scales,
                          int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                          const nvfp4_gate_params* gate,
                          void* y, int32_t y_dtype, int64_t ldy,
                          uint8_t* a_codes_out, uint8_t* a_scales_out, void* stream);

/*
 * nvfp4_w4a4_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without a_codes_out/a_scales_out, the same kernels and results.  The
 * shapes that run in two stages keep their quantized activations in the library's
 * one fixed device workspace of NVFP4_NOALLOC_WORKSPACE_BYTES, which each GPU holds
 * from the first such call until the process ends; they need
 * ceil(M*K/2 / 256)*256 + M*K/16 bytes of it, and a larger shape returns
 * NVFP4_ERR_INVALID_ARG before anything is enqueued (the fused decode and skinny
 * shapes use no workspace and have no such limit).  The call allocates and frees
 * nothing.  Calls that overlap on one GPU (on different streams, or from different
 * threads) share the workspace and race: serialize them.
 */
#define NVFP4_NOALLOC_WORKSPACE_BYTES (32ll << 20)
NVFP4_API int32_t nvfp4_w4a4_linear_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  const float* gscale_in, float* gscale_out,
                                  int64_t N, const uint8_t* w_codes, const uint8_t* w_scales,
                                  int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                                  const nvfp4_gate_params* gate,
                                  void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * Re-encoding of a fused weight onto one shared global scale: the alternative
 * repair of the fused-GEMM global-scale mismatch, where the per-segment epilogue
 * of nvfp4_w4a4_gemm is the other ("Why Gated DeltaNet Survives 4-Bit
 * Quantization" review page, strengths paragraph / the paper's section 6).
 * Every row is dequantized exactly with its segment's scale (e2m1 * s * g_seg)
 * and quantized again, by the numerics above, under the shared scale.  The
 * result is one NVFP4 tensor: a GEMM over it takes n_seg = 1 and the scale
 * written to gscale_out.  Blocks whose scale stays in the normal E4M3 range
 * keep their codes when the shared scale is the largest segment scale; their
 * scale bytes are re-rounded, so the re-encoding can cost up to 1/16 relative
 * per block (none when the scales differ by powers of two).
 *   codes, scales  device, packed weight [N][K/2], [N][K/16] (as packed by
 *                  nvfp4_pack_weight)
 *   n_seg, seg_end host segment table over the N rows (as for nvfp4_pack_weight)
 *   seg_gscale     device, n_seg fp32: the segment scales the weight was packed with
 *   gscale_shared  device, 1 fp32 (finite, > 0), or NULL: the largest segment scale
 *   codes_out, scales_out device outputs [N][K/2], [N][K/16]; may be the same
 *                  buffers as codes, scales (in place), otherwise must not overlap them
 *   gscale_out     device, 1 fp32 (output): the shared scale used; must not point
 *                  into seg_gscale nor equal gscale_shared (NVFP4_ERR_INVALID_ARG),
 *                  since the kernel writes it while other workgroups read those
 */
NVFP4_API int32_t nvfp4_requantize_weight(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                                int32_t n_seg, const int64_t* seg_end, const float* seg_gscale,
                                const float* gscale_shared, uint8_t* codes_out, uint8_t* scales_out,
                                float* gscale_out, void* stream);

/*
 * Detector of the global-scale mismatch (host only, nothing enqueued): for a
 * fused weight packed with the segment scales seg_gscale (host, n_seg fp32,
 * finite, > 0), a GEMM that applied the single scale g_used (finite, > 0) to
 * every segment would scale segment s's outputs by g_used / g_s.  Writes the
 * worst factor max_s max(g_used / g_s, g_s / g_used) (1.0 = no mismatch) to
 * *factor_out and that segment's index to *worst_out (either may be NULL).
 * The mismatch is silent in the outputs (review page, strengths paragraph), so
 * callers that fuse separately calibrated modules check this before launching a
 * single-scale GEMM.
 */
NVFP4_API int32_t nvfp4_segment_mismatch_factor(int32_t n_seg, const float* seg_gscale, float g_used,
                                      double* factor_out, int32_t* worst_out);

/*
 * Guard for single-scale launches (host only, nothing enqueued): returns NVFP4_OK
 * when the n_seg segment scales a fused weight was packed with (seg_gscale, host,
 * finite, > 0) are all equal, so that nvfp4_w4a4_gemm / nvfp4_w4a4_linear may run
 * it with n_seg == 1 and that one scale; otherwise NVFP4_ERR_INVALID_ARG, with the
 * offending segment and its ratio in the message.  The GEMM cannot make this check
 * itself: the segment scales it receives are device memory, and validation never
 * synchronizes.  The mismatch it catches is silent in the outputs ("Why Gated
 * DeltaNet Survives 4-Bit Quantization" review page, strengths paragraph / the
 * paper's section 6).
 */
NVFP4_API int32_t nvfp4_require_single_scale(int32_t n_seg, const float* seg_gscale);

/*
 * Rotated NVFP4 front end (SoloQ-N; "SoloQ: Calibration-Free Quantization for
 * Diffusion Language Models" page, "how it is used" and "assumptions and limits"
 * sections): every row x of the input is rotated, z = Pi x with the K-RPBH rotation
 * Pi = (Q_k (x) I_h) blkdiag(H_h D_1, ..., H_h D_k) P, quantized to NVFP4 by the
 * numerics above with global scales computed from the rotated rows, and given the
 * scale-only bias correction c_bc(z) = ||z||^2 / <q(z), z> (q(z) the dequantized
 * NVFP4 row; 1 when that product is 0).  Activations are rotated online (one
 * segment); a weight W is rotated offline the same way, row by row (its rows become
 * those of W' = W Pi^T), with one global scale per segment.
 *   x, x_dtype, rows, K, ldx   as for nvfp4_quantize_act / nvfp4_pack_weight
 *   h          block size: 512; K = k * h with k in {1, 2, 4, 8, 10}
 *              (NVFP4_ERR_UNSUPPORTED otherwise)
 *   perm       device int32 [K]: a permutation of 0..K-1, (P x)_i = x[perm[i]]
 *              (entries outside 0..K-1 are clamped; the result is then meaningless)
 *   signs      device int8 [K]: +1 or -1 (negative = -1), the diagonal of D_1..D_k in
 *              the permuted order
 *   Q          device fp32 [k][k] row-major: the cross-block mixer, block r of z is
 *              sum_s Q[r][s] (H_h D_s P x)_s
 *   n_seg, seg_end, seg_gscale_in  as for nvfp4_pack_weight (NULL scales = dynamic:
 *              fp32(amax / 2688) of each segment's rotated rows; activations: one segment)
 *   codes, scales   device outputs [rows][K/2], [rows][K/16]
 *   seg_gscale_out  device, n_seg fp32 (output)
 *   cbc_out    device, rows fp32 (output): c_bc of every row
 *   z_out      device fp32 [rows][K] or NULL: the rotated rows (16-byte aligned)
 * The rotation is evaluated in fp32 in one fixed order (gather and sign, the
 * Walsh-Hadamard butterflies at pair distance 1, 2, ..., h/2 with lower a + b and
 * upper a - b, one multiply by fp32(1/sqrt(h)), then left-to-right sums of
 * separately rounded products Q[r][s] y_s), so that the codes are reproducible.
 * In dynamic mode the rows are rotated twice (once for the global scale).
 */
NVFP4_API int32_t nvfp4_rotate_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, int64_t ldx,
                              int32_t h, const int32_t* perm, const int8_t* signs, const float* Q,
                              int32_t n_seg, const int64_t* seg_end, const float* seg_gscale_in,
                              uint8_t* codes, uint8_t* scales, float* seg_gscale_out, float* cbc_out,
                              float* z_out, void* stream);

/*
 * The GEMM of nvfp4_w4a4_gemm with the bias corrections of the rotated front end
 * folded into its epilogue (SoloQ page, "assumptions and limits": c_bc is absorbed by
 * the per-token and per-row scales): y[m,n] = fp32(fp32(acc * fp32(alpha_n *
 * col_scale[n])) * row_scale[m]) with alpha_n = g_a * g_w[segment(n)], rounded once
 * to y_dtype.  row_scale: device fp32 [M] (the activations' c_bc), col_scale: device
 * fp32 [N] (the weight rows' c_bc); both required.  No gate epilogue.  Other
 * arguments as for nvfp4_w4a4_gemm.
 */
NVFP4_API int32_t nvfp4_w4a4_gemm_rowcol(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                               int64_t M, int64_t N, int64_t K,
                               const uint8_t* w_codes, const uint8_t* w_scales,
                               int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                               const float* row_scale, const float* col_scale,
                               void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * Consumer of the GDN gate outputs: alpha = e^g and the gated delta rule ("Why
 * Gated DeltaNet Survives 4-Bit Quantization" review page: background section,
 * Eq. 2; mechanism step 2, Eq. 1; the spec list's state size K = V = 128).  Per
 * value head h and token t = 0 .. T-1, with key/query head kh = h / (n_v_heads /
 * n_k_heads) (consecutive value heads share a key head):
 *   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T,  o_t = S_t^T q_t / sqrt(d_k)
 * with alpha_t = e^{g_t}, in fp32.  The prediction that the write replaces is the
 * state before the decay, as the equation is printed.
 *   q, k      device fp32, [T][ldq], [T][ldk]: head kh at columns kh*d_k ..; 16-byte
 *             aligned, ldq and ldk multiples of 4 (NVFP4_ERR_UNSUPPORTED otherwise)
 *   v         device fp32, [T][ldv]: value head h at columns h*d_v ..
 *   gates     device fp32, [T][ldg]: the gate epilogue's rows [g_0..g_{H-1} | beta_0..beta_{H-1}]
 *             (H = n_v_heads, ldg >= 2 H), e.g. the output of nvfp4_w4a4_linear with a gate
 *   state_in  device fp32 [n_v_heads][d_k][d_v] or NULL (zero initial state)
 *   state_out device fp32 [n_v_heads][d_k][d_v] (output; may equal state_in)
 *   o         device fp32 [T][ldo] (output): value head h at columns h*d_v ..; must not
 *             overlap q, k, v or gates
 * Supported: d_k == 128, d_v a multiple of 8.  The token chain is sequential; heads
 * and state columns run in parallel.  Keys are expected normalized (unit L2 norm),
 * which with beta in (0, 1) keeps every step a contraction; nothing here normalizes.
 */
NVFP4_API int32_t nvfp4_gdn_gated_delta(const float* q, int64_t ldq, const float* k, int64_t ldk,
                              const float* v, int64_t ldv, const float* gates, int64_t ldg,
                              int64_t T, int32_t n_k_heads, int32_t n_v_heads, int32_t d_k, int32_t d_v,
                              const float* state_in, float* state_out, float* o, int64_t ldo,
                              void* stream);

/*
 * MXFP4 variant (the format the review page names as the next generalization,
 * future work / the paper's section 9): E2M1 codes packed as above, one E8M0 scale
 * byte b (value 2^(b-127)) per 32 elements, no global scale.  The format follows the
 * public OCP Microscaling definition: b = 127 + clamp(floor(log2 amax_block) - 2,
 * -127, 127) (byte 0 for a zero block), codes = RNE of x / 2^(b-127) onto the E2M1
 * magnitudes with ties to even, saturated at 6, sign bit of x.
 *
 * Quantization of rows of x (device, [M][ldx], F32 or BF16, K % 32 == 0):
 *   codes  device [M][K/2], scales device [M][K/32] (outputs)
 */
NVFP4_API int32_t nvfp4_mxfp4_quantize(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* codes, uint8_t* scales, void* stream);

/*
 * MXFP4 GEMM on the native block-scaled FP4 matrix instructions:
 * y[m,n] = sum_k e2m1 * 2^(sa-127) * e2m1 * 2^(sw-127), fp32 accumulation, rounded
 * once to y_dtype.
 *   a_codes, a_scales device [M][K/2], [M][K/32]; w_codes, w_scales device [N][K/2], [N][K/32]
 *   y device [M][ldy] of y_dtype (F32 or BF16), output
 *   K % 128 == 0, even ldy, even N for BF16 output, (M + 264) * ldy * sizeof(y) < 2^32,
 *   each packed operand < 2^31 bytes (NVFP4_ERR_UNSUPPORTED otherwise).
 */
NVFP4_API int32_t nvfp4_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, int64_t N, int64_t K,
                         const uint8_t* w_codes, const uint8_t* w_scales, void* y, int32_t y_dtype, int64_t ldy,
                         void* stream);

/*
 * Measurement helper, not part of the layer: a kernel that only issues f16 MFMA
 * 32x32x16 instructions (n_blocks workgroups of 4 waves, each wave 4 x iters of
 * them, 32768 FLOP each), so that a benchmark can report the matrix rate the chip
 * sustains beside its datasheet peak.  out: device, n_blocks * 256 fp32 (written).
 */
NVFP4_API int32_t nvfp4_bench_mfma_peak(int64_t iters, int32_t n_blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
