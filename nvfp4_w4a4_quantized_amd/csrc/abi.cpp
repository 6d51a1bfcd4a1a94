// C ABI of the NVFP4 W4A4 linear layer: host-side validation and dispatch.
// Every check happens before anything is enqueued; no call synchronizes.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return NVFP4_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(int32_t t) { return t == NVFP4_DTYPE_F32 ? 4 : 2; }

bool valid_dtype(int32_t t) { return t == NVFP4_DTYPE_F32 || t == NVFP4_DTYPE_BF16; }

// Device check: the kernels are built for gfx950 only.  Cached per device id.
int32_t check_device() {
  static std::mutex mu;
  static int cached[64];   // 0 unknown, 1 ok, 2 bad
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_DEVICE, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    cached[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (cached[dev] != 1) return fail(NVFP4_ERR_DEVICE, "current device is not gfx950 (MI355X)");
  return NVFP4_OK;
}

int32_t check_x(const void* x, int32_t dt, int64_t rows, int64_t K, int64_t ld, const char* name) {
  if (!x) return fail(NVFP4_ERR_INVALID_ARG, "%s is NULL", name);
  if (!valid_dtype(dt)) return fail(NVFP4_ERR_UNSUPPORTED, "%s dtype %d is not F32 or BF16", name, dt);
  if (rows <= 0 || K <= 0) return fail(NVFP4_ERR_INVALID_ARG, "%s shape must be positive (rows=%lld K=%lld)", name,
                                       (long long)rows, (long long)K);
  if (K % 16) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  if (ld < K) return fail(NVFP4_ERR_INVALID_ARG, "ld%s=%lld < K=%lld", name, (long long)ld, (long long)K);
  if (!aligned16(x) || (ld * (int64_t)dtype_size(dt)) % 16)
    return fail(NVFP4_ERR_UNSUPPORTED, "%s must be 16-byte aligned with 16-byte aligned rows", name);
  if (K / 8 > 0xFFFFFFFFll) return fail(NVFP4_ERR_UNSUPPORTED, "K too large");
  return NVFP4_OK;
}

int32_t check_packed(const uint8_t* codes, const uint8_t* scales, const char* name) {
  if (!codes || !scales) return fail(NVFP4_ERR_INVALID_ARG, "%s codes/scales pointer is NULL", name);
  if (!aligned16(codes) || !aligned16(scales))
    return fail(NVFP4_ERR_UNSUPPORTED, "%s codes/scales must be 16-byte aligned", name);
  return NVFP4_OK;
}

int32_t build_seg(int32_t n_seg, const int64_t* seg_end, int64_t N, const float* scales_or_null,
                  nvfp4::SegTable* out) {
  if (n_seg < 1 || n_seg > NVFP4_MAX_SEGMENTS)
    return fail(NVFP4_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, NVFP4_MAX_SEGMENTS);
  if (!seg_end) return fail(NVFP4_ERR_INVALID_ARG, "seg_end is NULL");
  std::memset(out, 0, sizeof(*out));
  out->n = n_seg;
  int64_t prev = 0;
  for (int i = 0; i < n_seg; ++i) {
    if (seg_end[i] <= prev)
      return fail(NVFP4_ERR_INVALID_ARG, "seg_end must be strictly increasing and positive (seg_end[%d]=%lld)", i,
                  (long long)seg_end[i]);
    prev = seg_end[i];
    out->end[i] = seg_end[i];
    if (scales_or_null) {
      const float v = scales_or_null[i];
      if (!std::isfinite(v) || v < 0.0f)
        return fail(NVFP4_ERR_INVALID_ARG, "segment scale %d is not finite and >= 0", i);
      out->scale[i] = v;
    }
  }
  if (prev != N)
    return fail(NVFP4_ERR_INVALID_ARG, "seg_end[last]=%lld must equal N=%lld", (long long)prev, (long long)N);
  return NVFP4_OK;
}

int32_t check_gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                          int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                          const nvfp4_gate_params* gate, const void* y, int32_t y_dtype, int64_t ldy,
                          nvfp4::GemmArgs* g) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "M, N, K must be positive (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 16) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  int32_t st = check_packed(w_codes, w_scales, "w");
  if (st) return st;
  if (!w_seg_gscale) return fail(NVFP4_ERR_INVALID_ARG, "w_seg_gscale is NULL");
  if (!y) return fail(NVFP4_ERR_INVALID_ARG, "y is NULL");
  if (!valid_dtype(y_dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "y dtype %d is not F32 or BF16", y_dtype);
  if (ldy < N) return fail(NVFP4_ERR_INVALID_ARG, "ldy=%lld < N=%lld", (long long)ldy, (long long)N);
  if (!aligned16(y)) return fail(NVFP4_ERR_UNSUPPORTED, "y must be 16-byte aligned");
  st = build_seg(n_seg, seg_end, N, nullptr, &g->seg);
  if (st) return st;
  g->gate = nvfp4::GateArgs{0, nullptr, nullptr};
  if (gate) {
    if (gate->n_heads <= 0) return fail(NVFP4_ERR_INVALID_ARG, "gate n_heads must be positive");
    if (N != 2 * (int64_t)gate->n_heads)
      return fail(NVFP4_ERR_INVALID_ARG, "gate epilogue needs N == 2*n_heads (N=%lld, n_heads=%d)", (long long)N,
                  gate->n_heads);
    if (y_dtype != NVFP4_DTYPE_F32) return fail(NVFP4_ERR_INVALID_ARG, "gate epilogue needs y_dtype F32");
    if (!gate->A_log || !gate->dt_bias) return fail(NVFP4_ERR_INVALID_ARG, "gate A_log/dt_bias is NULL");
    g->gate = nvfp4::GateArgs{gate->n_heads, gate->A_log, gate->dt_bias};
  }
  g->M = M;
  g->N = N;
  g->K = K;
  g->w_codes = w_codes;
  g->w_scales = w_scales;
  g->w_seg_gscale = w_seg_gscale;
  g->y = const_cast<void*>(y);
  g->y_type = y_dtype == NVFP4_DTYPE_F32 ? nvfp4::OutType::F32 : nvfp4::OutType::BF16;
  g->ldy = ldy;
  return NVFP4_OK;
}

nvfp4::InType in_type(int32_t dt) { return dt == NVFP4_DTYPE_F32 ? nvfp4::InType::F32 : nvfp4::InType::BF16; }

// Enqueue activation quantization (validated arguments).
hipError_t enqueue_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const float* gscale_in, uint8_t* codes, uint8_t* scales, float* gscale_out,
                             hipStream_t s) {
  nvfp4::SegTable one{};
  one.n = 1;
  one.end[0] = M;
  hipError_t e;
  const float* gvec;
  float* gcopy = nullptr;
  if (gscale_in) {
    gvec = gscale_in;
    gcopy = gscale_out;            // the quantizer hands the static scale back
  } else {
    e = nvfp4::launch_fill(gscale_out, 1, nullptr, s);
    if (e != hipSuccess) return e;
    e = nvfp4::launch_amax_gscale(x, in_type(x_dtype), M, K, ldx, gscale_out, s);
    if (e != hipSuccess) return e;
    gvec = gscale_out;
  }
  return nvfp4::launch_quant_rows(x, in_type(x_dtype), M, K, ldx, gvec, one, codes, scales, gcopy, s);
}

// The fused decode GEMV holds x as f16 in LDS: M * K * 2 bytes.
constexpr int64_t kGemvMaxM = 8;
constexpr int64_t kGemvLdsBudget = 56 * 1024;

bool linear_fused_gemv(int64_t M, int64_t K, int32_t x_dtype) {
  if (nvfp4::gemv_stream_fits(M, K, in_type(x_dtype))) return true;
  return M <= kGemvMaxM && K % 128 == 0 && M * K * 2 <= kGemvLdsBudget;
}

// Whether nvfp4_w4a4_linear runs this shape in one fused kernel (no activation
// codes in memory) rather than in two stages.
bool linear_fused(int64_t M, int64_t N, int64_t K, int32_t x_dtype) {
  return linear_fused_gemv(M, K, x_dtype) || nvfp4::linear_skinny_fits(M, N, K);
}

// The whole layer.  ws_codes/ws_scales: where the two-stage shapes keep the
// quantized activations (the caller's a_codes_out/a_scales_out, or the fixed
// workspace); codes_out/scales_out: the caller's optional copy on the fused paths.
int32_t linear_impl(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* gscale_in,
                    float* gscale_out, nvfp4::GemmArgs g, uint8_t* codes_out, uint8_t* scales_out,
                    uint8_t* ws_codes, uint8_t* ws_scales, hipStream_t s) {
  if (linear_fused_gemv(M, K, x_dtype)) {
    nvfp4::GemvArgs p{};
    p.x = x;
    p.x_type = in_type(x_dtype);
    p.ldx = ldx;
    p.gscale_in = gscale_in;
    p.gscale_out = gscale_out;
    p.a_codes_out = codes_out;
    p.a_scales_out = scales_out;
    p.g = g;
    return hip_status(nvfp4::launch_gemv_fused(p, s), "nvfp4_w4a4_linear (fused decode) launch");
  }
  if (nvfp4::linear_skinny_fits(M, g.N, K)) {
    hipError_t e = hipSuccess;
    const float* g_used = gscale_in;
    // dynamic mode: one workgroup (M tokens or fewer) takes the amax itself; more
    // tokens run an amax pass over x first
    const bool amax_in_kernel = !gscale_in && M <= nvfp4::linear_skinny_tokens_per_wg();
    if (!gscale_in && !amax_in_kernel) {
      e = nvfp4::launch_fill(gscale_out, 1, nullptr, s);
      if (e == hipSuccess) e = nvfp4::launch_amax_gscale(x, in_type(x_dtype), M, K, ldx, gscale_out, s);
      if (e != hipSuccess) return hip_status(e, "nvfp4_w4a4_linear amax launch");
      g_used = gscale_out;
    }
    nvfp4::GemvArgs p{};
    p.x = x;
    p.x_type = in_type(x_dtype);
    p.ldx = ldx;
    p.gscale_in = g_used;
    p.gscale_out = (gscale_in || amax_in_kernel) ? gscale_out : nullptr;
    p.a_codes_out = codes_out;
    p.a_scales_out = scales_out;
    p.g = g;
    return hip_status(nvfp4::launch_linear_skinny(p, s), "nvfp4_w4a4_linear (fused skinny) launch");
  }
  hipError_t e = enqueue_quant_act(x, x_dtype, M, K, ldx, gscale_in, ws_codes, ws_scales, gscale_out, s);
  if (e != hipSuccess) return hip_status(e, "nvfp4_w4a4_linear quantize launch");
  g.a_codes = ws_codes;
  g.a_scales = ws_scales;
  g.a_gscale = gscale_out;
  return hip_status(nvfp4::launch_gemm_tiled(g, s), "nvfp4_w4a4_linear gemm launch");
}

// Offset of the scale bytes in the fixed workspace, and the bytes a two-stage
// shape needs there.
int64_t noalloc_scales_offset(int64_t M, int64_t K) { return ((M * (K / 2)) + 255) / 256 * 256; }
int64_t noalloc_bytes(int64_t M, int64_t K) { return noalloc_scales_offset(M, K) + M * (K / 16); }

}  // namespace

extern "C" {

int32_t nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

int32_t nvfp4_quantize_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* gscale_in, uint8_t* codes, uint8_t* scales, float* gscale_out,
                           void* stream) {
  int32_t st = check_x(x, x_dtype, M, K, ldx, "x");
  if (st) return st;
  st = check_packed(codes, scales, "activation");
  if (st) return st;
  if (!gscale_out) return fail(NVFP4_ERR_INVALID_ARG, "gscale_out is NULL");
  st = check_device();
  if (st) return st;
  return hip_status(enqueue_quant_act(x, x_dtype, M, K, ldx, gscale_in, codes, scales, gscale_out,
                                      static_cast<hipStream_t>(stream)),
                    "nvfp4_quantize_act launch");
}

int32_t nvfp4_pack_weight(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t ldw, int32_t n_seg,
                          const int64_t* seg_end, const float* seg_gscale_in, uint8_t* codes, uint8_t* scales,
                          float* seg_gscale_out, void* stream) {
  int32_t st = check_x(w, w_dtype, N, K, ldw, "w");
  if (st) return st;
  st = check_packed(codes, scales, "weight");
  if (st) return st;
  if (!seg_gscale_out) return fail(NVFP4_ERR_INVALID_ARG, "seg_gscale_out is NULL");
  nvfp4::SegTable seg;
  st = build_seg(n_seg, seg_end, N, seg_gscale_in, &seg);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (seg_gscale_in) {
    e = nvfp4::launch_fill(seg_gscale_out, n_seg, &seg, s);
  } else {
    e = nvfp4::launch_fill(seg_gscale_out, n_seg, nullptr, s);
    int64_t start = 0;
    for (int i = 0; i < n_seg && e == hipSuccess; ++i) {
      const char* base = static_cast<const char*>(w) + start * ldw * (int64_t)dtype_size(w_dtype);
      e = nvfp4::launch_amax_gscale(base, in_type(w_dtype), seg.end[i] - start, K, ldw, seg_gscale_out + i, s);
      start = seg.end[i];
    }
  }
  if (e == hipSuccess) e = nvfp4::launch_quant_rows(w, in_type(w_dtype), N, K, ldw, seg_gscale_out, seg, codes, scales, nullptr, s);
  return hip_status(e, "nvfp4_pack_weight launch");
}

int32_t nvfp4_w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale, int64_t M,
                        int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int32_t n_seg,
                        const int64_t* seg_end, const float* w_seg_gscale, const nvfp4_gate_params* gate, void* y,
                        int32_t y_dtype, int64_t ldy, void* stream) {
  nvfp4::GemmArgs g{};
  int32_t st = check_packed(a_codes, a_scales, "activation");
  if (st) return st;
  if (!a_gscale) return fail(NVFP4_ERR_INVALID_ARG, "a_gscale is NULL");
  st = check_gemm_common(M, N, K, w_codes, w_scales, n_seg, seg_end, w_seg_gscale, gate, y, y_dtype, ldy, &g);
  if (st) return st;
  st = check_device();
  if (st) return st;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_gscale = a_gscale;
  return hip_status(nvfp4::launch_gemm_tiled(g, static_cast<hipStream_t>(stream)), "nvfp4_w4a4_gemm launch");
}

int32_t nvfp4_w4a4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const float* gscale_in,
                          float* gscale_out, int64_t N, const uint8_t* w_codes, const uint8_t* w_scales,
                          int32_t n_seg, const int64_t* seg_end, const float* w_seg_gscale,
                          const nvfp4_gate_params* gate, void* y, int32_t y_dtype, int64_t ldy, uint8_t* a_codes_out,
                          uint8_t* a_scales_out, void* stream) {
  int32_t st = check_x(x, x_dtype, M, K, ldx, "x");
  if (st) return st;
  if (!gscale_out) return fail(NVFP4_ERR_INVALID_ARG, "gscale_out is NULL");
  if ((a_codes_out == nullptr) != (a_scales_out == nullptr))
    return fail(NVFP4_ERR_INVALID_ARG, "a_codes_out and a_scales_out must both be given or both be NULL");
  if (a_codes_out) {
    st = check_packed(a_codes_out, a_scales_out, "activation");
    if (st) return st;
  }
  nvfp4::GemmArgs g{};
  st = check_gemm_common(M, N, K, w_codes, w_scales, n_seg, seg_end, w_seg_gscale, gate, y, y_dtype, ldy, &g);
  if (st) return st;
  if (!linear_fused(M, N, K, x_dtype) && !a_codes_out)
    return fail(NVFP4_ERR_INVALID_ARG,
                "this shape (M=%lld, N=%lld, K=%lld) runs in two stages and needs a_codes_out/a_scales_out",
                (long long)M, (long long)N, (long long)K);
  st = check_device();
  if (st) return st;
  return linear_impl(x, x_dtype, M, K, ldx, gscale_in, gscale_out, g, a_codes_out, a_scales_out, a_codes_out,
                     a_scales_out, static_cast<hipStream_t>(stream));
}

int32_t nvfp4_w4a4_linear_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  const float* gscale_in, float* gscale_out, int64_t N, const uint8_t* w_codes,
                                  const uint8_t* w_scales, int32_t n_seg, const int64_t* seg_end,
                                  const float* w_seg_gscale, const nvfp4_gate_params* gate, void* y,
                                  int32_t y_dtype, int64_t ldy, void* stream) {
  int32_t st = check_x(x, x_dtype, M, K, ldx, "x");
  if (st) return st;
  if (!gscale_out) return fail(NVFP4_ERR_INVALID_ARG, "gscale_out is NULL");
  nvfp4::GemmArgs g{};
  st = check_gemm_common(M, N, K, w_codes, w_scales, n_seg, seg_end, w_seg_gscale, gate, y, y_dtype, ldy, &g);
  if (st) return st;
  const bool fused = linear_fused(M, N, K, x_dtype);
  if (!fused && noalloc_bytes(M, K) > nvfp4::kNoallocScratchBytes)
    return fail(NVFP4_ERR_INVALID_ARG,
                "M=%lld, K=%lld needs %lld bytes of activation workspace; the fixed workspace holds %lld "
                "(use nvfp4_w4a4_linear with caller buffers)",
                (long long)M, (long long)K, (long long)noalloc_bytes(M, K), (long long)nvfp4::kNoallocScratchBytes);
  st = check_device();
  if (st) return st;
  uint8_t* ws = nullptr;
  if (!fused) {
    void* p = nullptr;
    const hipError_t e = nvfp4::noalloc_scratch(&p);
    if (e != hipSuccess) return hip_status(e, "nvfp4_w4a4_linear_noalloc workspace lookup");
    ws = static_cast<uint8_t*>(p);
  }
  return linear_impl(x, x_dtype, M, K, ldx, gscale_in, gscale_out, g, nullptr, nullptr, ws,
                     ws ? ws + noalloc_scales_offset(M, K) : nullptr, static_cast<hipStream_t>(stream));
}

int32_t nvfp4_requantize_weight(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, int32_t n_seg,
                                const int64_t* seg_end, const float* seg_gscale, const float* gscale_shared,
                                uint8_t* codes_out, uint8_t* scales_out, float* gscale_out, void* stream) {
  if (N <= 0 || K <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "N, K must be positive (N=%lld K=%lld)", (long long)N, (long long)K);
  if (K % 16) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  int32_t st = check_packed(codes, scales, "weight");
  if (st) return st;
  st = check_packed(codes_out, scales_out, "output");
  if (st) return st;
  if (!seg_gscale) return fail(NVFP4_ERR_INVALID_ARG, "seg_gscale is NULL");
  if (!gscale_out) return fail(NVFP4_ERR_INVALID_ARG, "gscale_out is NULL");
  // the kernel writes *gscale_out while other workgroups still read the segment
  // scales and the shared scale: it must alias neither
  if (n_seg >= 1 && n_seg <= NVFP4_MAX_SEGMENTS && gscale_out >= seg_gscale && gscale_out < seg_gscale + n_seg)
    return fail(NVFP4_ERR_INVALID_ARG, "gscale_out must not point into seg_gscale");
  if (gscale_out == gscale_shared) return fail(NVFP4_ERR_INVALID_ARG, "gscale_out must not alias gscale_shared");
  // in place, or no overlap at all (a partial overlap would let one lane read bytes
  // that another has already rewritten)
  const uintptr_t cb = (uintptr_t)codes, co = (uintptr_t)codes_out, sb = (uintptr_t)scales, so = (uintptr_t)scales_out;
  const uintptr_t ncode = (uintptr_t)(N * (K / 2)), nscale = (uintptr_t)(N * (K / 16));
  if (cb != co && cb < co + ncode && co < cb + ncode)
    return fail(NVFP4_ERR_INVALID_ARG, "codes_out partially overlaps codes");
  if (sb != so && sb < so + nscale && so < sb + nscale)
    return fail(NVFP4_ERR_INVALID_ARG, "scales_out partially overlaps scales");
  if (N * (K / 16) >= (int64_t(1) << 31)) return fail(NVFP4_ERR_UNSUPPORTED, "N * K / 16 must be < 2^31");
  nvfp4::SegTable seg;
  st = build_seg(n_seg, seg_end, N, nullptr, &seg);
  if (st) return st;
  st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_requantize(codes, scales, N, K, seg, seg_gscale, gscale_shared, codes_out,
                                             scales_out, gscale_out, static_cast<hipStream_t>(stream)),
                    "nvfp4_requantize_weight launch");
}

int32_t nvfp4_segment_mismatch_factor(int32_t n_seg, const float* seg_gscale, float g_used, double* factor_out,
                                      int32_t* worst_out) {
  if (n_seg < 1 || n_seg > NVFP4_MAX_SEGMENTS)
    return fail(NVFP4_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, NVFP4_MAX_SEGMENTS);
  if (!seg_gscale) return fail(NVFP4_ERR_INVALID_ARG, "seg_gscale is NULL");
  if (!std::isfinite(g_used) || !(g_used > 0.0f)) return fail(NVFP4_ERR_INVALID_ARG, "g_used must be finite and > 0");
  double worst = 0.0;
  int32_t at = 0;
  for (int32_t i = 0; i < n_seg; ++i) {
    const float g = seg_gscale[i];
    if (!std::isfinite(g) || !(g > 0.0f)) return fail(NVFP4_ERR_INVALID_ARG, "segment scale %d must be finite and > 0", i);
    const double r = (double)g_used / (double)g;
    const double f = r >= 1.0 ? r : 1.0 / r;
    if (f > worst) {
      worst = f;
      at = i;
    }
  }
  if (factor_out) *factor_out = worst;
  if (worst_out) *worst_out = at;
  return ok();
}

int32_t nvfp4_require_single_scale(int32_t n_seg, const float* seg_gscale) {
  double factor = 0.0;
  int32_t worst = 0;
  const int32_t st = nvfp4_segment_mismatch_factor(n_seg, seg_gscale, n_seg >= 1 && seg_gscale ? seg_gscale[0] : 1.0f,
                                                   &factor, &worst);
  if (st) return st;
  if (factor != 1.0)
    return fail(NVFP4_ERR_INVALID_ARG,
                "the weight has more than one distinct segment scale (segment %d is %.6g times segment 0's): a "
                "GEMM launched with n_seg == 1 would mis-scale it; pass its segment table",
                worst, (double)seg_gscale[worst] / (double)seg_gscale[0]);
  return ok();
}

int32_t nvfp4_gdn_gated_delta(const float* q, int64_t ldq, const float* k, int64_t ldk, const float* v, int64_t ldv,
                              const float* gates, int64_t ldg, int64_t T, int32_t n_k_heads, int32_t n_v_heads,
                              int32_t d_k, int32_t d_v, const float* state_in, float* state_out, float* o,
                              int64_t ldo, void* stream) {
  if (!q || !k || !v || !gates || !state_out || !o)
    return fail(NVFP4_ERR_INVALID_ARG, "q, k, v, gates, state_out and o must not be NULL");
  if (T <= 0 || n_k_heads <= 0 || n_v_heads <= 0 || d_k <= 0 || d_v <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "T, head counts and head dimensions must be positive");
  if (n_v_heads % n_k_heads)
    return fail(NVFP4_ERR_INVALID_ARG, "n_v_heads=%d is not a multiple of n_k_heads=%d", n_v_heads, n_k_heads);
  if (!nvfp4::gdn_shape_ok(d_k, d_v))
    return fail(NVFP4_ERR_UNSUPPORTED, "the recurrence supports d_k == 128 and d_v a multiple of 8 (d_k=%d d_v=%d)",
                d_k, d_v);
  if (ldq < (int64_t)n_k_heads * d_k || ldk < (int64_t)n_k_heads * d_k || ldv < (int64_t)n_v_heads * d_v ||
      ldo < (int64_t)n_v_heads * d_v || ldg < 2 * (int64_t)n_v_heads)
    return fail(NVFP4_ERR_INVALID_ARG, "a row stride is shorter than its row");
  if (!aligned16(q) || !aligned16(k) || ldq % 4 || ldk % 4)
    return fail(NVFP4_ERR_UNSUPPORTED, "q and k must be 16-byte aligned with 16-byte aligned rows");
  if ((int64_t)n_v_heads * (d_v / 8) >= (int64_t(1) << 31)) return fail(NVFP4_ERR_UNSUPPORTED, "too many heads");
  const int64_t lim = int64_t(1) << 31;
  if (T * ldq * 4 >= lim || T * ldk * 4 >= lim || T * ldv * 4 >= lim || T * ldg * 4 >= lim || T * ldo >= lim)
    return fail(NVFP4_ERR_UNSUPPORTED, "each of q, k, v, gates must span < 2^31 bytes");
  int32_t st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_gdn_delta(q, ldq, k, ldk, v, ldv, gates, ldg, T, n_k_heads, n_v_heads, d_v,
                                            state_in, state_out, o, ldo, static_cast<hipStream_t>(stream)),
                    "nvfp4_gdn_gated_delta launch");
}

int32_t nvfp4_rotate_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, int64_t ldx, int32_t h,
                              const int32_t* perm, const int8_t* signs, const float* Q, int32_t n_seg,
                              const int64_t* seg_end, const float* seg_gscale_in, uint8_t* codes, uint8_t* scales,
                              float* seg_gscale_out, float* cbc_out, float* z_out, void* stream) {
  int32_t st = check_x(x, x_dtype, rows, K, ldx, "x");
  if (st) return st;
  st = check_packed(codes, scales, "output");
  if (st) return st;
  if (!perm || !signs || !Q) return fail(NVFP4_ERR_INVALID_ARG, "perm, signs and Q must not be NULL");
  if (!seg_gscale_out || !cbc_out) return fail(NVFP4_ERR_INVALID_ARG, "seg_gscale_out and cbc_out must not be NULL");
  if (!nvfp4::rotate_shape_ok(K, h))
    return fail(NVFP4_ERR_UNSUPPORTED, "the rotation supports h = 512 and K = k * 512 with k in {1, 2, 4, 8, 10} "
                "(K=%lld h=%d)", (long long)K, h);
  if (z_out && (reinterpret_cast<uintptr_t>(z_out) & 15u))
    return fail(NVFP4_ERR_UNSUPPORTED, "z_out must be 16-byte aligned");
  nvfp4::SegTable seg;
  st = build_seg(n_seg, seg_end, rows, seg_gscale_in, &seg);
  if (st) return st;
  st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_rotate_quant(x, in_type(x_dtype), rows, K, ldx, perm, signs, Q, seg,
                                               seg_gscale_in == nullptr, codes, scales, seg_gscale_out, cbc_out,
                                               z_out, static_cast<hipStream_t>(stream)),
                    "nvfp4_rotate_quantize launch");
}

int32_t nvfp4_w4a4_gemm_rowcol(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale, int64_t M,
                               int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int32_t n_seg,
                               const int64_t* seg_end, const float* w_seg_gscale, const float* row_scale,
                               const float* col_scale, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  nvfp4::GemmArgs g{};
  int32_t st = check_packed(a_codes, a_scales, "activation");
  if (st) return st;
  if (!a_gscale) return fail(NVFP4_ERR_INVALID_ARG, "a_gscale is NULL");
  if (!row_scale || !col_scale) return fail(NVFP4_ERR_INVALID_ARG, "row_scale and col_scale must not be NULL");
  st = check_gemm_common(M, N, K, w_codes, w_scales, n_seg, seg_end, w_seg_gscale, nullptr, y, y_dtype, ldy, &g);
  if (st) return st;
  st = check_device();
  if (st) return st;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_gscale = a_gscale;
  g.row_scale = row_scale;
  g.col_scale = col_scale;
  return hip_status(nvfp4::launch_gemm_tiled(g, static_cast<hipStream_t>(stream)), "nvfp4_w4a4_gemm_rowcol launch");
}

int32_t nvfp4_bench_mfma_peak(int64_t iters, int32_t n_blocks, float* out, void* stream) {
  if (iters <= 0 || n_blocks <= 0 || !out) return fail(NVFP4_ERR_INVALID_ARG, "iters, n_blocks > 0 and out needed");
  int32_t st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_mfma_peak(iters, n_blocks, out, static_cast<hipStream_t>(stream)),
                    "nvfp4_bench_mfma_peak launch");
}

int32_t nvfp4_mxfp4_quantize(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                             uint8_t* scales, void* stream) {
  int32_t st = check_x(x, x_dtype, M, K, ldx, "x");
  if (st) return st;
  if (K % 32) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld is not a multiple of 32 (MXFP4 block)", (long long)K);
  st = check_packed(codes, scales, "mxfp4");
  if (st) return st;
  if (M * (K / 32) >= (int64_t(1) << 32)) return fail(NVFP4_ERR_UNSUPPORTED, "M * K / 32 must be < 2^32");
  st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_mx_quant(x, in_type(x_dtype), M, K, ldx, codes, scales,
                                           static_cast<hipStream_t>(stream)),
                    "nvfp4_mxfp4_quantize launch");
}

int32_t nvfp4_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, int64_t N, int64_t K,
                         const uint8_t* w_codes, const uint8_t* w_scales, void* y, int32_t y_dtype, int64_t ldy,
                         void* stream) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "M, N, K must be positive (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 32) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld is not a multiple of 32 (MXFP4 block)", (long long)K);
  if (K % 128) return fail(NVFP4_ERR_UNSUPPORTED, "the MXFP4 GEMM needs K %% 128 == 0 (K=%lld)", (long long)K);
  int32_t st = check_packed(a_codes, a_scales, "a");
  if (st) return st;
  st = check_packed(w_codes, w_scales, "w");
  if (st) return st;
  if (!y) return fail(NVFP4_ERR_INVALID_ARG, "y is NULL");
  if (!valid_dtype(y_dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "y dtype %d is not F32 or BF16", y_dtype);
  if (ldy < N) return fail(NVFP4_ERR_INVALID_ARG, "ldy=%lld < N=%lld", (long long)ldy, (long long)N);
  if (!aligned16(y)) return fail(NVFP4_ERR_UNSUPPORTED, "y must be 16-byte aligned");
  if (M * (K / 2) >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_UNSUPPORTED, "each packed operand must be < 2^31 bytes");
  const int64_t esz = y_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ldy % 2 || (y_dtype == NVFP4_DTYPE_BF16 && N % 2))
    return fail(NVFP4_ERR_UNSUPPORTED, "the MXFP4 GEMM needs an even ldy (and an even N for bf16 output)");
  if ((M + 264) * ldy * esz >= (int64_t(1) << 32))
    return fail(NVFP4_ERR_UNSUPPORTED, "the MXFP4 GEMM output must span < 4 GiB ((M + 264) * ldy * size)");
  st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_mx_gemm(a_codes, a_scales, w_codes, w_scales, M, N, K, y,
                                          y_dtype == NVFP4_DTYPE_BF16, ldy, static_cast<hipStream_t>(stream)),
                    "nvfp4_mxfp4_gemm launch");
}

}  // extern "C"
