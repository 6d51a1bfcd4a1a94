"""Plain CPU oracle for the NVFP4 W4A4 linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The HIP library never uses it; the two share no code, tables or
helpers.  Everything here is numpy in float64 (plus exact rational arithmetic in
a few helpers) and is meant to be checked against the pages by eye.

Sources (the pages are cited by title and section):

* [GDN-4bit review] "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4
  for the Recurrent Half of a Hybrid 27B LLM" (review page).
  - Background section (the paper's section 1): an NVFP4 tensor is 4-bit E2M1
    values, one E4M3 scale for every 16-element block, and one FP32 scale for
    the whole tensor.  The Key Numbers list restates the same composition.
  - Mechanism step 1 (the paper's sections 2 and 5.1): the largest magnitude in a
    block sets that block's scale, so an outlier only coarsens the other 15
    elements of its own block; within a block max/RMS can be at most sqrt(16)=4.
  - Mechanism set-up (the paper's section 5): fake quantization = quantize,
    dequantize, then continue in high precision.
  - Mechanism step 2 (the paper's section 2, Eq. 1): the GDN gates
    g = -exp(A_log) * softplus(a + dt_bias), alpha = exp(g), beta = sigmoid(b).
  - Strengths paragraph (the paper's section 6): modules calibrated one by one
    but served through one fused GEMM need their own global scales; a single
    scale silently corrupts the gates.
* [GDN-4bit abstract] the same paper's abstract (podcast page and abstract
  page): the repair of the global-scale mismatch for fused GEMMs over
  per-module-calibrated NVFP4 checkpoints.
* [SoloQ page] "SoloQ: Calibration-Free Quantization for Diffusion Language
  Models", usage/assumptions section: its NVFP4 variant computes the per-tensor
  global scale and the 16-coordinate block scales from the tensor itself
  (dynamic mode).

Readings where the pages are silent (each is also listed in the design doc):

R1  E2M1 = 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    subnormal.  Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; code bit 3 is the sign.
R2  E4M3 is the OCP "FN" variant: bias 7, subnormals m*2^-9, no infinity,
    0x7F/0xFF are NaN, largest finite 448 (byte 0x7E).
R3  The global scale g is a *decode* multiplier.  Dynamic mode:
    g = fp32(amax / (6*448)) with one fp32 round-to-nearest division; g = 0 for
    an all-zero tensor.  Static (calibrated) mode: g is given.
R4  Block scale: t = a_b / (6 g), the exact quotient, rounded once to E4M3 with
    round-to-nearest-even and saturated at 448.  A zero block, g = 0, or
    t <= 2^-10 gives scale byte 0x00.
R5  Element code: r = |x| / (s g), the exact quotient, saturated at 6, rounded
    once to the E2M1 magnitudes with ties to the even code; the sign bit is the
    sign bit of x (so -0.0 and negatives that round to zero give code 0x8).
    With s = 0 every magnitude code is 0.
R6  Packing: byte j of a row = code[2j] | code[2j+1] << 4 (low nibble = even
    element).  Scales are plain row-major [rows x K/16] bytes.
R7  GEMM: Y = deq(A) deq(W)^T with deq(x) = e2m1 * s * g, evaluated in float64;
    each output column uses the global scale of its weight segment.
R8  Output rounding: once, round-to-nearest-even, to bf16 or fp32.
R9  softplus(z) = log(1 + e^z), evaluated as max(z,0) + log1p(exp(-|z|)).

Why float64 is exact enough for R4/R5: the quotients are compared with
midpoints that have at most 5 (E4M3) or 3 (E2M1) significant bits, times a
value with at most 28 significant bits.  A quotient that is not exactly on a
midpoint is at least ~2^-33 (relative) away from it, far more than the 2^-53
error of one float64 division, so rounding the float64 quotient gives the same
answer as rounding the exact one.  The tests pin this against exact rational
(Fraction) brute force.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16                 # elements per scale block
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GLOBAL_DIVISOR = np.float32(6.0 * 448.0)   # 2688, exact in fp32


# ----------------------------------------------------------------------------
# Format definitions (R1, R2)
# ----------------------------------------------------------------------------

def e2m1_value(code):
    """Value of 4-bit E2M1 code(s): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    mag = np.where(exp == 0, man * 0.5, np.ldexp(1.0 + man / 2.0, exp - 1))
    return np.where(sign == 1, -mag, mag)


def e4m3_value(byte):
    """Value of E4M3 (OCP FN) byte(s): sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0."""
    b = np.asarray(byte, dtype=np.int64)
    sign = (b >> 7) & 1
    exp = (b >> 3) & 15
    man = b & 7
    mag = np.where(exp == 0, np.ldexp(man.astype(np.float64), -9),
                   np.ldexp(1.0 + man / 8.0, exp - 7))
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# Sorted non-negative representable magnitudes; index == code (E2M1) or byte (E4M3).
_E2M1_MAGS = e2m1_value(np.arange(8))             # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_MAGS = e4m3_value(np.arange(0x7F))          # bytes 0x00..0x7E, 0 .. 448


def _round_to_grid_rne(v, grid):
    """Index of the grid value nearest to v (v >= 0 float64, v <= grid[-1]);
    an exact tie goes to the even index (= the even code / byte).

    The midpoint between neighbours is exact in float64 (few significant bits),
    so comparing v with it decides the rounding exactly.
    """
    v = np.asarray(v, dtype=np.float64)
    hi = np.searchsorted(grid, v, side="left")          # grid[hi] >= v
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    mid = (grid[lo] + grid[hi]) / 2.0
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(grid[hi] == v, hi, idx).astype(np.int64)


def e4m3_rne_sat(t):
    """Byte of the E4M3 value nearest to t >= 0 (ties to even byte), saturated at 448 (0x7E)."""
    t = np.minimum(np.asarray(t, dtype=np.float64), E4M3_MAX)
    return _round_to_grid_rne(t, _E4M3_MAGS)


def e2m1_rne_sat(r):
    """Magnitude code (0..7) of the E2M1 value nearest to r >= 0 (ties to even code), saturated at 6."""
    r = np.minimum(np.asarray(r, dtype=np.float64), E2M1_MAX)
    return _round_to_grid_rne(r, _E2M1_MAGS)


# ----------------------------------------------------------------------------
# Global scale (R3)
# ----------------------------------------------------------------------------

def global_scale(amax):
    """Dynamic-mode global scale: fp32(amax / 2688), one IEEE fp32 division.

    amax is the largest |x| of a bf16/fp32 tensor, hence exactly an fp32 value.
    [SoloQ page, usage section: scales derived from the tensor itself]
    """
    a = np.float32(amax)
    if a == 0:
        return np.float32(0.0)
    with np.errstate(over="ignore", under="ignore"):
        return np.float32(a / GLOBAL_DIVISOR)


def tensor_amax(x64):
    return float(np.max(np.abs(x64))) if x64.size else 0.0


# ----------------------------------------------------------------------------
# Quantization (R4, R5, R6)
# ----------------------------------------------------------------------------

def quantize_rows(x64, g_rows):
    """NVFP4-quantize the rows of x64 [R, K] (float64, exact input values).

    g_rows: fp32 global scale for every row (array [R]; one tensor = one value
    repeated, a fused weight = its segment's value).
    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16]).

    Steps, in the pages' order [GDN-4bit review, background and mechanism
    step 1]: per 16-element block take the largest magnitude, derive the E4M3
    block scale from it under the global scale, then round every element of
    the block to E2M1 and pack two codes per byte.
    """
    x64 = np.asarray(x64, dtype=np.float64)
    R, K = x64.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    g = np.asarray(g_rows, dtype=np.float32).astype(np.float64).reshape(R, 1)
    blocks = x64.reshape(R, K // BLOCK, BLOCK)
    a_b = np.max(np.abs(blocks), axis=2)                      # exact
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = a_b / (6.0 * g)                                   # 6*g is exact in float64
    zero = (g == 0) | (a_b == 0)
    t = np.where(zero, 0.0, t)
    sbyte = e4m3_rne_sat(t)                                   # 0x00..0x7E
    s = _E4M3_MAGS[sbyte]                                     # [R, K/16]
    sg = s * g                                                # exact (4 + 24 bits)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = np.abs(blocks) / sg[:, :, None]
    r = np.where((sg == 0)[:, :, None], 0.0, r)
    mag = e2m1_rne_sat(r)
    sign = np.signbit(blocks).astype(np.int64)
    code = (sign << 3) | mag                                  # [R, K/16, 16]
    code = code.reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbyte.astype(np.uint8)


def unpack_codes(packed):
    """[R, K/2] bytes -> [R, K] 4-bit codes (low nibble = even element)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    R, H = p.shape
    out = np.empty((R, 2 * H), dtype=np.int64)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def dequantize_rows(packed, scales, g_rows=None):
    """Fake-quantization decode [GDN-4bit review, mechanism set-up]:
    x_hat = e2m1 * s (* g if g_rows is given), exact in float64."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    s = e4m3_value(np.asarray(scales, dtype=np.uint8)).reshape(R, K // BLOCK, 1)
    v = e2m1_value(codes).reshape(R, K // BLOCK, BLOCK) * s
    v = v.reshape(R, K)
    if g_rows is not None:
        v = v * np.asarray(g_rows, dtype=np.float32).astype(np.float64).reshape(R, 1)
    return v


def quantize_activation(x64, gscale=None):
    """Activation quantization.  gscale None = dynamic mode (g from the tensor's
    amax, [SoloQ page]); otherwise the calibrated fp32 global scale.
    Returns (codes, scales, g)."""
    g = global_scale(tensor_amax(x64)) if gscale is None else np.float32(gscale)
    R = x64.shape[0]
    codes, scales = quantize_rows(x64, np.full(R, g, dtype=np.float32))
    return codes, scales, g


def segment_rows(seg_end, N):
    """Segment index of each of the N weight rows (= output columns)."""
    seg_end = np.asarray(seg_end, dtype=np.int64)
    if seg_end.ndim != 1 or len(seg_end) == 0 or seg_end[-1] != N or np.any(np.diff(seg_end) <= 0) or seg_end[0] <= 0:
        raise ValueError("bad segment table")
    return np.searchsorted(seg_end, np.arange(N), side="right")


def pack_weight(w64, seg_end, seg_gscale=None):
    """Weight packing with one global scale per fused-output segment
    [GDN-4bit review, strengths paragraph (paper section 6); GDN-4bit abstract].
    seg_gscale None = per-segment dynamic scale fp32(amax_seg/2688).
    Returns (codes, scales, g_seg float32[S])."""
    N = w64.shape[0]
    seg = segment_rows(seg_end, N)
    S = len(seg_end)
    if seg_gscale is None:
        g_seg = np.array([global_scale(tensor_amax(w64[seg == i])) for i in range(S)], dtype=np.float32)
    else:
        g_seg = np.asarray(seg_gscale, dtype=np.float32).reshape(S)
    codes, scales = quantize_rows(w64, g_seg[seg])
    return codes, scales, g_seg


# ----------------------------------------------------------------------------
# GEMM + epilogues (R7, R8, R9)
# ----------------------------------------------------------------------------

def gemm_f64(a_codes, a_scales, a_g, w_codes, w_scales, seg_end, w_g_seg):
    """Y64 = deq(A) @ deq(W)^T in float64; column n uses its segment's scale."""
    M = a_codes.shape[0]
    N = w_codes.shape[0]
    a_hat = dequantize_rows(a_codes, a_scales, np.full(M, a_g, dtype=np.float32))
    seg = segment_rows(seg_end, N)
    w_hat = dequantize_rows(w_codes, w_scales, np.asarray(w_g_seg, dtype=np.float32)[seg])
    return a_hat @ w_hat.T


def softplus_f64(z):
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid_f64(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def gate_epilogue_f64(y64, A_log, dt_bias):
    """GDN gates, Eq. 1 [GDN-4bit review, mechanism step 2]:
    columns [0, H) are the a-heads, [H, 2H) the b-heads; returns [g | beta]."""
    A_log = np.asarray(A_log, dtype=np.float32).astype(np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float32).astype(np.float64)
    H = A_log.shape[0]
    if y64.shape[1] != 2 * H:
        raise ValueError("gate epilogue needs N == 2 * n_heads")
    z = y64[:, :H] + dt_bias[None, :]
    g = -np.exp(A_log)[None, :] * softplus_f64(z)
    beta = sigmoid_f64(y64[:, H:])
    return np.concatenate([g, beta], axis=1)


def round_to_bf16(y):
    """Round float64 values once, to nearest-even, onto bf16 (8 significant
    bits); result returned as float64.  Overflow beyond bf16 range is not
    handled (never reached by this layer)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    nz = (y != 0) & np.isfinite(y)
    m, e = np.frexp(y[nz])                 # y = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                # bf16 normal exponent floor (2^-126 = 0.5*2^-125)
    q = np.rint(np.ldexp(y[nz], 8 - e))    # np.rint = round half to even
    out[nz] = np.ldexp(q, e - 8)
    out[~nz] = y[~nz]
    return out


def f64_to_bf16_bits(y):
    """bf16 bit patterns (uint16) of float64 values, rounded once (RNE)."""
    v = round_to_bf16(y).astype(np.float32)          # exact: value already on the bf16 grid
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def round_output(y64, out_dtype):
    """R8: round once to the output dtype; returns float64 of the rounded values."""
    if out_dtype == "bf16":
        return round_to_bf16(y64)
    if out_dtype == "f32":
        return np.asarray(y64, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(out_dtype)


def linear_reference(a_codes, a_scales, a_g, w_codes, w_scales, seg_end, w_g_seg,
                     out_dtype, gate=None):
    """The whole forward on quantized operands: GEMM, optional gate epilogue,
    one rounding to the output dtype.  Returns (y_rounded_f64, y64_unrounded)."""
    y64 = gemm_f64(a_codes, a_scales, a_g, w_codes, w_scales, seg_end, w_g_seg)
    if gate is not None:
        y64 = gate_epilogue_f64(y64, gate["A_log"], gate["dt_bias"])
    return round_output(y64, out_dtype), y64


# ----------------------------------------------------------------------------
# Error bounds used by the parity tests
# ----------------------------------------------------------------------------

U32 = 2.0 ** -24
F32_TINY = 2.0 ** -149          # smallest fp32 subnormal


def ulp(y, out_dtype):
    """Spacing of the output format at |y| (normal range)."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    mbits = 8 if out_dtype == "bf16" else 24
    e = np.floor(np.log2(np.where(y > 0, y, 1.0)))
    e = np.maximum(e, -126)
    sp = np.ldexp(1.0, (e - (mbits - 1)).astype(np.int64))
    return np.where(y > 0, sp, np.ldexp(1.0, -126 - (mbits - 1)))


def gemm_abs_product(a_codes, a_scales, w_codes, w_scales):
    """|A_s| @ |W_s|^T: the scale-decoded operands without global scales, in
    absolute value (the sum that bounds fp32 accumulation error)."""
    a_s = np.abs(dequantize_rows(a_codes, a_scales))
    w_s = np.abs(dequantize_rows(w_codes, w_scales))
    return a_s @ w_s.T


def gemm_elem_bound(y64, abs_prod, alpha_cols, K, out_dtype):
    """Per-element bound on |Y_gpu - round(Y64)| for an fp32-accumulated GEMM:
    one output ulp + gamma_K * |alpha| * (|A_s| |W_s|^T) + 2u |Y64|."""
    gamma = K * U32 / (1.0 - K * U32)
    alpha = np.abs(np.asarray(alpha_cols, dtype=np.float64))[None, :]
    return ulp(round_output(y64, out_dtype), out_dtype) + gamma * alpha * abs_prod + 2 * U32 * np.abs(y64)


def gate_elem_bound(y64_gemm, gemm_bound, A_log, dt_bias, out_rounded):
    """Per-element bound for the gate outputs [g | beta] (fp32):
    |dg| <= e^A_log * sigmoid(z) * (E_a + u(|y| + |dt_bias|)) + 8u|g| + ulp(g)
            + (1 + e^A_log) * 2^-149,
    |dbeta| <= beta(1-beta) * E_b + 8u*beta + ulp(beta) + 2 * 2^-149.
    The u(|y|+|dt_bias|) term covers the fp32 rounding of z = y + dt_bias; 8u
    covers the relative error of the fp32 exp/log1p/divide; the 2^-149 terms
    cover results in the fp32 subnormal range (z below about -87), where each
    fp32 rounding costs up to half a subnormal spacing in absolute terms and
    the one of softplus is then multiplied by e^A_log."""
    A_log = np.asarray(A_log, dtype=np.float32).astype(np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float32).astype(np.float64)
    H = A_log.shape[0]
    ya, yb = y64_gemm[:, :H], y64_gemm[:, H:]
    z = ya + dt_bias[None, :]
    sig_z = sigmoid_f64(z)
    g = -np.exp(A_log)[None, :] * softplus_f64(z)
    beta = sigmoid_f64(yb)
    bg = np.exp(A_log)[None, :] * sig_z * (gemm_bound[:, :H] + U32 * (np.abs(ya) + np.abs(dt_bias)[None, :])) \
        + 8 * U32 * np.abs(g) + ulp(out_rounded[:, :H], "f32") + (1.0 + np.exp(A_log))[None, :] * F32_TINY
    bb = beta * (1 - beta) * gemm_bound[:, H:] + 8 * U32 * beta + ulp(out_rounded[:, H:], "f32") + 2 * F32_TINY
    return np.concatenate([bg, bb], axis=1)


# ----------------------------------------------------------------------------
# Harmonization onto one shared global scale, and the mismatch factor
# ----------------------------------------------------------------------------

def requantize_shared_scale(codes, scales, seg_end, g_seg, g_shared=None):
    """Re-encode a weight packed with one global scale per fused-output segment
    onto one global scale for the whole fused weight: the alternative repair of
    the fused-GEMM global-scale mismatch, where the per-segment epilogue is the
    other [GDN-4bit review, strengths paragraph (the paper's section 6);
    GDN-4bit abstract].

    Reading (the pages name the mismatch and its repair, not a re-encoding
    recipe): every row is dequantized exactly with its own segment's scale,
    x_hat = e2m1 * s * g_seg[seg(row)], and quantized again with the shared
    scale by the same steps as any NVFP4 tensor (quantize_rows).  g_shared
    defaults to the largest segment scale, so no block scale needs more range
    than it had.  float64 stays exact: x_hat has <= 2 + 4 + 24 significant bits,
    compared with midpoints times <= 31-bit values (see the module docstring).

    Returns (codes', scales', g_shared float32)."""
    g_seg = np.asarray(g_seg, dtype=np.float32)
    N = np.asarray(codes).shape[0]
    seg = segment_rows(seg_end, N)
    x_hat = dequantize_rows(codes, scales, g_seg[seg])
    gs = np.float32(np.max(g_seg)) if g_shared is None else np.float32(g_shared)
    c2, s2 = quantize_rows(x_hat, np.full(N, gs, dtype=np.float32))
    return c2, s2, gs


def segment_mismatch_factor(g_seg, g_used):
    """Factor by which a fused GEMM that applies the one global scale g_used to
    every segment mis-scales the worst segment's outputs: max over segments of
    max(g_used / g_s, g_s / g_used) (1.0 when every segment has scale g_used);
    also returns that segment's index.  [GDN-4bit review, strengths paragraph:
    the mismatch is silent, so it has to be detected]"""
    g = np.asarray(g_seg, dtype=np.float32).astype(np.float64)
    u = float(np.float32(g_used))
    f = np.maximum(u / g, g / u)
    worst = int(np.argmax(f))
    return float(f[worst]), worst


# ----------------------------------------------------------------------------
# MXFP4: the next format the pages name (E2M1 elements, one power-of-two scale
# per 32 elements)
# ----------------------------------------------------------------------------
#
# [GDN-4bit review, future work (the paper's section 9 / "range extension"):
# generalize beyond NVFP4 to FP6 and MXFP.]  The pages name the format only.
# Readings (the public OCP Microscaling format definition, not the pages):
# M1  block = 32 consecutive elements of a row; scale = E8M0 byte b (value
#     2^(b - 127)); elements E2M1 as in R1, packed as in R6.
# M2  shared exponent = floor(log2(amax_block)) - 2 (2 = exponent of E2M1's
#     largest value 6 = 1.5 * 2^2), clamped to [-127, 127]; a zero block gets
#     byte 0 and magnitude codes 0.
# M3  element code = RNE of x / 2^shared onto the E2M1 magnitudes (ties to even),
#     saturated at 6 (quotients in [6, 8) occur), sign bit = sign bit of x.
# M4  no global scale; GEMM Y = deq(A) deq(W)^T in float64, rounded once (R8).

MX_BLOCK = 32


def mx_quantize_rows(x64):
    """MXFP4-quantize the rows of x64 [R, K] (float64 of exact fp32/bf16 inputs,
    K % 32 == 0).  Returns (codes uint8 [R, K/2], scales uint8 [R, K/32]).
    Steps: per 32-element block the largest magnitude sets the shared power of
    two (M2), every element is rounded onto E2M1 under it (M3), then packed (R6)."""
    x64 = np.asarray(x64, dtype=np.float64)
    R, K = x64.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x64.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))        # amax = m 2^e, 0.5 <= m < 1
    shared = np.clip(e - 1 - 2, -127, 127)                 # floor(log2 amax) - 2
    shared = np.where(amax > 0, shared, -127)
    q = np.abs(blocks) / np.ldexp(1.0, shared)[:, :, None]  # exact: division by a power of two
    mag = e2m1_rne_sat(q)
    sign = np.signbit(blocks).astype(np.int64)
    code = ((sign << 3) | mag).reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (shared + 127).astype(np.uint8)


def mx_dequantize_rows(packed, scales):
    """x_hat = e2m1 * 2^(scale byte - 127), exact in float64."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127).reshape(R, K // MX_BLOCK, 1)
    return (e2m1_value(codes).reshape(R, K // MX_BLOCK, MX_BLOCK) * s).reshape(R, K)


def mx_gemm_f64(a_codes, a_scales, w_codes, w_scales):
    """Y64 = deq(A) @ deq(W)^T in float64 (M4)."""
    return mx_dequantize_rows(a_codes, a_scales) @ mx_dequantize_rows(w_codes, w_scales).T
