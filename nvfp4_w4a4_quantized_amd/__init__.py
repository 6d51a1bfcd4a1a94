"""Python binding of libnvfp4.so, the NVFP4 W4A4 linear layer for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI declared in include/nvfp4.h.  torch tensors supply device memory and the
current HIP stream.  The functions carry the C names and raise Nvfp4Error with the
library's message when a call returns an error status.

Importing this package loads the library and raises ImportError if it has not
been built (``python nvfp4_w4a4_quantized_amd/build.py``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARG = 1
NVFP4_ERR_UNSUPPORTED = 2
NVFP4_ERR_HIP = 3
NVFP4_ERR_DEVICE = 4
NVFP4_DTYPE_F32 = 0
NVFP4_DTYPE_BF16 = 1
NVFP4_MAX_SEGMENTS = 64

EXPORTED = ["nvfp4_abi_version", "nvfp4_last_error", "nvfp4_quantize_act", "nvfp4_pack_weight",
            "nvfp4_w4a4_gemm", "nvfp4_w4a4_linear", "nvfp4_w4a4_linear_noalloc", "nvfp4_requantize_weight", "nvfp4_segment_mismatch_factor",
            "nvfp4_require_single_scale", "nvfp4_rotate_quantize", "nvfp4_w4a4_gemm_rowcol",
            "nvfp4_gdn_gated_delta", "nvfp4_mxfp4_quantize", "nvfp4_mxfp4_gemm", "nvfp4_bench_mfma_peak"]


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"nvfp4 status {status}: {msg}")
        self.status = status


class GateParams(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python nvfp4_w4a4_quantized_amd/build.py` "
                          "(the NVFP4 layer has no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.nvfp4_abi_version.restype = I32
    lib.nvfp4_abi_version.argtypes = []
    lib.nvfp4_last_error.restype = ctypes.c_char_p
    lib.nvfp4_last_error.argtypes = []
    lib.nvfp4_quantize_act.restype = I32
    lib.nvfp4_quantize_act.argtypes = [P, I32, I64, I64, I64, P, P, P, P, P]
    lib.nvfp4_pack_weight.restype = I32
    lib.nvfp4_pack_weight.argtypes = [P, I32, I64, I64, I64, I32, P, P, P, P, P, P]
    lib.nvfp4_w4a4_gemm.restype = I32
    lib.nvfp4_w4a4_gemm.argtypes = [P, P, P, I64, I64, I64, P, P, I32, P, P, P, P, I32, I64, P]
    lib.nvfp4_w4a4_linear.restype = I32
    lib.nvfp4_w4a4_linear.argtypes = [P, I32, I64, I64, I64, P, P, I64, P, P, I32, P, P, P, P, I32, I64, P, P, P]
    lib.nvfp4_w4a4_linear_noalloc.restype = I32
    lib.nvfp4_w4a4_linear_noalloc.argtypes = [P, I32, I64, I64, I64, P, P, I64, P, P, I32, P, P, P, P, I32, I64, P]
    lib.nvfp4_requantize_weight.restype = I32
    lib.nvfp4_requantize_weight.argtypes = [P, P, I64, I64, I32, P, P, P, P, P, P, P]
    lib.nvfp4_segment_mismatch_factor.restype = I32
    lib.nvfp4_segment_mismatch_factor.argtypes = [I32, P, ctypes.c_float, P, P]
    lib.nvfp4_require_single_scale.restype = I32
    lib.nvfp4_require_single_scale.argtypes = [I32, P]
    lib.nvfp4_rotate_quantize.restype = I32
    lib.nvfp4_rotate_quantize.argtypes = [P, I32, I64, I64, I64, I32, P, P, P, I32, P, P, P, P, P, P, P, P]
    lib.nvfp4_w4a4_gemm_rowcol.restype = I32
    lib.nvfp4_w4a4_gemm_rowcol.argtypes = [P, P, P, I64, I64, I64, P, P, I32, P, P, P, P, P, I32, I64, P]
    lib.nvfp4_gdn_gated_delta.restype = I32
    lib.nvfp4_gdn_gated_delta.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I32, I32, I32, I32, P, P, P, I64, P]
    lib.nvfp4_bench_mfma_peak.restype = I32
    lib.nvfp4_bench_mfma_peak.argtypes = [I64, I32, P, P]
    lib.nvfp4_mxfp4_quantize.restype = I32
    lib.nvfp4_mxfp4_quantize.argtypes = [P, I32, I64, I64, I64, P, P, P]
    lib.nvfp4_mxfp4_gemm.restype = I32
    lib.nvfp4_mxfp4_gemm.argtypes = [P, P, I64, I64, I64, P, P, P, I32, I64, P]
    return lib


lib = _load()


def nvfp4_abi_version() -> int:
    return int(lib.nvfp4_abi_version())


def nvfp4_last_error() -> str:
    return lib.nvfp4_last_error().decode()


def _check(status: int) -> None:
    if status != NVFP4_OK:
        raise Nvfp4Error(status, nvfp4_last_error())


# ----------------------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return NVFP4_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return NVFP4_DTYPE_BF16
    raise Nvfp4Error(NVFP4_ERR_UNSUPPORTED, f"dtype {t.dtype} is not float32 or bfloat16")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise Nvfp4Error(NVFP4_ERR_INVALID_ARG, f"{name} must be 2-D with unit column stride")
    return t.shape[0], t.shape[1], t.stride(0)


def _seg_array(seg_end: Sequence[int]):
    arr = (ctypes.c_int64 * len(seg_end))(*[int(v) for v in seg_end])
    return arr, len(seg_end)


def _gate(gate):
    if gate is None:
        return None
    A_log, dt_bias = gate
    return GateParams(int(A_log.numel()), A_log.data_ptr(), dt_bias.data_ptr())


def empty_packed(rows: int, K: int, device="cuda"):
    """Device buffers (codes [rows, K/2], scales [rows, K/16]) for a packed operand."""
    torch = _torch()
    return (torch.empty((rows, K // 2), dtype=torch.uint8, device=device),
            torch.empty((rows, K // 16), dtype=torch.uint8, device=device))


def nvfp4_quantize_act(x, gscale_in, codes, scales, gscale_out, stream=None) -> None:
    """Quantize activations x [M, K] (bf16/fp32).  gscale_in None = dynamic mode."""
    M, K, ldx = _rows(x, "x")
    _check(lib.nvfp4_quantize_act(x.data_ptr(), _dtype_code(x), M, K, ldx, _ptr(gscale_in), codes.data_ptr(),
                                  scales.data_ptr(), gscale_out.data_ptr(), _stream(stream)))


def nvfp4_pack_weight(w, seg_end, seg_gscale_in, codes, scales, seg_gscale_out, stream=None) -> None:
    """Pack weight w [N, K] with per-segment global scales.  seg_gscale_in: list of
    host floats (calibrated) or None (per-segment amax)."""
    N, K, ldw = _rows(w, "w")
    seg, n_seg = _seg_array(seg_end)
    gin = None
    if seg_gscale_in is not None:
        gin = (ctypes.c_float * n_seg)(*[float(v) for v in seg_gscale_in])
    _check(lib.nvfp4_pack_weight(w.data_ptr(), _dtype_code(w), N, K, ldw, n_seg, seg, gin, codes.data_ptr(),
                                 scales.data_ptr(), seg_gscale_out.data_ptr(), _stream(stream)))


def nvfp4_w4a4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_end, w_seg_gscale, y, gate=None,
                    stream=None) -> None:
    """y = GEMM of packed operands with the per-segment epilogue (and the gate
    epilogue if gate = (A_log, dt_bias) is given)."""
    M, half_k = a_codes.shape
    N = w_codes.shape[0]
    _, _, ldy = _rows(y, "y")
    seg, n_seg = _seg_array(seg_end)
    g = _gate(gate)
    _check(lib.nvfp4_w4a4_gemm(a_codes.data_ptr(), a_scales.data_ptr(), a_gscale.data_ptr(), M, N, 2 * half_k,
                               w_codes.data_ptr(), w_scales.data_ptr(), n_seg, seg, w_seg_gscale.data_ptr(),
                               ctypes.byref(g) if g is not None else None, y.data_ptr(), _dtype_code(y), ldy,
                               _stream(stream)))


def nvfp4_w4a4_linear(x, gscale_in, gscale_out, w_codes, w_scales, seg_end, w_seg_gscale, y, gate=None,
                      a_codes_out=None, a_scales_out=None, stream=None) -> None:
    """The whole layer: quantize x, GEMM, epilogues."""
    M, K, ldx = _rows(x, "x")
    N = w_codes.shape[0]
    _, _, ldy = _rows(y, "y")
    seg, n_seg = _seg_array(seg_end)
    g = _gate(gate)
    _check(lib.nvfp4_w4a4_linear(x.data_ptr(), _dtype_code(x), M, K, ldx, _ptr(gscale_in), gscale_out.data_ptr(),
                                 N, w_codes.data_ptr(), w_scales.data_ptr(), n_seg, seg, w_seg_gscale.data_ptr(),
                                 ctypes.byref(g) if g is not None else None, y.data_ptr(), _dtype_code(y), ldy,
                                 _ptr(a_codes_out), _ptr(a_scales_out), _stream(stream)))


def nvfp4_w4a4_linear_noalloc(x, gscale_in, gscale_out, w_codes, w_scales, seg_end, w_seg_gscale, y, gate=None,
                              stream=None) -> None:
    """The whole layer with no caller workspace: two-stage shapes keep their
    quantized activations in the library's fixed device workspace."""
    M, K, ldx = _rows(x, "x")
    N = w_codes.shape[0]
    _, _, ldy = _rows(y, "y")
    seg, n_seg = _seg_array(seg_end)
    g = _gate(gate)
    _check(lib.nvfp4_w4a4_linear_noalloc(x.data_ptr(), _dtype_code(x), M, K, ldx, _ptr(gscale_in),
                                         gscale_out.data_ptr(), N, w_codes.data_ptr(), w_scales.data_ptr(), n_seg,
                                         seg, w_seg_gscale.data_ptr(), ctypes.byref(g) if g is not None else None,
                                         y.data_ptr(), _dtype_code(y), ldy, _stream(stream)))


def nvfp4_requantize_weight(codes, scales, seg_end, seg_gscale, gscale_shared, codes_out, scales_out, gscale_out,
                            stream=None) -> None:
    """Re-encode a packed weight with per-segment global scales (device seg_gscale)
    onto one shared scale (device 1-element tensor, or None: the largest segment
    scale).  codes_out/scales_out may be codes/scales themselves (in place)."""
    N, half_k = codes.shape
    seg, n_seg = _seg_array(seg_end)
    _check(lib.nvfp4_requantize_weight(codes.data_ptr(), scales.data_ptr(), N, 2 * half_k, n_seg, seg,
                                       seg_gscale.data_ptr(), _ptr(gscale_shared), codes_out.data_ptr(),
                                       scales_out.data_ptr(), gscale_out.data_ptr(), _stream(stream)))


def nvfp4_segment_mismatch_factor(seg_gscale: Sequence[float], g_used: float):
    """(worst factor, segment index) by which a single-scale fused GEMM using g_used
    would mis-scale a weight packed with the host segment scales seg_gscale."""
    n = len(seg_gscale)
    arr = (ctypes.c_float * n)(*[float(v) for v in seg_gscale])
    f = ctypes.c_double(0.0)
    w = ctypes.c_int32(0)
    _check(lib.nvfp4_segment_mismatch_factor(n, arr, ctypes.c_float(g_used), ctypes.byref(f), ctypes.byref(w)))
    return f.value, w.value


def nvfp4_require_single_scale(seg_gscale: Sequence[float]) -> None:
    """Raises Nvfp4Error unless every host segment scale of a fused weight is the
    same, i.e. unless a single-scale GEMM (one segment) over it is exact."""
    n = len(seg_gscale)
    arr = (ctypes.c_float * max(n, 1))(*[float(v) for v in seg_gscale])
    _check(lib.nvfp4_require_single_scale(n, arr))


def nvfp4_rotate_quantize(x, perm, signs, Q, codes, scales, seg_gscale_out, cbc_out, seg_end=None,
                          seg_gscale_in=None, z_out=None, h=512, stream=None) -> None:
    """Rotate the rows of x (K-RPBH: perm int32 [K], signs int8 [K], Q fp32 [k, k], all
    on the device), quantize them to NVFP4 with scales from the rotated rows (or the
    host seg_gscale_in), and write the bias-correction factor of every row."""
    rows, K, ldx = _rows(x, "x")
    seg, n_seg = _seg_array([rows] if seg_end is None else seg_end)
    gin = None
    if seg_gscale_in is not None:
        gin = (ctypes.c_float * n_seg)(*[float(v) for v in seg_gscale_in])
    _check(lib.nvfp4_rotate_quantize(x.data_ptr(), _dtype_code(x), rows, K, ldx, h, perm.data_ptr(), signs.data_ptr(),
                                     Q.data_ptr(), n_seg, seg, gin, codes.data_ptr(), scales.data_ptr(),
                                     seg_gscale_out.data_ptr(), cbc_out.data_ptr(), _ptr(z_out), _stream(stream)))


def nvfp4_w4a4_gemm_rowcol(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_end, w_seg_gscale, row_scale,
                           col_scale, y, stream=None) -> None:
    """The block-scaled GEMM with per-row and per-column output factors."""
    M, half_k = a_codes.shape
    N = w_codes.shape[0]
    _, _, ldy = _rows(y, "y")
    seg, n_seg = _seg_array(seg_end)
    _check(lib.nvfp4_w4a4_gemm_rowcol(a_codes.data_ptr(), a_scales.data_ptr(), a_gscale.data_ptr(), M, N, 2 * half_k,
                                      w_codes.data_ptr(), w_scales.data_ptr(), n_seg, seg, w_seg_gscale.data_ptr(),
                                      row_scale.data_ptr(), col_scale.data_ptr(), y.data_ptr(), _dtype_code(y), ldy,
                                      _stream(stream)))


def nvfp4_gdn_gated_delta(q, k, v, gates, n_k_heads, n_v_heads, state_in, state_out, o, d_k=128,
                          stream=None) -> None:
    """The gated delta rule over T tokens: q, k [T, >= n_k_heads*d_k], v and o
    [T, >= n_v_heads*d_v], gates [T, >= 2*n_v_heads] ([g | beta] rows), states
    [n_v_heads, d_k, d_v] (state_in None = zeros); all fp32 on the device."""
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (gates, "gates"), (state_out, "state_out"), (o, "o")):
        if t.dtype != torch.float32:
            raise Nvfp4Error(NVFP4_ERR_UNSUPPORTED, f"{name} must be float32")
    if state_in is not None and (state_in.dtype != torch.float32 or not state_in.is_contiguous()):
        raise Nvfp4Error(NVFP4_ERR_UNSUPPORTED, "state_in must be contiguous float32")
    if not state_out.is_contiguous():
        raise Nvfp4Error(NVFP4_ERR_INVALID_ARG, "state_out must be contiguous")
    T, _, ldq = _rows(q, "q")
    _, _, ldk = _rows(k, "k")
    _, _, ldv = _rows(v, "v")
    _, _, ldg = _rows(gates, "gates")
    _, _, ldo = _rows(o, "o")
    d_v = state_out.shape[-1]
    _check(lib.nvfp4_gdn_gated_delta(q.data_ptr(), ldq, k.data_ptr(), ldk, v.data_ptr(), ldv, gates.data_ptr(), ldg,
                                     T, n_k_heads, n_v_heads, d_k, d_v, _ptr(state_in), state_out.data_ptr(),
                                     o.data_ptr(), ldo, _stream(stream)))


def empty_mx_packed(rows: int, K: int, device="cuda"):
    """Device buffers (codes [rows, K/2], scales [rows, K/32]) for an MXFP4 operand."""
    torch = _torch()
    return (torch.empty((rows, K // 2), dtype=torch.uint8, device=device),
            torch.empty((rows, K // 32), dtype=torch.uint8, device=device))


def nvfp4_mxfp4_quantize(x, codes, scales, stream=None) -> None:
    """MXFP4-quantize x [M, K] (bf16/fp32, K % 32 == 0)."""
    M, K, ldx = _rows(x, "x")
    _check(lib.nvfp4_mxfp4_quantize(x.data_ptr(), _dtype_code(x), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                                    _stream(stream)))


def nvfp4_mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, y, stream=None) -> None:
    """y = MXFP4 GEMM of packed operands (K % 128 == 0)."""
    M, half_k = a_codes.shape
    N = w_codes.shape[0]
    _, _, ldy = _rows(y, "y")
    _check(lib.nvfp4_mxfp4_gemm(a_codes.data_ptr(), a_scales.data_ptr(), M, N, 2 * half_k, w_codes.data_ptr(),
                                w_scales.data_ptr(), y.data_ptr(), _dtype_code(y), ldy, _stream(stream)))


def nvfp4_bench_mfma_peak(iters: int, n_blocks: int, out, stream=None) -> None:
    """Measurement helper: n_blocks x 4 waves issuing 4 * iters f16 MFMA 32x32x16 each."""
    _check(lib.nvfp4_bench_mfma_peak(int(iters), int(n_blocks), out.data_ptr(), _stream(stream)))
