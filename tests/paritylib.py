"""Helpers shared by the GPU parity tests: run the HIP path through the binding,
run the oracle on the same raw inputs, compare (bit-exact for codes/scales/global
scales, within the stated tolerance for GEMM outputs)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import nvfp4 as O

REL_FRO_TOL = 1e-3


def dev_x(values_f32: np.ndarray, bf16_bits=None, device="cuda"):
    """Device tensor of the layer input: bf16 from bit patterns, else fp32."""
    if bf16_bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(device)


def x64_of(values_f32: np.ndarray) -> np.ndarray:
    return np.asarray(values_f32, dtype=np.float32).astype(np.float64)


def gpu_quantize(nv, xt, gscale=None):
    M, K = xt.shape
    codes, scales = nv.empty_packed(M, K, xt.device)
    gout = torch.empty(1, dtype=torch.float32, device=xt.device)
    gin = None if gscale is None else torch.tensor([gscale], dtype=torch.float32, device=xt.device)
    nv.nvfp4_quantize_act(xt, gin, codes, scales, gout)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), np.float32(gout.cpu().numpy()[0])


def gpu_pack(nv, wt, seg_end, seg_gscale=None):
    N, K = wt.shape
    codes, scales = nv.empty_packed(N, K, wt.device)
    gout = torch.empty(len(seg_end), dtype=torch.float32, device=wt.device)
    nv.nvfp4_pack_weight(wt, seg_end, seg_gscale, codes, scales, gout)
    torch.cuda.synchronize()
    return codes, scales, gout


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{what}: {len(bad)} mismatching bytes, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}"


def oracle_reference(ac, as_, ag, wc, ws, seg_end, gw, out_dtype, gate=None, rows=None, cols=None):
    """Oracle output (rounded), unrounded Y64 and per-element bound, optionally
    restricted to a subset of rows of A and columns (= rows of W)."""
    if rows is not None:
        ac, as_ = ac[rows], as_[rows]
    seg = O.segment_rows(seg_end, wc.shape[0])
    gw_rows = np.asarray(gw, dtype=np.float32)[seg]
    if cols is not None:
        wc, ws, gw_rows = wc[cols], ws[cols], gw_rows[cols]
    M = ac.shape[0]
    a_hat = O.dequantize_rows(ac, as_, np.full(M, ag, dtype=np.float32))
    w_hat = O.dequantize_rows(wc, ws, gw_rows)
    y64 = a_hat @ w_hat.T
    absprod = O.gemm_abs_product(ac, as_, wc, ws)
    alpha = np.float64(np.float32(ag)) * gw_rows.astype(np.float64)
    K = ac.shape[1] * 2
    if gate is None:
        yref = O.round_output(y64, out_dtype)
        bound = O.gemm_elem_bound(y64, absprod, alpha, K, out_dtype)
        return yref, y64, bound
    A_log, dt_bias = gate
    out64 = O.gate_epilogue_f64(y64, A_log, dt_bias)
    yref = O.round_output(out64, "f32")
    gb = O.gemm_elem_bound(y64, absprod, alpha, K, "f32")
    bound = O.gate_elem_bound(y64, gb, A_log, dt_bias, yref)
    return yref, out64, bound


def y_to_f64(yt) -> np.ndarray:
    return yt.float().cpu().numpy().astype(np.float64)


def assert_within_tolerance(y_gpu, yref, bound, what):
    err = np.abs(y_gpu - yref)
    denom = np.linalg.norm(yref)
    rel = np.linalg.norm(y_gpu - yref) / (denom if denom > 0 else 1.0)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    assert rel <= REL_FRO_TOL, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO_TOL}"
    worst = np.unravel_index(np.argmax(err / bound), err.shape) if err.size else None
    assert ratio <= 1.0, f"{what}: max err/bound {ratio:.3f} at {worst} (got {y_gpu[worst]}, want {yref[worst]})"
    return rel, ratio
