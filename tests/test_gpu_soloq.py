"""GPU parity of the rotated NVFP4 front end (SoloQ page: K-RPBH rotation, NVFP4
with scales from the rotated tensor, scale-only bias correction) and of the GEMM
with the bias corrections in its epilogue, through the C ABI, against the oracle.

The rotated values are compared bit for bit with the oracle's fp32 evaluation of
the rotation (both follow one fixed fp32 order), so codes, scale bytes and global
scales must be bit-exact.  c_bc is a ratio of two fp32 sums of non-negative terms
over K elements: each sum is within gamma_K of exact, the block-scale and global
scale products and the division add 4 roundings, so |dc|/c <= 2 gamma_K + 4u."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as O
from oracle import soloq as S
from synth import workloads as W
from tests import paritylib as P

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _c_tol(K):
    g = K * U / (1 - K * U)
    return 2 * g + 4 * U


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_w4a4_quantized_amd as nvmod
    return nvmod


def _params_dev(p):
    return (torch.from_numpy(p["perm"]).cuda(), torch.from_numpy(p["signs"]).cuda(), torch.from_numpy(p["Q"]).cuda())


def _gpu_rotate(nv, xt, p, seg_end=None, seg_g=None, with_z=True):
    rows, K = xt.shape
    perm, signs, Q = _params_dev(p)
    codes, scales = nv.empty_packed(rows, K, "cuda")
    n_seg = 1 if seg_end is None else len(seg_end)
    g = torch.empty(n_seg, dtype=torch.float32, device="cuda")
    c = torch.empty(rows, dtype=torch.float32, device="cuda")
    z = torch.empty((rows, K), dtype=torch.float32, device="cuda") if with_z else None
    nv.nvfp4_rotate_quantize(xt, perm, signs, Q, codes, scales, g, c, seg_end=seg_end, seg_gscale_in=seg_g, z_out=z)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), scales.cpu().numpy(), g.cpu().numpy(), c.cpu().numpy().astype(np.float64),
            None if z is None else z.cpu().numpy())


def _x_case(rows, K, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 60
    if dtype == "bf16":
        bits = W._to_bf16_bits(x)
        return W.bf16_bits_to_f32(bits), P.dev_x(None, bits)
    return x, P.dev_x(x)


@pytest.mark.parametrize("rows,K,dtype,mode", [
    (37, 1024, "bf16", "dynamic"),
    (37, 1024, "bf16", "static"),
    (5, 512, "f32", "dynamic"),
    (130, 2048, "f32", "static"),
    (64, 4096, "bf16", "dynamic"),
    (9, 5120, "bf16", "dynamic"),
])
def test_rotate_quantize_matches_oracle(nv, rows, K, dtype, mode):
    xv, xt = _x_case(rows, K, rows * 13 + K, dtype)
    p = W.krpbh_params(K, 512, seed=K + rows)
    g_static = [0.21] if mode == "static" else None
    gc, gs, gg, gcb, gz = _gpu_rotate(nv, xt, p, seg_g=g_static)
    oc, os_, og, ocb, oz = S.rotate_quantize(xv, p["perm"], p["signs"], p["Q"], 512, seg_gscale=g_static)
    assert np.array_equal(gz.view(np.uint32), oz.view(np.uint32)), "rotated rows differ from the fp32 order"
    assert np.array_equal(gg, og), (gg, og)
    P.assert_bytes_equal(gs, os_, "scales")
    P.assert_bytes_equal(gc, oc, "codes")
    assert np.all(np.abs(gcb - ocb) <= _c_tol(K) * np.abs(ocb)), np.max(np.abs(gcb - ocb) / ocb)


def test_rotate_quantize_weight_segments(nv):
    # a fused weight rotated offline: two segments with their own dynamic scales,
    # and the same weight with calibrated scales
    rng = np.random.default_rng(3)
    w = np.concatenate([rng.standard_normal((40, 1024)) * 0.02, rng.standard_normal((56, 1024)) * 0.08]).astype(np.float32)
    p = W.krpbh_params(1024, 512, seed=4)
    for seg_g in (None, [1e-4, 3e-4]):
        gc, gs, gg, gcb, gz = _gpu_rotate(nv, P.dev_x(w), p, seg_end=[40, 96], seg_g=seg_g)
        oc, os_, og, ocb, oz = S.rotate_quantize(w, p["perm"], p["signs"], p["Q"], 512, seg_end=[40, 96],
                                                 seg_gscale=seg_g)
        assert np.array_equal(gz.view(np.uint32), oz.view(np.uint32))
        assert np.array_equal(gg, og)
        P.assert_bytes_equal(gc, oc, "weight codes")
        P.assert_bytes_equal(gs, os_, "weight scales")
        assert np.all(np.abs(gcb - ocb) <= _c_tol(1024) * np.abs(ocb))


def test_rotate_quantize_without_z_and_zero_rows(nv):
    # rows of zeros: scale bytes 0, codes keep the sign of zero, c_bc = 1
    xv, xt = _x_case(20, 1024, 5, "bf16")
    xv[3] = 0.0
    xt[3] = 0.0
    p = W.krpbh_params(1024, 512, seed=6)
    gc, gs, gg, gcb, _ = _gpu_rotate(nv, xt, p, with_z=False)
    oc, os_, og, ocb, _ = S.rotate_quantize(xv, p["perm"], p["signs"], p["Q"], 512)
    P.assert_bytes_equal(gc, oc, "codes")
    P.assert_bytes_equal(gs, os_, "scales")
    assert gcb[3] == 1.0 and ocb[3] == 1.0


def _rowcol_check(nv, M, N, K, seg_end, out_dtype, seed, rows=None, cols=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 60
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    p = W.krpbh_params(K, 512, seed=seed + 1)
    xt, wt = P.dev_x(x), P.dev_x(w)
    perm, signs, Q = _params_dev(p)
    ac, as_ = nv.empty_packed(M, K, "cuda")
    wc, ws = nv.empty_packed(N, K, "cuda")
    ag = torch.empty(1, dtype=torch.float32, device="cuda")
    wg = torch.empty(len(seg_end), dtype=torch.float32, device="cuda")
    cx = torch.empty(M, dtype=torch.float32, device="cuda")
    cw = torch.empty(N, dtype=torch.float32, device="cuda")
    nv.nvfp4_rotate_quantize(wt, perm, signs, Q, wc, ws, wg, cw, seg_end=seg_end)
    nv.nvfp4_rotate_quantize(xt, perm, signs, Q, ac, as_, ag, cx)
    y = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    nv.nvfp4_w4a4_gemm_rowcol(ac, as_, ag, wc, ws, seg_end, wg, cx, cw, y)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    oxc, oxs, oxg, ocx, _ = S.rotate_quantize(x, p["perm"], p["signs"], p["Q"], 512)
    owc, ows, owg, ocw, _ = S.rotate_quantize(w, p["perm"], p["signs"], p["Q"], 512, seg_end=seg_end)
    assert np.array_equal(ac.cpu().numpy(), oxc) and np.array_equal(wc.cpu().numpy(), owc)
    seg = O.segment_rows(seg_end, N)
    a_hat = O.dequantize_rows(oxc[rows], oxs[rows], np.full(len(rows), oxg[0], dtype=np.float32))
    w_hat = O.dequantize_rows(owc[cols], ows[cols], owg[seg[cols]])
    y64 = (a_hat @ w_hat.T) * ocx[rows][:, None] * ocw[cols][None, :]
    alpha = np.float64(oxg[0]) * owg[seg[cols]].astype(np.float64)
    absprod = O.gemm_abs_product(oxc[rows], oxs[rows], owc[cols], ows[cols])
    bound = S.rowcol_elem_bound(y64, absprod, alpha, ocx[rows], ocw[cols], K, out_dtype)
    bound = bound + (2 * _c_tol(K)) * np.abs(y64)          # the two fp32 c_bc factors
    yref = O.round_output(y64, out_dtype)
    y_gpu = P.y_to_f64(y[torch.from_numpy(rows).cuda()])[:, cols]
    P.assert_within_tolerance(y_gpu, yref, bound, f"rowcol M={M} N={N} K={K}")


def test_gemm_rowcol_small_tiles(nv):
    _rowcol_check(nv, 300, 200, 1024, [64, 200], "bf16", seed=7)
    _rowcol_check(nv, 77, 96, 512, [96], "f32", seed=8)


def test_gemm_rowcol_big_tiles_ragged(nv):
    # M, N >= 512: the 256 x 256 kernel, ragged edges
    _rowcol_check(nv, 700, 600, 1024, [256, 600], "bf16", seed=9)
    _rowcol_check(nv, 512, 768, 2048, [768], "f32", seed=10)


def test_rotated_layer_full_size_sampled(nv):
    """The rotated front end on the GDN in_proj activations at full size (8192 x 5120,
    dynamic scales: the global scale comes from all rotated rows) in the launch
    configuration the benchmark times; the oracle checks the global scale over the
    whole tensor and the bytes, rotated values and c_bc of sampled rows."""
    wl = W.generate("gdn_in_proj_8192x16384x5120", with_weight=False)
    xv, xt = W.x_values_f32(wl), P.dev_x(None, wl.data["x_bf16"])
    p = W.krpbh_params(5120, 512, seed=0)
    gc, gs, gg, gcb, gz = _gpu_rotate(nv, xt, p)
    amax = 0.0
    for r0 in range(0, 8192, 1024):
        amax = max(amax, float(np.max(np.abs(S.rotate_f32(xv[r0:r0 + 1024], p["perm"], p["signs"], p["Q"], 512)))))
    og = O.global_scale(amax)
    assert gg[0] == og
    rows = np.unique(np.append(np.random.default_rng(11).choice(8192, 48, replace=False), 8191))
    oc, os_, _, ocb, oz = S.rotate_quantize(xv[rows], p["perm"], p["signs"], p["Q"], 512, seg_gscale=[og])
    assert np.array_equal(gz[rows].view(np.uint32), oz.view(np.uint32))
    P.assert_bytes_equal(gc[rows], oc, "codes (sampled)")
    P.assert_bytes_equal(gs[rows], os_, "scales (sampled)")
    assert np.all(np.abs(gcb[rows] - ocb) <= _c_tol(5120) * np.abs(ocb))
