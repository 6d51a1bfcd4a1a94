"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.  Codes, scale bytes and global scales must be bit-exact; GEMM and
gate outputs must be within 1e-3 relative Frobenius error and within the
per-element bound computed by the oracle."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as O
from synth import workloads as W
from tests import paritylib as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_w4a4_quantized_amd as nvmod
    return nvmod


def _x_inputs(wl):
    xv = W.x_values_f32(wl)
    return xv, P.dev_x(xv, wl.data.get("x_bf16"))


# ----------------------------------------------------------------------------- quantization

@pytest.mark.parametrize("name,M", [
    ("tiny_linear_64x128x256", None),
    ("decode_gemv_4x16384x5120", None),
    ("gdn_in_proj_8192x16384x5120", 203),
    ("gdn_gates_32768x96x5120", 130),
    ("mlp_gate_up_32768x34816x5120", 77),
])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_quantize_act_matches_oracle(nv, name, M, mode):
    wl = W.generate(name, M=M, with_weight=False)
    xv, xt = _x_inputs(wl)
    x64 = P.x64_of(xv)
    g_static = np.float32(0.0371) if mode == "static" else None
    oc, os_, og = O.quantize_activation(x64, g_static)
    gc, gs, gg = P.gpu_quantize(nv, xt, None if g_static is None else float(g_static))
    assert gg == og, (gg, og)
    P.assert_bytes_equal(gs, os_, "scales")
    P.assert_bytes_equal(gc, oc, "codes")


def _adversarial_inputs():
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows.append([6.0] + mids + [-m for m in mids] + [0.0])       # E2M1 ties with s = 1
    rows.append([6.375, 1.0, -0.0, 0.125] + [0.0] * 12)           # E4M3 tie 1.0625 -> 1.0
    rows.append([0.0] * 8 + [-0.0] * 8)                           # zero block with -0
    rows.append([1e-3, -1e-3, 6.0] + [0.0] * 13)                  # tiny values round to +-0
    rows.append([3.0, -2.9990234375, 2.5, 0.5] * 4)               # values on and near grid points
    rows.append([1e-30, -3e-31] + [0.0] * 14)                     # scale underflows to 0
    rows.append([5e4, -4.9e4, 1.0, -1.0] * 4)                     # large values, static overflow
    arr = np.array(rows, dtype=np.float32)
    rng = np.random.default_rng(21)
    rnd = (rng.standard_normal((5, 16)) * np.array([[1e-3], [1.0], [37.0], [1e4], [3e-5]])).astype(np.float32)
    return np.concatenate([arr, rnd], axis=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g", [1.0, 0.0371, 2.0, 1e-5, 40.0, None])
def test_quantize_adversarial(nv, dtype, g):
    x = _adversarial_inputs()
    x = np.tile(x, (1, 4))                                        # K = 64
    if dtype == "bf16":
        bits = W._to_bf16_bits(x)
        xv = W.bf16_bits_to_f32(bits)
        xt = P.dev_x(xv, bits)
    else:
        xv, xt = x, P.dev_x(x)
    oc, os_, og = O.quantize_activation(P.x64_of(xv), None if g is None else np.float32(g))
    gc, gs, gg = P.gpu_quantize(nv, xt, g)
    assert gg == og
    P.assert_bytes_equal(gs, os_, "scales")
    P.assert_bytes_equal(gc, oc, "codes")


def test_quantize_near_midpoints_dense(nv):
    """Values placed exactly on and 1..3 fp32 ulps around every E2M1 midpoint under
    non-trivial block scales: exercises the exact fix-up path."""
    rng = np.random.default_rng(22)
    g = np.float32(0.0173)
    rows = []
    for _ in range(64):
        sb = int(rng.integers(0x20, 0x7F))
        s = float(O.e4m3_value(sb))
        blk = np.zeros(16, dtype=np.float64)
        blk[0] = 6 * s * float(g)                                 # sets the block scale to s
        mids = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], size=15)
        vals = (mids * s * float(g)).astype(np.float32)
        d = rng.integers(-3, 4, size=15)
        vals = vals.view(np.int32) + d.astype(np.int32)
        blk[1:] = vals.view(np.float32) * rng.choice([-1, 1], size=15)
        rows.append(blk.astype(np.float32))
    x = np.stack(rows)
    x = np.tile(x, (1, 2))
    oc, os_, og = O.quantize_activation(P.x64_of(x), g)
    gc, gs, gg = P.gpu_quantize(nv, P.dev_x(x), float(g))
    P.assert_bytes_equal(gs, os_, "scales")
    P.assert_bytes_equal(gc, oc, "codes")


def test_quantize_strided_rows_and_ragged(nv):
    rng = np.random.default_rng(23)
    for M, K in [(1, 16), (3, 48), (17, 272), (5, 528)]:
        full = (rng.standard_normal((M, K + 32)) * 3).astype(np.float32)
        xt = P.dev_x(full)[:, :K]                                 # ldx = K + 32
        oc, os_, og = O.quantize_activation(P.x64_of(full[:, :K]))
        gc, gs, gg = P.gpu_quantize(nv, xt)
        assert gg == og
        P.assert_bytes_equal(gs, os_, f"scales {M}x{K}")
        P.assert_bytes_equal(gc, oc, f"codes {M}x{K}")


def test_quantize_deterministic(nv):
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=512, with_weight=False)
    _, xt = _x_inputs(wl)
    a = P.gpu_quantize(nv, xt)
    b = P.gpu_quantize(nv, xt)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


# ----------------------------------------------------------------------------- weight packing

@pytest.mark.parametrize("seg_end,sigma,static", [
    ([256, 512, 1280, 2048], [0.02, 0.04, 0.01, 0.08], False),
    ([48, 96], [0.02, 0.02], False),
    ([1024, 2048], [0.02, 0.08], True),
    ([130], [0.02], False),
])
def test_pack_weight_matches_oracle(nv, seg_end, sigma, static):
    rng = np.random.default_rng(31)
    K = 512
    parts, start = [], 0
    for e, sg in zip(seg_end, sigma):
        parts.append(rng.standard_normal((e - start, K)).astype(np.float32) * np.float32(sg))
        start = e
    w = np.concatenate(parts)
    w64 = w.astype(np.float64)
    gin = None
    if static:
        g0 = O.global_scale(O.tensor_amax(w64[:seg_end[0]]))
        gin = [float(g0), float(np.float32(4) * g0)]
    oc, os_, og = O.pack_weight(w64, seg_end, gin)
    gc, gs, gg = P.gpu_pack(nv, P.dev_x(w), seg_end, gin)
    assert np.array_equal(gg.cpu().numpy(), og)
    P.assert_bytes_equal(gs.cpu().numpy(), os_, "weight scales")
    P.assert_bytes_equal(gc.cpu().numpy(), oc, "weight codes")


# ----------------------------------------------------------------------------- GEMM

def _run_layer(nv, wl, use_linear, out_rows=None, seg_gscale=None, act_static=None):
    """Pack W, quantize X, run the GEMM on the GPU; return everything the oracle check needs."""
    xv, xt = _x_inputs(wl)
    w = wl.data["w32"]
    wt = P.dev_x(w)
    wc, ws, wg = P.gpu_pack(nv, wt, wl.seg_end, seg_gscale)
    M, N = xt.shape[0], w.shape[0]
    y_dtype = torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32
    y = torch.empty((M, N), dtype=y_dtype, device="cuda")
    gate = None
    if wl.gate_heads:
        gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    gin = None if act_static is None else torch.tensor([act_static], dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, wl.K, "cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    if use_linear:
        nv.nvfp4_w4a4_linear(xt, gin, gout, wc, ws, wl.seg_end, wg, y, gate=gate, a_codes_out=ac, a_scales_out=as_)
    else:
        nv.nvfp4_quantize_act(xt, gin, ac, as_, gout)
        nv.nvfp4_w4a4_gemm(ac, as_, gout, wc, ws, wl.seg_end, wg, y, gate=gate)
    torch.cuda.synchronize()
    return dict(xv=xv, w=w, y=y, ac=ac.cpu().numpy(), as_=as_.cpu().numpy(), ag=np.float32(gout.item()),
                wc=wc.cpu().numpy(), ws=ws.cpu().numpy(), wg=wg.cpu().numpy())


def _oracle_side(wl, r, seg_gscale=None, act_static=None, rows=None, cols=None):
    x64 = P.x64_of(r["xv"])
    ac, as_, ag = O.quantize_activation(x64, None if act_static is None else np.float32(act_static))
    w64 = r["w"].astype(np.float64)
    wc, ws, wg = O.pack_weight(w64, wl.seg_end, seg_gscale)
    assert ag == r["ag"] and np.array_equal(wg, r["wg"])
    P.assert_bytes_equal(r["ac"], ac, "activation codes")
    P.assert_bytes_equal(r["as_"], as_, "activation scales")
    P.assert_bytes_equal(r["wc"], wc, "weight codes")
    P.assert_bytes_equal(r["ws"], ws, "weight scales")
    gate = (wl.data["A_log"], wl.data["dt_bias"]) if wl.gate_heads else None
    return P.oracle_reference(ac, as_, ag, wc, ws, wl.seg_end, wg, wl.y_dtype, gate=gate, rows=rows, cols=cols)


def _shrink(wl, N_seg_end=None, sigma=None, M=None, seed=0):
    """Replace the weight by a smaller one with the same segment structure."""
    rng = np.random.default_rng(seed + 100)
    if N_seg_end is not None:
        wl.seg_end = N_seg_end
    if sigma is not None:
        wl.seg_sigma = sigma
    parts, start = [], 0
    for e, sg in zip(wl.seg_end, wl.seg_sigma):
        parts.append(rng.standard_normal((e - start, wl.K)).astype(np.float32) * np.float32(sg))
        start = e
    wl.data["w32"] = np.concatenate(parts)
    wl.N = wl.seg_end[-1]
    return wl


@pytest.mark.parametrize("use_linear", [False, True])
def test_gemm_tiny_config(nv, use_linear):
    wl = W.generate("tiny_linear_64x128x256")
    r = _run_layer(nv, wl, use_linear)
    yref, _, bound = _oracle_side(wl, r)
    P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, "tiny")


@pytest.mark.parametrize("use_linear", [False, True])
@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_gemm_decode_config_full(nv, use_linear, mode):
    wl = W.generate("decode_gemv_4x16384x5120")
    act = 0.0415 if mode == "static" else None
    r = _run_layer(nv, wl, use_linear, act_static=act)
    cols = np.sort(np.random.default_rng(1).choice(wl.N, 2048, replace=False))
    yref, _, bound = _oracle_side(wl, r, act_static=act, cols=cols)
    P.assert_within_tolerance(P.y_to_f64(r["y"])[:, cols], yref, bound, "decode")


def test_gemm_gdn_in_proj_segments(nv):
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=267, with_weight=False)
    _shrink(wl, [256, 512, 1280, 2048])
    r = _run_layer(nv, wl, use_linear=True, act_static=0.04)
    yref, _, bound = _oracle_side(wl, r, act_static=0.04)
    P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, "gdn_in_proj")


def test_gemm_gates_epilogue(nv):
    wl = W.generate("gdn_gates_32768x96x5120", M=300)
    r = _run_layer(nv, wl, use_linear=True)
    yref, _, bound = _oracle_side(wl, r)
    y = P.y_to_f64(r["y"])
    P.assert_within_tolerance(y, yref, bound, "gates")
    assert np.all(y[:, :48] < 0) and np.all((y[:, 48:] >= 0) & (y[:, 48:] <= 1))


def test_gemm_mlp_gate_up_scales_4x_apart(nv):
    wl = W.generate("mlp_gate_up_32768x34816x5120", M=150, with_weight=False)
    _shrink(wl, [512, 1024])
    g0 = O.global_scale(O.tensor_amax(wl.data["w32"][:512].astype(np.float64)))
    seg_g = [float(g0), float(np.float32(4) * g0)]
    r = _run_layer(nv, wl, use_linear=True, seg_gscale=seg_g)
    yref, _, bound = _oracle_side(wl, r, seg_gscale=seg_g)
    P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, "mlp")


@pytest.mark.parametrize("M", [1, 3, 17])
@pytest.mark.parametrize("N,seg_end", [(48, [48]), (96, [48, 96]), (130, [2, 130])])
@pytest.mark.parametrize("K", [16, 48, 272, 640])
def test_gemm_ragged_shapes(nv, M, N, seg_end, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    x = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    x[:, rng.integers(0, K)] *= 40
    bits = W._to_bf16_bits(x)
    xv = W.bf16_bits_to_f32(bits)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wl = W.Workload(name="ragged", M=M, N=N, K=K, x_dtype="bf16", y_dtype="bf16", seg_end=seg_end,
                    seg_sigma=[0.02] * len(seg_end), n_hot=1, hot_gain=(40, 40))
    wl.data.update(x32=x, x_bf16=bits, w32=w)
    for use_linear in (False, True):
        r = _run_layer(nv, wl, use_linear)
        yref, _, bound = _oracle_side(wl, r)
        P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, f"ragged M={M} N={N} K={K} linear={use_linear}")


def test_gemm_deterministic(nv):
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=200, with_weight=False)
    _shrink(wl, [256, 512, 1280, 2048])
    r1 = _run_layer(nv, wl, use_linear=False)
    r2 = _run_layer(nv, wl, use_linear=False)
    assert torch.equal(r1["y"], r2["y"])


def test_linear_codes_equal_two_stage(nv):
    """The fused decode path writes the same activation codes as the stand-alone quantizer."""
    wl = W.generate("decode_gemv_4x16384x5120")
    r1 = _run_layer(nv, wl, use_linear=True)
    r2 = _run_layer(nv, wl, use_linear=False)
    assert np.array_equal(r1["ac"], r2["ac"]) and np.array_equal(r1["as_"], r2["as_"]) and r1["ag"] == r2["ag"]
    y1, y2 = P.y_to_f64(r1["y"]), P.y_to_f64(r2["y"])
    assert np.linalg.norm(y1 - y2) / np.linalg.norm(y2) < 1e-3


# ----------------------------------------------------------------------------- large-tile kernel and full sizes

def test_gemm_big_tile_ragged(nv):
    """M, N >= 512 select the 256 x 256 kernel; ragged edges in both dimensions."""
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=700, with_weight=False)
    _shrink(wl, [300, 1000, 1300], sigma=[0.02, 0.05, 0.01])
    for use_linear in (False, True):
        r = _run_layer(nv, wl, use_linear, act_static=0.04)
        yref, _, bound = _oracle_side(wl, r, act_static=0.04)
        P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, f"big tile linear={use_linear}")


def _cut_k(wl, K):
    """Keep the first K columns of X and W (a shorter reduction, same value mix)."""
    wl.K = K
    for key in ("x32", "x_bf16", "w32"):
        if key in wl.data:
            wl.data[key] = np.ascontiguousarray(wl.data[key][:, :K])
    return wl


@pytest.mark.parametrize("M,seg_end,K", [
    (4100, [1200, 3000, 4500], 640),      # 17 x 18 = 306 tiles: workgroups with two tiles, ragged in M and N
    (4352, [2176, 4352], 256),            # 289 tiles, four K steps
])
def test_gemm_big_tile_several_tiles_per_workgroup(nv, M, seg_end, K):
    """More 256 x 256 tiles than compute units (a second round of workgroups), ragged
    last tiles in both dimensions, a short K; sampled rows include every row of the
    last row tile and sampled columns every column of the last column tile and the
    segment boundaries."""
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=M, with_weight=False)
    _cut_k(wl, K)
    _shrink(wl, seg_end, sigma=[0.02, 0.05, 0.01][:len(seg_end)])
    N = wl.N
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False), np.arange((M - 1) // 256 * 256, M)]))
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), np.arange((N - 1) // 256 * 256, N),
                                     np.asarray(seg_end[:-1]) - 1, np.asarray(seg_end[:-1])]))
    r = _run_layer(nv, wl, False, act_static=0.04)
    yref, _, bound = _oracle_side(wl, r, act_static=0.04, rows=rows, cols=cols)
    y = P.y_to_f64(r["y"])[rows][:, cols]
    P.assert_within_tolerance(y, yref, bound, f"several tiles per workgroup M={M} N={N} K={K}")


def _full_size_check(nv, name, seg_ratio=False, n_rows=24, n_cols=None, seed=5):
    """Full-size run in bench.py's launch configuration (quantize + GEMM, static
    activation scale from a dynamic pre-pass); the oracle checks sampled rows
    (bit-exact activation and weight bytes for them) and the outputs there."""
    wl = W.generate(name)
    xv, xt = _x_inputs(wl)
    w = wl.data["w32"]
    w64_seg_amax = [O.tensor_amax(w[s0:s1].astype(np.float64))
                    for s0, s1 in zip([0] + wl.seg_end[:-1], wl.seg_end)]
    seg_g = None
    if seg_ratio:
        g0 = O.global_scale(w64_seg_amax[0])
        seg_g = [float(np.float32(r) * g0) for r in wl.seg_scale_ratio]
    wt = P.dev_x(w)
    wc, ws, wg = P.gpu_pack(nv, wt, wl.seg_end, seg_g)
    del wt
    M, N = wl.M, wl.N
    gstat = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, wl.K, "cuda")
    nv.nvfp4_quantize_act(xt, None, ac, as_, gstat)
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32, device="cuda")
    gate = None
    if wl.gate_heads:
        gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    nv.nvfp4_quantize_act(xt, gstat, ac, as_, gout)
    nv.nvfp4_w4a4_gemm(ac, as_, gout, wc, ws, wl.seg_end, wg, y, gate=gate)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, n_rows, replace=False))
    rows[-1] = M - 1
    cols = np.arange(N) if n_cols is None else np.sort(rng.choice(N, n_cols, replace=False))
    # oracle: global scales from the full tensors, bytes of the sampled rows only
    ag = O.global_scale(O.tensor_amax(P.x64_of(xv)))
    assert ag == np.float32(gout.item())
    if seg_g is None:
        og = np.array([O.global_scale(a) for a in w64_seg_amax], dtype=np.float32)
    else:
        og = np.asarray(seg_g, dtype=np.float32)
    assert np.array_equal(og, wg.cpu().numpy())
    oac, oas = O.quantize_rows(P.x64_of(xv[rows]), np.full(len(rows), ag, dtype=np.float32))
    P.assert_bytes_equal(ac[torch.from_numpy(rows).cuda()].cpu().numpy(), oac, "activation codes (sampled)")
    P.assert_bytes_equal(as_[torch.from_numpy(rows).cuda()].cpu().numpy(), oas, "activation scales (sampled)")
    seg = O.segment_rows(wl.seg_end, N)
    owc, ows = O.quantize_rows(w[cols].astype(np.float64), og[seg[cols]])
    P.assert_bytes_equal(wc[torch.from_numpy(cols).cuda()].cpu().numpy(), owc, "weight codes (sampled)")
    P.assert_bytes_equal(ws[torch.from_numpy(cols).cuda()].cpu().numpy(), ows, "weight scales (sampled)")
    # outputs at the sampled rows x columns
    gseg = og[seg[cols]]
    a_hat = O.dequantize_rows(oac, oas, np.full(len(rows), ag, dtype=np.float32))
    w_hat = O.dequantize_rows(owc, ows, gseg)
    y64 = a_hat @ w_hat.T
    absprod = O.gemm_abs_product(oac, oas, owc, ows)
    alpha = np.float64(ag) * gseg.astype(np.float64)
    y_gpu = P.y_to_f64(y[torch.from_numpy(rows).cuda()])[:, cols]
    if gate is None:
        yref = O.round_output(y64, wl.y_dtype)
        bound = O.gemm_elem_bound(y64, absprod, alpha, wl.K, wl.y_dtype)
    else:
        out64 = O.gate_epilogue_f64(y64, wl.data["A_log"], wl.data["dt_bias"])
        yref = O.round_output(out64, "f32")
        bound = O.gate_elem_bound(y64, O.gemm_elem_bound(y64, absprod, alpha, wl.K, "f32"),
                                  wl.data["A_log"], wl.data["dt_bias"], yref)
    P.assert_within_tolerance(y_gpu, yref, bound, name)


def test_full_gdn_in_proj_sampled(nv):
    _full_size_check(nv, "gdn_in_proj_8192x16384x5120")


def test_full_gdn_gates_sampled(nv):
    _full_size_check(nv, "gdn_gates_32768x96x5120", n_rows=256)


def test_full_mlp_gate_up_sampled(nv):
    _full_size_check(nv, "mlp_gate_up_32768x34816x5120", seg_ratio=True, n_rows=16, n_cols=4096)


@pytest.mark.parametrize("M", [1, 2, 5, 8])
@pytest.mark.parametrize("K", [512, 2048, 5120])
@pytest.mark.parametrize("xdt,mode", [("bf16", "dynamic"), ("bf16", "static"), ("f32", "dynamic")])
def test_decode_stream_shapes(nv, M, K, xdt, mode):
    """Decode shapes on the streaming GEMV (K % 512 == 0): ragged N, several token
    counts, both input dtypes, dynamic and static activation scales."""
    rng = np.random.default_rng(M * 7919 + K)
    N = 1000
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 60
    bits = W._to_bf16_bits(x) if xdt == "bf16" else None
    xv = W.bf16_bits_to_f32(bits) if xdt == "bf16" else x
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wl = W.Workload(name="decode", M=M, N=N, K=K, x_dtype=xdt, y_dtype="bf16", seg_end=[300, N],
                    seg_sigma=[0.02, 0.02], n_hot=1, hot_gain=(60, 60))
    wl.data.update(x32=x, w32=w)
    if bits is not None:
        wl.data["x_bf16"] = bits
    act = 0.05 if mode == "static" else None
    r = _run_layer(nv, wl, use_linear=True, act_static=act)
    yref, _, bound = _oracle_side(wl, r, act_static=act)
    P.assert_within_tolerance(P.y_to_f64(r["y"]), yref, bound, f"decode M={M} K={K} {xdt} {mode}")


def _skinny_case(M, N, seg_end, K, xdt, seed, gate_heads=0, y_dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 50
    bits = W._to_bf16_bits(x) if xdt == "bf16" else None
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wl = W.Workload(name="skinny", M=M, N=N, K=K, x_dtype=xdt, y_dtype=y_dtype, seg_end=seg_end,
                    seg_sigma=[0.02] * len(seg_end), n_hot=1, hot_gain=(50, 50), gate_heads=gate_heads)
    wl.data.update(x32=x, w32=w)
    if bits is not None:
        wl.data["x_bf16"] = bits
    if gate_heads:
        wl.data["A_log"] = rng.uniform(0.0, 2.7, gate_heads).astype(np.float32)
        wl.data["dt_bias"] = (rng.standard_normal(gate_heads) * 0.5).astype(np.float32)
    return wl


@pytest.mark.parametrize("M,N,seg_end,K,xdt,gate_heads,y_dtype", [
    (300, 96, [48, 96], 5120, "bf16", 48, "f32"),      # GDN gates shape, ragged M, gate epilogue
    (13, 17, [17], 256, "f32", 0, "bf16"),             # one chunk, one 32-column tile, fp32 input
    (129, 128, [64, 128], 512, "bf16", 0, "bf16"),     # four column tiles, two segments
    (200, 40, [8, 40], 768, "f32", 0, "f32"),          # three chunks, fp32 in and out
    (9, 96, [48, 96], 1024, "bf16", 48, "f32"),        # just above the decode GEMV's token limit
    (128, 96, [48, 96], 5120, "bf16", 48, "f32"),      # the most tokens one workgroup takes (dynamic: amax in-kernel)
])
@pytest.mark.parametrize("mode", ["static", "dynamic"])
@pytest.mark.parametrize("codes_out", [True, False])
def test_linear_skinny_fused(nv, M, N, seg_end, K, xdt, gate_heads, y_dtype, mode, codes_out):
    """The fused skinny-N linear (x read once, quantized in registers) against the
    oracle: global scale and (when requested) codes bit-exact, outputs within the
    GEMM tolerance."""
    _check_linear(nv, M, N, seg_end, K, xdt, gate_heads, y_dtype, mode, codes_out, "skinny")


@pytest.mark.parametrize("M,N,seg_end,K,xdt,gate_heads,y_dtype", [
    (4, 96, [48, 96], 5120, "bf16", 48, "f32"),        # decode GEMV with the gate epilogue
    (1, 1000, [300, 1000], 2048, "f32", 0, "f32"),     # one token, fp32 in and out, ragged N
    (8, 520, [256, 520], 1024, "bf16", 0, "bf16"),     # eight tokens, ragged last workgroup
    (3, 200, [200], 1536, "bf16", 0, "bf16"),          # three tokens, three 512-element K slices
    (6, 200, [200], 1536, "bf16", 0, "bf16"),          # K % 1024 != 0 with more than four tokens
    (4, 130, [64, 130], 8192, "bf16", 0, "bf16"),      # sixteen K slices (the most), ragged N, two segments
    (2, 64, [64], 1024, "f32", 0, "f32"),              # two K slices (the fewest), fp32 in and out
    (4, 1, [1], 2048, "bf16", 0, "bf16"),              # one output row: every other weight row clamped
    (3, 17, [5, 17], 1536, "bf16", 0, "f32"),          # 17 rows, two segments, a partial row group
])
@pytest.mark.parametrize("mode", ["static", "dynamic"])
@pytest.mark.parametrize("codes_out", [True, False])
def test_linear_decode_fused(nv, M, N, seg_end, K, xdt, gate_heads, y_dtype, mode, codes_out):
    """The fused decode GEMV (M <= 8) through nvfp4_w4a4_linear against the oracle:
    global scale and (when requested) codes bit-exact, outputs within the GEMM
    tolerance."""
    _check_linear(nv, M, N, seg_end, K, xdt, gate_heads, y_dtype, mode, codes_out, "decode")


@pytest.mark.parametrize("M,N,K,xdt", [
    (3, 200, 2048, "bf16"),     # the 4x4x4 decode kernel (four K slices)
    (6, 130, 1024, "bf16"),     # the two-role decode kernel (more than four tokens)
    (2, 64, 1536, "f32"),       # the 4x4x4 decode kernel, fp32 rows
    (40, 96, 512, "bf16"),      # the fused skinny kernel
])
@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_linear_fused_strided_x(nv, M, N, K, xdt, mode):
    """The fused paths of nvfp4_w4a4_linear on x rows longer than their data (a column
    slice of a wider tensor, ldx = K + 64): codes bit-exact, outputs within the GEMM
    tolerance, against the oracle on the slice."""
    rng = np.random.default_rng(M * 131 + K)
    full = rng.standard_normal((M, K + 64)).astype(np.float32)
    full[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40
    bits = W._to_bf16_bits(full) if xdt == "bf16" else None
    xv = W.bf16_bits_to_f32(bits) if xdt == "bf16" else full
    xt = P.dev_x(xv, bits)[:, :K]
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    seg_end = [N // 2, N]
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end, None)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    act = 0.0391 if mode == "static" else None
    gin = None if act is None else torch.tensor([act], dtype=torch.float32, device="cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_w4a4_linear(xt, gin, gout, wc, ws, seg_end, wg, y, a_codes_out=ac, a_scales_out=as_)
    torch.cuda.synchronize()
    oc, os_, og = O.quantize_activation(P.x64_of(xv[:, :K]), None if act is None else np.float32(act))
    owc, ows, owg = O.pack_weight(w.astype(np.float64), seg_end)
    assert np.float32(gout.item()) == og
    P.assert_bytes_equal(ac.cpu().numpy(), oc, "activation codes")
    P.assert_bytes_equal(as_.cpu().numpy(), os_, "activation scales")
    yref, _, bound = P.oracle_reference(oc, os_, og, owc, ows, seg_end, owg, "bf16")
    P.assert_within_tolerance(P.y_to_f64(y), yref, bound, f"strided x M={M} N={N} K={K} {xdt} {mode}")


def _check_linear(nv, M, N, seg_end, K, xdt, gate_heads, y_dtype, mode, codes_out, what):
    wl = _skinny_case(M, N, seg_end, K, xdt, seed=M * 31 + N * 7 + K, gate_heads=gate_heads, y_dtype=y_dtype)
    act = 0.0457 if mode == "static" else None
    xv, xt = _x_inputs(wl)
    wt = P.dev_x(wl.data["w32"])
    wc, ws, wg = P.gpu_pack(nv, wt, wl.seg_end, None)
    y = torch.empty((M, N), dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32, device="cuda")
    gate = None
    if gate_heads:
        gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    gin = None if act is None else torch.tensor([act], dtype=torch.float32, device="cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    ac = as_ = None
    if codes_out:
        ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_w4a4_linear(xt, gin, gout, wc, ws, wl.seg_end, wg, y, gate=gate, a_codes_out=ac, a_scales_out=as_)
    torch.cuda.synchronize()
    oc, os_, og = O.quantize_activation(P.x64_of(xv), None if act is None else np.float32(act))
    owc, ows, owg = O.pack_weight(wl.data["w32"].astype(np.float64), wl.seg_end)
    assert np.float32(gout.item()) == og
    if codes_out:
        P.assert_bytes_equal(ac.cpu().numpy(), oc, "activation codes")
        P.assert_bytes_equal(as_.cpu().numpy(), os_, "activation scales")
    ogate = (wl.data["A_log"], wl.data["dt_bias"]) if gate_heads else None
    yref, _, bound = P.oracle_reference(oc, os_, og, owc, ows, wl.seg_end, owg, y_dtype, gate=ogate)
    P.assert_within_tolerance(P.y_to_f64(y), yref, bound, f"{what} M={M} N={N} K={K} {xdt} {mode}")


def _near_midpoint_rows(rng, M, K, g, xdt):
    """M x K activations whose 16-element blocks sit on E2M1 midpoints under chosen block
    scales.  Element 0 of a block is 6 s g, which fixes the block scale to s; the other
    15 are midpoints m s g (m in 0.25 .. 5) with random signs.  fp32: each moved 0..3 ulps
    either way (the bracket's fix-up decides them).  bf16: g is a power of two, so m s g
    has <= 7 significant bits and is an exact bf16 value: every such element is a tie."""
    x = np.zeros((M, K), dtype=np.float32)
    for r in range(M):
        for b in range(K // 16):
            s = float(O.e4m3_value(int(rng.integers(0x20, 0x7F))))
            blk = np.empty(16, dtype=np.float32)
            blk[0] = np.float32(6 * s * g)
            mids = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], size=15)
            v = (mids * s * g).astype(np.float32)
            if xdt == "f32":
                v = (v.view(np.int32) + rng.integers(-3, 4, size=15).astype(np.int32)).view(np.float32)
            blk[1:] = v * rng.choice([-1, 1], size=15).astype(np.float32)
            x[r, 16 * b:16 * b + 16] = blk
    return x


@pytest.mark.parametrize("M,N,K,xdt", [
    (70, 96, 512, "f32"),       # fused skinny kernel
    (70, 96, 512, "bf16"),
    (4, 64, 1024, "f32"),       # decode GEMV, MFMA 4x4x4
    (4, 64, 1024, "bf16"),
    (7, 64, 1024, "bf16"),      # decode GEMV, 5..8 tokens
])
def test_linear_fused_near_midpoints(nv, M, N, K, xdt):
    """Activations on and around E2M1 midpoints through the fused linear kernels, which
    quantize x in registers: codes and scales bit-exact with the oracle (the near-midpoint
    fix-up decides every flagged element), outputs within the GEMM tolerance."""
    rng = np.random.default_rng(M * 101 + K + (7 if xdt == "bf16" else 0))
    g = 0.0173 if xdt == "f32" else 2.0 ** -6
    x = _near_midpoint_rows(rng, M, K, g, xdt)
    if xdt == "bf16":
        bits = W._to_bf16_bits(x)
        xv = W.bf16_bits_to_f32(bits)
        assert np.array_equal(xv, x)                                # every value exact in bf16
        xt = P.dev_x(xv, bits)
    else:
        xv, xt = x, P.dev_x(x)
    w = rng.standard_normal((N, K)).astype(np.float32)
    seg_end = [N]
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end, None)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gin = torch.tensor([g], dtype=torch.float32, device="cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_w4a4_linear(xt, gin, gout, wc, ws, seg_end, wg, y, a_codes_out=ac, a_scales_out=as_)
    torch.cuda.synchronize()
    oc, os_, og = O.quantize_activation(P.x64_of(xv), np.float32(g))
    owc, ows, owg = O.pack_weight(w.astype(np.float64), seg_end)
    P.assert_bytes_equal(as_.cpu().numpy(), os_, "activation scales")
    P.assert_bytes_equal(ac.cpu().numpy(), oc, "activation codes")
    yref, _, bound = P.oracle_reference(oc, os_, og, owc, ows, seg_end, owg, "bf16")
    P.assert_within_tolerance(P.y_to_f64(y), yref, bound, f"near-midpoint M={M} N={N} K={K} {xdt}")


def test_linear_skinny_equals_two_stage(nv):
    """Fused skinny path and the two-stage path (quantize, then GEMM) agree to the
    GEMM tolerance on the same inputs; their activation codes are identical."""
    wl = _skinny_case(257, 96, [48, 96], 2048, "bf16", seed=11, gate_heads=48, y_dtype="f32")
    xv, xt = _x_inputs(wl)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(wl.data["w32"]), wl.seg_end, None)
    gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    y1 = torch.empty((257, 96), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    g1 = torch.empty(1, dtype=torch.float32, device="cuda")
    g2 = torch.empty_like(g1)
    ac1, as1 = nv.empty_packed(257, 2048, "cuda")
    ac2, as2 = nv.empty_packed(257, 2048, "cuda")
    nv.nvfp4_w4a4_linear(xt, None, g1, wc, ws, wl.seg_end, wg, y1, gate=gate, a_codes_out=ac1, a_scales_out=as1)
    nv.nvfp4_quantize_act(xt, None, ac2, as2, g2)
    nv.nvfp4_w4a4_gemm(ac2, as2, g2, wc, ws, wl.seg_end, wg, y2, gate=gate)
    torch.cuda.synchronize()
    assert g1.item() == g2.item()
    assert torch.equal(ac1, ac2) and torch.equal(as1, as2)
    a, b = y1.double(), y2.double()
    assert float(torch.linalg.norm(a - b) / torch.linalg.norm(b)) < 1e-5


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_full_gdn_gates_fused_linear_sampled(nv, mode):
    """The GDN gate projections at full size (32768 x 96 x 5120) through
    nvfp4_w4a4_linear, i.e. the fused skinny kernel in the launch configuration the
    benchmark times (static: a calibrated scale equal to this tensor's amax-derived
    one, no codes written), and again with the activation codes requested (and in
    dynamic mode).  One sampled token from every 128-token workgroup range plus the
    last token: codes, scale bytes and the global scale bit-exact, outputs within the
    gate bound (Eq. 1 of the review page, mechanism step 2)."""
    name = "gdn_gates_32768x96x5120"
    wl = W.generate(name)
    xv, xt = _x_inputs(wl)
    w = wl.data["w32"]
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), wl.seg_end, None)
    M, N, K = wl.M, wl.N, wl.K
    gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    ag = O.global_scale(O.tensor_amax(P.x64_of(xv)))
    gin = torch.tensor([float(ag)], dtype=torch.float32, device="cuda") if mode == "static" else None
    outs = []
    for with_codes in ((False, True) if mode == "static" else (True,)):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        gout = torch.empty(1, dtype=torch.float32, device="cuda")
        ac = as_ = None
        if with_codes:
            ac, as_ = nv.empty_packed(M, K, "cuda")
        nv.nvfp4_w4a4_linear(xt, gin, gout, wc, ws, wl.seg_end, wg, y, gate=gate, a_codes_out=ac, a_scales_out=as_)
        torch.cuda.synchronize()
        assert np.float32(gout.item()) == ag
        outs.append((y, ac, as_))
    rng = np.random.default_rng(17)
    rows = np.arange(0, M, 128) + rng.integers(0, 128, M // 128)
    rows = np.unique(np.append(rows, M - 1))
    rsel = torch.from_numpy(rows).cuda()
    oac, oas = O.quantize_rows(P.x64_of(xv[rows]), np.full(len(rows), ag, dtype=np.float32))
    owc, ows, owg = O.pack_weight(w.astype(np.float64), wl.seg_end)
    assert np.array_equal(owg, wg.cpu().numpy())
    yref, _, bound = P.oracle_reference(oac, oas, ag, owc, ows, wl.seg_end, owg, "f32",
                                        gate=(wl.data["A_log"], wl.data["dt_bias"]))
    for y, ac, as_ in outs:
        if ac is not None:
            P.assert_bytes_equal(ac[rsel].cpu().numpy(), oac, "activation codes (sampled)")
            P.assert_bytes_equal(as_[rsel].cpu().numpy(), oas, "activation scales (sampled)")
        P.assert_within_tolerance(P.y_to_f64(y[rsel]), yref, bound, f"gates fused {mode}")
    if len(outs) == 2:
        assert torch.equal(outs[0][0], outs[1][0])      # writing the codes does not change y


# ----------------------------------------------------------------------------- degenerate input

@pytest.mark.parametrize("M,N,seg_end,K,gate_heads,route", [
    (4, 640, [320, 640], 1024, 0, "linear"),          # decode GEMV (fused quantize)
    (300, 96, [48, 96], 512, 48, "linear"),           # skinny fused kernel with the gate epilogue
    (600, 640, [256, 640], 512, 0, "two_stage"),      # quantizer + 256 x 256 GEMM
])
def test_all_zero_activation(nv, M, N, seg_end, K, gate_heads, route):
    """An all-zero activation tensor (some entries -0.0) in dynamic mode: amax 0 gives
    g = 0, every block scale byte 0 and codes that keep only the sign of zero; the
    GEMM output is exactly 0 (the gate epilogue then gives its value at 0)."""
    rng = np.random.default_rng(3)
    x = np.zeros((M, K), dtype=np.float32)
    x[rng.random((M, K)) < 0.3] = -0.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end)
    gate = None
    if gate_heads:
        A_log = rng.uniform(-1.0, 2.7, gate_heads).astype(np.float32)
        dt_bias = rng.uniform(-3.0, 3.0, gate_heads).astype(np.float32)
        gate = (torch.from_numpy(A_log).cuda(), torch.from_numpy(dt_bias).cuda())
    y = torch.full((M, N), 7.0, dtype=torch.float32 if gate_heads else torch.bfloat16, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    gout = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    if route == "linear":
        nv.nvfp4_w4a4_linear(xt, None, gout, wc, ws, seg_end, wg, y, gate=gate, a_codes_out=ac, a_scales_out=as_)
    else:
        nv.nvfp4_quantize_act(xt, None, ac, as_, gout)
        nv.nvfp4_w4a4_gemm(ac, as_, gout, wc, ws, seg_end, wg, y, gate=gate)
    torch.cuda.synchronize()
    x64 = xt.float().cpu().numpy().astype(np.float64)
    oac, oas, og = O.quantize_activation(x64)
    assert og == 0.0 and gout.item() == 0.0
    P.assert_bytes_equal(ac.cpu().numpy(), oac, "codes of an all-zero tensor")
    P.assert_bytes_equal(as_.cpu().numpy(), oas, "scales of an all-zero tensor")
    owc, ows, owg = O.pack_weight(w.astype(np.float64), seg_end)
    yref, _, bound = P.oracle_reference(oac, oas, og, owc, ows, seg_end, owg, "f32" if gate_heads else "bf16",
                                        gate=None if gate is None else (A_log, dt_bias))
    got = P.y_to_f64(y)
    if gate_heads:
        P.assert_within_tolerance(got, yref, bound, "gate epilogue at y = 0")
    else:
        assert np.array_equal(got, np.zeros_like(got)), "GEMM of an all-zero activation is not exactly 0"
