"""GPU parity of the shared-scale re-encoding of a fused weight
(nvfp4_requantize_weight) against the oracle on the same seeded inputs: codes,
scale bytes and the shared scale bit-exact; a GEMM over the re-encoded weight
(one segment) within the usual tolerance of the oracle on the same bytes."""

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


def _weight(seg_end, sigma, K, seed):
    rng = np.random.default_rng(seed)
    parts, start = [], 0
    for e, sg in zip(seg_end, sigma):
        parts.append(rng.standard_normal((e - start, K)).astype(np.float32) * np.float32(sg))
        start = e
    return np.concatenate(parts)


def _gpu_requant(nv, wc, ws, seg_end, wg, shared=None, in_place=False):
    N, half_k = wc.shape
    if in_place:
        co, so = wc, ws
    else:
        co, so = nv.empty_packed(N, 2 * half_k, wc.device)
    gout = torch.empty(1, dtype=torch.float32, device=wc.device)
    gin = None if shared is None else torch.tensor([shared], dtype=torch.float32, device=wc.device)
    nv.nvfp4_requantize_weight(wc, ws, seg_end, wg, gin, co, so, gout)
    torch.cuda.synchronize()
    return co, so, gout


CASES = {
    # GDN in_proj structure (q, k, v, z), distinct per-segment amax scales
    "gdn_in_proj_like": ([128, 256, 640, 1024], [0.02, 0.04, 0.01, 0.08], 5120),
    # MLP gate/up with calibrated scales 4x apart (set below)
    "mlp_scales_4x": ([256, 512], [0.02, 0.08], 5120),
    # GDN gates a, b
    "gates_a_b": ([48, 96], [0.02, 0.03], 5120),
    # ragged: 3 segments, 3 blocks per row, subnormal-scale and zero blocks
    "ragged_tiny": ([3, 5, 9], [0.02, 0.3, 0.005], 48),
}


@pytest.mark.parametrize("shared", [None, 1.37])
@pytest.mark.parametrize("case", sorted(CASES))
def test_requantize_matches_oracle(nv, case, shared):
    seg_end, sigma, K = CASES[case]
    w = _weight(seg_end, sigma, K, seed=41)
    if case == "ragged_tiny":
        w[1, 16:32] *= 1e-3
        w[6, :16] = 0.0
    w64 = w.astype(np.float64)
    gin = None
    if case == "mlp_scales_4x":
        g0 = O.global_scale(O.tensor_amax(w64[:256]))
        gin = [float(g0), float(np.float32(4) * g0)]
    oc, os_, og = O.pack_weight(w64, seg_end, gin)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end, gin)
    P.assert_bytes_equal(wc.cpu().numpy(), oc, "packed codes")
    P.assert_bytes_equal(ws.cpu().numpy(), os_, "packed scales")
    g_shared = None if shared is None else np.float32(shared * float(og.max()))
    rc, rs, rg = O.requantize_shared_scale(oc, os_, seg_end, og, g_shared)
    co, so, gout = _gpu_requant(nv, wc, ws, seg_end, wg, None if g_shared is None else float(g_shared))
    assert np.float32(gout.item()) == rg
    P.assert_bytes_equal(so.cpu().numpy(), rs, "re-encoded scales")
    P.assert_bytes_equal(co.cpu().numpy(), rc, "re-encoded codes")
    if case == "mlp_scales_4x" and shared is None:
        # scales a power of two apart: the re-encoding is lossless (codes kept)
        P.assert_bytes_equal(co.cpu().numpy(), oc, "codes kept")


def test_requantize_in_place_equals_out_of_place(nv):
    seg_end, sigma, K = CASES["gdn_in_proj_like"]
    w = _weight(seg_end, sigma, K, seed=42)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end)
    co, so, g1 = _gpu_requant(nv, wc, ws, seg_end, wg)
    ic, is_, g2 = _gpu_requant(nv, wc.clone(), ws.clone(), seg_end, wg, in_place=True)
    assert torch.equal(co, ic) and torch.equal(so, is_) and g1.item() == g2.item()


@pytest.mark.parametrize("name", ["gdn_in_proj_8192x16384x5120", "mlp_gate_up_32768x34816x5120"])
def test_requantize_full_size_sampled(nv, name):
    """Full-size fused weights, re-encoded on the GPU; sampled rows of every segment
    re-encoded by the oracle from the same packed bytes."""
    wl = W.generate(name, M=1)
    w = wl.data["w32"]
    gin = None
    if wl.seg_scale_ratio is not None:
        g0 = O.global_scale(O.tensor_amax(w[:wl.seg_end[0]].astype(np.float64)))
        gin = [float(np.float32(r) * g0) for r in wl.seg_scale_ratio]
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), wl.seg_end, gin)
    co, so, gout = _gpu_requant(nv, wc, ws, wl.seg_end, wg)
    og = wg.cpu().numpy()
    assert np.float32(gout.item()) == og.max()
    rng = np.random.default_rng(7)
    starts = [0] + list(wl.seg_end[:-1])
    rows = np.concatenate([np.sort(rng.choice(np.arange(s, e), 16, replace=False))
                           for s, e in zip(starts, wl.seg_end)])
    sub_end = list(np.cumsum([16] * len(wl.seg_end)))
    rc, rs, rg = O.requantize_shared_scale(wc[rows].cpu().numpy(), ws[rows].cpu().numpy(), sub_end, og)
    P.assert_bytes_equal(so[rows].cpu().numpy(), rs, "re-encoded scales (sampled rows)")
    P.assert_bytes_equal(co[rows].cpu().numpy(), rc, "re-encoded codes (sampled rows)")
    if gin is not None:
        assert torch.equal(co, wc)          # scales 4x apart: every code kept


def test_gemm_over_requantized_weight(nv):
    """The re-encoded weight is one NVFP4 tensor: a single-segment GEMM over it
    matches the oracle on the same bytes, and stays within 1/16 (the largest
    re-rounding of a block scale) of the per-segment epilogue's result."""
    seg_end, sigma, K = CASES["gdn_in_proj_like"]
    w = _weight(seg_end, sigma, K, seed=43)
    x, _ = W.random_rows(300, K, seed=44, dtype="f32")
    xt = P.dev_x(x)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end)
    co, so, gsh = _gpu_requant(nv, wc, ws, seg_end, wg)
    ac, as_, ag = P.gpu_quantize(nv, xt)
    act, ast, agt = (torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(),
                     torch.tensor([ag], dtype=torch.float32, device="cuda"))
    N = seg_end[-1]
    y1 = torch.empty((300, N), dtype=torch.float32, device="cuda")
    nv.nvfp4_w4a4_gemm(act, ast, agt, co, so, [N], gsh, y1)
    y4 = torch.empty((300, N), dtype=torch.float32, device="cuda")
    nv.nvfp4_w4a4_gemm(act, ast, agt, wc, ws, seg_end, wg, y4)
    torch.cuda.synchronize()
    yref, _, bound = P.oracle_reference(ac, as_, ag, co.cpu().numpy(), so.cpu().numpy(), [N],
                                        gsh.cpu().numpy(), "f32")
    P.assert_within_tolerance(P.y_to_f64(y1), yref, bound, "single-segment GEMM over the re-encoded weight")
    d = np.linalg.norm(P.y_to_f64(y1) - P.y_to_f64(y4)) / np.linalg.norm(P.y_to_f64(y4))
    print(f"re-encoded vs per-segment epilogue: relative Frobenius difference {d:.3e}")
    assert 0 < d < 1 / 16
