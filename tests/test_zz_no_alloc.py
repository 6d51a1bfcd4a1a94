"""nvfp4_w4a4_linear_noalloc (the entry point for callers that cannot allocate)
against nvfp4_w4a4_linear with caller buffers: identical outputs and global
scales on two calls in a row, the second smaller, on the two-stage path (which
uses the fixed workspace) and on the fused paths, in both activation-scale modes;
and against the oracle within the layer's tolerance."""

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


def _case(M, N, K, seed, seg_end, gate_heads=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 60
    bits = W._to_bf16_bits(x)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    gate = None
    if gate_heads:
        gate = (rng.uniform(0.0, 2.7, gate_heads).astype(np.float32),
                (rng.standard_normal(gate_heads) * 0.5).astype(np.float32))
    return W.bf16_bits_to_f32(bits), bits, w, gate


def _run_both(nv, M, N, K, seed, seg_end, mode, gate_heads=0):
    xv, bits, w, gate = _case(M, N, K, seed, seg_end, gate_heads)
    xt = P.dev_x(xv, bits)
    wc, ws, wg = P.gpu_pack(nv, P.dev_x(w), seg_end, None)
    ydt = torch.float32 if gate_heads else torch.bfloat16
    gin = torch.tensor([0.043], dtype=torch.float32, device="cuda") if mode == "static" else None
    gdev = None if gate is None else tuple(torch.from_numpy(a).cuda() for a in gate)
    y_ref = torch.full((M, N), float("nan"), dtype=ydt, device="cuda")
    y_na = torch.full((M, N), float("nan"), dtype=ydt, device="cuda")
    g_ref = torch.empty(1, dtype=torch.float32, device="cuda")
    g_na = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_w4a4_linear(xt, gin, g_ref, wc, ws, seg_end, wg, y_ref, gate=gdev, a_codes_out=ac, a_scales_out=as_)
    nv.nvfp4_w4a4_linear_noalloc(xt, gin, g_na, wc, ws, seg_end, wg, y_na, gate=gdev)
    torch.cuda.synchronize()
    assert g_na.item() == g_ref.item()
    assert torch.equal(y_na.view(torch.int16) if ydt == torch.bfloat16 else y_na.view(torch.int32),
                       y_ref.view(torch.int16) if ydt == torch.bfloat16 else y_ref.view(torch.int32))
    # and the layer's tolerance against the oracle
    x64 = xv.astype(np.float64)
    oc, os_, og = O.quantize_activation(x64, None if gin is None else np.float32(0.043))
    owc, ows, owg = O.pack_weight(w.astype(np.float64), seg_end)
    assert np.float32(g_na.item()) == og
    yref, _, bound = P.oracle_reference(oc, os_, og, owc, ows, seg_end, owg, "f32" if gate_heads else "bf16",
                                        gate=gate)
    P.assert_within_tolerance(P.y_to_f64(y_na), yref, bound, f"noalloc M={M} N={N} K={K}")


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_noalloc_two_stage_twice_second_smaller(nv, mode):
    # the two-stage path keeps its activations in the fixed workspace: a large call
    # (scales at a high offset in it) and then a smaller one over the same memory
    _run_both(nv, 1024, 640, 5120, 1, [256, 640], mode)
    _run_both(nv, 203, 300, 1024, 2, [300], mode)


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_noalloc_fused_paths_twice_second_smaller(nv, mode):
    _run_both(nv, 600, 96, 5120, 3, [48, 96], mode, gate_heads=48)      # skinny, gate epilogue
    _run_both(nv, 130, 96, 1024, 4, [48, 96], mode, gate_heads=48)
    _run_both(nv, 8, 1000, 2048, 5, [300, 1000], mode)                  # decode
    _run_both(nv, 3, 520, 1024, 6, [520], mode)


def test_noalloc_rejects_oversize_two_stage_shape(nv):
    M, N, K = 16384, 256, 4096            # 37.7 MB of activation workspace > 32 MiB
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wc, ws = nv.empty_packed(N, K, "cuda")
    wg = torch.ones(1, dtype=torch.float32, device="cuda")
    y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_w4a4_linear_noalloc(x, None, g, wc, ws, [N], wg, y)
    assert e.value.status == nv.NVFP4_ERR_INVALID_ARG and "workspace" in str(e.value)
    # the largest two-stage shape that fits still runs
    M2 = (32 << 20) // (K // 2 + K // 16) - 16
    nv.nvfp4_w4a4_linear_noalloc(x[:M2], None, g, wc, ws, [N], wg, y[:M2])
    torch.cuda.synchronize()
