"""GPU parity of the MXFP4 variant (quantizer and GEMM on the native block-scaled
FP4 MFMA) against the oracle on the same seeded inputs: codes and E8M0 scale bytes
bit-exact; GEMM outputs within 1e-3 relative Frobenius error and within the
per-element bound of fp32 accumulation of exact products."""

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


def _gpu_mx_quant(nv, xt):
    M, K = xt.shape
    c, s = nv.empty_mx_packed(M, K, xt.device)
    nv.nvfp4_mxfp4_quantize(xt, c, s)
    torch.cuda.synchronize()
    return c, s


def _adversarial():
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    x[1, 32:64] *= np.float32(1e-38)                       # subnormal block maximum
    x[2, :32] = np.float32(2.0 ** 120)                     # clamped exponent region
    x[3, 64:96] = np.float32(6.0 * 2.0 ** -3)              # quotients exactly 6 / ties below
    x[3, 70] = np.float32(0.25 * 2.0 ** -3)                # tie 0.25 -> 0
    x[3, 71] = np.float32(2.5 * 2.0 ** -3)                 # tie 2.5 -> 2
    x[4, :32] = np.float32(7.99)                           # saturation at 6
    x[5, :] = np.ldexp(1.0, rng.integers(-60, 60, 256)).astype(np.float32)
    return x


@pytest.mark.parametrize("kind", ["residual_bf16", "tiny_f32", "adversarial_f32"])
def test_mx_quantize_matches_oracle(nv, kind):
    if kind == "residual_bf16":
        wl = W.generate("gdn_in_proj_8192x16384x5120", M=300, with_weight=False)
        xv = W.x_values_f32(wl)
        xt = P.dev_x(xv, wl.data["x_bf16"])
    elif kind == "tiny_f32":
        xv = W.generate("tiny_linear_64x128x256").data["x32"]
        xt = P.dev_x(xv)
    else:
        xv = _adversarial()
        xt = P.dev_x(xv)
    oc, os_ = O.mx_quantize_rows(xv.astype(np.float64))
    gc, gs = _gpu_mx_quant(nv, xt)
    P.assert_bytes_equal(gs.cpu().numpy(), os_, "E8M0 scales")
    P.assert_bytes_equal(gc.cpu().numpy(), oc, "codes")


def _mx_reference(ac, as_, wc, ws, out_dtype):
    y64 = O.mx_gemm_f64(ac, as_, wc, ws)
    absprod = np.abs(O.mx_dequantize_rows(ac, as_)) @ np.abs(O.mx_dequantize_rows(wc, ws)).T
    K = ac.shape[1] * 2
    bound = O.gemm_elem_bound(y64, absprod, np.ones(wc.shape[0]), K, out_dtype)
    return O.round_output(y64, out_dtype), bound


@pytest.mark.parametrize("M,N,K", [(300, 520, 256), (64, 128, 128), (512, 512, 5120), (257, 1000, 1024)])
@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
def test_mx_gemm_matches_oracle(nv, M, N, K, y_dtype):
    rng = np.random.default_rng(62)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(40.0)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ac, as_ = _gpu_mx_quant(nv, P.dev_x(x))
    wc, ws = _gpu_mx_quant(nv, P.dev_x(w))
    y = torch.empty((M, N), dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32, device="cuda")
    nv.nvfp4_mxfp4_gemm(ac, as_, wc, ws, y)
    torch.cuda.synchronize()
    yref, bound = _mx_reference(ac.cpu().numpy(), as_.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), y_dtype)
    P.assert_within_tolerance(P.y_to_f64(y), yref, bound, f"mxfp4 {M}x{N}x{K}")


def test_mx_gemm_full_gdn_in_proj_sampled(nv):
    """The GDN in_proj shape (8192 x 16384 x 5120, bf16 out) in MXFP4: sampled rows
    and columns against the oracle on the same bytes."""
    wl = W.generate("gdn_in_proj_8192x16384x5120")
    xt = P.dev_x(None, wl.data["x_bf16"])
    wt = P.dev_x(wl.data["w32"])
    ac, as_ = _gpu_mx_quant(nv, xt)
    wc, ws = _gpu_mx_quant(nv, wt)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    nv.nvfp4_mxfp4_gemm(ac, as_, wc, ws, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(63)
    rows = np.sort(rng.choice(wl.M, 24, replace=False))
    cols = np.sort(rng.choice(wl.N, 512, replace=False))
    yref, bound = _mx_reference(ac[rows].cpu().numpy(), as_[rows].cpu().numpy(), wc[cols].cpu().numpy(),
                                ws[cols].cpu().numpy(), "bf16")
    P.assert_within_tolerance(P.y_to_f64(y)[rows][:, cols], yref, bound, "mxfp4 in_proj sampled")
