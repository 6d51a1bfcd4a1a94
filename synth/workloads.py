"""Seeded synthetic inputs for the NVFP4 W4A4 linear layer.

Shared by the tests, the benchmark and the oracle checks.  This module draws
random numbers and nothing else: it holds none of the method's arithmetic (no
scales, no rounding to NVFP4).  The only conversion it performs is the
round-to-nearest-even cast of fp32 draws to bf16 inputs (done by torch).

Recipe (stands in for the residual-stream activations and trained weights the
pages measure on, which are not available):

* numpy PCG64 ``default_rng(seed)``, seed 0 by default; draw order: X base,
  hot-channel indices, hot-channel gains, then W segment by segment, then the
  gate parameters A_log and dt_bias.
* Residual-stream-like X: N(0, 1) base, round(1% of K) hot channels (51 for
  K = 5120) chosen without replacement and fixed across tokens, each scaled by
  a gain drawn from U(30, 100).  The pages report max/RMS 63.5 and heavy
  outlier channels for the mid-layer residual stream ["Why Gated DeltaNet
  Survives 4-Bit Quantization" review page, mechanism step 1, Table 2].
* Weights: N(0, sigma_seg) per fused segment.
* Gate parameters: A_log ~ U(0, 2.7), dt_bias ~ N(0, 0.5), fp32.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HIDDEN = 5120


@dataclass
class Workload:
    name: str
    M: int
    N: int
    K: int
    x_dtype: str                     # "f32" or "bf16"
    y_dtype: str                     # "f32" or "bf16"
    seg_end: list                    # cumulative segment ends over N
    seg_sigma: list                  # weight std per segment
    n_hot: int
    hot_gain: tuple                  # (lo, hi) or (g, g)
    act_mode: str = "static"         # "static" (calibrated g_a) or "dynamic"
    # calibrated weight scales given as ratios to segment 0's amax-derived
    # scale (None = every segment takes its own amax-derived scale)
    seg_scale_ratio: Optional[list] = None
    gate_heads: int = 0
    description: str = ""
    data: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_linear_64x128x256": dict(
        M=64, N=128, K=256, x_dtype="f32", y_dtype="f32", seg_end=[128], seg_sigma=[0.02],
        n_hot=2, hot_gain=(100.0, 100.0), act_mode="dynamic",
        description="tiny NVFP4 W4A4 linear, fp32 in/out, both operands quantized in dynamic mode"),
    "decode_gemv_4x16384x5120": dict(
        M=4, N=16384, K=HIDDEN, x_dtype="bf16", y_dtype="bf16", seg_end=[16384], seg_sigma=[0.02],
        n_hot=51, hot_gain=(30.0, 100.0),
        description="decode-shaped GEMV, one weight segment, bf16 out"),
    "gdn_in_proj_8192x16384x5120": dict(
        M=8192, N=16384, K=HIDDEN, x_dtype="bf16", y_dtype="bf16",
        seg_end=[2048, 4096, 10240, 16384], seg_sigma=[0.02, 0.04, 0.01, 0.08],
        n_hot=51, hot_gain=(30.0, 100.0),
        description="prefill fused GDN input projection q,k,v,z with per-segment global scales"),
    "gdn_gates_32768x96x5120": dict(
        M=32768, N=96, K=HIDDEN, x_dtype="bf16", y_dtype="f32", seg_end=[48, 96], seg_sigma=[0.02, 0.02],
        n_hot=51, hot_gain=(30.0, 100.0), gate_heads=48,
        description="GDN gate projections a,b (skinny N) with the fused gate epilogue, fp32 out"),
    "mlp_gate_up_32768x34816x5120": dict(
        M=32768, N=34816, K=HIDDEN, x_dtype="bf16", y_dtype="bf16", seg_end=[17408, 34816],
        seg_sigma=[0.02, 0.08], n_hot=51, hot_gain=(30.0, 100.0), seg_scale_ratio=[1.0, 4.0],
        description="fused MLP gate/up at long prefill, segment scales 4x apart, bf16 out"),
}


def workload(name: str) -> Workload:
    d = dict(WORKLOADS[name])
    return Workload(name=name, **d)


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 view of bf16 bit patterns (a widening, no rounding)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def generate(name: str, M: Optional[int] = None, seed: int = 0, with_weight: bool = True) -> Workload:
    """Draw the inputs of workload `name`.  M overrides the number of tokens
    (rows of X) for reduced-size tests; everything else keeps its shape.

    Fills wl.data with:
      x32      fp32 [M, K]   (the fp32 draw; for bf16 workloads the value
                              actually used is x_bf16 widened)
      x_bf16   uint16 [M, K] bf16 bit patterns (bf16 workloads only)
      w32      fp32 [N, K]
      A_log, dt_bias  fp32 [H] (gate workload only)
    """
    wl = workload(name)
    if M is not None:
        wl.M = int(M)
    rng = np.random.default_rng(seed)
    K = wl.K
    x = rng.standard_normal((wl.M, K), dtype=np.float32)
    hot = rng.choice(K, size=wl.n_hot, replace=False)
    lo, hi = wl.hot_gain
    gains = (np.full(wl.n_hot, lo) if lo == hi else rng.uniform(lo, hi, wl.n_hot)).astype(np.float32)
    x[:, hot] *= gains[None, :]
    wl.data["hot_channels"] = hot
    wl.data["x32"] = x
    if wl.x_dtype == "bf16":
        wl.data["x_bf16"] = _to_bf16_bits(x)
    if with_weight:
        parts = []
        start = 0
        for end, sigma in zip(wl.seg_end, wl.seg_sigma):
            parts.append(rng.standard_normal((end - start, K), dtype=np.float32) * np.float32(sigma))
            start = end
        wl.data["w32"] = np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]
    if wl.gate_heads:
        H = wl.gate_heads
        wl.data["A_log"] = rng.uniform(0.0, 2.7, H).astype(np.float32)
        wl.data["dt_bias"] = (rng.standard_normal(H) * 0.5).astype(np.float32)
    return wl


def x_values_f32(wl: Workload) -> np.ndarray:
    """The activation values as the layer sees them (bf16 widened, or fp32)."""
    if wl.x_dtype == "bf16":
        return bf16_bits_to_f32(wl.data["x_bf16"])
    return wl.data["x32"]


def random_rows(n_rows: int, k: int, seed: int, dtype: str = "bf16", scale: float = 1.0):
    """Plain N(0, scale) rows for ragged-shape tests; returns (x32, bits or None)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_rows, k), dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        b = _to_bf16_bits(x)
        return bf16_bits_to_f32(b), b
    return x, None


# --------------------------------------------------------------------------- GDN recurrence inputs

GDN_HEADS = dict(n_k_heads=16, n_v_heads=48, d_k=128, d_v=128)


def gdn_recurrence_inputs(T: int, n_k_heads: int = 16, n_v_heads: int = 48, d_k: int = 128, d_v: int = 128,
                          seed: int = 0, with_state: bool = False) -> dict:
    """Seeded inputs of the gated delta-rule recurrence (fp32 arrays).

    Recipe: keys and queries N(0, 1) per head, divided by their L2 norm (unit vectors,
    computed in float64 and stored as fp32); values N(0, 1); the gate output row
    [g | beta] with g = -10^U(-5, 1.3) (decays from alpha ~ 0.99999, the long
    horizons of a trained model, to alpha ~ e^-20) and beta ~ U(0.02, 0.98); an
    initial state N(0, 0.1) when asked.  Draw order: q, k, v, g, beta, state.
    """
    rng = np.random.default_rng(seed)

    def unit(shape):
        a = rng.standard_normal(shape)
        return (a / np.linalg.norm(a, axis=-1, keepdims=True)).astype(np.float32)

    q = unit((T, n_k_heads, d_k))
    k = unit((T, n_k_heads, d_k))
    v = rng.standard_normal((T, n_v_heads, d_v), dtype=np.float32)
    g = (-(10.0 ** rng.uniform(-5.0, 1.3, (T, n_v_heads)))).astype(np.float32)
    beta = rng.uniform(0.02, 0.98, (T, n_v_heads)).astype(np.float32)
    out = dict(q=q, k=k, v=v, gates=np.concatenate([g, beta], axis=1))
    if with_state:
        out["state0"] = (rng.standard_normal((n_v_heads, d_k, d_v)) * 0.1).astype(np.float32)
    return out


# --------------------------------------------------------------------------- rotation parameters

def krpbh_params(d: int, h: int = 512, seed: int = 0) -> dict:
    """Random draws of a K-RPBH rotation of dimension d = k h: a uniform random
    permutation perm (int32 [d]), Rademacher signs (int8 [d], +-1) and a Haar-random
    orthogonal k x k matrix Q (fp32), drawn as the Q factor of a QR decomposition of
    an N(0, 1) matrix with the signs of R's diagonal moved into Q (the standard way
    to sample the Haar measure).  Draw order: perm, signs, the Gaussian matrix."""
    if d % h:
        raise ValueError("d must be a multiple of h")
    rng = np.random.default_rng(seed)
    perm = rng.permutation(d).astype(np.int32)
    signs = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    k = d // h
    A = rng.standard_normal((k, k))
    q, r = np.linalg.qr(A)
    q = q * np.sign(np.diag(r))[None, :]
    return dict(perm=perm, signs=signs, Q=q.astype(np.float32), h=h)
