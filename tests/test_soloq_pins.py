"""Pins of the rotated NVFP4 front end's oracle (SoloQ page: the K-RPBH rotation,
Proposition 1, the scale-only bias correction) against the printed matrix form
built from library primitives, exact enumeration, closed forms and statistics.
CPU only."""

import itertools
import math

import numpy as np
import pytest
from scipy.linalg import block_diag, hadamard

from oracle import nvfp4 as O
from oracle import soloq as S
from synth import workloads as W


def _dense_pi(p):
    """Pi as the printed product (Q_k (x) I_h) blkdiag(H_h D_1 .. H_h D_k) P, from
    numpy/scipy primitives: np.kron, scipy's block_diag and hadamard."""
    h, Q, perm, signs = p["h"], p["Q"].astype(np.float64), p["perm"], p["signs"].astype(np.float64)
    d = len(perm)
    k = d // h
    H = hadamard(h) / math.sqrt(h)
    P = np.zeros((d, d))
    P[np.arange(d), perm] = 1.0                     # (P x)_i = x[perm[i]]
    blocks = [H @ np.diag(signs[i * h:(i + 1) * h]) for i in range(k)]
    return np.kron(Q, np.eye(h)) @ block_diag(*blocks) @ P


@pytest.mark.parametrize("d,h", [(12, 4), (64, 16), (96, 32), (16, 16)])
def test_rotation_equals_the_printed_matrix_product(d, h):
    p = W.krpbh_params(d, h, seed=d + h)
    x = np.random.default_rng(1).standard_normal((5, d))
    want = x @ _dense_pi(p).T
    got = S.rotate_f64(x, p["perm"], p["signs"], p["Q"], h)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_rotation_is_orthogonal_and_preserves_linear_layers():
    p = W.krpbh_params(5120, 512, seed=3)
    I = np.eye(5120)[:640]
    rows = S.rotate_f64(I, p["perm"], p["signs"], p["Q"], 512)      # rows of Pi^T
    # Q_k is stored in fp32, so Pi is orthogonal to fp32 precision (k terms of ~2^-24)
    assert np.allclose(rows @ rows.T, np.eye(640), atol=1e-6)
    Q = p["Q"].astype(np.float64)
    assert np.allclose(Q @ Q.T, np.eye(10), atol=1e-6)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5120))
    w = rng.standard_normal((7, 5120))
    xr = S.rotate_f64(x, p["perm"], p["signs"], p["Q"], 512)
    wr = S.rotate_f64(w, p["perm"], p["signs"], p["Q"], 512)      # rows of W' = W Pi^T
    assert np.allclose(xr @ wr.T, x @ w.T, rtol=1e-5, atol=1e-4)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)


def test_one_block_is_rpbh():
    # k = 1: Q_1 = [+-1], so Pi = +-H D P (the permuted block-Hadamard rotation)
    p = W.krpbh_params(64, 64, seed=5)
    x = np.random.default_rng(6).standard_normal((4, 64))
    H = hadamard(64) / 8.0
    want = float(p["Q"][0, 0]) * (x[:, p["perm"]] * p["signs"]) @ H.T
    assert abs(abs(float(p["Q"][0, 0])) - 1) < 1e-6
    assert np.allclose(S.rotate_f64(x, p["perm"], p["signs"], p["Q"], 64), want, atol=1e-12)


def test_proposition_1_conditional_variance_by_enumerating_the_signs():
    # the variance over all Rademacher sign patterns of every rotated coordinate equals
    # (1/h) sum_j Q_rj^2 M_j, M_j the energy of block j of P x (exact enumeration, d = 8)
    h, k = 4, 2
    p = W.krpbh_params(h * k, h, seed=7)
    x = np.random.default_rng(8).standard_normal(h * k)
    x /= np.linalg.norm(x)
    px = x[p["perm"]]
    M = np.array([np.sum(px[j * h:(j + 1) * h] ** 2) for j in range(k)])
    second = np.zeros(h * k)
    for bits in itertools.product([-1.0, 1.0], repeat=h * k):
        z = S.rotate_f64(x[None, :], p["perm"], np.array(bits), p["Q"], h)[0]
        second += z ** 2
    second /= 2 ** (h * k)
    Q = p["Q"].astype(np.float64)
    for r in range(k):
        want = np.sum(Q[r] ** 2 * M) / h
        assert np.allclose(second[r * h:(r + 1) * h], want, rtol=1e-12)


def test_proposition_1_expectation_over_haar_mixers_is_one_over_d():
    # a unit vector with one dominant coordinate: averaged over independent draws of
    # Q_k, D and P the rotated coordinates have second moment 1/d
    d, h = 64, 8
    x = np.full(d, 0.05)
    x[3] = 1.0
    x /= np.linalg.norm(x)
    acc = np.zeros(d)
    n = 3000
    for s in range(n):
        p = W.krpbh_params(d, h, seed=1000 + s)
        acc += S.rotate_f64(x[None, :], p["perm"], p["signs"], p["Q"], h)[0] ** 2
    m = acc / n
    assert abs(np.mean(m) * d - 1) < 1e-6                           # the norm is preserved
    assert np.max(np.abs(m * d - 1)) < 0.15                         # every coordinate ~ 1/d


def test_fp32_evaluation_is_within_its_rounding_bound():
    # reading S3's fp32 order against the float64 rotation: per row,
    # ||z32 - z64||_2 <= (log2 h + 2 + 2k) u ||x||_2 (each butterfly stage adds at most
    # u of the running norm, the scaling one more, the mix 2k roundings of Q-weighted
    # terms of norm ||x||).  The bound is not vacuous (the observed error is a few
    # percent of it) and plausible mistakes in the fp32 order break it: a missing
    # butterfly stage, the scaling applied twice, the mixer transposed.
    p = W.krpbh_params(5120, 512, seed=9)
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=24, with_weight=False)
    x = W.x_values_f32(wl)
    z32 = S.rotate_f32(x, p["perm"], p["signs"], p["Q"], 512).astype(np.float64)
    z64 = S.rotate_f64(x, p["perm"], p["signs"], p["Q"], 512)
    u = 2.0 ** -24
    bound = (9 + 2 + 2 * 10) * u * np.linalg.norm(x.astype(np.float64), axis=1)
    err = np.linalg.norm(z32 - z64, axis=1)
    assert np.all(err <= bound), (err / bound).max()
    assert np.median(err / bound) > 0.01
    wrong = [
        S.rotate_f32(x, p["perm"], p["signs"], p["Q"].T.copy(), 512),           # mixer transposed
        S.rotate_f32(x, p["perm"], p["signs"], p["Q"], 512) / np.float32(np.sqrt(512)),   # scaled twice
        S.rotate_f32(x, np.argsort(p["perm"]).astype(np.int32), p["signs"], p["Q"], 512),   # P^T for P
    ]
    for bad in wrong:
        assert np.any(np.linalg.norm(bad.astype(np.float64) - z64, axis=1) > bound)


def test_fp32_butterflies_match_the_transform_matrix_on_exact_inputs():
    # small integers: every butterfly sum is exact in fp32, so the fp32 evaluation
    # equals the float64 product with scipy's Hadamard matrix up to the final scaling
    p = W.krpbh_params(64, 64, seed=10)
    p["Q"][:] = 1.0
    p["signs"][:] = 1
    x = np.random.default_rng(11).integers(-8, 9, (3, 64)).astype(np.float32)
    got = S.rotate_f32(x, np.arange(64), p["signs"], p["Q"], 64).astype(np.float64)
    want = (x.astype(np.float64) @ hadamard(64).T) * float(np.float32(1 / 8.0))
    assert np.array_equal(got, want)


def test_bias_correction_closed_forms():
    # on-grid z: q(z) = z and c = 1; c q(z) restores the component along z exactly;
    # a power-of-two rescaling of z leaves c unchanged; z = 0 gives 1
    g = np.float32(2.0 ** -3)
    vals = np.array([0.5, 1, 1.5, 2, 3, 4, 6, -6] * 4, dtype=np.float64) * float(g)
    codes, scales = O.quantize_rows(vals[None, :], np.array([g], dtype=np.float32))
    assert S.bias_correction(vals[None, :], codes, scales, [g])[0] == 1.0
    rng = np.random.default_rng(12)
    z = rng.standard_normal((6, 256)) * rng.uniform(0.1, 10, (6, 1))
    z[:, 5] *= 40
    cz, sz, gz = O.quantize_activation(z)
    c = S.bias_correction(z, cz, sz, np.full(6, gz))
    q = O.dequantize_rows(cz, sz, np.full(6, gz, dtype=np.float32))
    assert np.allclose(np.einsum("ij,ij->i", c[:, None] * q, z), np.einsum("ij,ij->i", z, z), rtol=1e-13)
    assert np.all(np.abs(c - 1) < 0.05) and np.all(c != 1)
    cz2, sz2, gz2 = O.quantize_activation(z * 8.0)
    assert np.array_equal(S.bias_correction(z * 8.0, cz2, sz2, np.full(6, gz2)), c)
    zero = np.zeros((1, 32))
    c0, s0 = O.quantize_rows(zero, np.array([0.0], dtype=np.float32))
    assert S.bias_correction(zero, c0, s0, [0.0])[0] == 1.0


def test_rotate_quantize_segments_and_gemm_reference():
    p = W.krpbh_params(1024, 512, seed=13)
    rng = np.random.default_rng(14)
    w = np.concatenate([rng.standard_normal((40, 1024)) * 0.02, rng.standard_normal((24, 1024)) * 0.08]).astype(np.float32)
    wc, ws, gw, cw, zw = S.rotate_quantize(w, p["perm"], p["signs"], p["Q"], 512, seg_end=[40, 64])
    z64 = zw.astype(np.float64)
    assert gw[0] == O.global_scale(np.max(np.abs(z64[:40]))) and gw[1] == O.global_scale(np.max(np.abs(z64[40:])))
    x = rng.standard_normal((9, 1024)).astype(np.float32)
    xc, xs, gx, cx, zx = S.rotate_quantize(x, p["perm"], p["signs"], p["Q"], 512)
    y = S.gemm_rowcol_f64(xc, xs, gx[0], cx, wc, ws, [40, 64], gw, cw)
    # the rotated, quantized, bias-corrected layer approximates x w^T
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.2
    # without the correction factors it is the plain NVFP4 GEMM of the rotated operands
    y0 = O.gemm_f64(xc, xs, gx[0], wc, ws, [40, 64], gw)
    assert np.allclose(y, y0 * cx[:, None] * cw[None, :], rtol=1e-15)
