"""Plain CPU oracle of the rotated NVFP4 front end (SoloQ-N): the K-RPBH rotation
of activations (online) and weights (offline), NVFP4 with scales computed from the
rotated tensor itself, and the scale-only bias correction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The HIP library never uses it; the two share no code.

Source: "SoloQ: Calibration-Free Quantization for Diffusion Language Models" page
(the SoloQ page):
* "how it is used" section: the rotation Pi = (Q_k (x) I_h) blkdiag(H_h D_1, ...,
  H_h D_k) P, with H_h the normalized Walsh-Hadamard matrix, D_i Rademacher sign
  diagonals, P a uniform random permutation and Q_k a Haar-random orthogonal
  cross-block mixer; Proposition 1: the conditional variance over the signs of a
  rotated coordinate is (1/h) sum_j Q_rj^2 M_j (M_j the block energies), whose
  expectation over a Haar Q_k is exactly 1/d for a unit vector; k = 1 gives RPBH.
* "assumptions and limits" section: for y = W x the weight is rotated offline,
  W' = W Pi^T, the activation online, x' = Pi x, then both are quantized; SoloQ-N
  puts native NVFP4 (E2M1, a per-tensor global scale and 16-coordinate block
  scales, computed from the tensor itself) on the rotated representation and adds
  the scale-only bias correction c_bc(z) = ||z||^2 / <q(z), z>, which restores the
  component along z exactly and folds into the per-token / per-row scales.

Readings (each also listed in the design doc):
S1  P as a gather: (P x)_i = x[perm[i]]; D_i acts on block i of the permuted vector;
    block i = coordinates i*h .. i*h + h - 1; (Q_k (x) I_h) z has block r equal to
    sum_s Q[r, s] z_block_s (the Kronecker product with the block index outer).
S2  H_h is the Sylvester-ordered Hadamard matrix divided by sqrt(h).
S3  Where the rotated value decides a code, both sides use it as computed in fp32
    in this order (the kernel's precision): gather, sign, the butterflies of the
    fast Walsh-Hadamard transform stage by stage (pair distance 1, 2, 4, ..., h/2;
    lower <- a + b, upper <- a - b), one multiply by fp32(1/sqrt(h)), then the
    cross-block mix as a left-to-right fp32 sum of fp32 products
    Q[r, 0] y_0 + Q[r, 1] y_1 + ...  The float64 rotation is the exact reference
    that this fp32 evaluation is pinned against.
S4  NVFP4 on the rotated rows follows the NVFP4 oracle (dynamic global scale
    fp32(amax / 2688) over the rotated tensor, or over each weight segment).
S5  c_bc uses q(z) = the dequantized NVFP4 value e2m1 * s * g; it is 1 when
    <q(z), z> = 0 (all of z quantizes to zero).  It is applied in the GEMM
    epilogue as one fp32 factor per activation row and one per weight row:
    y[m, n] = c_x[m] * c_w[n] * g_a * g_w * sum_k deq(a) deq(w).
S6  Block size h = 512 for K = 5120 (k = 10 blocks), the block size the page uses as
    its example (18944 = 512 x 37).
"""

from __future__ import annotations

import numpy as np

from oracle import nvfp4 as O


def _blocks(y, h):
    R, d = y.shape
    if d % h:
        raise ValueError("d must be a multiple of h")
    return y.reshape(R, d // h, h)


def hadamard_normalized(h):
    """Sylvester Hadamard matrix H_h / sqrt(h) (S2), built by doubling."""
    H = np.ones((1, 1))
    while H.shape[0] < h:
        H = np.block([[H, H], [H, -H]])
    if H.shape[0] != h:
        raise ValueError("h must be a power of two")
    return H / np.sqrt(h)


def rotate_f64(x, perm, signs, Q, h):
    """Pi x for every row of x [R, d], in float64 (the exact reference):
    gather by perm, Rademacher signs, H_h on every block, then mix block r as
    sum_s Q[r, s] block_s."""
    x = np.asarray(x, dtype=np.float64)
    y = x[:, np.asarray(perm)] * np.asarray(signs, dtype=np.float64)[None, :]
    yb = _blocks(y, h) @ hadamard_normalized(h).T            # H_h D_s x_s per block
    z = np.einsum("rs,nsj->nrj", np.asarray(Q, dtype=np.float64), yb)
    return z.reshape(x.shape[0], -1)


def rotate_f32(x, perm, signs, Q, h):
    """Pi x evaluated in fp32 in the order of reading S3 (numpy float32 arithmetic:
    every operation rounds once, to nearest even)."""
    f = np.float32
    x = np.asarray(x, dtype=f)
    y = (x[:, np.asarray(perm)] * np.asarray(signs, dtype=f)[None, :]).astype(f)
    R, d = y.shape
    yb = _blocks(y, h).copy()
    length = 1
    while length < h:
        v = yb.reshape(R, d // h, h // (2 * length), 2, length)
        a = v[:, :, :, 0, :].copy()
        b = v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = a + b
        v[:, :, :, 1, :] = a - b
        length *= 2
    yb = (yb * f(1.0 / np.sqrt(h))).astype(f)
    Qf = np.asarray(Q, dtype=f)
    k = d // h
    z = np.empty_like(yb)
    for r in range(k):
        acc = Qf[r, 0] * yb[:, 0, :]
        for s in range(1, k):
            acc = (acc + Qf[r, s] * yb[:, s, :]).astype(f)
        z[:, r, :] = acc
    return z.reshape(R, d)


def bias_correction(z, codes, scales, g_rows):
    """c_bc(z) = ||z||^2 / <q(z), z> per row (S5), float64; 1 where <q(z), z> = 0."""
    z = np.asarray(z, dtype=np.float64)
    q = O.dequantize_rows(codes, scales, g_rows)
    num = np.einsum("ij,ij->i", z, z)
    den = np.einsum("ij,ij->i", q, z)
    out = np.ones_like(num)
    nz = den != 0
    out[nz] = num[nz] / den[nz]
    return out


def rotate_quantize(x, perm, signs, Q, h, seg_end=None, seg_gscale=None):
    """The SoloQ-N front end for the rows of x (activations: one segment; a fused
    weight: its segments): rotate in fp32 (S3), NVFP4-quantize with global scales
    from the rotated rows themselves (or the given ones), bias-correction factors.
    Returns (codes, scales, g_seg float32[S], c_bc float64[R], z float32[R, d])."""
    z = rotate_f32(x, perm, signs, Q, h)
    R = z.shape[0]
    seg_end = [R] if seg_end is None else list(seg_end)
    seg = O.segment_rows(seg_end, R)
    z64 = z.astype(np.float64)
    if seg_gscale is None:
        g = np.array([O.global_scale(O.tensor_amax(z64[seg == i])) for i in range(len(seg_end))], dtype=np.float32)
    else:
        g = np.asarray(seg_gscale, dtype=np.float32)
    codes, scales = O.quantize_rows(z64, g[seg])
    c = bias_correction(z64, codes, scales, g[seg])
    return codes, scales, g, c, z


def gemm_rowcol_f64(a_codes, a_scales, a_g, c_x, w_codes, w_scales, seg_end, w_g_seg, c_w):
    """y = c_x[m] c_w[n] (deq(A) deq(W)^T) in float64 (S5)."""
    y = O.gemm_f64(a_codes, a_scales, a_g, w_codes, w_scales, seg_end, w_g_seg)
    return y * np.asarray(c_x, dtype=np.float64)[:, None] * np.asarray(c_w, dtype=np.float64)[None, :]


def rowcol_elem_bound(y64, abs_prod, alpha_cols, c_x, c_w, K, out_dtype):
    """Per-element bound for the epilogue fp32((acc * fp32(alpha_n * c_w[n])) * c_x[m])
    rounded to the output: the plain GEMM bound with alpha replaced by
    alpha c_w c_x, plus 2u|Y64| for the two further fp32 roundings."""
    a = np.abs(np.asarray(alpha_cols, dtype=np.float64) * np.asarray(c_w, dtype=np.float64))
    b = O.gemm_elem_bound(y64, abs_prod * np.abs(np.asarray(c_x, dtype=np.float64))[:, None], a, K, out_dtype)
    return b + 2 * O.U32 * np.abs(y64)
