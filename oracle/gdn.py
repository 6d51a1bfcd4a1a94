"""Plain CPU oracle of the Gated DeltaNet gate consumer: alpha = e^g and the
delta-rule recurrence fed by the NVFP4 layer's gate outputs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The HIP library never uses it; the two share no code.  numpy, float64.

Source: "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
Recurrent Half of a Hybrid 27B LLM" (review page):
* background section, the recurrence (Eq. 2): per head the state S (d_k x d_v)
  decays by alpha_t and is then written along the key k_t with strength beta_t,
  replacing what the state predicted for k_t (S_{t-1}^T k_t) by v_t; the read-out
  is o_t = S_t^T q_t / sqrt(d_k);
* mechanism step 2, Eq. 1: alpha_t = e^{g_t} with g_t the decay gate
  -exp(A_log) softplus(a_t + dt_bias), beta_t = sigmoid(b_t), i.e. the [g | beta]
  outputs of the fused gate epilogue;
* mechanism step 3 (the paper's section 5.3): the write overwrites the state
  along the current key direction, which is why errors are forgotten;
* the spec list: GDN state K = V = 128.

Readings (each also listed in the design doc):
G1  The recurrence is taken exactly as printed: the prediction that the write
    replaces is S_{t-1}^T k_t, the state before the decay, so that
    S_t = (alpha_t I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.
G2  Head layout of the hybrid model's GDN (from the fused in_proj segments q, k
    2048 and v 6144 wide and the 48 gate heads, with K = V = 128): 16 key/query
    heads and 48 value heads; value head h reads key/query head h // 3
    (consecutive value heads share a key head).
G3  Keys and queries reach the recurrence already normalized (unit L2 norm per
    head); the pages do not say how, and with beta <= 1 a unit key keeps every
    eigenvalue of alpha I - beta k k^T inside [-1, 1].  The synthetic inputs draw
    them that way; the recurrence itself does not normalize.
G4  The initial state is zero unless one is given.
"""

from __future__ import annotations

import numpy as np


def gate_alpha(g):
    """alpha = e^g (Eq. 1): the per-token, per-head decay from the gate output g."""
    return np.exp(np.asarray(g, dtype=np.float64))


def split_gates(gates, n_v_heads):
    """The fused gate epilogue's output row [g_0..g_{H-1} | beta_0..beta_{H-1}] ->
    (g [T, H], beta [T, H]) in float64."""
    gt = np.asarray(gates, dtype=np.float64)
    return gt[:, :n_v_heads], gt[:, n_v_heads:2 * n_v_heads]


def delta_rule(q, k, v, alpha, beta, state0=None):
    """Eq. 2, token by token, in float64.

    q, k   [T, Hk, dk]     queries and keys per key head
    v      [T, Hv, dv]     values per value head (Hv a multiple of Hk)
    alpha, beta [T, Hv]    decay and write strength per token and value head
    state0 [Hv, dk, dv] or None (zeros)
    Returns (o [T, Hv, dv], S_T [Hv, dk, dv]) with o_t = S_t^T q_t / sqrt(dk).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    if Hv % Hk:
        raise ValueError("value heads must be a multiple of key heads")
    kh = np.arange(Hv) // (Hv // Hk)                 # G2: key head of each value head
    S = np.zeros((Hv, dk, dv)) if state0 is None else np.array(state0, dtype=np.float64)
    o = np.empty((T, Hv, dv))
    scale = 1.0 / np.sqrt(dk)
    for t in range(T):
        kt = k[t, kh]                                # [Hv, dk]
        qt = q[t, kh]
        pred = np.einsum("hkv,hk->hv", S, kt)        # S_{t-1}^T k_t
        write = beta[t][:, None] * (v[t] - pred)     # beta_t (v_t - S_{t-1}^T k_t)
        S = alpha[t][:, None, None] * S + kt[:, :, None] * write[:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, qt) * scale
    return o, S


def gated_delta_from_gates(q, k, v, gates, state0=None):
    """The consumer as a whole: [g | beta] from the gate epilogue -> alpha = e^g ->
    the recurrence."""
    Hv = v.shape[1]
    g, beta = split_gates(gates, Hv)
    return delta_rule(q, k, v, gate_alpha(g), beta, state0)


def recurrence_flops(T, Hv, dk, dv):
    """Arithmetic of the recurrence per call: per token and value head the
    prediction S^T k (2 dk dv), the decayed rank-one write (3 dk dv: the decay
    multiply, the product and the add) and the read-out S^T q (2 dk dv)."""
    return 7.0 * T * Hv * dk * dv
