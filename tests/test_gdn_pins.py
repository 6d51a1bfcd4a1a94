"""Pins of the GDN gate-consumer oracle (alpha = e^g and the delta-rule recurrence,
Eq. 2 of the review page) against closed forms, exact rational arithmetic in a
different formulation (transition matrices), and the overwrite/erasure properties
the page describes.  CPU only."""

import math
from fractions import Fraction

import numpy as np

from oracle import gdn as G
from synth import workloads as W


def test_alpha_closed_forms_and_gate_split():
    assert G.gate_alpha(0.0) == 1.0
    assert G.gate_alpha(math.log(0.5)) == 0.5
    a = G.gate_alpha(np.array([-1e-5, -20.0]))
    assert 0 < a[1] < a[0] < 1
    gates = np.arange(12, dtype=np.float32).reshape(2, 6)
    g, b = G.split_gates(gates, 3)
    assert np.array_equal(g, gates[:, :3]) and np.array_equal(b, gates[:, 3:])


def test_identity_when_nothing_is_written_or_forgotten():
    inp = W.gdn_recurrence_inputs(9, 2, 6, 8, 5, seed=1, with_state=True)
    T = 9
    ones, zeros = np.ones((T, 6)), np.zeros((T, 6))
    o, S = G.delta_rule(inp["q"], inp["k"], inp["v"], ones, zeros, inp["state0"])
    S0 = inp["state0"].astype(np.float64)
    assert np.array_equal(S, S0)
    kh = np.arange(6) // 3
    want = np.einsum("hkv,thk->thv", S0, inp["q"].astype(np.float64)[:, kh]) / math.sqrt(8)
    assert np.allclose(o, want, rtol=1e-14, atol=0)


def test_pure_decay_closed_form():
    inp = W.gdn_recurrence_inputs(7, 1, 2, 4, 3, seed=2, with_state=True)
    alpha = np.array([[0.5, 0.25], [0.75, 1.0], [0.5, 0.5], [1.0, 0.125],
                      [0.25, 0.5], [0.5, 1.0], [0.75, 0.75]])
    _, S = G.delta_rule(inp["q"], inp["k"], inp["v"], alpha, np.zeros((7, 2)), inp["state0"])
    want = np.prod(alpha, axis=0)[:, None, None] * inp["state0"].astype(np.float64)
    assert np.array_equal(S, want)                      # powers of two: exact


def _rational_transition_form(k, v, alpha, beta, S0):
    """S_T by transition matrices in exact rationals: S_t = A_t S_{t-1} + B_t with
    A_t = alpha_t I - beta_t k_t k_t^T and B_t = beta_t k_t v_t^T (one key head)."""
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    S = [[Fraction(x) for x in row] for row in S0]
    for t in range(T):
        A = [[(alpha[t] if i == j else 0) - beta[t] * k[t][i] * k[t][j] for j in range(dk)] for i in range(dk)]
        S = [[sum(A[i][m] * S[m][c] for m in range(dk)) + beta[t] * k[t][i] * v[t][c] for c in range(dv)]
             for i in range(dk)]
    return S


def test_exact_against_rational_transition_matrices():
    rng = np.random.default_rng(3)
    T, dk, dv = 5, 4, 3
    half = [Fraction(-1, 2), Fraction(0), Fraction(1, 2)]
    k = [[half[i] for i in rng.integers(0, 3, dk)] for _ in range(T)]
    v = [[Fraction(int(i)) for i in rng.integers(-3, 4, dv)] for _ in range(T)]
    alpha = [Fraction(int(n), 4) for n in rng.integers(1, 5, T)]
    beta = [Fraction(int(n), 4) for n in rng.integers(0, 5, T)]
    S0 = [[Fraction(int(i), 2) for i in rng.integers(-4, 5, dv)] for _ in range(dk)]
    want = _rational_transition_form(k, v, alpha, beta, S0)
    f = lambda a: np.array(a, dtype=np.float64)
    q = np.zeros((T, 1, dk))
    _, S = G.delta_rule(q, f(k)[:, None, :], f(v)[:, None, :], f(alpha)[:, None], f(beta)[:, None],
                        f(S0)[None])
    assert np.array_equal(S[0], f(want))                # dyadic inputs: float64 is exact here


def test_write_overwrites_along_the_key():
    # alpha = beta = 1 and a unit key: after the write the state answers v_t for k_t,
    # and every direction orthogonal to k_t is left as it was
    inp = W.gdn_recurrence_inputs(1, 1, 1, 16, 6, seed=4, with_state=True)
    k = inp["k"].astype(np.float64)
    _, S = G.delta_rule(inp["q"], k, inp["v"], np.ones((1, 1)), np.ones((1, 1)), inp["state0"])
    assert np.allclose(S[0].T @ k[0, 0], inp["v"][0, 0], atol=1e-12)
    u = np.random.default_rng(5).standard_normal(16)
    u -= (u @ k[0, 0]) * k[0, 0]
    assert np.allclose(u @ S[0], u @ inp["state0"][0].astype(np.float64), atol=1e-12)


def test_orthonormal_keys_erase_the_initial_state():
    # the active erasure of the review page's mechanism step 3: keys that sweep an
    # orthonormal basis with full write strength leave no trace of the old state,
    # S_T = sum_t k_t v_t^T whatever S_0 was
    dk, dv = 8, 5
    basis, _ = np.linalg.qr(np.random.default_rng(6).standard_normal((dk, dk)))
    k = basis.T[:, None, :]
    v = np.random.default_rng(7).standard_normal((dk, 1, dv))
    one = np.ones((dk, 1))
    for s0 in (np.zeros((1, dk, dv)), np.random.default_rng(8).standard_normal((1, dk, dv)) * 10):
        _, S = G.delta_rule(np.zeros((dk, 1, dk)), k, v, one, one, s0)
        assert np.allclose(S[0], np.einsum("tk,tv->kv", k[:, 0], v[:, 0]), atol=1e-12)


def test_linear_in_state_and_values():
    inp = W.gdn_recurrence_inputs(12, 2, 4, 8, 6, seed=9, with_state=True)
    g, b = G.split_gates(inp["gates"], 4)
    a = G.gate_alpha(g)
    v2 = np.random.default_rng(10).standard_normal(inp["v"].shape)
    o1, S1 = G.delta_rule(inp["q"], inp["k"], inp["v"], a, b, inp["state0"])
    o2, S2 = G.delta_rule(inp["q"], inp["k"], v2, a, b, None)
    o3, S3 = G.delta_rule(inp["q"], inp["k"], inp["v"].astype(np.float64) + v2, a, b, inp["state0"])
    assert np.allclose(o3, o1 + o2, rtol=1e-12, atol=1e-12) and np.allclose(S3, S1 + S2, rtol=1e-12, atol=1e-12)


def test_value_heads_share_consecutive_key_heads():
    # reading G2: value head h reads key/query head h // (Hv / Hk), i.e. the key heads
    # repeated (not tiled) across the value heads
    inp = W.gdn_recurrence_inputs(6, 2, 6, 8, 4, seed=11)
    g, b = G.split_gates(inp["gates"], 6)
    a = G.gate_alpha(g)
    o, S = G.delta_rule(inp["q"], inp["k"], inp["v"], a, b)
    rep = lambda x: np.repeat(x, 3, axis=1)
    o_r, S_r = G.delta_rule(rep(inp["q"]), rep(inp["k"]), inp["v"], a, b)
    assert np.array_equal(o, o_r) and np.array_equal(S, S_r)
    tile = lambda x: np.tile(x, (1, 3, 1))
    o_t, _ = G.delta_rule(tile(inp["q"]), tile(inp["k"]), inp["v"], a, b)
    assert not np.allclose(o, o_t)


def test_contraction_keeps_the_state_bounded():
    # unit keys and beta <= 1: every step is a contraction plus a bounded write, so
    # ||S_t|| stays within ||S_0|| + sum of the writes (no growth from the recurrence)
    inp = W.gdn_recurrence_inputs(300, 1, 3, 16, 8, seed=12, with_state=True)
    g, b = G.split_gates(inp["gates"], 3)
    _, S = G.delta_rule(inp["q"], inp["k"], inp["v"], G.gate_alpha(g), b, inp["state0"])
    bound = np.linalg.norm(inp["state0"], axis=(1, 2)) + np.sum(
        b * np.linalg.norm(inp["v"], axis=2), axis=0) * 2
    assert np.all(np.linalg.norm(S, axis=(1, 2)) <= bound)


def test_read_out_sees_the_tokens_own_write():
    # o_t reads S_t (after token t's write): from a zero state with alpha = beta = 1 and
    # q_t = k_t, the first output is v_1 / sqrt(dk)
    inp = W.gdn_recurrence_inputs(1, 1, 1, 16, 6, seed=13)
    k = inp["k"].astype(np.float64)
    o, _ = G.delta_rule(k, k, inp["v"], np.ones((1, 1)), np.ones((1, 1)))
    assert np.allclose(o[0, 0], inp["v"][0, 0] / 4.0, atol=1e-12)
