"""GPU parity of the GDN gate consumer (alpha = e^g and the gated delta rule, Eq. 2 of
the review page) through the C ABI against the float64 oracle on the same seeded
inputs.  Tolerance: the layer's 1e-3 relative Frobenius error on the outputs and on
the final state, plus a sup-norm check (max |error| <= 1e-4 of the largest
reference magnitude).  The kernel computes in fp32: each token's update rounds
O(d_k) terms, and with unit keys and beta < 1 every step is a contraction, so the
rounding errors do not grow along the token chain; the measured errors are ~1e-6."""

import numpy as np
import pytest
import torch

from oracle import gdn as G
from synth import workloads as W

pytestmark = pytest.mark.gpu

REL_FRO = 1e-3
SUP_REL = 1e-4


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_w4a4_quantized_amd as nvmod
    return nvmod


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _gpu(nv, inp, Hk, Hv, state_in=None, pad=0, in_place=False):
    """Run the recurrence on the device; q/k/v/o/gates as 2-D row-major arrays whose
    rows may be padded by `pad` elements (strides larger than the rows)."""
    T = inp["q"].shape[0]
    dv = inp["v"].shape[2]

    def mat(x, width):
        m = np.zeros((T, width + pad), dtype=np.float32)
        m[:, :width] = x.reshape(T, width)
        return _dev(m)[:, :width]
    q = mat(inp["q"], Hk * 128)
    k = mat(inp["k"], Hk * 128)
    v = mat(inp["v"], Hv * dv)
    gates = mat(inp["gates"], 2 * Hv)
    o = torch.full((T, Hv * dv + pad), float("nan"), dtype=torch.float32, device="cuda")[:, :Hv * dv]
    s_in = None if state_in is None else _dev(state_in)
    s_out = s_in if in_place else torch.empty((Hv, 128, dv), dtype=torch.float32, device="cuda")
    nv.nvfp4_gdn_gated_delta(q, k, v, gates, Hk, Hv, s_in, s_out, o)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64).reshape(T, Hv, dv), s_out.cpu().numpy().astype(np.float64)


def _check(got, want, what):
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    sup = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300)
    assert np.all(np.isfinite(got)), what
    assert err <= REL_FRO, f"{what}: relative Frobenius error {err:.3e}"
    assert sup <= SUP_REL, f"{what}: sup-norm error {sup:.3e} of the largest magnitude"
    return err


@pytest.mark.parametrize("T,Hk,Hv,dv,with_state", [
    (1, 1, 1, 8, False),          # one token, one column group
    (5, 2, 6, 32, True),          # shared key heads, initial state, a tail shorter than a block
    (64, 1, 3, 128, False),       # one whole 64-token block
    (131, 2, 6, 16, True),        # two blocks and an odd tail (a token pair cut by the end)
    (300, 2, 2, 128, True),       # one value head per key head
])
def test_gdn_matches_oracle(nv, T, Hk, Hv, dv, with_state):
    inp = W.gdn_recurrence_inputs(T, Hk, Hv, 128, dv, seed=T * 7 + Hv, with_state=with_state)
    s0 = inp.get("state0")
    o, S = _gpu(nv, inp, Hk, Hv, s0)
    oo, oS = G.gated_delta_from_gates(inp["q"], inp["k"], inp["v"], inp["gates"], s0)
    _check(o, oo, f"o T={T}")
    _check(S, oS, f"state T={T}")


def test_gdn_strided_rows_and_in_place_state(nv):
    # rows longer than their data (like column slices of a wider projection output),
    # and the final state written over the initial one
    inp = W.gdn_recurrence_inputs(97, 2, 6, 128, 24, seed=3, with_state=True)
    o, S = _gpu(nv, inp, 2, 6, inp["state0"], pad=20, in_place=True)
    oo, oS = G.gated_delta_from_gates(inp["q"], inp["k"], inp["v"], inp["gates"], inp["state0"])
    _check(o, oo, "o strided")
    _check(S, oS, "state in place")


def test_gdn_extreme_gates(nv):
    # alpha = 1 exactly (g = 0) with full-strength writes, and alpha ~ e^-60 (state
    # wiped every token): the kernel follows the oracle at both ends
    inp = W.gdn_recurrence_inputs(70, 1, 3, 128, 16, seed=5, with_state=True)
    inp["gates"][:, 0] = 0.0
    inp["gates"][:, 3] = 0.999
    inp["gates"][:, 1] = -60.0
    o, S = _gpu(nv, inp, 1, 3, inp["state0"])
    oo, oS = G.gated_delta_from_gates(inp["q"], inp["k"], inp["v"], inp["gates"], inp["state0"])
    _check(o, oo, "o extreme gates")
    _check(S, oS, "state extreme gates")


def test_gdn_full_size_sampled_heads(nv):
    """The recurrence workload at full size (8192 tokens, 16 key heads, 48 value heads,
    d_k = d_v = 128) in the launch configuration the benchmark times; the oracle
    follows the value heads of two key heads (the first and the last) over all
    tokens, the last 64-token block included."""
    T = 8192
    inp = W.gdn_recurrence_inputs(T, **W.GDN_HEADS, seed=0)
    o, S = _gpu(nv, inp, 16, 48)
    for j in (0, 15):
        hv = slice(3 * j, 3 * j + 3)
        gates = np.concatenate([inp["gates"][:, hv], inp["gates"][:, 48 + 3 * j:48 + 3 * j + 3]], axis=1)
        oo, oS = G.gated_delta_from_gates(inp["q"][:, j:j + 1], inp["k"][:, j:j + 1], inp["v"][:, hv], gates)
        _check(o[:, hv], oo, f"o key head {j}")
        _check(S[hv], oS, f"state key head {j}")
