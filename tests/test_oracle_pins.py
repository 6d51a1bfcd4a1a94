"""Pins of the CPU oracle against things other than itself: golden tables,
torch's own float8 (E4M3FN) implementation, exact rational brute force,
closed forms and invariants.  CPU only."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4 as O
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


E2M1_GOLDEN = {int(c): float(v) for c, v in _read_table("e2m1_values.txt")}
CONST = {k: float(v) for k, v in _read_table("nvfp4_constants.txt")}
# E4M3 values from torch's float8_e4m3fn (an implementation independent of the oracle)
E4M3_TORCH = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# --------------------------------------------------------------------------- formats

def test_e2m1_table_matches_golden():
    for c, v in E2M1_GOLDEN.items():
        got = float(O.e2m1_value(c))
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)
    assert float(O.e2m1_value(7)) == CONST["e2m1_max"]


def test_e4m3_table_matches_torch_float8():
    mine = O.e4m3_value(np.arange(256))
    both_nan = np.isnan(mine) & np.isnan(E4M3_TORCH)
    assert np.all(both_nan | (mine == E4M3_TORCH))
    assert mine[int(CONST["e4m3_max_byte"])] == CONST["e4m3_max"]
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[1] == 2.0 ** -9
    assert np.all(np.diff(mine[:0x7F]) > 0)           # monotone in the byte


def test_e4m3_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(5)
    t = np.concatenate([
        rng.uniform(0, 448, 20000), np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 20000)),
        # exact midpoints between neighbouring E4M3 values, and their fp32 neighbours
        (E4M3_TORCH[0:0x7E] + E4M3_TORCH[1:0x7F]) / 2,
    ]).astype(np.float32)
    t = np.concatenate([t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1000))])
    t = t[(t >= 0) & (t <= 448)]
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = O.e4m3_rne_sat(t.astype(np.float64))
    assert np.array_equal(mine, ref)


def test_e4m3_saturates():
    assert O.e4m3_rne_sat(449.0) == 0x7E
    assert O.e4m3_rne_sat(1e9) == 0x7E
    assert O.e4m3_rne_sat(2.0 ** -10) == 0x00        # tie between 0 and 2^-9 -> even byte 0
    assert O.e4m3_rne_sat(np.nextafter(2.0 ** -10, 1)) == 0x01


def test_e2m1_tie_table():
    for mid, code, val in _read_table("e2m1_rne_ties.txt"):
        mid, code, val = float(mid), int(code), float(val)
        assert O.e2m1_rne_sat(mid) == code
        assert E2M1_GOLDEN[code] == val
        assert O.e2m1_rne_sat(np.nextafter(mid, 0)) <= code
        assert O.e2m1_rne_sat(np.nextafter(mid, 10)) >= code
        # just off the midpoint, the nearest grid value wins
        below = E2M1_GOLDEN[int(O.e2m1_rne_sat(np.nextafter(mid, 0)))]
        above = E2M1_GOLDEN[int(O.e2m1_rne_sat(np.nextafter(mid, 10)))]
        assert below < mid < above
    assert O.e2m1_rne_sat(7.3) == 7


# --------------------------------------------------------------------------- brute force

_E2M1_MAGS_F = [Fraction(E2M1_GOLDEN[c]) for c in range(8)]
_E4M3_F = [Fraction(float(E4M3_TORCH[b])) for b in range(0x7F)]


def _nearest_even(candidates, v):
    best = None
    for i, c in enumerate(candidates):
        d = abs(v - c)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0 and best[1] % 2 == 1):
            best = (d, i)
    return best[1]


def brute_quantize(rows, g):
    """Exact rational quantization by exhaustive search, independent of the oracle."""
    g = Fraction(float(np.float32(g)))
    codes_all, scales_all = [], []
    for row in rows:
        codes, scales = [], []
        for b0 in range(0, len(row), 16):
            blk = [Fraction(float(v)) for v in row[b0:b0 + 16]]
            a = max(abs(v) for v in blk)
            if g == 0 or a == 0:
                sb = 0
            else:
                t = min(a / (6 * g), Fraction(448))
                sb = _nearest_even(_E4M3_F, t)
            s = _E4M3_F[sb]
            scales.append(sb)
            for v, vf in zip(blk, row[b0:b0 + 16]):
                sign = 8 if math.copysign(1.0, float(vf)) < 0 else 0
                if s == 0:
                    mag = 0
                else:
                    r = min(abs(v) / (s * g), Fraction(6))
                    mag = _nearest_even(_E2M1_MAGS_F, r)
                codes.append(sign | mag)
        packed = [codes[i] | (codes[i + 1] << 4) for i in range(0, len(codes), 2)]
        codes_all.append(packed)
        scales_all.append(scales)
    return np.array(codes_all, dtype=np.uint8), np.array(scales_all, dtype=np.uint8)


def brute_global_scale(amax):
    """Nearest fp32 to amax/2688 (ties to even), by exact comparison of candidates."""
    q = Fraction(float(np.float32(amax))) / 2688
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-1)), f, np.nextafter(f, np.float32(1e30))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - q)
        even = (int(np.array(c, dtype=np.float32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return np.float32(best[1])


def _adversarial_rows():
    g = 1.0
    rows = []
    # E2M1 midpoints exactly, with a 6*s element so that s = 1 exactly
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows.append([6.0] + mids + [-m for m in mids] + [0.0])
    # E4M3 tie: a_b = 6 * 1.0625 (midpoint between 1.0 and 1.125) -> even byte 0x38
    rows.append([6.375, 1.0, -0.0, 0.1] + [0.0] * 12)
    # zero block, negative zeros, tiny values that round to zero
    rows.append([0.0] * 8 + [-0.0] * 8)
    rows.append([1e-3, -1e-3, 6.0] + [0.0] * 13)
    return np.array(rows, dtype=np.float64), g


def test_brute_force_tiny_random_and_adversarial():
    rng = np.random.default_rng(11)
    for trial in range(6):
        x = (rng.standard_normal((3, 64)) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
        x[0, rng.integers(0, 64)] *= 100
        x64 = x.astype(np.float64)
        g = O.global_scale(O.tensor_amax(x64))
        assert g == brute_global_scale(O.tensor_amax(x64))
        c, s = O.quantize_rows(x64, np.full(3, g, dtype=np.float32))
        bc, bs = brute_quantize(x, g)
        assert np.array_equal(c, bc) and np.array_equal(s, bs), trial
    x64, g = _adversarial_rows()
    c, s = O.quantize_rows(x64, np.full(len(x64), g, dtype=np.float32))
    bc, bs = brute_quantize(x64, g)
    assert np.array_equal(c, bc) and np.array_equal(s, bs)
    # spot values of the adversarial rows, worked by hand
    assert s[0, 0] == 0x38                             # scale 1.0
    assert c[0, 0] == (0x7 | (0 << 4))                 # 6.0 -> 7, 0.25 -> 0 (tie to even)
    assert c[0, 1] == (2 | (2 << 4))                   # 0.75 -> 1.0 (2), 1.25 -> 1.0 (2)
    assert s[1, 0] == 0x38                             # E4M3 tie 1.0625 -> 1.0
    assert s[2, 0] == 0 and np.all(c[2, :4] == 0) and np.all(c[2, 4:] == 0x88)
    assert c[3, 0] == (0x0 | (0x8 << 4))               # +1e-3 -> 0x0, -1e-3 -> 0x8


def test_brute_force_subnormal_scales_and_static_overflow():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((2, 32))).astype(np.float32)
    # large calibrated g: block scales land in the E4M3 subnormal range
    for g in [np.float32(0.05), np.float32(0.3), np.float32(2.0)]:
        c, s = O.quantize_rows(x.astype(np.float64), np.full(2, g, dtype=np.float32))
        bc, bs = brute_quantize(x, g)
        assert np.array_equal(c, bc) and np.array_equal(s, bs)
    # tiny calibrated g: t > 448 saturates the scale and then the elements at 6
    g = np.float32(1e-5)
    c, s = O.quantize_rows(x.astype(np.float64), np.full(2, g, dtype=np.float32))
    bc, bs = brute_quantize(x, g)
    assert np.array_equal(c, bc) and np.array_equal(s, bs)
    assert np.all(s == 0x7E)


# --------------------------------------------------------------------------- invariants

def test_round_trip_on_grid_values():
    rng = np.random.default_rng(3)
    R, K = 5, 64
    g = np.float32(0.0371)
    sbytes = rng.integers(0x08, 0x7F, size=(R, K // 16))          # normal E4M3 scales
    mags = rng.integers(0, 8, size=(R, K))
    signs = rng.integers(0, 2, size=(R, K))
    mags.reshape(R, K // 16, 16)[:, :, 3] = 7                      # a +-6 element in every block
    codes = (signs << 3) | mags
    s = E4M3_TORCH[sbytes]
    vals = np.array([[E2M1_GOLDEN[int(cc)] for cc in row] for row in codes]).reshape(R, K // 16, 16)
    x = (vals * s[:, :, None] * float(g)).reshape(R, K)            # exact in float64
    c, sc = O.quantize_rows(x, np.full(R, g, dtype=np.float32))
    assert np.array_equal(sc, sbytes)
    expect_packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    # +0.0 magnitudes keep their sign bit from the input
    assert np.array_equal(c, expect_packed)
    back = O.dequantize_rows(c, sc, np.full(R, g, dtype=np.float32))
    assert np.array_equal(back, x)


def test_block_structure_max_over_rms_and_one_hot():
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=16, with_weight=False)
    x = W.x_values_f32(wl).astype(np.float64)
    blocks = x.reshape(16, -1, int(CONST["block_size"]))
    rms = np.sqrt(np.mean(blocks ** 2, axis=2))
    ratio = np.max(np.abs(blocks), axis=2) / rms
    assert np.all(ratio <= CONST["block_max_over_rms"] + 1e-12)
    # a one-hot block reaches the bound exactly, and quantizes to a single +-6 code
    one = np.zeros((1, 16))
    one[0, 5] = -3.7
    c, s = O.quantize_rows(one, np.array([O.global_scale(3.7)], dtype=np.float32))
    codes = O.unpack_codes(c)[0]
    assert codes[5] == 0xF and np.all(np.delete(codes, 5) == 0)
    deq = O.dequantize_rows(c, s)[0]
    assert np.max(np.abs(deq)) / np.sqrt(np.mean(deq ** 2)) == 4.0


def test_block_max_gets_code_six_and_amax_block_gets_448():
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=32, with_weight=False)
    x = W.x_values_f32(wl).astype(np.float64)
    c, s, g = O.quantize_activation(x)
    codes = O.unpack_codes(c).reshape(32, -1, 16)
    blocks = x.reshape(32, -1, 16)
    arg = np.argmax(np.abs(blocks), axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0] & 7
    normal = s >= 0x08
    assert np.all(top[normal] == 7)
    amax_row, amax_col = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s[amax_row, amax_col // 16] == 0x7E
    assert g == brute_global_scale(O.tensor_amax(x))


def test_locality_static_mode():
    wl = W.generate("decode_gemv_4x16384x5120", with_weight=False)
    x = W.x_values_f32(wl).astype(np.float64)
    g = np.float32(0.05)
    c0, s0 = O.quantize_rows(x, np.full(4, g, dtype=np.float32))
    x2 = x.copy()
    x2[2, 1000] = 90.0                                  # an outlier in block 62 of row 2
    c1, s1 = O.quantize_rows(x2, np.full(4, g, dtype=np.float32))
    dc = np.argwhere(c0 != c1)
    ds = np.argwhere(s0 != s1)
    assert len(ds) == 1 and tuple(ds[0]) == (2, 1000 // 16)
    assert np.all(dc[:, 0] == 2) and np.all(dc[:, 1] // 8 == 1000 // 16)


def test_global_scale_brute_force_and_zero():
    rng = np.random.default_rng(4)
    for a in list(rng.uniform(1e-6, 1e4, 200).astype(np.float32)) + [np.float32(2688.0), np.float32(21.0)]:
        assert O.global_scale(a) == brute_global_scale(a)
    assert O.global_scale(0.0) == 0
    c, s, g = O.quantize_activation(np.zeros((2, 32)))
    assert g == 0 and np.all(s == 0) and np.all(c == 0)


# --------------------------------------------------------------------------- GEMM + epilogues

def _ongrid_operand(rng, R, K):
    """Rows of E2M1 values with a +-6 in every block, so that with g = 1 every
    block scale is exactly 1.0 and quantization is the identity."""
    vals = np.array([E2M1_GOLDEN[c] for c in range(16)])
    idx = rng.integers(0, 16, size=(R, K))
    idx.reshape(R, K // 16, 16)[:, :, 0] = rng.choice([7, 15], size=(R, K // 16))
    return vals[idx]


def test_gemm_equals_integer_matmul_when_scales_are_one():
    rng = np.random.default_rng(7)
    M, N, K = 5, 7, 48                                   # non-square: a transposed operand fails
    A = _ongrid_operand(rng, M, K)
    Wt = _ongrid_operand(rng, N, K)
    ac, as_ = O.quantize_rows(A, np.ones(M, dtype=np.float32))
    wc, ws = O.quantize_rows(Wt, np.ones(N, dtype=np.float32))
    assert np.all(as_ == 0x38) and np.all(ws == 0x38)
    y64 = O.gemm_f64(ac, as_, np.float32(1), wc, ws, [N], np.ones(1, dtype=np.float32))
    Ai = (A * 2).astype(np.int64)                        # E2M1 values are multiples of 1/2
    Wi = (Wt * 2).astype(np.int64)
    exact = [[sum(int(Ai[m, k]) * int(Wi[n, k]) for k in range(K)) for n in range(N)] for m in range(M)]
    assert np.array_equal(y64 * 4, np.array(exact, dtype=np.float64))


def test_segment_linearity_and_single_scale_mismatch():
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=8, with_weight=False)
    x = W.x_values_f32(wl)[:, :256].astype(np.float64)
    rng = np.random.default_rng(8)
    seg_end = [16, 32, 80, 128]
    sig = np.repeat([0.02, 0.04, 0.01, 0.08], np.diff([0] + seg_end))
    w = rng.standard_normal((128, 256)) * sig[:, None]
    w = w.astype(np.float32).astype(np.float64)
    ac, as_, ag = O.quantize_activation(x)
    wc, ws, gseg = O.pack_weight(w, seg_end)
    assert len(set(gseg.tolist())) == 4
    y = O.gemm_f64(ac, as_, ag, wc, ws, seg_end, gseg)
    # multiplying one segment's global scale by 2^3 multiplies exactly its columns by 8
    g2 = gseg.copy()
    g2[2] = g2[2] * np.float32(8)
    y2 = O.gemm_f64(ac, as_, ag, wc, ws, seg_end, g2)
    cols = np.arange(128)
    in2 = (cols >= 32) & (cols < 80)
    assert np.array_equal(y2[:, in2], 8 * y[:, in2]) and np.array_equal(y2[:, ~in2], y[:, ~in2])
    # applying segment 0's scale to every segment (a single-scale fused GEMM)
    # scales segment s's outputs by g[0]/g[s]: the mismatch the per-segment epilogue removes
    y1 = O.gemm_f64(ac, as_, ag, wc, ws, seg_end, np.full(4, gseg[0], dtype=np.float32))
    seg = O.segment_rows(seg_end, 128)
    ratio = gseg[0].astype(np.float64) / gseg.astype(np.float64)
    assert np.allclose(y1, y * ratio[seg][None, :], rtol=1e-12, atol=0)
    assert not np.allclose(y1, y, rtol=1e-2)


def test_pack_weight_dynamic_segment_scales():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((96, 64)) * 0.02).astype(np.float32).astype(np.float64)
    w[60] *= 5
    wc, ws, g = O.pack_weight(w, [48, 96])
    assert g[0] == brute_global_scale(np.max(np.abs(w[:48])))
    assert g[1] == brute_global_scale(np.max(np.abs(w[48:])))
    with pytest.raises(ValueError):
        O.segment_rows([48, 48, 96], 96)
    with pytest.raises(ValueError):
        O.segment_rows([50], 96)


def test_gate_epilogue_closed_forms():
    from scipy.special import expit
    H = 4
    A_log = np.array([0.0, 1.0, 2.7, 0.3], dtype=np.float32)
    dt = np.zeros(H, dtype=np.float32)
    y = np.zeros((1, 2 * H))
    out = O.gate_epilogue_f64(y, A_log, dt)
    assert np.allclose(out[0, :H], -np.exp(A_log.astype(np.float64)) * math.log(2), rtol=1e-15)
    assert np.all(out[0, H:] == 0.5)
    rng = np.random.default_rng(10)
    y = rng.standard_normal((50, 2 * H)) * 20
    dt = rng.standard_normal(H).astype(np.float32)
    out = O.gate_epilogue_f64(y, A_log, dt)
    z = y[:, :H] + dt.astype(np.float64)
    ref_g = -np.exp(A_log.astype(np.float64)) * np.logaddexp(0.0, z)
    assert np.allclose(out[:, :H], ref_g, rtol=1e-13)
    assert np.allclose(out[:, H:], expit(y[:, H:]), rtol=1e-13)
    # alpha = e^g in (0, 1) <=> g < 0; beta in (0, 1) (checked where float64 can resolve it)
    assert np.all(out[:, :H] < 0)
    mod = O.gate_epilogue_f64(y / 10, A_log, dt)
    alpha = np.exp(mod[:, :H])
    assert np.all((alpha > 0) & (alpha < 1)) and np.all((mod[:, H:] > 0) & (mod[:, H:] < 1))
    with pytest.raises(ValueError):
        O.gate_epilogue_f64(np.zeros((1, 7)), A_log, dt)


def test_bf16_rounding_matches_torch_and_ties():
    rng = np.random.default_rng(13)
    v = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-30, 30, 20000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(v.astype(np.float64)), ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert O.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    # a float64 value just above a bf16 tie that an fp32 intermediate would turn into a tie
    y = 1 + 2 ** -8 + 2 ** -40
    assert O.round_to_bf16(np.array([y]))[0] == 1 + 2 ** -7


def test_error_bound_admits_fp32_gemm_and_rejects_planted_error():
    wl = W.generate("tiny_linear_64x128x256")
    x = W.x_values_f32(wl).astype(np.float64)
    w = wl.data["w32"].astype(np.float64)
    ac, as_, ag = O.quantize_activation(x)
    wc, ws, gw = O.pack_weight(w, wl.seg_end)
    yref, y64 = O.linear_reference(ac, as_, ag, wc, ws, wl.seg_end, gw, "f32")
    # an fp32 GEMM the way a GPU does it: exact scale-decoded operands, fp32 sums, fp32 alpha
    a_s = O.dequantize_rows(ac, as_).astype(np.float32)
    w_s = O.dequantize_rows(wc, ws).astype(np.float32)
    acc = a_s @ w_s.T
    alpha = np.float32(ag) * gw[0]
    ygpu = (acc * alpha).astype(np.float64)
    bound = O.gemm_elem_bound(y64, O.gemm_abs_product(ac, as_, wc, ws), np.full(128, alpha), wl.K, "f32")
    assert np.all(np.abs(ygpu - yref) <= bound)
    rel = np.linalg.norm(ygpu - yref) / np.linalg.norm(yref)
    assert rel < 1e-5
    planted = ygpu.copy()
    planted[3, 7] *= 1.01
    assert np.any(np.abs(planted - yref) > bound)


def _seq_fp32_acc(a_s, w_s):
    """fp32 accumulation in plain k order (one rounding per partial sum)."""
    acc = np.zeros((a_s.shape[0], w_s.shape[0]), np.float32)
    for k in range(a_s.shape[1]):
        acc = acc + np.outer(a_s[:, k], w_s[:, k]).astype(np.float32)
    return acc


def _to_bf16_f64(y32):
    """fp32 -> bf16 by torch's own RNE cast (independent of the oracle), as float64."""
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_error_bound_bf16_output_admits_fp32_gemm_and_is_tight():
    # bf16-output branch of the per-element bound: an fp32 GEMM (exact scale-decoded
    # operands, fp32 sums in BLAS order and in plain k order, fp32 alpha and multiply)
    # rounded to bf16 by torch lies within it; a planted 2-ulp bf16 error is flagged at
    # most elements (a bound 10x too loose would flag none)
    wl = W.generate("gdn_in_proj_8192x16384x5120", M=32, with_weight=False)
    x = W.x_values_f32(wl).astype(np.float64)
    rng = np.random.default_rng(7)
    N = 192
    w = (rng.standard_normal((N, wl.K)) * 0.02).astype(np.float32).astype(np.float64)
    ac, as_, ag = O.quantize_activation(x)
    wc, ws, gw = O.pack_weight(w, [N])
    yref, y64 = O.linear_reference(ac, as_, ag, wc, ws, [N], gw, "bf16")
    a_s = O.dequantize_rows(ac, as_).astype(np.float32)
    w_s = O.dequantize_rows(wc, ws).astype(np.float32)
    alpha = np.float32(ag) * np.float32(gw[0])
    bound = O.gemm_elem_bound(y64, O.gemm_abs_product(ac, as_, wc, ws), np.full(N, alpha, np.float64), wl.K, "bf16")
    for acc in (a_s @ w_s.T, _seq_fp32_acc(a_s, w_s)):
        yb = _to_bf16_f64((acc * alpha).astype(np.float32))
        assert np.all(np.abs(yb - yref) <= bound)
        # bf16 spacing at each reference value, from torch's bf16 grid
        up = torch.from_numpy(yref.astype(np.float32)).to(torch.bfloat16)
        ulp = (torch.nextafter(up, torch.full_like(up, float("inf"))) - up).double().abs().numpy()
        planted = yb + 2 * ulp
        assert np.mean(np.abs(planted - yref) > bound) >= 0.25
    assert np.median(bound / ulp) < 3.0


def test_gate_bound_admits_fp32_epilogue_and_rejects_planted_errors():
    # the gate outputs' bound against an fp32 emulation of the GPU epilogue: fp32 GEMM
    # sums, y = acc * alpha in fp32, z = y + dt_bias in fp32, numpy's float32
    # exp/log1p, g = -exp(A_log) * softplus(z), beta = 1/(1+e^-y) evaluated without
    # overflow.  Adversarial parameters: A_log at 0 and 2.7, dt_bias from -100 to 100 and
    # near 0, head weights from 0.002 to 0.5 so that y spans tiny to +-100 (subnormal
    # outputs included).  Planted errors of 1e-3 relative in g and in beta are flagged,
    # and so is a sigmoid that overflows e^-y to give 0 for y < -88.
    wl = W.generate("gdn_gates_32768x96x5120", M=64)
    x = W.x_values_f32(wl).astype(np.float64)
    H = 48
    rng = np.random.default_rng(11)
    A_log = np.linspace(0.0, 2.7, H).astype(np.float32)
    dt = np.concatenate([np.linspace(-100, 100, 24), rng.standard_normal(24) * 0.01]).astype(np.float32)
    sig = np.concatenate([np.geomspace(0.002, 0.2, 48), np.geomspace(0.002, 0.5, 48)])
    w = (rng.standard_normal((96, wl.K)) * sig[:, None]).astype(np.float32).astype(np.float64)
    ac, as_, ag = O.quantize_activation(x)
    wc, ws, gw = O.pack_weight(w, [48, 96])
    y64 = O.gemm_f64(ac, as_, ag, wc, ws, [48, 96], gw)
    out64 = O.gate_epilogue_f64(y64, A_log, dt)
    yref = O.round_output(out64, "f32")
    alpha = (np.float32(ag) * gw[np.repeat([0, 1], 48)]).astype(np.float32)
    gb = O.gemm_elem_bound(y64, O.gemm_abs_product(ac, as_, wc, ws), alpha.astype(np.float64), wl.K, "f32")
    bound = O.gate_elem_bound(y64, gb, A_log, dt, yref)
    a_s = O.dequantize_rows(ac, as_).astype(np.float32)
    w_s = O.dequantize_rows(wc, ws).astype(np.float32)
    f32 = np.float32

    def epilogue(acc, stable_sigmoid=True):
        y = (acc * alpha[None, :]).astype(f32)
        z = (y[:, :H] + dt[None, :]).astype(f32)
        with np.errstate(over="ignore"):
            sp = (np.maximum(z, f32(0)) + np.log1p(np.exp(-np.abs(z)))).astype(f32)
            g = (-np.exp(A_log)[None, :] * sp).astype(f32)
            yb = y[:, H:]
            if stable_sigmoid:
                e = np.exp(-np.abs(yb))
                r = f32(1) / (f32(1) + e)
                beta = np.where(yb >= 0, r, e * r).astype(f32)
            else:
                beta = (f32(1) / (f32(1) + np.exp(-yb))).astype(f32)
        return np.concatenate([g, beta], axis=1).astype(np.float64), y

    for acc in (a_s @ w_s.T, _seq_fp32_acc(a_s, w_s)):
        emu, y = epilogue(acc)
        assert np.all(np.abs(emu - yref) <= bound)
    # the inputs reach the extremes they are meant to
    assert y[:, :H].min() + dt.min() < -87 and y[:, :H].max() + dt.max() > 87
    assert y[:, H:].min() < -88 and np.any((yref[:, H:] > 0) & (yref[:, H:] < 2.0 ** -126))
    for sl in (slice(0, H), slice(H, 2 * H)):
        planted = emu.copy()
        planted[:, sl] *= 1.0 + 1e-3
        flagged = np.abs(planted[:, sl] - yref[:, sl]) > bound[:, sl]
        assert np.mean(flagged) >= 0.1, np.mean(flagged)
    overflowing, _ = epilogue(a_s @ w_s.T, stable_sigmoid=False)
    assert np.any(np.abs(overflowing - yref) > bound)


# --------------------------------------------------------------------------- shared-scale re-encoding

def _xhat_rows(codes, scales, g_rows):
    """Exact dequantized values (Python floats: <= 30 significant bits) from the
    golden E2M1 table and torch's E4M3 values, independent of the oracle."""
    rows = []
    for r in range(codes.shape[0]):
        g = float(np.float32(g_rows[r]))
        row = []
        for j, byte in enumerate(codes[r]):
            for c in (int(byte) & 15, int(byte) >> 4):
                k = len(row)
                s = float(E4M3_TORCH[int(scales[r, k // 16])])
                v = E2M1_GOLDEN[c] * s * g
                row.append(math.copysign(abs(v), -1.0) if c & 8 else v)
        rows.append(row)
    return rows


def test_requantize_shared_scale_brute_force():
    """Bytes of the re-encoding equal exhaustive rational quantization of the exact
    dequantized values under the shared scale (subnormal block scales included)."""
    rng = np.random.default_rng(21)
    seg_end = [3, 5, 8]
    w = rng.standard_normal((8, 64)) * np.repeat([0.02, 0.3, 0.005], [3, 2, 3])[:, None]
    w[1, 16:32] *= 1e-3                                    # blocks with subnormal scales
    w[6, 0:16] = 0.0                                       # a zero block
    w[6, 0] = -0.0
    w64 = w.astype(np.float32).astype(np.float64)
    c, s, g = O.pack_weight(w64, seg_end)
    seg = O.segment_rows(seg_end, 8)
    assert len(set(g.tolist())) == 3
    for g_shared in (None, np.float32(g.max() * np.float32(1.7))):
        c2, s2, gs = O.requantize_shared_scale(c, s, seg_end, g, g_shared)
        assert gs == (g.max() if g_shared is None else g_shared)
        bc, bs = brute_quantize(_xhat_rows(c, s, g[seg]), gs)
        assert np.array_equal(c2, bc) and np.array_equal(s2, bs)


def test_requantize_identity_and_power_of_two_shift():
    """Same scale: the re-encoding is the identity on normal-scale blocks (their
    largest element has code 6, so amax = 6 s g).  Shared scale 2^k g_s: codes
    unchanged and every scale byte lowered by 8k (exponent field - k) while the
    shifted scale stays normal."""
    rng = np.random.default_rng(22)
    w64 = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32).astype(np.float64)
    c, s, g = O.pack_weight(w64, [16])
    assert s.min() >= 8 + 16                               # normal, and still normal after -16
    c1, s1, g1 = O.requantize_shared_scale(c, s, [16], g)
    assert g1 == g[0] and np.array_equal(c1, c) and np.array_equal(s1, s)
    c2, s2, g2 = O.requantize_shared_scale(c, s, [16], g, g[0] * np.float32(4))
    assert np.array_equal(c2, c) and np.array_equal(s2.astype(int), s.astype(int) - 16)


def test_requantize_keeps_codes_and_rerounds_scales():
    """Under a larger shared scale a normal-scale block keeps its codes and its
    scale becomes E4M3-RNE(s g_s / g_shared): the block maximum (code 6) gives
    t' = s g_s / g_shared exactly, and the re-rounded scale moves the element
    quotients by at most 1/16, less than the 12.5 % to the nearest E2M1 midpoint."""
    rng = np.random.default_rng(23)
    seg_end = [32, 64]
    w = rng.standard_normal((64, 128)) * np.repeat([0.02, 0.0826], 32)[:, None]
    c, s, g = O.pack_weight(w.astype(np.float32).astype(np.float64), seg_end)
    c2, s2, gs = O.requantize_shared_scale(c, s, seg_end, g)
    assert gs == g[1] and 2.0 < g[1] / g[0] < 4.0        # not a power of two
    assert s[:32].min() >= 8 + 24                          # scales stay normal after / 4
    assert np.array_equal(c2, c)
    assert np.array_equal(s2[32:], s[32:])
    gF = [Fraction(float(v)) for v in g]
    for r in range(32):
        for b in range(s.shape[1]):
            t = _E4M3_F[int(s[r, b])] * gF[0] / Fraction(float(gs))
            assert s2[r, b] == _nearest_even(_E4M3_F, t)


def test_segment_mismatch_factor():
    g = np.array([1.5e-5, 6.0e-5], dtype=np.float32)      # up scale = 4 x gate scale
    assert O.segment_mismatch_factor(g, g[0]) == (4.0, 1)
    assert O.segment_mismatch_factor(g, g[1]) == (4.0, 0)
    assert O.segment_mismatch_factor(np.full(3, g[0]), g[0]) == (1.0, 0)
    f, worst = O.segment_mismatch_factor(np.array([1.0, 3.0, 0.25], dtype=np.float32), 1.0)
    assert (f, worst) == (4.0, 2)


def test_requantize_code_table_identity_range():
    """The kept-codes range used by the re-encoding kernel: with rho = s g_s /
    (s' g_shared), every E2M1 magnitude v has RNE(v rho) = v exactly when
    7/8 <= rho < 7/6 (checked by exact rational rounding at the ends, just outside
    them and inside)."""
    mags = [Fraction(E2M1_GOLDEN[c]) for c in range(8)]

    def kept(rho):
        return all(_nearest_even(_E2M1_MAGS_F, min(v * rho, Fraction(6))) == c for c, v in enumerate(mags))

    eps = Fraction(1, 2 ** 40)
    assert kept(Fraction(7, 8)) and kept(Fraction(7, 6) - eps) and kept(Fraction(1))
    assert not kept(Fraction(7, 8) - eps) and not kept(Fraction(7, 6))
    for k in range(1, 50):
        rho = Fraction(7, 8) + (Fraction(7, 6) - Fraction(7, 8)) * k / 50
        assert kept(rho)


# --------------------------------------------------------------------------- MXFP4

def brute_mx_quantize(rows):
    """Exact rational MXFP4 quantization: the shared exponent from the exact binary
    exponent of the block maximum, codes by exhaustive nearest-even search."""
    codes_all, scales_all = [], []
    for row in rows:
        codes, scales = [], []
        for b0 in range(0, len(row), 32):
            blk = [Fraction(float(v)) for v in row[b0:b0 + 32]]
            a = max(abs(v) for v in blk)
            if a == 0:
                e = -127
            else:
                e = 0
                while Fraction(2) ** (e + 1) <= a:
                    e += 1
                while Fraction(2) ** e > a:
                    e -= 1
                e = max(-127, min(127, e - 2))
            scales.append(e + 127)
            X = Fraction(2) ** e
            for v, vf in zip(blk, row[b0:b0 + 32]):
                sign = 8 if math.copysign(1.0, float(vf)) < 0 else 0
                codes.append(sign | _nearest_even(_E2M1_MAGS_F, min(abs(v) / X, Fraction(6))))
        codes_all.append([codes[i] | (codes[i + 1] << 4) for i in range(0, len(codes), 2)])
        scales_all.append(scales)
    return np.array(codes_all, dtype=np.uint8), np.array(scales_all, dtype=np.uint8)


def test_mx_quantize_brute_force():
    rng = np.random.default_rng(51)
    x = rng.standard_normal((6, 128)).astype(np.float32) * np.float32(3.0)
    x[1, :32] *= np.float32(1e-30)                         # tiny block (large negative exponent)
    x[2, 32:64] = 0.0                                      # zero block
    x[2, 40] = -0.0
    x[3, 64:96] = np.float32(6.0) * np.float32(2.0 ** 5)   # block of maxima: quotient exactly 6
    x[4, 0] = np.float32(7.9)                              # quotient just under 8 saturates to 6
    x[5, :32] = np.float32(2.0 ** 100)                     # large exponent
    c, s = O.mx_quantize_rows(x.astype(np.float64))
    bc, bs = brute_mx_quantize(x)
    assert np.array_equal(c, bc) and np.array_equal(s, bs)


def test_mx_scale_rule_and_round_trip():
    """amax / 2^shared lies in [4, 8) for every non-zero block; values on the grid
    (e2m1 * 2^e with a block maximum of 4 or 6) re-quantize to the same bytes."""
    rng = np.random.default_rng(52)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-20, 20, size=(16, 1)))).astype(np.float32)
    c, s = O.mx_quantize_rows(x.astype(np.float64))
    amax = np.abs(x.astype(np.float64)).reshape(16, 8, 32).max(axis=2)
    ratio = amax / np.ldexp(1.0, s.astype(np.int64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))
    xh = O.mx_dequantize_rows(c, s)
    c2, s2 = O.mx_quantize_rows(xh)
    top = np.abs(xh).reshape(16, 8, 32).max(axis=2) / np.ldexp(1.0, s.astype(np.int64) - 127)
    ok = np.isin(top, [4.0, 6.0])                          # blocks whose maximum kept exponent e+2
    assert ok.mean() > 0.9
    assert np.array_equal(s2[ok], s[ok])
    rows_ok = ok.all(axis=1)
    assert np.array_equal(c2[rows_ok], c[rows_ok])


def test_mx_gemm_integer_matmul_at_unit_scale():
    rng = np.random.default_rng(53)
    A = rng.choice(np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6]), size=(5, 64))
    Wt = rng.choice(np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -6, -4]), size=(7, 64))
    A[:, ::32] = 6.0                                       # every block max = 6: shared exponent 0
    Wt[:, ::32] = -6.0
    ac, as_ = O.mx_quantize_rows(A)
    wc, ws = O.mx_quantize_rows(Wt)
    assert np.all(as_ == 127) and np.all(ws == 127)
    y = O.mx_gemm_f64(ac, as_, wc, ws)
    Ai, Wi = (A * 2).astype(np.int64), (Wt * 2).astype(np.int64)
    assert np.array_equal(y * 4, (Ai @ Wi.T).astype(np.float64))
