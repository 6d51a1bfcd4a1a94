"""The C-ABI library builds, loads and exports every symbol include/nvfp4.h declares,
and its host-side validation rejects bad arguments before touching the GPU.
CPU only: no compute call reaches a kernel here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    lib_path = os.path.join(ROOT, "nvfp4_w4a4_quantized_amd", "libnvfp4.so")
    if not os.path.exists(lib_path):
        import __graft_entry__
        __graft_entry__.build()
    import nvfp4_w4a4_quantized_amd as nvmod
    return nvmod


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]+?\b(nvfp4_\w+)\s*\(", src)))


def test_header_declarations_are_exported(nv):
    names = _declared()
    assert names == sorted(nv.EXPORTED)
    for n in names:
        assert hasattr(nv.lib, n), n
    ver = int(re.search(r"#define NVFP4_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert nv.nvfp4_abi_version() == ver


FAKE = ctypes.c_void_p(1 << 20)        # a 16-byte aligned non-null address, never dereferenced
FAKE_ODD = ctypes.c_void_p((1 << 20) + 4)


def _q(nv, x=FAKE, dt=1, M=4, K=64, ld=64, gin=None, codes=FAKE, scales=FAKE, gout=FAKE):
    return nv.lib.nvfp4_quantize_act(x, dt, M, K, ld, gin, codes, scales, gout, None)


def test_quantize_act_validation(nv):
    assert _q(nv, x=None) == nv.NVFP4_ERR_INVALID_ARG and "NULL" in nv.nvfp4_last_error()
    assert _q(nv, K=60, ld=64) == nv.NVFP4_ERR_INVALID_ARG and "multiple of 16" in nv.nvfp4_last_error()
    assert _q(nv, M=0) == nv.NVFP4_ERR_INVALID_ARG
    assert _q(nv, M=-3) == nv.NVFP4_ERR_INVALID_ARG
    assert _q(nv, ld=48) == nv.NVFP4_ERR_INVALID_ARG
    assert _q(nv, dt=7) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(nv, x=FAKE_ODD) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(nv, ld=68) == nv.NVFP4_ERR_UNSUPPORTED            # bf16 rows not 16-byte aligned
    assert _q(nv, codes=None) == nv.NVFP4_ERR_INVALID_ARG
    assert _q(nv, gout=None) == nv.NVFP4_ERR_INVALID_ARG


def _segs(vals):
    return (ctypes.c_int64 * len(vals))(*vals), len(vals)


def test_pack_weight_validation(nv):
    def call(seg_vals, gin=None, N=96):
        seg, n = _segs(seg_vals)
        g = None if gin is None else (ctypes.c_float * len(gin))(*gin)
        return nv.lib.nvfp4_pack_weight(FAKE, 0, N, 64, 64, n, seg, g, FAKE, FAKE, FAKE, None)
    assert call([48, 48, 96]) == nv.NVFP4_ERR_INVALID_ARG and "increasing" in nv.nvfp4_last_error()
    assert call([50]) == nv.NVFP4_ERR_INVALID_ARG and "equal N" in nv.nvfp4_last_error()
    assert call([0, 96]) == nv.NVFP4_ERR_INVALID_ARG
    assert call([48, 96], gin=[1.0, float("nan")]) == nv.NVFP4_ERR_INVALID_ARG
    assert call([48, 96], gin=[1.0, -2.0]) == nv.NVFP4_ERR_INVALID_ARG
    assert call(list(range(1, 66)), N=65) == nv.NVFP4_ERR_INVALID_ARG      # more than 64 segments
    seg, n = _segs([96])
    assert nv.lib.nvfp4_pack_weight(FAKE, 0, 96, 64, 64, 0, seg, None, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert nv.lib.nvfp4_pack_weight(FAKE, 0, 96, 64, 64, 1, None, None, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG


def _gemm(nv, M=4, N=96, K=64, seg_vals=(48, 96), gate=None, y_dtype=1, ldy=96, y=FAKE, a=FAKE, ag=FAKE):
    seg, n = _segs(list(seg_vals))
    g = ctypes.byref(gate) if gate is not None else None
    return nv.lib.nvfp4_w4a4_gemm(a, FAKE, ag, M, N, K, FAKE, FAKE, n, seg, FAKE, g, y, y_dtype, ldy, None)


def test_gemm_validation(nv):
    assert _gemm(nv, K=40) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, N=0, seg_vals=(1,)) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, ldy=50) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, seg_vals=(48, 90)) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, a=None) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, ag=None) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, y=None) == nv.NVFP4_ERR_INVALID_ARG
    assert _gemm(nv, y_dtype=5) == nv.NVFP4_ERR_UNSUPPORTED
    assert _gemm(nv, y=FAKE_ODD) == nv.NVFP4_ERR_UNSUPPORTED
    bad = nv.GateParams(40, FAKE.value, FAKE.value)            # N != 2 * n_heads
    assert _gemm(nv, gate=bad, y_dtype=0) == nv.NVFP4_ERR_INVALID_ARG and "2*n_heads" in nv.nvfp4_last_error()
    good = nv.GateParams(48, FAKE.value, FAKE.value)
    assert _gemm(nv, gate=good, y_dtype=1) == nv.NVFP4_ERR_INVALID_ARG      # gate needs fp32 output
    nul = nv.GateParams(48, None, FAKE.value)
    assert _gemm(nv, gate=nul, y_dtype=0) == nv.NVFP4_ERR_INVALID_ARG


def test_linear_validation(nv):
    seg, n = _segs([4096])
    # two-stage shape without workspace for the activation codes
    st = nv.lib.nvfp4_w4a4_linear(FAKE, 1, 512, 256, 256, None, FAKE, 4096, FAKE, FAKE, n, seg, FAKE, None,
                                  FAKE, 1, 4096, None, None, None)
    assert st == nv.NVFP4_ERR_INVALID_ARG and "a_codes_out" in nv.nvfp4_last_error()
    st = nv.lib.nvfp4_w4a4_linear(FAKE, 1, 4, 256, 256, None, FAKE, 4096, FAKE, FAKE, n, seg, FAKE, None,
                                  FAKE, 1, 4096, FAKE, None, None)
    assert st == nv.NVFP4_ERR_INVALID_ARG
    st = nv.lib.nvfp4_w4a4_linear(FAKE, 1, 4, 256, 256, None, None, 4096, FAKE, FAKE, n, seg, FAKE, None,
                                  FAKE, 1, 4096, None, None, None)
    assert st == nv.NVFP4_ERR_INVALID_ARG


def test_linear_noalloc_validation(nv):
    seg, n = _segs([256])

    def call(M=4096, N=256, K=4096):
        return nv.lib.nvfp4_w4a4_linear_noalloc(FAKE, 1, M, K, K, None, FAKE, N, FAKE, FAKE, n, seg, FAKE, None, FAKE,
                                                1, N, None)
    assert call(M=16384) == nv.NVFP4_ERR_INVALID_ARG and "workspace" in nv.nvfp4_last_error()
    assert call(M=0) == nv.NVFP4_ERR_INVALID_ARG
    assert call(K=72) == nv.NVFP4_ERR_INVALID_ARG


def test_binding_rejects_wrong_dtype(nv):
    import torch
    x = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_quantize_act(x, None, x, x, x)


def test_requantize_weight_validation(nv):
    def call(N=96, K=64, seg_vals=(48, 96), codes=FAKE, scales=FAKE, sg=FAKE, co=None, so=None,
             gout=ctypes.c_void_p(1 << 23)):
        seg, n = _segs(list(seg_vals))
        co = ctypes.c_void_p((1 << 24)) if co is None else co
        so = ctypes.c_void_p((1 << 25)) if so is None else so
        return nv.lib.nvfp4_requantize_weight(codes, scales, N, K, n, seg, sg, None, co, so, gout, None)
    assert call(K=40) == nv.NVFP4_ERR_INVALID_ARG and "multiple of 16" in nv.nvfp4_last_error()
    assert call(N=0, seg_vals=(1,)) == nv.NVFP4_ERR_INVALID_ARG
    assert call(seg_vals=(48, 90)) == nv.NVFP4_ERR_INVALID_ARG and "equal N" in nv.nvfp4_last_error()
    assert call(codes=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(sg=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(gout=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(co=FAKE_ODD) == nv.NVFP4_ERR_UNSUPPORTED
    # output codes starting 16 bytes into the input codes: a partial overlap
    assert call(co=ctypes.c_void_p(FAKE.value + 16)) == nv.NVFP4_ERR_INVALID_ARG and "overlap" in nv.nvfp4_last_error()
    assert call(so=ctypes.c_void_p(FAKE.value + 16)) == nv.NVFP4_ERR_INVALID_ARG and "overlap" in nv.nvfp4_last_error()
    # the shared scale written over a segment scale that other workgroups still read
    sg = ctypes.c_void_p(1 << 26)
    assert call(sg=sg, gout=sg) == nv.NVFP4_ERR_INVALID_ARG and "seg_gscale" in nv.nvfp4_last_error()
    assert call(sg=sg, gout=ctypes.c_void_p(sg.value + 4)) == nv.NVFP4_ERR_INVALID_ARG
    seg, n = _segs([48, 96])
    assert nv.lib.nvfp4_requantize_weight(FAKE, FAKE, 96, 64, n, seg, sg, FAKE, ctypes.c_void_p(1 << 24),
                                          ctypes.c_void_p(1 << 25), FAKE, None) == nv.NVFP4_ERR_INVALID_ARG
    assert "gscale_shared" in nv.nvfp4_last_error()


def test_segment_mismatch_factor_matches_oracle(nv):
    import numpy as np
    from oracle import nvfp4 as O
    rng = np.random.default_rng(3)
    cases = [([1.5e-5, 6.0e-5], 1.5e-5), ([2.0, 2.0, 2.0], 2.0), ([1.0, 3.0, 0.25], 1.0)]
    cases += [(list(rng.uniform(1e-6, 1e-3, size=n).astype(np.float32)), float(np.float32(rng.uniform(1e-6, 1e-3))))
              for n in (1, 4, 64)]
    for g, used in cases:
        f, worst = nv.nvfp4_segment_mismatch_factor(g, used)
        of, ow = O.segment_mismatch_factor(g, used)
        assert worst == ow and f == of, (g, used, f, of)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_segment_mismatch_factor([1.0, float("inf")], 1.0)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_segment_mismatch_factor([1.0], 0.0)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_segment_mismatch_factor([1.0] * 65, 1.0)


def test_single_scale_guard(nv):
    """A single-scale launch over a fused weight whose segments were packed with
    different global scales is refused by the host guard; equal scales pass."""
    nv.nvfp4_require_single_scale([0.5])
    nv.nvfp4_require_single_scale([2.0e-5] * 4)
    for scales in ([1.5e-5, 6.0e-5], [1.0, 1.0, 1.0000001], [3.0, 3.0, 0.75, 3.0]):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_require_single_scale(scales)
        assert e.value.status == nv.NVFP4_ERR_INVALID_ARG and "more than one distinct" in str(e.value)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_require_single_scale([])
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_require_single_scale([1.0, float("nan")])
    assert nv.lib.nvfp4_require_single_scale(2, None) == nv.NVFP4_ERR_INVALID_ARG


def test_rotate_quantize_validation(nv):
    seg, n = _segs([64])

    def call(x=FAKE, rows=64, K=1024, ld=1024, h=512, perm=FAKE, codes=FAKE, cbc=FAKE, z=None, segs=(seg, n)):
        return nv.lib.nvfp4_rotate_quantize(x, 1, rows, K, ld, h, perm, FAKE, FAKE, segs[1], segs[0], None, codes,
                                            FAKE, FAKE, cbc, z, None)
    assert call(K=1536, ld=1536) == nv.NVFP4_ERR_UNSUPPORTED and "512" in nv.nvfp4_last_error()   # k = 3
    assert call(h=256) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(K=8192, ld=8192) == nv.NVFP4_ERR_UNSUPPORTED                                       # k = 16
    assert call(perm=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(cbc=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(codes=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(x=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(rows=0) == nv.NVFP4_ERR_INVALID_ARG
    assert call(z=FAKE_ODD) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(segs=_segs([32, 60])) == nv.NVFP4_ERR_INVALID_ARG        # segments must end at rows


def test_gemm_rowcol_validation(nv):
    seg, n = _segs([128])

    def call(rs=FAKE, cs=FAKE, M=64, N=128, K=256):
        return nv.lib.nvfp4_w4a4_gemm_rowcol(FAKE, FAKE, FAKE, M, N, K, FAKE, FAKE, n, seg, FAKE, rs, cs, FAKE, 1, N,
                                             None)
    assert call(rs=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(cs=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(K=40) == nv.NVFP4_ERR_INVALID_ARG
    assert call(N=100) == nv.NVFP4_ERR_INVALID_ARG                        # segment table != N


def test_gdn_gated_delta_validation(nv):
    def call(q=FAKE, k=FAKE, v=FAKE, g=FAKE, T=64, Hk=2, Hv=6, dk=128, dv=128, ldq=256, ldk=256, ldv=768, ldg=12,
             ldo=768, s_out=FAKE, o=FAKE):
        return nv.lib.nvfp4_gdn_gated_delta(q, ldq, k, ldk, v, ldv, g, ldg, T, Hk, Hv, dk, dv, None, s_out, o, ldo,
                                            None)
    assert call(q=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(o=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(s_out=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(T=0) == nv.NVFP4_ERR_INVALID_ARG
    assert call(Hv=5) == nv.NVFP4_ERR_INVALID_ARG and "multiple" in nv.nvfp4_last_error()
    assert call(dk=64, ldq=128, ldk=128) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(dv=12, ldv=72, ldo=72) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(ldq=200) == nv.NVFP4_ERR_INVALID_ARG
    assert call(ldg=11) == nv.NVFP4_ERR_INVALID_ARG
    assert call(ldo=700) == nv.NVFP4_ERR_INVALID_ARG
    assert call(q=FAKE_ODD) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(ldk=258) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(T=1 << 20, ldv=768) == nv.NVFP4_ERR_UNSUPPORTED          # byte extents past 2^31


def test_mxfp4_validation(nv):
    q = lambda K=64, ld=64, codes=FAKE: nv.lib.nvfp4_mxfp4_quantize(FAKE, 1, 4, K, ld, codes, FAKE, None)
    assert q(K=48, ld=48) == nv.NVFP4_ERR_INVALID_ARG and "multiple of 32" in nv.nvfp4_last_error()
    assert q(codes=None) == nv.NVFP4_ERR_INVALID_ARG
    g = lambda M=4, N=64, K=256, y=FAKE, ldy=64, dt=1: nv.lib.nvfp4_mxfp4_gemm(FAKE, FAKE, M, N, K, FAKE, FAKE, y, dt,
                                                                                 ldy, None)
    assert g(K=96) == nv.NVFP4_ERR_UNSUPPORTED and "128" in nv.nvfp4_last_error()
    assert g(K=80) == nv.NVFP4_ERR_INVALID_ARG
    assert g(M=0) == nv.NVFP4_ERR_INVALID_ARG
    assert g(y=None) == nv.NVFP4_ERR_INVALID_ARG
    assert g(ldy=32) == nv.NVFP4_ERR_INVALID_ARG
    assert g(dt=9) == nv.NVFP4_ERR_UNSUPPORTED
    assert g(N=63, ldy=64) == nv.NVFP4_ERR_UNSUPPORTED and "even" in nv.nvfp4_last_error()   # bf16 pairs
    assert g(N=63, ldy=63, dt=0) == nv.NVFP4_ERR_UNSUPPORTED                                   # odd ldy
    assert g(M=1 << 20, N=4096, ldy=4096, K=128) == nv.NVFP4_ERR_UNSUPPORTED                  # > 4 GiB output
