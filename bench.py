"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

Headline (value): TFLOP/s of the prefill fused GDN input projection
M=8192, N=16384 (4 segments: q,k 2048; v,z 6144), K=5120, bf16 in/out, including
the activation quantization (calibrated activation global scale).  One step =
nvfp4_quantize_act + nvfp4_w4a4_gemm (quantize, block-scaled GEMM, per-segment
epilogue).  Also reported: the same with dynamic activation scaling (amax pass
included), the decode GEMV (M=4, N=16384, K=5120) in GB/s of packed weight
traffic with weight copies rotated past the 256 MB infinity cache, the GDN gates
and MLP gate/up workloads, the shared-scale re-encoding of fused weights, the
MXFP4 variant on the in_proj shape, the tiny linear's call latency, the GDN gate
consumer (gated delta rule over 8192 tokens), the achievable HBM and MFMA rates
measured by a plain copy and an MFMA-only kernel, and the CPU oracle's throughput on
a bounded row sample of the headline workload.  Every timed workload reports the
mean and the median, 10th and 90th percentiles of per-call HIP-event times.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--all]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 NVFP4 GEMM TFLOPS incl. act-quant (M=8192,K=5120); decode GB/s"
PEAK_MFMA_F16_TFLOPS = 2500.0          # MI355X dense f16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0                 # MI355X HBM3E
OTHER_WORKLOADS = ["gdn_gates_32768x96x5120", "mlp_gate_up_32768x34816x5120"]
COPY_BYTES = 256 << 20                 # calibration copy for the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gdn_in_proj_traffic.json")
KERNEL_SOURCES = ["nvfp4_w4a4_quantized_amd/csrc/gemm.hip", "nvfp4_w4a4_quantized_amd/csrc/kernel_common.hpp",
                  "nvfp4_w4a4_quantized_amd/csrc/nvfp4_device.hpp", "nvfp4_w4a4_quantized_amd/csrc/launch.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_if_current():
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def setup_layer(nv, wl, seg_gscale=None):
    import torch
    from synth import workloads as W
    xt = dev_bf16(wl.data["x_bf16"]) if wl.x_dtype == "bf16" else torch.from_numpy(wl.data["x32"]).cuda()
    wt = torch.from_numpy(wl.data["w32"]).cuda()
    wc, ws = nv.empty_packed(wl.N, wl.K, "cuda")
    wg = torch.empty(len(wl.seg_end), dtype=torch.float32, device="cuda")
    nv.nvfp4_pack_weight(wt, wl.seg_end, seg_gscale, wc, ws, wg)
    torch.cuda.synchronize()
    del wt
    return xt, wc, ws, wg


def timed_steps(step, steps):
    """Wall time per step (ms) of exactly `steps` back-to-back steps, bracketed by
    device synchronizations; nothing but the steps' own launches is enqueued."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def settle(step, seconds=0.4):
    """Run `step` untimed for about `seconds`, before the warm-up steps, so that the
    GPU has reached the clock it holds under this load when timing starts."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def dist(ms_values):
    """mean / median / p10 / p90 of per-call times (ms)."""
    a = np.asarray(ms_values, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p10": round(float(np.percentile(a, 10)), 5), "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


def event_times(call, n):
    """HIP-event duration (ms) of each of n calls, events on the launch stream."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def event_breakdown(step, steps):
    """Mean HIP-event durations (ms) of the two launches of a step, measured in a
    separate pass after the timed one (event records between launches would add
    their own gaps to the timed steps)."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    first = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    second = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    event_breakdown.last = dict(total=[e[0].elapsed_time(e[2]) for e in evs], first=[e[0].elapsed_time(e[1]) for e in evs],
                                second=[e[1].elapsed_time(e[2]) for e in evs])
    return first, second


def time_prefill(nv, xt, wc, ws, wg, seg_end, steps, warmup, static_g, y_dtype):
    """Time `steps` steps of quantize + GEMM.  Returns wall ms/step and the mean
    HIP-event durations of the quantize (and amax) part and of the GEMM launch."""
    import torch
    M, K = xt.shape
    N = wc.shape[0]
    ac, as_ = nv.empty_packed(M, K, "cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=y_dtype, device="cuda")
    gin = static_g
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nv.nvfp4_quantize_act(xt, gin, ac, as_, gout, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nv.nvfp4_w4a4_gemm(ac, as_, gout, wc, ws, seg_end, wg, y, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    settle(step)
    for _ in range(warmup):
        step()
    wall = timed_steps(step, steps)
    q_ms, g_ms = event_breakdown(step, max(steps, 50))
    return wall, q_ms, g_ms, y


def time_decode(nv, steps, warmup):
    """Fused decode GEMV (M=4) with weight copies rotated so that the working set
    exceeds twice the 256 MB infinity cache."""
    import torch
    from synth import workloads as W
    wl = W.generate("decode_gemv_4x16384x5120")
    xt, wc, ws, wg = setup_layer(nv, wl)
    n_sets = 12                                   # 12 x 47.2 MB = 566 MB of packed weight
    copies = [(wc.clone(), ws.clone()) for _ in range(n_sets)]
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    gstat = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(wl.M, wl.K, "cuda")
    nv.nvfp4_quantize_act(xt, None, ac, as_, gstat)           # calibrated scale = this tensor's
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        c, s = copies[i % n_sets]
        nv.nvfp4_w4a4_linear(xt, gstat, gout, c, s, wl.seg_end, wg, y, stream=stream)
    # steady state: back-to-back calls on rotated weights, one event pair around them
    n = max(steps, 120)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        c, s = copies[i % n_sets]
        nv.nvfp4_w4a4_linear(xt, gstat, gout, c, s, wl.seg_end, wg, y, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    per_call = e0.elapsed_time(e1) / n
    # single-call times (an event pair around each call, rotated weights)
    def one(i):
        c, s = copies[i % n_sets]
        nv.nvfp4_w4a4_linear(xt, gstat, gout, c, s, wl.seg_end, wg, y, stream=stream)
    single = np.array(event_times(one, 240))
    w_bytes = wl.N * wl.K // 2 + wl.N * wl.K // 16
    alg_bytes = w_bytes + wl.M * wl.K * 2 + wl.M * wl.N * 2
    gbps = alg_bytes / (per_call * 1e-3) / 1e9
    return dict(workload=wl.name, us_per_call=round(per_call * 1e3, 3), gbps=round(gbps, 1),
                frac_hbm=round(gbps / PEAK_HBM_GBPS, 4), algorithmic_bytes=alg_bytes,
                single_call_us_median=round(float(np.median(single)) * 1e3, 3),
                single_call_us={k: (round(v * 1e3, 3) if k != "n" else v) for k, v in dist(single).items()},
                rotated_weight_sets=n_sets, calls=n, act_scale="static",
                timing="back-to-back calls, rotated weight copies, one event pair around all calls")


def time_config(nv, name, steps, warmup):
    """Another prefill-shaped workload, timed like the headline: one step =
    nvfp4_quantize_act (calibrated activation scale) + nvfp4_w4a4_gemm, with
    HIP events around each launch on the launch stream.  Calibrated weight
    scales (segment scales 4x apart) are derived on the GPU: segment 0 is packed
    once in dynamic mode and its amax-derived scale is read back."""
    import torch
    from synth import workloads as W
    wl = W.generate(name)
    seg_g = None
    if wl.seg_scale_ratio is not None:
        _, _, _, wg0 = setup_layer(nv, wl)
        g0 = float(wg0[0].item())
        seg_g = [float(np.float32(r) * np.float32(g0)) for r in wl.seg_scale_ratio]
        del wg0
    xt, wc, ws, wg = setup_layer(nv, wl, seg_g)
    wl.data.pop("w32", None)
    wl.data.pop("x32", None)
    M, N, K = wl.M, wl.N, wl.K
    gate = None
    if wl.gate_heads:
        gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    gstat = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_quantize_act(xt, None, ac, as_, gstat)
    y = torch.empty((M, N), dtype=torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    gout = torch.empty(1, dtype=torch.float32, device="cuda")

    fused = N <= 128 and K % 256 == 0          # the fused skinny-N linear: x read once
    # HBM-bound (fused) workloads alternate between two copies of x so that the working
    # set (2 x 335 MB) exceeds twice the 256 MB infinity cache
    xs = [xt, xt.clone()] if fused else [xt]
    turn = [0]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if fused:
            xi = xs[turn[0] % len(xs)]
            turn[0] += 1
            nv.nvfp4_w4a4_linear(xi, gstat, gout, wc, ws, wl.seg_end, wg, y, gate=gate, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        else:
            nv.nvfp4_quantize_act(xt, gstat, ac, as_, gout, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            nv.nvfp4_w4a4_gemm(ac, as_, gout, wc, ws, wl.seg_end, wg, y, gate=gate, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    settle(step)
    for _ in range(warmup):
        step()
    wall = timed_steps(step, steps)
    q_ms, g_ms = event_breakdown(step, max(steps, 50))
    step_dist = dist(event_breakdown.last["total"])
    flops = 2.0 * M * N * K
    ybytes = M * N * (2 if wl.y_dtype == "bf16" else 4)
    packed = lambda rows: rows * K // 2 + rows * K // 16
    two_stage_bytes = M * K * 2 + 2 * packed(M) + packed(N) + ybytes      # x in, codes out, codes + W in, y out
    fused_bytes = M * K * 2 + packed(N) + ybytes                           # x in, W in, y out
    mode = ("fused quantize + GEMM (nvfp4_w4a4_linear), static activation scale" if fused
            else "two-stage, static activation scale")
    breakdown = {"linear": round(q_ms, 4)} if fused else {"quantize_act": round(q_ms, 4), "gemm": round(g_ms, 4)}
    out = dict(workload=name, M=M, N=N, K=K, segments=wl.seg_end, mode=mode,
               ms_per_step=round(wall, 4), tflops=round(flops / (wall * 1e-3) / 1e12, 2),
               breakdown_ms=breakdown, step_ms=step_dist,
               input_sets=len(xs),
               algorithmic_bytes={"two_stage": two_stage_bytes, "fused_minimum": fused_bytes})
    if fused:
        gbps = fused_bytes / (wall * 1e-3) / 1e9
        kgbps = fused_bytes / (q_ms * 1e-3) / 1e9
        out.update(bound="hbm", gbps_vs_fused_minimum=round(gbps, 1), frac_hbm=round(gbps / PEAK_HBM_GBPS, 4),
                   kernel_gbps=round(kgbps, 1), kernel_frac_hbm=round(kgbps / PEAK_HBM_GBPS, 4))
    else:
        out.update(bound="mfma", frac_mfma=round(flops / (wall * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
                   gemm_tflops=round(flops / (g_ms * 1e-3) / 1e12, 2))
    del xt, xs, wc, ws, ac, as_, y
    torch.cuda.empty_cache()
    return out


def time_tiny(nv, calls=200):
    """The tiny linear (64 x 128 x 256, fp32 in and out, dynamic scales for both
    operands): latency of one nvfp4_w4a4_linear call (one launch: the fused skinny
    kernel takes the activation amax itself), HIP events around each call."""
    import torch
    from synth import workloads as W
    wl = W.generate("tiny_linear_64x128x256")
    xt = torch.from_numpy(wl.data["x32"]).cuda()
    wt = torch.from_numpy(wl.data["w32"]).cuda()
    wc, ws = nv.empty_packed(wl.N, wl.K, "cuda")
    wg = torch.empty(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_pack_weight(wt, wl.seg_end, None, wc, ws, wg)
    y = torch.empty((wl.M, wl.N), dtype=torch.float32, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    call = lambda i: nv.nvfp4_w4a4_linear(xt, None, g, wc, ws, wl.seg_end, wg, y)
    for i in range(20):
        call(i)
    d = dist(event_times(call, calls))
    return dict(workload=wl.name, mode="nvfp4_w4a4_linear, dynamic activation scale (amax inside the fused kernel)",
                latency_us={k: (round(v * 1e3, 2) if k != "n" else v) for k, v in d.items()},
                bound="launch latency")


PEAK_FP32_VALU_TFLOPS = 157.3          # MI355X vector fp32 (packed); unpacked FMA: half of it


def time_gdn(nv, steps, warmup):
    """The GDN gate consumer: nvfp4_gdn_gated_delta over 8192 tokens with 16 key and
    48 value heads, d_k = d_v = 128 (one sequence), inputs resident in HBM."""
    import torch
    from synth import workloads as W
    T = 8192
    hd = W.GDN_HEADS
    inp = W.gdn_recurrence_inputs(T, **hd, seed=0)
    q = torch.from_numpy(inp["q"].reshape(T, -1)).cuda()
    k = torch.from_numpy(inp["k"].reshape(T, -1)).cuda()
    v = torch.from_numpy(inp["v"].reshape(T, -1)).cuda()
    gates = torch.from_numpy(inp["gates"]).cuda()
    Hk, Hv, dk, dv = hd["n_k_heads"], hd["n_v_heads"], hd["d_k"], hd["d_v"]
    o = torch.empty((T, Hv * dv), dtype=torch.float32, device="cuda")
    st = torch.empty((Hv, dk, dv), dtype=torch.float32, device="cuda")
    call = lambda i: nv.nvfp4_gdn_gated_delta(q, k, v, gates, Hk, Hv, None, st, o)
    settle(lambda: call(0), 0.3)
    for i in range(warmup):
        call(i)
    d = dist(event_times(call, max(steps, 20)))
    flops = 7.0 * T * Hv * dk * dv          # S^T k, the decayed rank-one write, S^T q
    bytes_ = 4 * T * (2 * Hk * dk + 2 * Hv * dv + 2 * Hv) + 4 * Hv * dk * dv
    ms = d["median"]
    return dict(workload="gdn_gated_delta_8192tok_16x48heads_128x128",
                mode="alpha = e^g and the gated delta rule (Eq. 2), fp32, one sequence", ms=d,
                tokens_per_s=round(T / (ms * 1e-3), 1), tflops=round(flops / (ms * 1e-3) / 1e12, 3),
                bound="alu (sequential token chain)", peak_fp32_vector_tflops=PEAK_FP32_VALU_TFLOPS,
                frac_fp32_vector=round(flops / (ms * 1e-3) / 1e12 / PEAK_FP32_VALU_TFLOPS, 4),
                algorithmic_bytes=bytes_, gbps=round(bytes_ / (ms * 1e-3) / 1e9, 1),
                us_per_token=round(ms * 1e3 / T, 4))


def time_rotated(nv, steps, warmup):
    """The rotated NVFP4 front end on the GDN in_proj shape (8192 x 16384 x 5120, 4
    weight segments): the weight is rotated and packed once (offline); one step =
    nvfp4_rotate_quantize of the activations (dynamic: a rotate+amax pass, then rotate,
    quantize and c_bc) + nvfp4_w4a4_gemm_rowcol (the GEMM with the c_bc factors)."""
    import torch
    from synth import workloads as W
    wl = W.generate("gdn_in_proj_8192x16384x5120")
    M, N, K = wl.M, wl.N, wl.K
    p = W.krpbh_params(K, 512, seed=0)
    perm, signs, Q = (torch.from_numpy(p[n]).cuda() for n in ("perm", "signs", "Q"))
    xt = dev_bf16(wl.data["x_bf16"])
    wt = torch.from_numpy(wl.data["w32"]).cuda()
    wl.data.clear()
    wc, ws = nv.empty_packed(N, K, "cuda")
    wg = torch.empty(len(wl.seg_end), dtype=torch.float32, device="cuda")
    cw = torch.empty(N, dtype=torch.float32, device="cuda")
    nv.nvfp4_rotate_quantize(wt, perm, signs, Q, wc, ws, wg, cw, seg_end=wl.seg_end)
    torch.cuda.synchronize()
    del wt
    ac, as_ = nv.empty_packed(M, K, "cuda")
    ag = torch.empty(1, dtype=torch.float32, device="cuda")
    cx = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nv.nvfp4_rotate_quantize(xt, perm, signs, Q, ac, as_, ag, cx, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nv.nvfp4_w4a4_gemm_rowcol(ac, as_, ag, wc, ws, wl.seg_end, wg, cx, cw, y, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    settle(step)
    for _ in range(warmup):
        step()
    wall = timed_steps(step, steps)
    r_ms, g_ms = event_breakdown(step, max(steps, 20))
    flops = 2.0 * M * N * K
    rot_bytes = 2 * (M * K * 2) + M * K // 2 + M * K // 16 + 4 * M     # x read twice, codes, scales, c_bc
    del xt, wc, ws, ac, as_, y
    torch.cuda.empty_cache()
    return dict(workload="rotated_gdn_in_proj_8192x16384x5120",
                mode="K-RPBH rotation (h = 512, k = 10) + NVFP4 (dynamic) + c_bc, then the GEMM with c_bc factors",
                ms_per_step=round(wall, 4), tflops=round(flops / (wall * 1e-3) / 1e12, 2),
                breakdown_ms={"rotate_quantize": round(r_ms, 4), "gemm_rowcol": round(g_ms, 4)},
                step_ms=dist(event_breakdown.last["total"]),
                gemm_tflops=round(flops / (g_ms * 1e-3) / 1e12, 2),
                rotate_gbps=round(rot_bytes / (r_ms * 1e-3) / 1e9, 1), rotate_algorithmic_bytes=rot_bytes)


def achievable_peaks(nv):
    """Rates the chip sustains here, beside the datasheet peaks: a plain 1 GiB device
    copy (bytes read + written per second) and a kernel that only issues f16 MFMAs."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    copy_ms = dist(event_times(lambda i: dst.copy_(src), 20))["median"]
    del src, dst
    blocks, iters = 256 * 4, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    nv.nvfp4_bench_mfma_peak(2000, blocks, out)
    mf_ms = dist(event_times(lambda i: nv.nvfp4_bench_mfma_peak(iters, blocks, out), 5))["median"]
    mflops = blocks * 4 * iters * 4 * 32768.0
    torch.cuda.empty_cache()
    return {"hbm_copy_gbps": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "hbm_copy_frac_of_datasheet": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_f16_tflops": round(mflops / (mf_ms * 1e-3) / 1e12, 1),
            "mfma_f16_frac_of_datasheet": round(mflops / (mf_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            "how": "torch copy of 1 GiB (2 GiB moved); MFMA 32x32x16 f16 only, 1024 workgroups x 4 waves"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


REQUANT_WORKLOADS = ["gdn_in_proj_8192x16384x5120", "mlp_gate_up_32768x34816x5120"]


def time_requantize(nv, name, steps, warmup):
    """Re-encoding of a fused weight onto one shared global scale
    (nvfp4_requantize_weight, out of place): back-to-back calls with HIP events
    around them on the launch stream; GB/s of the algorithmic bytes (packed weight
    read + written once)."""
    import torch
    from synth import workloads as W
    wl = W.generate(name, M=1)
    seg_g = None
    if wl.seg_scale_ratio is not None:
        _, _, _, wg0 = setup_layer(nv, wl)
        g0 = float(wg0[0].item())
        seg_g = [float(np.float32(r) * np.float32(g0)) for r in wl.seg_scale_ratio]
    _, wc, ws, wg = setup_layer(nv, wl, seg_g)
    wl.data.clear()
    N, K = wl.N, wl.K
    alg = 2 * (N * K // 2 + N * K // 16)
    # rotated input/output sets: the working set exceeds twice the 256 MB infinity cache
    n_sets = max(2, -(-600_000_000 // alg))
    sets = [((wc, ws) if i == 0 else (wc.clone(), ws.clone())) + nv.empty_packed(N, K, "cuda") for i in range(n_sets)]
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        c, sc, co, so = sets[i % n_sets]
        nv.nvfp4_requantize_weight(c, sc, wl.seg_end, wg, None, co, so, gout, stream=stream)

    for i in range(warmup):
        call(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kept = float((sets[0][2] == wc).float().mean().item())
    gbps = alg / (ms * 1e-3) / 1e9
    del wc, ws, sets
    torch.cuda.empty_cache()
    return dict(workload=f"requantize_weight_{N}x{K}", source=name, segments=wl.seg_end,
                segment_scales="calibrated, 4x apart" if seg_g else "per-segment amax",
                us_per_call=round(ms * 1e3, 2), rotated_sets=n_sets, algorithmic_bytes=alg, bound="hbm",
                gbps=round(gbps, 1),
                frac_hbm=round(gbps / PEAK_HBM_GBPS, 4), codes_kept_fraction=round(kept, 6))


PEAK_MFMA_FP4_TFLOPS = 10100.0         # MI355X dense FP4 MFMA


def time_mxfp4(nv, steps, warmup):
    """MXFP4 variant on the GDN in_proj shape (8192 x 16384 x 5120, bf16 in/out): one
    step = nvfp4_mxfp4_quantize(x) + nvfp4_mxfp4_gemm, the weight quantized once
    beforehand; HIP events around each launch on the launch stream."""
    import torch
    from synth import workloads as W
    wl = W.generate("gdn_in_proj_8192x16384x5120")
    M, N, K = wl.M, wl.N, wl.K
    xt = dev_bf16(wl.data["x_bf16"])
    wt = torch.from_numpy(wl.data["w32"]).cuda()
    wl.data.clear()
    wc, ws = nv.empty_mx_packed(N, K, "cuda")
    nv.nvfp4_mxfp4_quantize(wt, wc, ws)
    del wt
    ac, as_ = nv.empty_mx_packed(M, K, "cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nv.nvfp4_mxfp4_quantize(xt, ac, as_, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nv.nvfp4_mxfp4_gemm(ac, as_, wc, ws, y, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    wall = timed_steps(step, steps)
    q_ms, g_ms = event_breakdown(step, steps)
    flops = 2.0 * M * N * K
    gt = flops / (g_ms * 1e-3) / 1e12
    del xt, wc, ws, ac, as_, y
    torch.cuda.empty_cache()
    return dict(workload="mxfp4_gdn_in_proj_8192x16384x5120", M=M, N=N, K=K,
                mode="MXFP4 quantize (activation) + GEMM on the block-scaled FP4 MFMA, bf16 out",
                ms_per_step=round(wall, 4), tflops=round(flops / (wall * 1e-3) / 1e12, 2),
                breakdown_ms={"mx_quantize": round(q_ms, 4), "mx_gemm": round(g_ms, 4)}, bound="mfma",
                gemm_tflops=round(gt, 2), peak_fp4_tflops=PEAK_MFMA_FP4_TFLOPS,
                frac_fp4_peak=round(gt / PEAK_MFMA_FP4_TFLOPS, 4))


def profile_target(nv, target, launches):
    """Launch one kernel of the path a few times and nothing else, for counter runs
    (rocprofv3 --pmc): first a plain copy of COPY_BYTES (the calibration kernel whose
    HBM bytes are known: COPY_BYTES read + COPY_BYTES written), then `launches`
    launches of the target:
      gemm   - nvfp4_w4a4_gemm on the GDN in_proj workload (8192 x 16384 x 5120)
      quant  - nvfp4_quantize_act on the same activations (static scale)
      decode - nvfp4_w4a4_linear, decode GEMV 4 x 16384 x 5120
      gates  - nvfp4_w4a4_linear, fused GDN gates 32768 x 96 x 5120
      requant - nvfp4_requantize_weight on the GDN in_proj weight (16384 x 5120)
      mxgemm - nvfp4_mxfp4_gemm on the GDN in_proj shape (MXFP4 operands)
      gdn    - nvfp4_gdn_gated_delta, 8192 tokens, 16 key / 48 value heads
      rotate - nvfp4_rotate_quantize (dynamic) on the GDN in_proj activations"""
    import torch
    from synth import workloads as W
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if target == "rotate":
        wl = W.generate("gdn_in_proj_8192x16384x5120", with_weight=False)
        p = W.krpbh_params(wl.K, 512, seed=0)
        perm, signs, Q = (torch.from_numpy(p[n]).cuda() for n in ("perm", "signs", "Q"))
        xt = dev_bf16(wl.data["x_bf16"])
        ac, as_ = nv.empty_packed(wl.M, wl.K, "cuda")
        ag = torch.empty(1, dtype=torch.float32, device="cuda")
        cx = torch.empty(wl.M, dtype=torch.float32, device="cuda")
        for _ in range(launches):
            nv.nvfp4_rotate_quantize(xt, perm, signs, Q, ac, as_, ag, cx)
        torch.cuda.synchronize()
        print(f"profile target rotate: {launches} calls (rotate+amax, rotate+quantize) on 8192 x 5120", flush=True)
        return
    if target == "gdn":
        T = 8192
        hd = W.GDN_HEADS
        inp = W.gdn_recurrence_inputs(T, **hd, seed=0)
        q, k, v = (torch.from_numpy(inp[n].reshape(T, -1)).cuda() for n in ("q", "k", "v"))
        gates = torch.from_numpy(inp["gates"]).cuda()
        o = torch.empty_like(v)
        st = torch.empty((hd["n_v_heads"], hd["d_k"], hd["d_v"]), dtype=torch.float32, device="cuda")
        for _ in range(launches):
            nv.nvfp4_gdn_gated_delta(q, k, v, gates, hd["n_k_heads"], hd["n_v_heads"], None, st, o)
        torch.cuda.synchronize()
        print(f"profile target gdn: {launches} launches of the gated delta rule over {T} tokens", flush=True)
        return
    name = {"gemm": "gdn_in_proj_8192x16384x5120", "quant": "gdn_in_proj_8192x16384x5120",
            "decode": "decode_gemv_4x16384x5120", "gates": "gdn_gates_32768x96x5120",
            "requant": "gdn_in_proj_8192x16384x5120", "mxgemm": "gdn_in_proj_8192x16384x5120"}[target]
    wl = W.generate(name)
    xt, wc, ws, wg = setup_layer(nv, wl)
    M, N, K = wl.M, wl.N, wl.K
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_quantize_act(xt, None, ac, as_, g)            # calibrated scale: this tensor's own
    y = torch.empty((M, N), dtype=torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32, device="cuda")
    gout = torch.empty(1, dtype=torch.float32, device="cuda")
    gate = None
    if wl.gate_heads:
        gate = (torch.from_numpy(wl.data["A_log"]).cuda(), torch.from_numpy(wl.data["dt_bias"]).cuda())
    torch.cuda.synchronize()
    co, so = nv.empty_packed(N, K, "cuda")
    if target == "mxgemm":
        xc, xs = nv.empty_mx_packed(M, K, "cuda")
        mwc, mws = nv.empty_mx_packed(N, K, "cuda")
        nv.nvfp4_mxfp4_quantize(xt, xc, xs)
        nv.nvfp4_mxfp4_quantize(torch.from_numpy(wl.data["w32"]).cuda(), mwc, mws)
        torch.cuda.synchronize()
    for _ in range(launches):
        if target == "mxgemm":
            nv.nvfp4_mxfp4_gemm(xc, xs, mwc, mws, y)
        elif target == "requant":
            nv.nvfp4_requantize_weight(wc, ws, wl.seg_end, wg, None, co, so, gout)
        elif target == "gemm":
            nv.nvfp4_w4a4_gemm(ac, as_, g, wc, ws, wl.seg_end, wg, y)
        elif target == "quant":
            nv.nvfp4_quantize_act(xt, g, ac, as_, gout)
        else:
            nv.nvfp4_w4a4_linear(xt, g, gout, wc, ws, wl.seg_end, wg, y, gate=gate)
    torch.cuda.synchronize()
    print(f"profile target {target}: {launches} launches of {name} after a {COPY_BYTES >> 20} MiB copy", flush=True)


def cpu_baseline(wl, static_g, target_s=10.0):
    """The oracle as it stands, timed on the host on a bounded row sample of the
    headline workload: quantize the sampled rows of X, dequantize-then-GEMM in
    float64, round to bf16.  Weight packing by the oracle is done once, untimed."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import nvfp4 as O
    from synth import workloads as W
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        wc, ws, wg = O.pack_weight(wl.data["w32"].astype(np.float64), wl.seg_end)
        pack_s = time.perf_counter() - t0
        x = W.x_values_f32(wl)

        def run(rows):
            t = time.perf_counter()
            ac, as_, ag = O.quantize_activation(x[:rows].astype(np.float64), static_g)
            O.linear_reference(ac, as_, ag, wc, ws, wl.seg_end, wg, "bf16")
            return time.perf_counter() - t

        rows, t = 64, run(64)
        while t < target_s and rows < wl.M:           # grow the sample until it takes >= target_s
            rows = min(wl.M, rows * 2)
            t = run(rows)
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    flops = 2.0 * rows * wl.N * wl.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(min(cores, used)), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{rows} of {wl.M} rows of the GDN in_proj workload (N={wl.N}, K={wl.K}): oracle "
                      f"quantize + float64 dequantize-GEMM + bf16 rounding, {t:.1f} s; oracle weight "
                      f"packing ({pack_s:.1f} s) untimed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dynamic", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="time only the decode GEMV (no JSON contract line)")
    ap.add_argument("--no-configs", action="store_true", help="skip the GDN-gates and MLP gate/up workloads")
    ap.add_argument("--configs-only", action="store_true", help="time only the GDN-gates and MLP gate/up workloads")
    ap.add_argument("--profile-target", choices=["gemm", "quant", "decode", "gates", "requant", "mxgemm", "gdn", "rotate"],
                    help="for counter runs: a calibration copy, then a few launches of one kernel (no JSON line)")
    ap.add_argument("--launches", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this layer is benchmarked on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_w4a4_quantized_amd as nv
    from synth import workloads as W

    torch.cuda.set_device(0)
    if args.profile_target:
        profile_target(nv, args.profile_target, args.launches)
        return
    if args.decode_only:
        print(json.dumps({"decode": time_decode(nv, args.steps, args.warmup)}), flush=True)
        return
    if args.configs_only:
        ow = [time_config(nv, n, args.steps, args.warmup) for n in OTHER_WORKLOADS]
        ow += [time_requantize(nv, n, max(args.steps, 20), 5) for n in REQUANT_WORKLOADS]
        ow.append(time_mxfp4(nv, args.steps, args.warmup))
        print(json.dumps({"other_workloads": ow}), flush=True)
        return
    log("generating the GDN in_proj workload (8192 x 16384 x 5120)")
    wl = W.generate("gdn_in_proj_8192x16384x5120")
    xt, wc, ws, wg = setup_layer(nv, wl)
    M, N, K = wl.M, wl.N, wl.K
    # calibrated activation scale: this tensor's own amax-derived scale, computed once
    gstat = torch.empty(1, dtype=torch.float32, device="cuda")
    ac, as_ = nv.empty_packed(M, K, "cuda")
    nv.nvfp4_quantize_act(xt, None, ac, as_, gstat)
    torch.cuda.synchronize()
    del ac, as_
    flops = 2.0 * M * N * K

    log("timing prefill (static activation scale)")
    wall, q_ms, g_ms, _ = time_prefill(nv, xt, wc, ws, wg, wl.seg_end, args.steps, args.warmup, gstat,
                                       torch.bfloat16)
    value = flops / (wall * 1e-3) / 1e12
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gdn_in_proj_8192x16384x5120", "M": M, "N": N, "K": K,
                   "segments": wl.seg_end, "act_scale": "static", "x_dtype": "bf16", "y_dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_MFMA_F16_TFLOPS, 4),
                     "traffic": traffic_if_current(), "kernel": "k_gemm_big (256x256 tile, bf16 out)",
                     "kernel_ms": round(g_ms, 4)},
        "breakdown_ms": {"quantize_act": round(q_ms, 4), "gemm": round(g_ms, 4)},
        "step_ms": dist(event_breakdown.last["total"]),
        "gemm_ms": dist(event_breakdown.last["second"]),
    }
    if not args.no_dynamic:
        log("timing prefill (dynamic activation scale)")
        wall_d, qd_ms, gd_ms, _ = time_prefill(nv, xt, wc, ws, wg, wl.seg_end, args.steps, args.warmup, None,
                                               torch.bfloat16)
        out["dynamic_act_scale"] = {"value": round(flops / (wall_d * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                                    "ms_per_step": round(wall_d, 4), "amax_and_quantize_ms": round(qd_ms, 4)}
    del xt, wc, ws
    torch.cuda.empty_cache()
    if not args.no_decode:
        log("timing decode GEMV (4 x 16384 x 5120)")
        out["decode"] = time_decode(nv, args.steps, args.warmup)
    if not args.no_configs:
        out["other_workloads"] = []
        for n in OTHER_WORKLOADS:
            log(f"timing {n}")
            out["other_workloads"].append(time_config(nv, n, args.steps, args.warmup))
    if not args.no_configs:
        log("timing the MXFP4 variant on the GDN in_proj shape")
        out["other_workloads"].append(time_mxfp4(nv, args.steps, args.warmup))
        for n in REQUANT_WORKLOADS:
            log(f"timing the shared-scale re-encoding of the {n} weight")
            out["other_workloads"].append(time_requantize(nv, n, max(args.steps, 20), 5))
    if not args.no_configs:
        log("timing the tiny linear (64 x 128 x 256)")
        out["tiny_linear"] = time_tiny(nv)
        log("timing the rotated front end on the GDN in_proj shape")
        out["other_workloads"].append(time_rotated(nv, args.steps, args.warmup))
        log("timing the GDN gate consumer (8192 tokens, 48 heads)")
        out["gdn_recurrence"] = time_gdn(nv, args.steps, 3)
        log("measuring achievable HBM and MFMA rates")
        out["achievable_peaks"] = achievable_peaks(nv)
    if not args.no_cpu:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(wl, np.float32(gstat.item()))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
