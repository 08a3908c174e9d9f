"""Benchmark of the attention forward (or backward) on one MI355X; prints ONE JSON line.

A step is one sdpa_forward call (scores, scale, mask, online softmax, weighted sum of V: the whole fused attention)
over the long-sequence workload B=4, h=8, n_q=n_k=4096, d_k=d_v=64, bf16, unmasked, with Q/K/V ~ N(0,1) seeded and
already resident in HBM. Metric: attention TFLOP/s = 4*B*h*n_q*n_k*d_k / time, against the bf16 dense MFMA peak.
The line also carries the ceilings measured on the chip after the timed region (dense MFMA, v_exp_f32, LDS reads,
copy bandwidth) and the softmax's exp2 throughput (one per visible score) against the measured exp ceiling.

With a backward workload (--workload sdpa_bwd_bf16_b4_h8_n4096, sdpa_bwd_causal_bf16_b4_h8_n4096, or the head widths
32 and 128: sdpa_bwd_bf16_b4_h16_n4096_d32, sdpa_bwd_bf16_b4_h4_n4096_d128) a step is one sdpa_backward call
(pre-pass, dK/dV, dQ) on the same tensors plus a seeded upstream gradient, with the training forward's float32
output and log-sum-exp computed once before the timed region; metric: backward TFLOP/s = 10*B*h*n_q*n_k*d_k / time
(the five n_q x n_k x d_k products the gradient needs).

With --workload sdpa_padded_bf16_b4_h8_n4096 a step is one sdpa_forward_padded call on the same tensors treated as a
length bucket (real key counts per batch entry in the workload); metric: TFLOP/s over the real (query, key) pairs.

With --workload sdpa_window_bf16_b4_h8_n4096_w256 a step is one sdpa_forward_window call (radius 256); metric:
TFLOP/s over the band's (query, key) pairs.
With --workload mha_self_bf16_b32_n128_dm512 a step is one mha_forward (B=32, n=128, d_model=512, h=8); metric:
TFLOP/s over its products (projections, attention, W^O).
With --workload encoder_layer_bf16_b32_n128_dm512 a step is one encoder_layer_forward (B=32, n=128, d_model=512,
h=8, d_ff=2048); metric: TFLOP/s over the layer's products, with tokens/s beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

# The CPU baseline's BLAS thread count: the cores this process may run on, unless the environment already fixes it.
# Set before numpy (and its BLAS) is first imported.
_AFFINITY = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(_AFFINITY))

METRIC = "attention TFLOP/s (4·B·h·n_q·n_k·d_k) at h={h},d_k={d_k}; % of bf16 MFMA peak"
METRIC_WINDOW = "restricted self-attention TFLOP/s over the band's pairs (4·B·h·pairs·d_k) at h=8,d_k=64; % of bf16 MFMA peak"
METRIC_PADDED = "attention TFLOP/s over real keys (4·h·n_q·Σ_b kv_len[b]·d_k) at h=8,d_k=64; % of bf16 MFMA peak"
METRIC_ENC = "encoder layer TFLOP/s (projections, attention, W^O, FFN) at d_model=512,h=8,d_ff=2048; % of bf16 MFMA peak"
METRIC_MHA = ("multi-head attention TFLOP/s (Q/K/V projections + attention + W^O) at d_model={d_model},h={h}; % of bf16 "
              "MFMA peak")
METRIC_BWD = "attention backward TFLOP/s (10·B·h·n_q·n_k·d_k) at h={h},d_k={d_k}; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector (the fp32 path runs on the VALU)
PROFILES = ROOT / "profiles"


def flops_metric(w):
    return 4.0 * w["B"] * w["h"] * w["n_q"] * w["n_k"] * w["d_k"]


def _pairs(w):
    # causal: only the n(n+1)/2 allowed (query, key) pairs do work
    return w["n_q"] * (w["n_q"] + 1) / 2 if w["causal"] else w["n_q"] * w["n_k"]


def flops_algorithmic(w):
    return 2.0 * w["B"] * w["h"] * _pairs(w) * (w["d_k"] + w["d_v"])


def flops_window(w):
    """4 * B * h * (allowed (query, key) pairs) * d_k for a band of radius w around each query."""
    n, r = w["n_q"], w["window"]
    pairs = sum(min(n - 1, i + r) - max(0, i - r) + 1 for i in range(n))
    return 4.0 * w["B"] * w["h"] * pairs * w["d_k"]


def flops_padded(w):
    # only (query, real key) pairs: 4 * h * n_q * sum_b kv_len[b] * d_k
    return 4.0 * w["h"] * w["n_q"] * sum(min(max(L, 0), w["n_k"]) for L in w["kv_len"]) * w["d_k"]


def flops_encoder(w):
    """Products of one encoder layer: Q/K/V and W^O projections, attention (4 n^2 d per head), FFN (two GEMMs)."""
    M, d, ff = w["B"] * w["n_q"], w["d_model"], w["d_ff"]
    return (2.0 * M * d * 3 * d + 4.0 * w["B"] * w["h"] * w["n_q"] * w["n_k"] * w["d_k"] + 2.0 * M * d * d
            + 4.0 * M * d * ff)


def flops_mha(w):
    """Products of mha_forward: Q/K/V projections, attention (4 n_q n_k d_k per head), W^O."""
    Mq, Mk, d = w["B"] * w["n_q"], w["B"] * w["n_k"], w["d_model"]
    return (2.0 * Mq * d * d + 4.0 * Mk * d * d + 4.0 * w["B"] * w["h"] * w["n_q"] * w["n_k"] * w["d_k"]
            + 2.0 * Mq * d * d)


def flops_metric_bwd(w):
    return 10.0 * w["B"] * w["h"] * w["n_q"] * w["n_k"] * w["d_k"]


def flops_algorithmic_bwd(w):
    # S = Q K^T, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q over the allowed pairs
    return 2.0 * w["B"] * w["h"] * _pairs(w) * (3 * w["d_k"] + 2 * w["d_v"])


def hbm_bytes_bwd(w):
    # read Q, K, V, O, dO (and lse); write dQ, dK, dV. O is the float32 output of the training forward pass (the
    # operand D = dO . O is formed from), 4 bytes an element in both dtypes.
    es = 2 if w["dtype"] == "bf16" else 4
    nq, nk = w["n_q"], w["n_k"]
    return w["B"] * w["h"] * (es * (3 * nq * w["d_k"] + 4 * nk * w["d_k"]) + 4 * nq * w["d_v"] + 4 * nq)


def hbm_bytes(w):
    es = 2 if w["dtype"] == "bf16" else 4
    return es * w["B"] * w["h"] * (w["n_q"] * w["d_k"] + w["n_k"] * (w["d_k"] + w["d_v"]) + w["n_q"] * w["d_v"])


KERNEL_SOURCES = ("transformer_head_scaled_02_amd/csrc/attn_fwd_bf16.hip",
                  "transformer_head_scaled_02_amd/csrc/attn_fwd_pp_bf16.hip",
                  "transformer_head_scaled_02_amd/csrc/attn_tile.h",
                  "transformer_head_scaled_02_amd/csrc/device_common.h")


def kernel_source_hash() -> str:
    """Hash of the kernel's code: comments and blank lines do not count, so a comment edit keeps the counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        text = re.sub(r"//[^\n]*", "", (ROOT / rel).read_text())
        h.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary for this workload's attention kernel, or None
    when there is none or the kernel source has changed since the counters were taken."""
    f = PROFILES / f"{workload}_hbm_traffic.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


PREWARM = {"ms": 0.0, "calls": 0}


def prewarm(step, ms: float):
    """Untimed calls for about `ms` milliseconds before the warm-up steps. Coming out of idle, the GPU raises its
    clock over the first few milliseconds of load (measured: the first 50 back-to-back long-sequence calls averaged
    161 us per call, the same calls a few milliseconds later 135 us), so a handful of warm-up calls still falls in
    that ramp; this brings the chip to the state a sustained workload runs in. Recorded in the output line."""
    import torch
    if ms <= 0:
        return
    t0 = time.perf_counter()
    calls = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        calls += 8
        torch.cuda.synchronize()
    PREWARM["ms"] = round((time.perf_counter() - t0) * 1e3, 1)
    PREWARM["calls"] += calls


def time_steps(step, steps: int, warmup: int, stream, prewarm_ms: float = 0.0):
    """Untimed pre-warm (about `prewarm_ms` milliseconds of calls), W untimed warm-up calls, then exactly K calls
    timed with HIP events recorded on `stream` (the stream the library launches on), bracketed by device
    synchronisation. Returns (ms per call, wall seconds of the region)."""
    import torch
    prewarm(step, prewarm_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def graph_replay(step, out, calls: int, loops: int = 7):
    """Short calls replayed from a HIP graph: `calls` back-to-back calls of `step` captured once (on a side stream,
    after eager warm-up calls there), the graph replayed `loops` times with HIP events around each replay, the output
    compared bitwise with the eager result after every replay. Host launch cost then no longer sits between the
    kernels, so the per-call time is the device-side figure. The entry points make no allocation, memset or
    synchronisation, which is what capture needs. Returns a dict, or None when calls <= 0."""
    import statistics

    import torch
    if calls <= 0:
        return None
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_call, same = [], True
    for _ in range(loops + 1):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) / calls)
        same = same and torch.equal(out, want)
    del g
    per_call = per_call[1:]  # the first replay also uploads the graph
    return {"calls_per_graph": calls, "loops": loops, "median_ms": round(statistics.median(per_call), 6),
            "min_ms": round(min(per_call), 6), "bitwise_equal_to_eager": bool(same)}


def repeat_median(step, stream, ms_hint: float, loops: int, min_ms: float = 5.0):
    """`loops` more timed loops after the main region, each of N back-to-back calls lasting at least `min_ms`; the
    median over loops of the per-call time is the steady-state figure (the main region's K calls can be too short to
    average out the clock ramp)."""
    import statistics

    import torch
    if loops <= 0:
        return None
    n = max(1, int(-(-min_ms // max(ms_hint, 1e-4))))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_call = []
    for _ in range(loops):
        e0.record(stream)
        for _ in range(n):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) / n)
    return {"loops": loops, "calls_per_loop": n, "median_ms": round(statistics.median(per_call), 5),
            "min_ms": round(min(per_call), 5), "max_ms": round(max(per_call), 5)}


def smi_snapshot():
    """Clock, power and temperature readings of the GPU as amd-smi (else rocm-smi) reports them, flattened to a few
    key/value pairs; None when neither tool answers. Best effort: the measurement does not depend on it."""
    import re
    import subprocess
    want = re.compile(r"(gfx|sclk|clk|clock|power|temp|hotspot|edge)", re.I)
    for cmd in (["amd-smi", "metric", "--clock", "--power", "--temperature", "--json"],
                ["rocm-smi", "--showclocks", "--showpower", "--showtemp", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            data = json.loads(r.stdout)
        except Exception:
            continue
        flat = {}

        def walk(x, path):
            if len(flat) >= 24:
                return
            if isinstance(x, dict):
                for k, v in x.items():
                    walk(v, f"{path}.{k}" if path else str(k))
            elif isinstance(x, list):
                for i, v in enumerate(x[:2]):
                    walk(v, f"{path}[{i}]")
            elif want.search(path) and x not in (None, "", "N/A"):
                flat[path] = x
        walk(data, "")
        if flat:
            return {"tool": cmd[0], "readings": flat}
    return None


def smi_under_load(step, seconds: float = 2.0):
    """An smi snapshot taken while `step` runs back to back (at least `seconds`, at most 30 s, until the snapshot is
    in): the clock the chip holds under this load, not at idle. Best effort, like smi_snapshot."""
    import threading

    import torch
    res = {}

    def sample():
        time.sleep(0.5)  # let the load settle first
        res["snap"] = smi_snapshot()

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0 < seconds or th.is_alive()) and time.perf_counter() - t0 < 30.0:
        for _ in range(64):
            step()
        torch.cuda.synchronize()
    th.join(timeout=30)
    return res.get("snap")


def host_cores():
    """What the CPU baseline could use: logical CPUs, the ones this process may run on, and the BLAS threads."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"os_cpu_count": os.cpu_count(), "affinity": _AFFINITY, "blas_threads": blas,
            "env": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}}


def copy_calibration(nbytes: int = 512 << 20, reps: int = 3):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline(w, x, budget_s: float):
    """Time the float64 oracle on whole heads of the same workload until about `budget_s` seconds are spent."""
    import numpy as np

    from oracle import sdpa_head
    host = host_cores()
    threads = host["blas_threads"] or int(os.environ.get("OMP_NUM_THREADS", _AFFINITY))
    Q, K, V = x["Q"].f64, x["K"].f64, x["V"].f64
    heads = [(b, hh) for b in range(w["B"]) for hh in range(w["h"])]
    done, t_total = 0, 0.0
    sdpa_head(Q[0, 0, :64], K[0, 0], V[0, 0], False)  # warm
    # whole heads, cycling over the workload's heads until the time budget is spent
    while t_total < budget_s:
        b, hh = heads[done % len(heads)]
        t0 = time.perf_counter()
        o = sdpa_head(Q[b, hh], K[b, hh], V[b, hh], w["causal"])
        t_total += time.perf_counter() - t0
        done += 1
        assert np.isfinite(o).all()
    per_head = flops_metric(w) / (w["B"] * w["h"])
    rec = {"value": per_head * done / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "host": host, "kind": "oracle",
           "sample": f"{done} head evaluations over the workload's {len(heads)} heads ({w['n_q']}x{w['n_k']} "
                     f"scores each, float64 NumPy), {t_total:.1f} s"}
    if w["n_q"] * w["n_k"] <= 4096 and w["B"] * w["h"] <= 64:
        # tiny heads (the fp32 single-head case): the pure-Python literal definition as well, one thread
        from oracle import sdpa_brute
        reps, tb = 0, 0.0
        while tb < min(2.0, budget_s):
            b, hh = heads[reps % len(heads)]
            t0 = time.perf_counter()
            sdpa_brute(Q[b, hh], K[b, hh], V[b, hh], w["causal"])
            tb += time.perf_counter() - t0
            reps += 1
        rec["brute_force"] = {"value": per_head * reps / tb / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"{reps} head evaluations of the pure-Python definition, {tb:.1f} s"}
    return rec


def cpu_baseline_bwd(w, x, budget_s: float):
    """Time the float64 oracle's backward pass on whole heads until about `budget_s` seconds are spent."""
    import numpy as np

    from oracle import sdpa_backward_head
    host = host_cores()
    threads = host["blas_threads"] or int(os.environ.get("OMP_NUM_THREADS", _AFFINITY))
    heads = [(b, hh) for b in range(w["B"]) for hh in range(w["h"])]
    done, t_total = 0, 0.0
    sdpa_backward_head(x["Q"].f64[0, 0, :64], x["K"].f64[0, 0, :64], x["V"].f64[0, 0, :64], x["dO"].f64[0, 0, :64])
    while t_total < budget_s:
        b, hh = heads[done % len(heads)]
        t0 = time.perf_counter()
        g = sdpa_backward_head(*(x[n].f64[b, hh] for n in ("Q", "K", "V", "dO")), w["causal"])
        t_total += time.perf_counter() - t0
        done += 1
        assert all(np.isfinite(a).all() for a in g)
    per_head = flops_metric_bwd(w) / (w["B"] * w["h"])
    return {"value": per_head * done / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "host": host, "kind": "oracle",
            "sample": f"{done} head backward evaluations over the workload's {len(heads)} heads ({w['n_q']}x{w['n_k']}"
                      f" scores each, float64 NumPy), {t_total:.1f} s"}


def bench_backward(args, w, x, m, dev):
    """Time sdpa_backward (three launches per step) on the workload; returns the JSON record."""
    import numpy as np
    import torch

    from oracle import sdpa_backward_head
    q, k, v, do = (dev(x[n]) for n in ("Q", "K", "V", "dO"))
    mask = "causal" if w["causal"] else "none"
    # the training path: the forward keeps its float32 output, from which the backward forms D = dO . O
    out, out32, lse = m.sdpa_forward_train(q, k, v, mask)
    o_for_d = out32 if out32 is not None else out
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.sdpa_backward_workspace_size(w["B"], w["h"], w["n_q"], w["n_k"], w["d_k"], w["d_v"]),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        m.sdpa_backward(q, k, v, o_for_d, do, lse, mask=mask, dq=dq, dk=dk, dv=dv, workspace=ws)

    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)

    # parity of the last timed step on one whole head (float64 oracle, same inputs)
    ref = sdpa_backward_head(*(x[n].f64[0, 0] for n in ("Q", "K", "V", "dO")), w["causal"])
    errs = {}
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        d = np.abs(g[0, 0].float().cpu().numpy().astype(np.float64) - r)
        errs[name] = {"nrms": float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(r * r))),
                      "max_rel": float(d.max() / np.abs(r).max())}

    value = flops_metric_bwd(w) / (ms * 1e-3) / 1e12
    achieved = flops_algorithmic_bwd(w) / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC_BWD.format(h=w["h"], d_k=w["d_k"]), "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded N(0,1) Q/K/V/dO, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "h": w["h"], "n_q": w["n_q"], "n_k": w["n_k"],
                   "d_k": w["d_k"], "d_v": w["d_v"], "mask": mask},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "sdpa_backward step (attn_bwd_pre + " + ("attn_bwd_dkdv_pp_bf16 + attn_bwd_dq_pp_bf16)"
                                                                     if w["d_k"] == 64 else
                                                                     "attn_bwd_dkdv_bf16 + attn_bwd_dq_bf16)"),
                     "algorithmic_hbm_bytes": hbm_bytes_bwd(w),
                     "algorithmic_hbm_GBps": round(hbm_bytes_bwd(w) / (ms * 1e-3) / 1e9, 1)},
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step_head0": errs,
    }


def bench_window(args, w, x, m, dev):
    """Time sdpa_forward_window; returns the JSON record."""
    import numpy as np
    import torch

    from oracle import sdpa_ref
    q, k, v = dev(x["Q"]), dev(x["K"]), dev(x["V"])
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    def step():
        m.sdpa_forward_window(q, k, v, w["window"], out=out)

    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)
    rows = np.array([0, 1, 255, 256, 2047, w["n_q"] - 1])
    ref = sdpa_ref(x["Q"].f64[0, 0, rows], x["K"].f64[0, 0], x["V"].f64[0, 0], q_index=rows, window=w["window"])
    err = np.abs(out[0, 0, rows].float().cpu().numpy() - ref)
    value = flops_window(w) / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC_WINDOW, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded N(0,1) Q/K/V, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "h": w["h"], "n_q": w["n_q"], "n_k": w["n_k"],
                   "d_k": w["d_k"], "d_v": w["d_v"], "window": w["window"]},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_fwd_bf16<64, 4, 1, 2, 4, true>"},
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step": {"max_abs": float(err.max()), "mean_abs": float(err.mean())},
    }


def bench_padded(args, w, x, m, dev):
    """Time sdpa_forward_padded on a length-bucketed batch; returns the JSON record."""
    import numpy as np
    import torch

    from oracle import sdpa_ref
    q, k, v = dev(x["Q"]), dev(x["K"]), dev(x["V"])
    lens = torch.tensor(w["kv_len"], dtype=torch.int32, device="cuda")
    out = torch.empty(w["B"], w["h"], w["n_q"], w["d_v"], dtype=q.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    def step():
        m.sdpa_forward_padded(q, k, v, lens, out=out)

    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)
    got = out.float().cpu().numpy()
    rows = np.array([0, 1, 127, 128, 2047, w["n_q"] - 1])
    errs = []
    for b in range(w["B"]):
        L = w["kv_len"][b]
        ref = sdpa_ref(x["Q"].f64[b, 0, rows], x["K"].f64[b, 0, :L], x["V"].f64[b, 0, :L], q_index=rows)
        errs.append(np.abs(got[b, 0, rows] - ref))
    err = np.stack(errs)
    value = flops_padded(w) / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC_PADDED, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded N(0,1) Q/K/V, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "h": w["h"], "n_q": w["n_q"], "n_k": w["n_k"],
                   "d_k": w["d_k"], "d_v": w["d_v"], "mask": "none", "kv_len": w["kv_len"]},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": "attn_fwd_bf16<64, 4, 2, 2, 3, false>"},
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step": {"max_abs": float(err.max()), "mean_abs": float(err.mean())},
    }


def bench_mha(args, w, x, m, dev):
    """Time mha_forward (three launches per step: projections, attention, W^O); returns the JSON record."""
    import numpy as np
    import torch

    from oracle import mha_ref
    xq = dev(x["Xq"])
    ws_t = [dev(x[nm]) for nm in ("Wq", "Wk", "Wv", "Wo")]
    out = torch.empty_like(xq)
    work = torch.empty(m.mha_workspace_size(w["B"], w["n_q"], w["n_k"], w["h"], w["d_k"], w["d_v"]), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        m.mha_forward(xq, xq, *ws_t, h=w["h"], out=out, workspace=work)

    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)
    ref = mha_ref(x["Xq"].f64[:2], x["Xq"].f64[:2], *(x[nm].f64 for nm in ("Wq", "Wk", "Wv", "Wo")), h=w["h"])
    d = np.abs(out[:2].float().cpu().numpy() - ref)
    value = flops_mha(w) / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC_MHA.format(d_model=w["d_model"], h=w["h"]), "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded inputs and weights, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "n": w["n_q"], "d_model": w["d_model"], "h": w["h"],
                   "d_k": w["d_k"], "mask": "none"},
        "tokens_per_s": round(w["B"] * w["n_q"] / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "mha_forward step (3 launches)"},
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step_first2": {"max_abs": float(d.max()), "mean_abs": float(d.mean())},
    }


def bench_encoder(args, w, x, m, dev):
    """Time encoder_layer_forward (six launches per step at this shape); returns the JSON record."""
    import numpy as np
    import torch

    from oracle import encoder_layer_ref
    names = ("Wq", "Wk", "Wv", "Wo", "ln1_gamma", "ln1_beta", "W1", "b1", "W2", "b2", "ln2_gamma", "ln2_beta")
    X = dev(x["X"])
    ts = [dev(x[nm]) for nm in names]
    out = torch.empty_like(X)
    ws = torch.empty(m.encoder_layer_workspace_size(w["B"], w["n_q"], w["d_model"], w["h"], w["d_ff"]),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        m.encoder_layer_forward(X, *ts, h=w["h"], eps=w["eps"], out=out, workspace=ws)

    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)
    ref = encoder_layer_ref(x["X"].f64[:2], *(x[nm].f64 for nm in names), w["h"], w["eps"])
    d = np.abs(out[:2].float().cpu().numpy() - ref)
    value = flops_encoder(w) / (ms * 1e-3) / 1e12
    tokens = w["B"] * w["n_q"] / (ms * 1e-3)
    return {
        "metric": METRIC_ENC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded inputs and layer weights, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "n": w["n_q"], "d_model": w["d_model"], "h": w["h"],
                   "d_ff": w["d_ff"], "mask": "none"},
        "tokens_per_s": round(tokens, 1),
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "encoder_layer_forward step (7 launches)"},
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step_first2": {"max_abs": float(d.max()), "mean_abs": float(d.mean())},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sdpa_bf16_b4_h8_n4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the measured-ceiling microbenchmarks")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--repeats", type=int, default=7,
                    help="timed loops of >= 5 ms each after the main region (their median is reported too)")
    ap.add_argument("--rotate-mb", type=float, default=0.0,
                    help="also time the call cycling over input/output copies totalling more than this many MiB")
    ap.add_argument("--no-smi", action="store_true", help="skip the amd-smi clock/power snapshots")
    ap.add_argument("--graph-below-ms", type=float, default=0.05,
                    help="calls shorter than this are also timed replayed from a HIP graph (graph_replay)")
    ap.add_argument("--sustain-s", type=float, default=2.0,
                    help="after the timed region, seconds of held load whose last calls are timed again (reported "
                         "beside the value)")
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="untimed calls for about this many milliseconds before the warm-up steps (the GPU's clock "
                         "ramps up over the first milliseconds of load)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path here is a single-GPU kernel library "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_head_scaled_02_amd as m
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    m.load_library()
    w = workloads.WORKLOADS[args.workload]
    if w["kind"] not in ("sdpa", "sdpa_bwd", "sdpa_padded", "sdpa_window", "encoder", "mha"):
        raise SystemExit("unknown bench workload kind")
    x = workloads.make_workload(args.workload)

    def dev(q):
        if q.dtype == "bf16":
            return torch.from_numpy(q.raw.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(q.raw).cuda()

    if w["kind"] == "sdpa_window":
        print(json.dumps(bench_window(args, w, x, m, dev)), flush=True)
        return
    if w["kind"] == "mha":
        print(json.dumps(bench_mha(args, w, x, m, dev)), flush=True)
        return
    if w["kind"] == "encoder":
        print(json.dumps(bench_encoder(args, w, x, m, dev)), flush=True)
        return
    if w["kind"] == "sdpa_padded":
        print(json.dumps(bench_padded(args, w, x, m, dev)), flush=True)
        return
    if w["kind"] == "sdpa_bwd":
        rec = bench_backward(args, w, x, m, dev)
        if not args.no_cpu_baseline:
            rec["cpu_baseline"] = cpu_baseline_bwd(w, x, args.cpu_budget)
        print(json.dumps(rec), flush=True)
        return

    q, k, v = dev(x["Q"]), dev(x["K"]), dev(x["V"])
    out = torch.empty(w["B"], w["h"], w["n_q"], w["d_v"], dtype=q.dtype, device="cuda")
    mask = "causal" if w["causal"] else "none"
    stream = torch.cuda.current_stream()

    def step():
        m.sdpa_forward(q, k, v, mask=mask, out=out)

    smi_before = None if args.no_smi else smi_snapshot()
    ms, wall = time_steps(step, args.steps, args.warmup, stream, args.prewarm_ms)
    reps = repeat_median(step, stream, ms, args.repeats)
    smi_load = None if args.no_smi else smi_under_load(step)

    # parity of the last timed output on sampled rows (float64 oracle, same inputs)
    from oracle import sdpa_ref
    got = out.float().cpu().numpy()
    rows = np.unique(np.array([0, 1, 127, 128, 2047, w["n_q"] - 1]).clip(0, w["n_q"] - 1))
    ref = np.stack([sdpa_ref(x["Q"].f64[b, hh, rows], x["K"].f64[b, hh], x["V"].f64[b, hh], w["causal"], q_index=rows)
                    for b, hh in ((0, 0), (w["B"] - 1, w["h"] - 1))])
    err = np.abs(np.stack([got[0, 0, rows], got[-1, -1, rows]]) - ref)

    # Cold-ish: the same calls cycling over copies of the inputs and outputs whose total exceeds --rotate-mb, so
    # that a call's operands have left the 256 MB last-level cache by the time they come round again.
    cold = None
    if args.rotate_mb > 0:
        per_set = hbm_bytes(w)
        nsets = min(1024, max(2, -(-int(args.rotate_mb * 2**20) // per_set)))
        sets = [(q.clone(), k.clone(), v.clone(), torch.empty_like(out)) for _ in range(nsets)]
        it = [0]

        def step_cold():
            qq, kk, vv, oo = sets[it[0] % nsets]
            it[0] += 1
            m.sdpa_forward(qq, kk, vv, mask=mask, out=oo)

        for _ in range(nsets):
            step_cold()
        torch.cuda.synchronize()
        rc = repeat_median(step_cold, stream, ms, max(args.repeats, 3), min_ms=max(5.0, 2.0 * nsets * ms))
        cold = {"buffer_sets": nsets, "bytes_cycled": nsets * per_set, **rc,
                "algorithmic_hbm_GBps": round(per_set / (rc["median_ms"] * 1e-3) / 1e9, 1)}
        del sets

    value = flops_metric(w) / (ms * 1e-3) / 1e12
    achieved = flops_algorithmic(w) / (ms * 1e-3) / 1e12
    # the roofline that bounds this shape: the matrix core when its arithmetic intensity (algorithmic FLOPs per
    # algorithmic byte) is above the ridge of the bf16 peak over the HBM peak, HBM otherwise
    intensity = flops_algorithmic(w) / hbm_bytes(w)
    dtype_peak = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_F32_TFLOPS
    if w["dtype"] != "bf16":
        kernel = f"attn_fwd_f32<{w['d_k']}>"
    elif w["d_k"] == 64 and not w["causal"] and w["n_q"] >= 512:
        kernel = "attn_fwd_pp_bf16 (eight-wave ping-pong)"
    else:
        kernel = f"attn_fwd_bf16<{w['d_k']}, ...>"
    traffic = measured_traffic(args.workload) if w["dtype"] == "bf16" else None
    if intensity * PEAK_HBM_GBS * 1e9 / 1e12 >= dtype_peak:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": dtype_peak, "unit": "TFLOP/s",
                "frac": round(achieved / dtype_peak, 4)}
    else:
        gbps = hbm_bytes(w) / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": traffic, "kernel_source_hash": kernel_source_hash(), "kernel": kernel,
                 "algorithmic_flops": flops_algorithmic(w), "algorithmic_hbm_bytes": hbm_bytes(w),
                 "arithmetic_intensity": round(intensity, 1),
                 "algorithmic_TFLOPs": round(achieved, 2),
                 "algorithmic_hbm_GBps": round(hbm_bytes(w) / (ms * 1e-3) / 1e9, 1)})
    rec = {
        "metric": METRIC.format(h=w["h"], d_k=w["d_k"]), "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic (seeded N(0,1) Q/K/V, no dataset)",
        "config": {"workload": args.workload, "B": w["B"], "h": w["h"], "n_q": w["n_q"], "n_k": w["n_k"],
                   "d_k": w["d_k"], "d_v": w["d_v"], "mask": mask},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "wall_s_timed_region": round(wall, 4),
        "timing_repeats": reps,
        "prewarm": dict(PREWARM),
        "parity_last_step": {"max_abs": float(err.max()), "mean_abs": float(err.mean())},
        "gpu_state": {"before": smi_before, "under_load": smi_load},
    }
    if reps is not None:
        rec["value_at_repeat_median"] = round(flops_metric(w) / (reps["median_ms"] * 1e-3) / 1e12, 2)
    if args.sustain_s > 0:
        # held load: calls back to back for sustain_s seconds, the last >= 5 ms of them timed (the clock a long run
        # settles at, warmth included)
        import torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.sustain_s:
            for _ in range(16):
                step()
            torch.cuda.synchronize()
        last = repeat_median(step, stream, ms, 1)
        rec["sustained"] = {"seconds": args.sustain_s, "ms_per_call_at_end": last["median_ms"],
                            "value_at_end": round(flops_metric(w) / (last["median_ms"] * 1e-3) / 1e12, 2)}
    if cold is not None:
        rec["cold"] = cold
    if ms < args.graph_below_ms:
        # launch-bound sizes: the same calls replayed from a HIP graph, the device-side per-call time
        gr = graph_replay(step, out, max(1, int(2.0 / max(ms, 1e-3))))
        gr["algorithmic_hbm_GBps"] = round(hbm_bytes(w) / (gr["median_ms"] * 1e-3) / 1e9, 1)
        rec["graph_replay"] = gr
    if not args.no_probes:
        # measured ceilings on this chip, taken after the timed region: dense bf16 MFMA throughput with every CU busy
        # (and the clock it holds under that load), the v_exp_f32 rate and device-to-device copy bandwidth
        tf, ghz = m.probe_mfma_bf16(iters=20000)
        rate, ghz_e = m.probe_exp_f32(iters=4000)
        lds_row, _ = m.probe_lds_read(False, iters=20000)
        lds_tr, _ = m.probe_lds_read(True, iters=20000)
        gbps = m.probe_hbm_copy(nbytes=1 << 30, reps=5)
        rec["measured_ceilings"] = {"mfma_bf16_tflops": round(tf, 1), "mfma_clock_ghz": round(ghz, 3),
                                    "exp2_per_clock_per_cu": round(rate, 2), "exp_clock_ghz": round(ghz_e, 3),
                                    "lds_read_bytes_per_clock_per_cu": {"ds_read_b128": round(lds_row, 1),
                                                                        "ds_read_b64_tr_b16": round(lds_tr, 1)},
                                    "hbm_copy_GBps": round(gbps, 1)}
        rec["pct_of_measured_mfma_ceiling"] = round(100 * value / tf, 2)
        # the second ceiling of the softmax: one exp2 per visible score against the chip's measured v_exp_f32 rate
        # (per CU per clock, at the clock it held under that probe, times the 256 CUs)
        exps = w["B"] * w["h"] * _pairs(w) / (ms * 1e-3)
        ceiling = rate * 256 * ghz_e * 1e9
        rec["exp_throughput"] = {"exp_per_s": round(exps / 1e12, 3), "measured_ceiling_per_s": round(ceiling / 1e12, 3),
                                 "unit": "1e12 exp2/s", "frac": round(exps / ceiling, 4),
                                 "count": "one exp2 per visible (query, key) score"}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
