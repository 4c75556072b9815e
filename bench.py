#!/usr/bin/env python3
"""Benchmark of the group-shared low-rank corrected W4A16 linear path on one MI355X.

A step is one pass of the whole path over one batch: the 32-layer LLaMA-2-7B-shaped decoder's
linear units (per layer the QKV group, the o_proj solo, the gate/up group and the down_proj solo)
at decode T = 1, rank 64, with the restore mask switching the correction on in 16 of the 32
layers (chosen beforehand by the library's GlowQ-S selection: g_ner of every layer and the
budgeted top-k with the layer-order fallback), run through one glowq_path_forward call.  Inputs
and weights are seeded synthetic data generated on the GPU and resident in HBM before the timed
region.

The JSON line also carries the dominant kernel's roofline (the fused decode kernel, measured with
HIP events on the launch stream), the fp64 CPU oracle timed on a bounded sample, and extra
measurements: the prefill pass (T = 512), the QKV decode group alone (T = 1, HBM TB/s) and the
gate/up prefill group (T = 2048, matrix-core TFLOP/s), plus the layerwise baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "corrected-W4 group fwd: tokens/s, HBM TB/s (T=1), MFMA TFLOP/s (T=2048)"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work
def unit_bytes(T, d, n_outs, r, restore, n_proj=1):
    """Bytes the path must move for one unit: packed W + (s, z), A_i and B once (or once per
    module for the layerwise form), X once, Y in fp16."""
    so = sum(n_outs)
    b = so * d // 2 + so * (d // 128) * 4 + T * d * 2 + T * so * 2
    if restore and r > 0:
        b += so * r * 2 + n_proj * r * d * 2
    return b


def unit_flops(T, d, n_outs, r, restore, n_proj=1):
    so = sum(n_outs)
    f = 2 * T * d * so
    if restore and r > 0:
        f += n_proj * 2 * T * d * r + 2 * T * r * so
    return f


# ------------------------------------------------------------------ workload on the GPU
# GlowQ-S fallback: layers whose g_ner lies within this fraction of the best score (in steps of it)
# count as equal and are taken in layer order
RESTORE_REL_TOL = 0.01


def select_path_mask(g, device, k=16, rel_tol=RESTORE_REL_TOL):
    """The path's restore set chosen by the library on the GPU (GlowQ-S): g_ner of every layer's
    seven modules (their fp16 weights regenerated, and the INT4-g128 form the path runs), then the
    budgeted top-k of the layers with the layer-order fallback for scores within rel_tol steps."""
    import torch
    import workload as W
    L = W.LLAMA2_7B["n_layers"]
    sums = torch.empty(L, 7, 2, dtype=torch.float64, device=device)
    ws = None
    for l in range(L):
        mods = [(w, g.QWeight.from_workload(W.rtn_quantize(w), device=device)) for w in W.llama2_path_weights(l, device)]
        if ws is None:
            ws = torch.empty(g.ner_workspace_bytes_batch([qw.n_out for _, qw in mods]), dtype=torch.uint8,
                             device=device)
        g.ner_sums_batch(mods, out=sums[l], workspace=ws)
        del mods
    scores, mask = g.restore_select(sums, k, rel_tol)
    torch.cuda.synchronize()
    return [bool(v) for v in mask.cpu()], [float(v) for v in scores.cpu()]


def build_path(T, device, keep_layers=(), layerwise=False, mask=None):
    import torch
    import workload as W
    from rank_error_compensation_amd import glowq as g

    units, descr, keep = [], [], {}
    t0 = time.time()
    for l in range(W.LLAMA2_7B["n_layers"]):
        layer_units, mask = W.llama2_path_inputs(T, device=device, layers=[l], layerwise=layerwise, mask=mask)
        for u in layer_units[l]:
            qws = [g.QWeight.from_workload(q, device=device) for q in u.weights]
            ys = [torch.empty(T, q.n_out, dtype=torch.float16, device=device) for q in u.weights]
            kind = g.UNIT_GROUP if u.kind == "group" else g.UNIT_SOLO
            pu = g.PathUnit(kind, u.x, qws, u.b, u.a, u.r, u.restore, ys)
            pu.b_layerwise = u.b_layerwise
            units.append(pu)
            descr.append((u.name, T, u.d, u.n_outs, u.r, u.restore))
        if l in keep_layers:
            keep[l] = layer_units[l]
        else:
            del layer_units
    torch.cuda.synchronize()
    log(f"[bench] built T={T} path: {len(units)} units in {time.time() - t0:.1f}s")
    return units, descr, mask, keep


def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graphed(fn):
    """fn's launches captured once in a HIP graph (torch's graph API on a side stream)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    torch.cuda.synchronize()
    return gr


def call_unit(u, g, ws, layerwise=False):
    if layerwise and u.kind == g.UNIT_GROUP:
        return g.layerwise_forward(u.x, u.weights, u.b_layerwise, u.a, u.r, u.restore, workspace=ws, y=u.y)
    if u.kind == g.UNIT_SOLO:
        return g.solo_forward(u.x, u.weights[0], u.b, u.a[0], u.r, u.restore, workspace=ws, y=u.y[0])
    return g.group_forward(u.x, u.weights, u.b, u.a, u.r, u.restore, workspace=ws, y=u.y)


def per_launch_events(units, descr, g, reps, layerwise=False):
    """Average device time of each unit's launch, from HIP events recorded on the launch stream
    around every call (one kernel per decode call)."""
    import torch
    n_proj = max(len(u.weights) for u in units) if layerwise else 1
    ws = g.make_workspace(max(u.x.shape[0] for u in units), max(u.r for u in units), n_proj)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in units]
    tot = [0.0] * len(units)
    for _ in range(2):
        for u in units:
            call_unit(u, g, ws, layerwise)
    torch.cuda.synchronize()
    for _ in range(reps):
        for (e0, e1), u in zip(ev, units):
            e0.record(stream)
            call_unit(u, g, ws, layerwise)
            e1.record(stream)
        torch.cuda.synchronize()
        for i, (e0, e1) in enumerate(ev):
            tot[i] += e0.elapsed_time(e1) * 1e-3
    return [t / reps for t in tot]


# ------------------------------------------------------------------ measured HBM traffic
def source_digest():
    """sha256 over the decode kernel's sources: counter readings are only valid for this code."""
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "handoff.h", "glowq_internal.h"):
        with open(os.path.join(ROOT, "rank_error_compensation_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None when the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "decode_path_T1_counters.txt")
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if line.startswith("traffic_bytes_per_launch=") or line.startswith("source_sha256="):
                    k, v = line.strip().split("=", 1)
                    kv[k] = v
        if kv.get("source_sha256") != source_digest():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline(keep, mask):
    """The fp64 oracle on a bounded sample of the same workload: one restored and one
    unrestored layer of the T = 1 path (weights copied from the GPU), scaled to 32 layers."""
    from oracle import glowq_ref as G
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info] + [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info
                                 if i.get("user_api") == "blas"})) or "unknown"
    except Exception:
        blas_threads, blas = 1, "unknown"
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    import torch
    t_layers = []
    for l, units in keep.items():
        cpu_units = []
        for u in units:
            for q in u.weights:
                q.q_packed = q.q_packed.cpu()
                q.s = q.s.cpu()
                q.z = q.z.cpu()
            u.x = u.x.cpu()
            u.a = [a.cpu() for a in u.a]
            u.b = u.b.cpu()
            cpu_units.append(u)
        t0 = time.perf_counter()
        G.path_forward({l: cpu_units}, mask)
        t_layers.append(time.perf_counter() - t0)
    t_pair = sum(t_layers)
    per_token = t_pair * (32 / len(t_layers))
    return {"value": round(1.0 / per_token, 4), "unit": "tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle on layers {sorted(keep)} (restored {[bool(mask[l]) for l in sorted(keep)]}) "
                      f"of the T=1 path, {t_pair:.1f}s, scaled x{32 // len(t_layers)} to the 32-layer step; "
                      f"BLAS {blas}, {blas_threads} threads; host: os.cpu_count() {os.cpu_count()}, "
                      f"{usable} usable by this process; dequantisation single-threaded numpy"}


# ------------------------------------------------------------------ extra measurements
def rotating_group(T, copies, g, device):
    """LLaMA-2-7B QKV group (d = 4096, 3 x 4096) with `copies` weight copies at distinct addresses (more than twice the
    256 MB last-level cache), cycled so that each call streams its weights from HBM."""
    import torch
    import workload as W
    u = W.llama2_qkv_unit(T, device=device)
    base = [g.QWeight.from_workload(q, device=device) for q in u.weights]
    sets = [base] + [[g.QWeight(w.q.clone(), w.sz.clone(), w.n_out, w.k_in, w.fmt) for w in base]
                     for _ in range(copies - 1)]
    a_sets = [u.a] + [[a.clone() for a in u.a] for _ in range(copies - 1)]
    ys = [torch.empty(T, w.n_out, dtype=torch.float16, device=device) for w in base]
    return u, sets, a_sets, ys


def extra_decode_qkv(g, T=1, reps=50):
    import torch
    copies = 20
    u, sets, a_sets, ys = rotating_group(T, copies, g, "cuda")
    ws = g.make_workspace(T, u.r)
    stream = torch.cuda.current_stream()
    for i in range(copies):
        g.group_forward(u.x, sets[i], u.b, a_sets[i], u.r, True, workspace=ws, y=ys)
    torch.cuda.synchronize()
    evs = []
    for k in range(reps * copies):
        i = k % copies
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.group_forward(u.x, sets[i], u.b, a_sets[i], u.r, True, workspace=ws, y=ys)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]
    t = statistics.median(ts)
    nb = unit_bytes(T, 4096, u.n_outs, u.r, True)
    return {"workload": f"llama2-7b QKV group decode T={T} r=64 (20 rotating weight copies)",
            "us_median": round(t * 1e6, 3), "tokens_per_s": round(T / t, 1),
            "alg_bytes": nb, "TB_per_s": round(nb / t / 1e12, 4), "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4)}


def extra_tiny_qkv(g, reps=200):
    """The tiny QKV group (d = 256, 3 x 256 outputs, T = 8, r = 16): a latency-bound launch.  Its
    correction factors are drawn as scaled Gaussians of the same shapes (their values do not change
    the launch)."""
    import torch
    import workload as W
    c = W.tiny_qkv_inputs(device="cuda")
    w = [g.QWeight.from_workload(q, device="cuda") for q in c["qw"]]
    a, b = W.gaussian_factors([q.n_out for q in c["qw"]], c["d"], c["r"], [q.err_sq for q in c["qw"]],
                              (0, 0, 0, 9), "cuda")
    ws = g.make_workspace(c["T"], c["r"])
    ys = [torch.empty(c["T"], q.n_out, dtype=torch.float16, device="cuda") for q in c["qw"]]
    stream = torch.cuda.current_stream()
    for _ in range(10):
        g.group_forward(c["x"], w, b, a, c["r"], True, workspace=ws, y=ys)
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.group_forward(c["x"], w, b, a, c["r"], True, workspace=ws, y=ys)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    t = statistics.median(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)
    return {"workload": "tiny QKV group d = 256, 3 x 256, T = 8, r = 16", "us_median": round(t * 1e6, 2),
            "tokens_per_s": round(c["T"] / t, 1)}


def extra_llama3(g, reps=10, min_bytes=600 << 20):
    """LLaMA-3.1-8B GQA units (QKV group 4096 -> 4096 + 1024 + 1024, gate/up group 4096 ->
    2 x 14336, solo down 14336 -> 4096) at T = 64 and 4096, r = 64 and 128: median time of one call
    between events; at T = 64 the call cycles over enough weight copies (>= 600 MB) that its
    weights stream from HBM."""
    import torch
    import workload as W
    stream = torch.cuda.current_stream()
    out = {}
    for r in (64, 128):
        for T in (64, 4096):
            units = W.llama3_gqa_units(T, r, device="cuda")
            for u in units:
                w0 = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
                wbytes = sum(w.q.numel() * w.q.element_size() + w.sz.numel() * w.sz.element_size() for w in w0)
                copies = max(1, -(-min_bytes // wbytes)) if T <= 64 else 1
                sets = [w0] + [[g.QWeight(w.q.clone(), w.sz.clone(), w.n_out, w.k_in, w.fmt) for w in w0]
                               for _ in range(copies - 1)]
                ws = g.make_workspace(T, r, 1)
                ys = [torch.empty(T, w.n_out, dtype=torch.float16, device="cuda") for w in w0]

                def call(i):
                    if u.kind == "solo":
                        g.solo_forward(u.x, sets[i][0], u.b, u.a[0], r, True, workspace=ws, y=ys[0])
                    else:
                        g.group_forward(u.x, sets[i], u.b, u.a, r, True, workspace=ws, y=ys)

                for i in range(copies):
                    call(i)
                torch.cuda.synchronize()
                evs = []
                for k in range(reps * copies):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    call(k % copies)
                    e1.record(stream)
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                t = statistics.median(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)
                nb = unit_bytes(T, u.d, u.n_outs, r, True)
                fl = unit_flops(T, u.d, u.n_outs, r, True)
                e = {"us": round(t * 1e6, 2), "tokens_per_s": round(T / t, 1),
                     "TB_per_s": round(nb / t / 1e12, 3), "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4),
                     "TFLOP_per_s": round(fl / t / 1e12, 1), "frac_mfma_f16_peak": round(fl / t / 1e12 / 2500.0, 4)}
                if copies > 1:
                    e["weight_copies"] = copies
                out[f"{u.name} T={T} r={r}"] = e
                del sets, w0, ws, ys
            del units
            torch.cuda.empty_cache()
    return out


def extra_prefill_gateup(g, reps=20):
    import torch
    import workload as W
    T = 2048
    u = W.llama2_gateup_unit(T, device="cuda", layerwise=True)
    w = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
    ws = g.make_workspace(T, u.r, 2)
    ys = [torch.empty(T, q.n_out, dtype=torch.float16, device="cuda") for q in w]
    stream = torch.cuda.current_stream()
    out = {}
    fns = (("group", lambda: g.group_forward(u.x, w, u.b, u.a, u.r, True, workspace=ws, y=ys)),
           ("layerwise", lambda: g.layerwise_forward(u.x, w, u.b_layerwise, u.a, u.r, True, workspace=ws, y=ys)))
    # the two are timed call by call, alternating, so that both see the same clock and power state
    # (the GEMM runs power-limited and the clock drifts over a run); median of the calls
    for _ in range(3):
        for _, fn in fns:
            fn()
    torch.cuda.synchronize()
    evs = {name: [] for name, _ in fns}
    for _ in range(reps):
        for name, fn in fns:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs[name].append((e0, e1))
    torch.cuda.synchronize()
    for name, _ in fns:
        t = statistics.median(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs[name])
        fl = unit_flops(T, 4096, u.n_outs, u.r, True, 1 if name == "group" else 2)
        out[name] = {"us": round(t * 1e6, 2), "tokens_per_s": round(T / t, 1),
                     "alg_TFLOP_per_s": round(unit_flops(T, 4096, u.n_outs, u.r, True) / t / 1e12, 2),
                     "frac_mfma_f16_peak": round(unit_flops(T, 4096, u.n_outs, u.r, True) / t / 1e12 / 2500.0, 4),
                     "flops_executed": fl}
    out["workload"] = "llama2-7b gate/up group prefill T=2048 r=64 (one call: projection + grouped GEMM)"
    return out


def paired_ci(fn_a, fn_b, trials=30, calls=10):
    """Interleaved paired timing of two call sequences on the launch stream: each trial times
    `calls` back-to-back calls of A and of B between HIP events, the order of the two alternating
    from trial to trial (clock and power drift cancel in the pairs).  Returns the per-call medians
    and the mean relative difference (B - A) / A per trial with its 95 % confidence interval
    (Student t over the trials); `significant` when the interval excludes zero."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn_a()
        fn_b()
    torch.cuda.synchronize()
    ta, tb = [], []
    for k in range(trials):
        order = ((fn_a, ta), (fn_b, tb)) if k % 2 == 0 else ((fn_b, tb), (fn_a, ta))
        for fn, acc in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                fn()
            e1.record(stream)
            e1.synchronize()
            acc.append(e0.elapsed_time(e1) * 1e3 / calls)
    rel = [(b - a) / a for a, b in zip(ta, tb)]
    n = len(rel)
    mean = sum(rel) / n
    sd = statistics.stdev(rel) if n > 1 else 0.0
    try:
        from scipy.stats import t as student_t
        q = float(student_t.ppf(0.975, n - 1))
    except Exception:
        q = 2.045
    half = q * sd / n ** 0.5
    return {"a_us_median": round(statistics.median(ta), 3), "b_us_median": round(statistics.median(tb), 3),
            "rel_diff_mean": round(mean, 5), "ci95": [round(mean - half, 5), round(mean + half, 5)],
            "significant": bool(mean - half > 0 or mean + half < 0), "trials": n, "calls_per_trial": calls}


def extra_group_vs_layerwise(g):
    """Group (one shared B, one projection) against layerwise (a B_i and a projection per module)
    on the same kernels at the same rank, paired interleaved trials with a 95 % CI of the relative
    difference (layerwise - group) / group: LLaMA-2-7B QKV decode T = 1 (rotating weight copies),
    gate/up prefill T = 2048, LLaMA-3.1-8B QKV at T = 64 (rotating copies) and gate/up at T = 4096."""
    import torch
    import workload as W
    out = {}
    # QKV decode, rotating copies so that the weights stream from HBM
    copies = 20
    u = W.llama2_qkv_unit(1, device="cuda", layerwise=True)
    base = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
    sets = [base] + [[g.QWeight(w.q.clone(), w.sz.clone(), w.n_out, w.k_in, w.fmt) for w in base] for _ in range(copies - 1)]
    ws = g.make_workspace(1, u.r, 3)
    ys = [torch.empty(1, w.n_out, dtype=torch.float16, device="cuda") for w in base]
    it = {"a": 0, "b": 0}

    def grp():
        it["a"] = (it["a"] + 1) % copies
        g.group_forward(u.x, sets[it["a"]], u.b, u.a, u.r, True, workspace=ws, y=ys)

    def lw():
        it["b"] = (it["b"] + 1) % copies
        g.layerwise_forward(u.x, sets[it["b"]], u.b_layerwise, u.a, u.r, True, workspace=ws, y=ys)

    out["qkv_decode_T1"] = paired_ci(grp, lw, trials=40, calls=20)
    del sets, base
    # gate/up prefill T = 2048
    u = W.llama2_gateup_unit(2048, device="cuda", layerwise=True)
    w = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
    ws = g.make_workspace(2048, u.r, 2)
    ys = [torch.empty(2048, q.n_out, dtype=torch.float16, device="cuda") for q in w]
    out["gateup_prefill_T2048"] = paired_ci(
        lambda: g.group_forward(u.x, w, u.b, u.a, u.r, True, workspace=ws, y=ys),
        lambda: g.layerwise_forward(u.x, w, u.b_layerwise, u.a, u.r, True, workspace=ws, y=ys), trials=30, calls=3)
    del w, ws, ys
    torch.cuda.empty_cache()
    # LLaMA-3.1-8B QKV (T = 64, rotating copies) and gate/up (T = 4096)
    for T, name in ((64, "qkv"), (4096, "gateup")):
        units = W.llama3_gqa_units(T, 64, device="cuda", layerwise=True, which=(name,))
        u = units[0]
        w0 = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
        ncp = 40 if T == 64 else 1
        sets = [w0] + [[g.QWeight(x.q.clone(), x.sz.clone(), x.n_out, x.k_in, x.fmt) for x in w0] for _ in range(ncp - 1)]
        ws = g.make_workspace(T, 64, len(w0))
        ys = [torch.empty(T, q.n_out, dtype=torch.float16, device="cuda") for q in w0]
        it = {"a": 0, "b": 0}

        def grp2():
            it["a"] = (it["a"] + 1) % ncp
            g.group_forward(u.x, sets[it["a"]], u.b, u.a, 64, True, workspace=ws, y=ys)

        def lw2():
            it["b"] = (it["b"] + 1) % ncp
            g.layerwise_forward(u.x, sets[it["b"]], u.b_layerwise, u.a, 64, True, workspace=ws, y=ys)

        out[f"llama3_{name}_T{T}"] = paired_ci(grp2, lw2, trials=30, calls=10 if T == 64 else 2)
        del sets, w0, ws, ys, units
        torch.cuda.empty_cache()
    out["how"] = ("a = group, b = layerwise; rel_diff = (layerwise - group) / group per trial; positive = group faster; "
                  "95 % Student-t interval over the trials")
    return out


def extra_w4a8(g, reps=20):
    """W4A8 (per-token int8 activations on the int8 matrix cores, fp16 correction): LLaMA-2-7B
    gate/up at T = 2048 (integer matrix-core ops against the 5.0 POP/s int8 peak) and QKV at
    T = 1 (HBM), with the W4A16 call of the same unit for comparison."""
    import torch
    import workload as W
    stream = torch.cuda.current_stream()
    out = {}
    for name, T, mk in (("gateup_T2048", 2048, W.llama2_gateup_unit), ("qkv_T1", 1, W.llama2_qkv_unit)):
        u = mk(T, device="cuda")
        w = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
        ws8 = torch.empty(g.w4a8_workspace_bytes(T, 4096, u.r), dtype=torch.uint8, device="cuda")
        ws16 = g.make_workspace(T, u.r, 1)
        ys = [torch.empty(T, q.n_out, dtype=torch.float16, device="cuda") for q in w]
        res = {}
        for tag, fn in (("w4a8", lambda: g.group_forward_w4a8(u.x, w, u.b, u.a, u.r, True, workspace=ws8, y=ys)),
                        ("w4a16", lambda: g.group_forward(u.x, w, u.b, u.a, u.r, True, workspace=ws16, y=ys))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t = statistics.median(ts)
            fl = unit_flops(T, 4096, u.n_outs, u.r, True)
            nb = unit_bytes(T, 4096, u.n_outs, u.r, True)
            e = {"us": round(t * 1e6, 2), "tokens_per_s": round(T / t, 1)}
            if T > 64:
                peak = 5000.0 if tag == "w4a8" else MFMA_F16_PEAK_TFLOPS
                e.update({"alg_TOP_per_s": round(fl / t / 1e12, 1), "peak_TOP_per_s": peak,
                          "frac_peak": round(fl / t / 1e12 / peak, 4)})
            else:
                e.update({"TB_per_s": round(nb / t / 1e12, 3), "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4)})
            res[tag] = e
        out[name] = res
        del w, ws8, ws16, ys
        torch.cuda.empty_cache()
    out["workload"] = "llama2-7b gate/up T=2048 and QKV T=1, r=64; W4A8 = int8 activation codes per token"
    return out


def mx_weight_bytes(fmt, n_outs, d):
    """Bytes of the quantised weights: INT4 codes + (z, s) pairs per 128 inputs, or MX codes
    (4 or 6 bits) + one scale byte per 32 inputs."""
    so = sum(n_outs)
    bits = {"int4": 4, "mxfp4": 4, "mxfp6_e2m3": 6, "mxfp6_e3m2": 6}[fmt]
    scale = so * (d // 128) * 4 if fmt == "int4" else so * (d // 32)
    return so * d * bits // 8 + scale


def extra_mx(g, reps=20, copies=20):
    """Microscaling weights (arXiv page, Table 13 datatypes) beside INT4-g128 on the same units:
    LLaMA-2-7B QKV decode at T = 1 (20 rotating weight copies, HBM-bound: algorithmic bytes with
    the format's own weight bytes) and gate/up prefill at T = 2048 (matrix-core bound)."""
    import torch
    import workload as W
    stream = torch.cuda.current_stream()
    out = {}
    for fmt in ("int4", "mxfp4", "mxfp6_e2m3"):
        res = {}
        u = W.llama2_qkv_unit(1, device="cuda", fmt=fmt)
        base = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
        sets = [base] + [[g.QWeight(w.q.clone(), w.sz.clone(), w.n_out, w.k_in, w.fmt) for w in base]
                         for _ in range(copies - 1)]
        ws = g.make_workspace(1, u.r)
        ys = [torch.empty(1, w.n_out, dtype=torch.float16, device="cuda") for w in base]
        for i in range(copies):
            g.group_forward(u.x, sets[i], u.b, u.a, u.r, True, workspace=ws, y=ys)
        torch.cuda.synchronize()
        evs = []
        for k in range(reps * copies):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.group_forward(u.x, sets[k % copies], u.b, u.a, u.r, True, workspace=ws, y=ys)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = statistics.median([e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs])
        nb = unit_bytes(1, 4096, u.n_outs, u.r, True) - mx_weight_bytes("int4", u.n_outs, 4096) + \
            mx_weight_bytes(fmt, u.n_outs, 4096)
        res["qkv_T1"] = {"us_median": round(t * 1e6, 3), "alg_bytes": nb, "TB_per_s": round(nb / t / 1e12, 4),
                         "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4)}
        if fmt in ("mxfp4", "mxfp6_e2m3"):
            ws8 = torch.empty(g.mx8_workspace_bytes(1, 4096, u.r), dtype=torch.uint8, device="cuda")
            for i in range(copies):
                g.group_forward_mx8(u.x, sets[i], u.b, u.a, u.r, True, workspace=ws8, y=ys)
            torch.cuda.synchronize()
            evs = []
            for k in range(reps * copies):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.group_forward_mx8(u.x, sets[k % copies], u.b, u.a, u.r, True, workspace=ws8, y=ys)
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            t8 = statistics.median([e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs])
            res["qkv_T1_x_mxfp8_activations"] = {"us_median": round(t8 * 1e6, 3), "TB_per_s": round(nb / t8 / 1e12, 4),
                                                 "frac_hbm_peak": round(nb / t8 / 1e12 / 8.0, 4)}
            del ws8
        del sets, base, ws, ys, u
        u = W.llama2_gateup_unit(2048, device="cuda", fmt=fmt)
        w = [g.QWeight.from_workload(q, device="cuda") for q in u.weights]
        ws = g.make_workspace(2048, u.r, 1)
        ys = [torch.empty(2048, q.n_out, dtype=torch.float16, device="cuda") for q in w]
        fn = graphed(lambda: g.group_forward(u.x, w, u.b, u.a, u.r, True, workspace=ws, y=ys)).replay
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = statistics.median(ts)
        fl = unit_flops(2048, 4096, u.n_outs, u.r, True)
        res["gateup_T2048"] = {"us_median": round(t * 1e6, 2), "TFLOP_per_s": round(fl / t / 1e12, 1),
                               "frac_mfma_f16_peak": round(fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        if fmt in ("mxfp4", "mxfp6_e2m3"):
            # the same weights against MXFP8 activations on the block-scaled matrix cores
            ws8 = torch.empty(g.mx8_workspace_bytes(2048, 4096, u.r), dtype=torch.uint8, device="cuda")
            fn8 = graphed(lambda: g.group_forward_mx8(u.x, w, u.b, u.a, u.r, True, workspace=ws8, y=ys)).replay
            for _ in range(3):
                fn8()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn8()
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t8 = statistics.median(ts)
            res["gateup_T2048_x_mxfp8_activations"] = {
                "us_median": round(t8 * 1e6, 2), "TFLOP_per_s": round(fl / t8 / 1e12, 1),
                "frac_mfma_fp8_peak": round(fl / t8 / 1e12 / 5000.0, 4),
                "how": "activations quantised to MXFP8 in the call, v_mfma_scale_f32_16x16x128_f8f6f4"}
            del ws8
        out[fmt] = res
        del w, ws, ys, u
        torch.cuda.empty_cache()
    out["workload"] = ("llama2-7b QKV T=1 (rotating copies) and gate/up T=2048, r=64, per weight format; "
                       "MX = OCP microscaling, 32-input blocks, E8M0 scales; x_mxfp8_activations = the same MX "
                       "weights against per-call MXFP8 activations (fp8 peak 5 PFLOP/s)")
    return out


def extra_moe(g, reps=10, copies=4):
    """Qwen1.5-MoE-A2.7B MLP: 60 experts, gate/up group 2048 -> 2 x 1408 and down 1408 -> 2048 per
    expert, top-4 routing, r = 64, one launch for all experts (plus the projection when
    correcting): per-expert shared basis and one basis for all experts, T = 1, 64 and 2048 tokens.
    Calls are captured in one HIP graph (32 at T <= 64, 4 at T = 2048, rotating over `copies` copies
    of every expert's weights and factors at T <= 64) and the graph's replay time is divided by their
    number, as the decode path spreads its graph launch over 128 launches. Bytes are the active experts' algorithmic bytes, flops the routed rows'."""
    import torch
    import workload as W
    stream = torch.cuda.current_stream()
    E, d, inter, r = 60, 2048, 1408, 64
    zx = lambda k: torch.zeros(1, k, dtype=torch.float16, device="cuda")
    gu = [W.make_unit(f"e{e}", "group", zx(d), [inter, inter], r, (0, 8, e), device="cuda") for e in range(E)]
    mods = [g.MoeModule.stack([g.QWeight.from_workload(u.weights[i]) for u in gu], [u.a[i] for u in gu])
            for i in range(2)]
    b_exp = torch.stack([u.b for u in gu]).contiguous()
    b_all = gu[0].b
    dn = [W.make_unit(f"d{e}", "solo", zx(inter), [d], r, (0, 9, e), device="cuda") for e in range(E)]
    dmods = [g.MoeModule.stack([g.QWeight.from_workload(u.weights[0]) for u in dn], [u.a[0] for u in dn])]
    db = torch.stack([u.b for u in dn]).contiguous()
    del gu, dn
    clone = lambda ms: [g.MoeModule(m.q.clone(), m.sz.clone(), None if m.a is None else m.a.clone(), m.n_out, m.k_in)
                        for m in ms]
    sets = [(mods, b_exp, dmods, db)] + [(clone(mods), b_exp.clone(), clone(dmods), db.clone())
                                         for _ in range(copies - 1)]

    def timed(calls, per_graph=32):
        # per_graph calls (rotating over the copies) captured in one graph, so that the graph's own
        # launch is spread over them as in the 128-launch decode path; median over replays / per_graph
        gr = graphed(lambda: [calls[k % len(calls)]() for k in range(per_graph)])
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return statistics.median(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs) / per_graph

    out = {}
    for T in (1, 64, 2048):
        nc = copies if T <= 64 else 1
        x = W.make_x(T, d, 0.77, (0, 10, T), device="cuda")
        rt, off = W.moe_routing(T, E, 4, (0, 10, T))
        rt, off = rt.cuda(), off.cuda()
        n = T * 4
        active = int((torch.diff(off) > 0).sum())
        ys = [torch.empty(n, inter, dtype=torch.float16, device="cuda") for _ in range(2)]
        res = {"routed_rows": n, "active_experts": active}
        for share, tag in ((0, "gateup_per_expert"), (1, "gateup_all_experts")):
            ws = g.make_workspace(1, 8, 1, min_bytes=g.moe_workspace_bytes(n, T, r, share))
            calls = [lambda c=c: g.moe_forward(x, E, sets[c][0], sets[c][1] if share == 0 else b_all, share, r, True, rt,
                                               off, n, workspace=ws, y=ys) for c in range(nc)]
            t = timed(calls, 32 if T <= 64 else 4)
            nb = active * unit_bytes(0, d, [inter, inter], r, True, 1 if share == 0 else 0) + (
                r * d * 2 if share == 1 else 0) + T * d * 2 + n * 2 * inter * 2
            fl = 2 * n * d * 2 * inter + (2 * n if share == 0 else 2 * T) * d * r + 2 * n * r * 2 * inter
            res[tag] = {"us": round(t * 1e6, 2), "tokens_per_s": round(T / t, 1),
                        "TB_per_s": round(nb / t / 1e12, 3), "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4),
                        "TFLOP_per_s": round(fl / t / 1e12, 1), "frac_mfma_f16_peak": round(fl / t / 1e12 / 2500.0, 4)}
            del calls, ws
        h = W.make_x(n, inter, 0.77, (0, 11, T), device="cuda")
        yd = [torch.empty(n, d, dtype=torch.float16, device="cuda")]
        ws = g.make_workspace(1, 8, 1, min_bytes=g.moe_workspace_bytes(n, n, r, 0))
        calls = [lambda c=c: g.moe_forward(h, E, sets[c][2], sets[c][3], 0, r, True, None, off, n, workspace=ws, y=yd)
                 for c in range(nc)]
        t = timed(calls, 32 if T <= 64 else 4)
        nb = active * unit_bytes(0, inter, [d], r, True) + n * inter * 2 + n * d * 2
        fl = 2 * n * inter * d + 2 * n * inter * r + 2 * n * r * d
        res["down_per_expert"] = {"us": round(t * 1e6, 2), "TB_per_s": round(nb / t / 1e12, 3),
                                  "frac_hbm_peak": round(nb / t / 1e12 / 8.0, 4), "TFLOP_per_s": round(fl / t / 1e12, 1),
                                  "frac_mfma_f16_peak": round(fl / t / 1e12 / 2500.0, 4)}
        out[f"T{T}"] = res
        del x, h, ys, yd, ws, calls
    out["workload"] = ("Qwen1.5-MoE-A2.7B MLP, 60 experts, gate/up 2 x 1408 over d = 2048, down 1408 -> 2048, "
                       "top-4, r=64; 32 calls per graph (4 at T = 2048), T <= 64 rotating 4 copies of all experts' weights "
                       "(T = 64 touches ~680 MB per cycle; at T = 1 the 4 active experts' ~46 MB per cycle can "
                       "stay in the 256 MB last-level cache)")
    del sets, mods, dmods, b_exp, db
    torch.cuda.empty_cache()
    return out


def extra_restore_selection(g, reps=3, k=16):
    """GlowQ-S selection over 32 LLaMA-2-7B-shaped layers (q, k, v, o, gate, up, down): the
    normalised error ratio of all 224 modules (fp16 W and its INT4-g128 form, both resident in
    HBM; one batch call) and the top-k choice of the layers, timed as one pass."""
    import torch
    import workload as W
    d, inter, L = 4096, 11008, 32
    shapes = [(d, d)] * 4 + [(inter, d)] * 2 + [(d, inter)]
    mods = []
    for l in range(L):
        for i, (O, kin) in enumerate(shapes):
            keys = (0, 5, l, i)
            w = W.make_w(O, kin, keys, W.outlier_columns(kin, keys), "cuda")
            mods.append((w, g.QWeight.from_workload(W.rtn_quantize(w))))
    torch.cuda.synchronize()
    sums = torch.empty(L * len(shapes), 2, dtype=torch.float64, device="cuda")
    ws = torch.empty(g.ner_workspace_bytes_batch([qw.n_out for _, qw in mods]), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        g.ner_sums_batch(mods, out=sums, workspace=ws)
        return g.restore_topk(sums.view(L, len(shapes), 2), k)

    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _, mask = run()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = statistics.median(ts)
    nb = sum(O * kin * 2 + O * kin // 2 + O * (kin // 128) * 4 for O, kin in shapes) * L
    out = {"workload": f"llama2-7b-shaped 32 layers x 7 modules: g_ner of every module + top-{k} layers",
           "ms": round(t * 1e3, 3), "alg_bytes": nb, "GB_per_s": round(nb / t / 1e9, 1),
           "frac_hbm_peak": round(nb / t / 1e9 / HBM_PEAK_GBS, 4), "restored": int(mask.sum())}
    del mods, sums, ws
    torch.cuda.empty_cache()
    return out


def extra_factor_solve(g, sigma32, reps=3, r=64, p=8, q=2):
    """Offline factor solve of the LLaMA-2-7B QKV group (m = 3 x 4096 stacked error rows, d = 4096):
    the quantisation errors of three generated fp16 weights, whitened by the calibration second
    moment measured in extra_second_moment, randomized SVD with k = r + p and q power iterations."""
    import torch
    import workload as W
    d = 4096
    errs = []
    for i in range(3):
        keys = (0, 6, 0, i)
        w = W.make_w(d, d, keys, W.outlier_columns(d, keys), "cuda")
        qw = W.rtn_quantize(w)
        w_hat = (qw.q.double() - qw.z.double().repeat_interleave(128, dim=1)) * qw.s.double().repeat_interleave(128, dim=1)
        errs.append(w.double() - w_hat)
    E = torch.cat(errs).contiguous()
    m = int(E.shape[0])
    k = r + p
    sigma = sigma32.double().contiguous()
    omega = torch.randn(d, k, generator=torch.Generator(device="cuda").manual_seed(0), device="cuda",
                        dtype=torch.float64)
    ws = torch.empty(int(g.lib().glowq_solve_workspace_bytes(m, d, k, r)), dtype=torch.uint8, device="cuda")
    g.solve_factors(E, sigma, omega, r, q, workspace=ws)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        A, B, S = g.solve_factors(E, sigma, omega, r, q, workspace=ws)  # synchronises
        ts.append(time.perf_counter() - t0)
    t = statistics.median(ts)
    # algorithmic flops: Cholesky d^3/3; products with the triangle L (d^2 k each: L Omega, L^T P
    # and L Z per power iteration, the final L^T P); with E_cat (2 m d k each: 2 + 2q of them);
    # Cholesky-QR bases (two passes of Gram + X R^-1, 8 n k^2 per basis); the small Gram, A and B
    flops = (d ** 3 / 3 + d * d * k * (2 + 2 * q) + 2 * m * d * k * (2 + 2 * q) + 8 * k * k * (m * (1 + q) + d * q)
             + 2 * k * k * d + 2 * m * k * r + 2 * r * d * k)
    out = {"workload": f"QKV group m = {m}, d = {d}, r = {r}, p = {p}, q = {q} (errors of generated LLaMA-2-7B-shaped "
                       "weights, Sigma_x from the calibration second moment)",
           "ms": round(t * 1e3, 2), "fp64_TFLOP_per_s": round(flops / t / 1e12, 2),
           "frac_fp64_peak": round(flops / t / 1e12 / 78.6, 4),
           "top_singular_value": float(S[0]), "r_th_singular_value": float(S[-1])}
    # the unit's restore score g_ec from the same errors and the solve's singular values
    ews = torch.empty(int(g.lib().glowq_ec_score_workspace_bytes(m, d)), dtype=torch.uint8, device="cuda")
    g.ec_score(E, sigma, S, r, workspace=ews)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        sc = g.ec_score(E, sigma, S, r, workspace=ews)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    t = statistics.median(ts)
    out["g_ec"] = {"ms": round(t * 1e3, 2), "fp64_TFLOP_per_s": round(m * d * d / t / 1e12, 2),
                   "frac_fp64_peak": round(m * d * d / t / 1e12 / 78.6, 4), "score": float(sc[2])}
    del E, sigma, omega, ws, A, B, ews
    torch.cuda.empty_cache()
    return out


def extra_second_moment(g, reps=5):
    """Offline factor solve, first step: Sigma_x = X^T X / N over 64 calibration sequences of 2048
    tokens at d = 4096 (the LLaMA-2-7B attention input), activations resident in HBM."""
    import torch
    import workload as W
    d, seqs, L = 4096, 64, 2048
    basis = W.haar_basis(d, 42, 0)
    x = torch.cat([W.make_x(L, d, 1.19, (42, q), device="cuda", basis=basis) for q in range(seqs)])
    N = int(x.shape[0])
    out = torch.empty(d, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(int(g.lib().glowq_second_moment_workspace_bytes(N, d)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    g.second_moment(x, out=out, workspace=ws)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.second_moment(x, out=out, workspace=ws)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = statistics.median(ts)
    sigma = out.clone()
    nb = -(-d // 256)                           # 256 x 256 lower-triangle tiles
    alg = N * d * (d + 1)                       # N d (d + 1) / 2 distinct products, 2 flops each
    executed = 2 * N * 256 * 256 * (nb * (nb + 1) // 2)
    del x, out, ws
    torch.cuda.empty_cache()
    return sigma, {"workload": f"Sigma_x = X^T X / N, N = {seqs} x {L} calibration tokens, d = {d}",
            "ms": round(t * 1e3, 3), "alg_TFLOP_per_s": round(alg / t / 1e12, 1),
            "executed_TFLOP_per_s": round(executed / t / 1e12, 1),
            "frac_mfma_f16_peak": round(executed / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


def achievable_peaks(reps=5):
    """The achievable peaks on this GPU, measured by the probe library: a streaming read of a
    4 GiB buffer (16 times the last-level cache) and a matrix-core-only fp16 loop."""
    import torch
    from rank_error_compensation_amd import probe
    stream = torch.cuda.current_stream()
    n = 4 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096 * 256 * 16, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hbm = 0.0
    for blocks in (512, 1024, 2048, 4096):  # best launch shape
        probe.read(src, sink, blocks)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            probe.read(src, sink, blocks)
        e1.record(stream)
        torch.cuda.synchronize()
        hbm = max(hbm, n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src
    mblocks, iters = 512, 10000
    msink = torch.empty(mblocks * 256 * 64, dtype=torch.uint8, device="cuda")
    probe.mfma_f16(iters // 10, msink, mblocks)
    torch.cuda.synchronize()
    e0.record(stream)
    fl = 0.0
    for _ in range(reps):
        fl += probe.mfma_f16(iters, msink, mblocks)
    e1.record(stream)
    torch.cuda.synchronize()
    mfma = fl / (e0.elapsed_time(e1) * 1e-3) / 1e12
    # the 16x16x32 instruction the GEMM kernels use, with 4 and 16 independent accumulators per wave
    shape_rates = {}
    ssink = torch.empty(1024 * 256 * 16, dtype=torch.uint8, device="cuda")
    for chains in (4, 16):
        probe.mfma_shape(1, chains, 100, ssink, 1024)
        torch.cuda.synchronize()
        e0.record(stream)
        fl = 0.0
        for _ in range(reps):
            fl += probe.mfma_shape(1, chains, 8000, ssink, 1024)
        e1.record(stream)
        torch.cuda.synchronize()
        shape_rates[f"mfma_16x16x32_f16_{chains}_chains_TFLOP_per_s"] = round(fl / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    torch.cuda.empty_cache()
    return {"hbm_read_GB_per_s": round(hbm, 1), "mfma_f16_TFLOP_per_s": round(mfma, 1), **shape_rates,
            "how": "probe library: 4 GiB nontemporal streaming read (best of 512..4096 workgroups of 256 "
                   "threads, 8 x 16 B in flight each); v_mfma_f32_32x32x16_f16 loop on registers (512 x 4 "
                   "waves, 4 independent chains each, sustained over 5 launches); v_mfma_f32_16x16x32_f16 loop with 4 "
                   "and 16 accumulators per wave (1024 x 4 waves): the 16x16x32 instruction needs about 16 "
                   "independent accumulators per wave to reach the full rate"}


def launch_sequence_floor(nbytes, reps=5):
    """Time of one pass of streaming reads with the decode step's launch sequence: one launch per
    unit reading that unit's algorithmic bytes (regions laid end to end, 3.6 GB in all, beyond the
    last-level cache), one workgroup per 32 KiB -- what separate launches of these sizes allow."""
    import torch
    from rank_error_compensation_amd import probe
    sizes = [(int(b) + 15) // 16 * 16 for b in nbytes]
    seq = probe.ReadSequence(sizes)
    src = torch.ones(seq.total, dtype=torch.uint8, device="cuda")
    sink = torch.empty(max((b + 32767) // 32768 for b in sizes) * 256 * 16, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    seq.run(src, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        seq.run(src, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, sink
    torch.cuda.empty_cache()
    return us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--event-reps", type=int, default=10)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB 5 times with a plain "
                         "device copy (a reference kernel of known traffic for hardware counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU (no multi-GPU path is built); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_error_compensation_amd import glowq as g
    g.lib()
    torch.cuda.set_device(0)
    dev = "cuda"

    # ---- headline: 32-layer path, decode T = 1, the restore set selected by the library
    T = 1
    t0 = time.time()
    sel_mask, sel_scores = select_path_mask(g, dev)
    log(f"[bench] restore set (g_ner, top-16, layer order within {RESTORE_REL_TOL} of the best): "
        f"layers {[l for l in range(32) if sel_mask[l]]}, scores {min(sel_scores):.6g} .. {max(sel_scores):.6g}, "
        f"{time.time() - t0:.1f}s")
    units, descr, mask, keep = build_path(T, dev, keep_layers=(), mask=sel_mask)
    first_off = next(l for l in range(32) if not mask[l])
    first_on = next(l for l in range(32) if mask[l])
    plan = g.PathPlan(units)
    nbytes = [unit_bytes(t, d, no, r, rs) for (_, t, d, no, r, rs) in descr]
    # timed region: K steps between two HIP events on the stream the library launches on
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        plan.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed = ev0.elapsed_time(ev1) * 1e-3
    ms = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed
    log(f"[bench] decode path: {ms * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), {value:.1f} tokens/s")

    # achievable peaks on this GPU (after the timed region, so that the matrix-core loop's heat
    # does not touch the headline)
    peaks = achievable_peaks()
    log(f"[bench] achievable peaks: {peaks}")

    # ---- dominant kernel: the fused decode kernel, one launch per unit (every launch of the step)
    launch_us = elapsed / args.steps / len(descr) * 1e6
    achieved = sum(nbytes) / (elapsed / args.steps) / 1e9
    durs = per_launch_events(units, descr, g, args.event_reps)  # per unit, single launch between events
    per_kind = {}
    for (name, t, d, no, r, rs), du, nb in zip(descr, durs, nbytes):
        k = f"{name}{'' if rs else '(no-restore)'}"
        e = per_kind.setdefault(k, {"launches": 0, "us": 0.0, "bytes": nb})
        e["launches"] += 1
        e["us"] += du * 1e6
    for k, e in per_kind.items():
        e["us"] = round(e["us"] / e["launches"], 3)
        e["GB_per_s"] = round(e["bytes"] / (e["us"] * 1e-6) / 1e9, 1)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "peak_measured": peaks["hbm_read_GB_per_s"],
                "frac_measured": round(achieved / peaks["hbm_read_GB_per_s"], 4),
                "kernel": "glowq::decode_kernel (fused projection + INT4 product + correction)",
                "launches_per_step": len(descr),
                "alg_bytes_per_launch_mean": int(sum(nbytes) / len(nbytes)),
                "launch_us_mean": round(launch_us, 3),
                "per_unit_single_launch_event_us": per_kind}
    floor_us = launch_sequence_floor(nbytes)
    roofline["launch_sequence_floor"] = {
        "us_per_step": round(floor_us, 1), "GB_per_s": round(sum(nbytes) / (floor_us * 1e-6) / 1e9, 1),
        "frac": round(floor_us / (elapsed / args.steps * 1e6), 4),
        "how": "probe library: the same 128 launches as plain streaming reads of each unit's algorithmic "
               "bytes, one workgroup of 256 threads per 32 KiB; frac = floor / decode step time"}
    log(f"[bench] decode kernel: {achieved:.0f} GB/s, {launch_us:.2f} us per launch over {len(descr)} launches; "
        f"streaming floor of the same launch sequence {floor_us:.1f} us/step")

    # ---- layerwise baseline on the same path
    extra = {}
    if not args.no_extras:
        del plan
        units_lw, descr_lw, _, _ = build_path(T, dev, layerwise=True, mask=sel_mask)
        ws_lw = g.make_workspace(T, 64, 3)

        def run_lw():
            for u in units_lw:
                call_unit(u, g, ws_lw, layerwise=True)

        def run_grp():
            for u in units_lw:
                call_unit(u, g, ws_lw, layerwise=False)

        # alternate the two schedules step by step (same clock and power state for both); the
        # per-step pairs give a 95 % interval of the relative difference
        # each schedule is captured in a HIP graph (128 launches issued from Python per step would
        # leave the GPU waiting for the host) and the replays are timed in pairs
        gr_grp, gr_lw = graphed(run_grp), graphed(run_lw)
        path_ci = paired_ci(gr_grp.replay, gr_lw.replay, trials=max(20, args.steps), calls=1)
        del gr_grp, gr_lw
        t_gr = path_ci["a_us_median"] * 1e-6
        t_lw = path_ci["b_us_median"] * 1e-6
        d_lw = d_gr = 0.0
        for _ in range(2):
            d_lw += sum(per_launch_events(units_lw, descr_lw, g, max(1, args.event_reps // 2), layerwise=True))
            d_gr += sum(per_launch_events(units_lw, descr_lw, g, max(1, args.event_reps // 2), layerwise=False))
        d_lw /= 2
        d_gr /= 2
        extra["layerwise_vs_group_T1_path"] = {
            "group_us_per_step_percall": round(t_gr * 1e6, 1), "layerwise_us_per_step_percall": round(t_lw * 1e6, 1),
            "group_kernel_sum_us": round(d_gr * 1e6, 1), "layerwise_kernel_sum_us": round(d_lw * 1e6, 1),
            "kernel_speedup": round(d_lw / d_gr, 4), "paired_steps_ci": path_ci}
        del units_lw
        torch.cuda.empty_cache()
        log(f"[bench] layerwise {d_lw * 1e6:.1f} us vs group {d_gr * 1e6:.1f} us (kernel sums)")

        # prefill pass
        units_p, descr_p, _, _ = build_path(512, dev, mask=sel_mask)
        plan_p = g.PathPlan(units_p)
        ksteps = max(3, args.steps // 10)
        ep = time_steps(plan_p.run, ksteps, 2)
        tp = ep / ksteps
        fl = sum(unit_flops(t, d, no, r, rs) for (_, t, d, no, r, rs) in descr_p)
        extra["prefill_path_T512"] = {"ms_per_step": round(tp * 1e3, 3), "tokens_per_s": round(512 / tp, 1),
                                      "alg_TFLOP_per_s": round(fl / tp / 1e12, 2),
                                      "frac_mfma_f16_peak": round(fl / tp / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        log(f"[bench] prefill path T=512: {tp * 1e3:.3f} ms, {fl / tp / 1e12:.1f} TFLOP/s")
        del plan_p, units_p
        torch.cuda.empty_cache()
        extra["tiny_qkv"] = extra_tiny_qkv(g)
        log(f"[bench] tiny QKV: {extra['tiny_qkv']}")
        for Tq in (1, 4, 16):
            extra[f"decode_qkv_T{Tq}"] = extra_decode_qkv(g, Tq)
            log(f"[bench] QKV decode T={Tq}: {extra[f'decode_qkv_T{Tq}']}")
        extra["llama3_gqa_units"] = extra_llama3(g)
        log(f"[bench] LLaMA-3.1-8B GQA units: {extra['llama3_gqa_units']}")
        extra["prefill_gateup_T2048"] = extra_prefill_gateup(g)
        for k in ("group", "layerwise"):
            e = extra["prefill_gateup_T2048"][k]
            e["frac_mfma_measured_peak"] = round(e["alg_TFLOP_per_s"] / peaks["mfma_f16_TFLOP_per_s"], 4)
        log(f"[bench] gate/up prefill T=2048: {extra['prefill_gateup_T2048']}")
        extra["group_vs_layerwise"] = extra_group_vs_layerwise(g)
        log(f"[bench] group vs layerwise: {extra['group_vs_layerwise']}")
        extra["w4a8"] = extra_w4a8(g)
        log(f"[bench] W4A8: {extra['w4a8']}")
        extra["moe_qwen15"] = extra_moe(g)
        log(f"[bench] MoE: {extra['moe_qwen15']}")
        extra["mx_formats"] = extra_mx(g)
        log(f"[bench] MX formats: {extra['mx_formats']}")
        extra["restore_selection_32L"] = extra_restore_selection(g)
        e = extra["restore_selection_32L"]
        e["frac_hbm_measured_peak"] = round(e["GB_per_s"] / peaks["hbm_read_GB_per_s"], 4)
        log(f"[bench] restore selection: {e}")
        sigma, extra["second_moment_calib"] = extra_second_moment(g)
        e = extra["second_moment_calib"]
        e["frac_mfma_measured_peak"] = round(e["executed_TFLOP_per_s"] / peaks["mfma_f16_TFLOP_per_s"], 4)
        log(f"[bench] second moment: {e}")
        extra["factor_solve_qkv"] = extra_factor_solve(g, sigma)
        del sigma
        log(f"[bench] factor solve: {extra['factor_solve_qkv']}")

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import glowq_ref  # noqa: F401  (oracle only in the CPU-baseline leg)
        _, _, mask2, keep = build_path_keep(T, dev, [first_on, first_off], sel_mask)
        cpu = cpu_baseline(keep, mask2)
        log(f"[bench] cpu oracle: {cpu}")

    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 5
        extra["copy_probe"] = {"bytes_read_per_copy": n, "bytes_written_per_copy": n,
                               "GB_per_s_read_plus_write": round(2 * n / t / 1e9, 1)}
        log(f"[bench] copy probe: {extra['copy_probe']}")

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama2-7b-32-layer-linear-path decode T=1 r=64 restore=16/32 layers",
                   "T": 1, "r": 64, "layers": 32, "d": 4096, "inter": 11008,
                   "units_per_step": len(descr), "weights": "INT4-g128 fp16 scale/zero",
                   "restore_set": {"how": f"g_ner on the GPU, top-16 layers, layer order within {RESTORE_REL_TOL} "
                                          "of the best score", "layers": [l for l in range(32) if sel_mask[l]]}},
        "roofline": roofline, "cpu_baseline": cpu, "achievable_peaks": peaks, "extra": extra,
    }
    print(json.dumps(line), flush=True)


def build_path_keep(T, device, layers, mask):
    """Only the requested layers of the path (for the CPU oracle sample)."""
    import workload as W
    keep = {}
    for l in layers:
        lu, mask = W.llama2_path_inputs(T, device=device, layers=[l], mask=mask)
        keep[l] = lu[l]
    return None, None, mask, keep


if __name__ == "__main__":
    main()
