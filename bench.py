"""Benchmark of the RAT+ layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

A step is one pass of the prefill hot path -- the gated recurrence (scan)
then dilated attention -- over one batch of the 1.5B-scale layer workload
(B=4, T=4096, H=16, d=128, D=16, full recurrence, bf16), with inputs already
resident in HBM.  Three input/output sets rotate so that consecutive steps
do not find their data in the 256 MB Infinity Cache.  ``value`` is prefill
tokens per second per layer, B*T / step time.

Per-kernel durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream), around a run of
back-to-back launches of that one kernel.  The JSON line also
carries the roofline of the dominant kernel, the oracle timed on the host
cores on a bounded sample (``cpu_baseline``) and, under ``extra``, the other
workloads: long prefill with a window (both recurrence readings), the 7.6B
hybrid prefill, the 2.6B decode at D = 64 and D = 16, the chunk-grid
attention on the 1.5B-scale prefill shape, the decode-loop step (the
recurrence update fused with decode attention) on the 2.6B decode shape,
and the layer backward of Active Recurrence Learning training (half of the
1.5B-scale batch at D = 1, half at D = 64).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

# kernel names as the profiler lists them (bf16, d = 128, full recurrence)
SCAN_KERNEL = "rat::scan_full_kernel<unsigned short, false, true>"  # bf16, no history, 256-token chunks
ATTN_KERNEL = "rat::attn_dilated_kernel<128, 4, 2, false, false, false>"  # the 1.5B plan: short residues, four waves

# launches timed per kernel (each between its own pair of HIP events)
MIN_TIMED = 50

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-extra", action="store_true", help="only the headline workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--launches", type=int, default=50,
                   help="launches timed per kernel, each between its own HIP events (profiled runs use fewer)")
    p.add_argument("--only", default=None, help="run one workload of --list by name (profiling)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


# ------------------------------------------------------------------ helpers
def progress(*parts):
    print("[bench]", *parts, file=sys.stderr, flush=True)


def time_launches(torch, fn, n, warmup):
    """Per-launch durations (ms) of ``fn(i)``: ``warmup`` untimed calls, then
    ``n`` calls, each between its own pair of HIP events recorded on the
    launch stream; returns median, p10, p90 and mean."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        fn(i)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    def pct(p):
        x = p * (len(ms) - 1)
        lo = int(x)
        hi = min(lo + 1, len(ms) - 1)
        return ms[lo] + (ms[hi] - ms[lo]) * (x - lo)

    return {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "mean": sum(ms) / len(ms), "n": len(ms)}


def stats_fields(prefix, st, nbytes=None, flops=None):
    """JSON fields of one kernel's launch statistics, its rates at the median."""
    out = {f"{prefix}_ms": st["median"], f"{prefix}_ms_p10": st["p10"], f"{prefix}_ms_p90": st["p90"],
           f"{prefix}_ms_mean": st["mean"], f"{prefix}_launches_timed": st["n"]}
    sec = st["median"] / 1e3
    if nbytes is not None:
        out[f"{prefix}_GBps"] = nbytes / sec / 1e9
        out[f"{prefix}_hbm_frac"] = nbytes / sec / 1e9 / HBM_PEAK_GBS
    if flops is not None:
        out[f"{prefix}_TFLOPs"] = flops / sec / 1e12
        out[f"{prefix}_mfma_frac"] = flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS
    return out


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when it is absent or was taken from other kernel sources."""
    path = os.path.join(PROFILES, "prefill_1.5B_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    from dilated_sparse_attention_amd.profiling import kernel_sources_hash

    if data.get("sources_hash") != kernel_sources_hash():
        return None
    ent = data.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("bytes_per_launch")


def attn_pairs(T, D, W):
    """(dilated pairs, local pairs) of one head: closed forms of the index-set
    sizes summed over the T queries."""
    M = [(T - r + D - 1) // D for r in range(min(D, T))]
    dil = sum(m * (m + 1) // 2 for m in M)
    loc = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
    return dil, loc


# ------------------------------------------------------------------ workloads
def prefill_units(w):
    """Algorithmic bytes / FLOPs of the scan and of the attention."""
    E = w.B * w.T * w.H * w.d
    s = 2 if "bfloat16" in str(w.dtype) else 4
    scan_bytes = 5 * E * s
    raw_heads = sum(1 for x in w.W if x > 0)
    attn_bytes = 4 * E * s + 2 * (E // w.H) * raw_heads * s
    pairs = 0
    for Dh, Wh in zip(w.D, w.W):
        a, b = attn_pairs(w.T, Dh, Wh)
        pairs += a + b
    attn_flops = 4 * w.d * pairs * w.B
    return scan_bytes, attn_bytes, attn_flops


def run_prefill(torch, rat, w, steps, warmup, mode=0, nsets=3):
    from dilated_sparse_attention_amd import inputs

    need_raw = any(x > 0 for x in w.W)
    sets = []
    for i in range(nsets):
        x = inputs.make_prefill(w, seed=i, device="cuda")
        ks = torch.empty_like(x["k"])
        vs = torch.empty_like(x["v"])
        out = torch.empty_like(x["q"])
        sets.append((x, ks, vs, out))
    D, W = list(w.D), list(w.W)

    def step(i):
        x, ks, vs, out = sets[i % nsets]
        rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=mode, k_state=ks, v_state=vs)
        rat.dilated_attn_prefill(x["q"], ks, vs, x["k"] if need_raw else None, x["v"] if need_raw else None,
                                 D=D, W=W, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / steps

    def launch(which, i):
        x, ks, vs, out = sets[i % nsets]
        if which == "scan":
            rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=mode, k_state=ks, v_state=vs)
        else:
            rat.dilated_attn_prefill(x["q"], ks, vs, x["k"] if need_raw else None, x["v"] if need_raw else None,
                                     D=D, W=W, out=out)

    n = max(steps, MIN_TIMED)
    scan_st = time_launches(torch, lambda i: launch("scan", i), n, warmup)
    attn_st = time_launches(torch, lambda i: launch("attn", i), n, warmup)
    del sets
    torch.cuda.empty_cache()
    return ms_step, wall, scan_st, attn_st


def run_decode(torch, rat, w, steps, warmup, nsets=3):
    from dilated_sparse_attention_amd import inputs

    sets = []
    for i in range(nsets):
        x = inputs.make_decode(w, seed=i, device="cuda")
        x["out"] = torch.empty_like(x["q"])
        sets.append(x)
    D, W = list(w.D), list(w.W)
    ws_bytes = rat.decode_workspace_bytes(w.B, w.H, w.d, w.T, D, W)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    def call(i):
        x = sets[i % nsets]
        rat.dilated_attn_decode(x["q"], x["kd"], x["vd"], x["kw"], x["vw"], w.T, D, W, out=x["out"],
                                workspace=ws if ws_bytes else None)

    st = time_launches(torch, call, max(steps, MIN_TIMED), warmup)
    nd = [(w.T + Dh - 1) // Dh for Dh in w.D]
    nw = [min(Wh, w.T) for Wh in w.W]
    s = 2
    nbytes = w.B * sum((a + b) * 2 * w.d * s for a, b in zip(nd, nw)) + 2 * w.B * w.H * w.d * s
    del sets
    torch.cuda.empty_cache()
    return st, nbytes


def chunk_units(w):
    """Algorithmic bytes / FLOPs of chunk-grid attention: q, every own state
    (k and v) and the output once, the chunk-end states once; query t scores
    its floor(t / D) chunk ends and its own state."""
    E = w.B * w.T * w.H * w.d
    s = 2
    ends = sum(w.T // Dh for Dh in w.D) * w.B * w.d  # chunk-end rows (p = cD - 1 <= T - 1), all heads
    nbytes = 4 * E * s + 2 * ends * s
    pairs = sum(sum(t // Dh + 1 for t in range(w.T)) for Dh in w.D)
    return nbytes, 4 * w.d * pairs * w.B


def run_chunk(torch, rat, w, steps, warmup, nsets=3):
    """Chunk-grid attention over the recurrence states of the prefill
    workload `w` (the states come from the scan kernel, outside the timed
    region), over rotating sets."""
    from dilated_sparse_attention_amd import inputs

    sets = []
    for i in range(nsets):
        x = inputs.make_prefill(w, seed=i, device="cuda")
        ks, vs = rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=w.modes[0])
        sets.append((x["q"], ks, vs, torch.empty_like(x["q"])))
        del x
    D = list(w.D)
    call = lambda i: rat.chunk_attn_prefill(*sets[i % nsets][:3], D=D, out=sets[i % nsets][3])  # noqa: E731
    st = time_launches(torch, call, max(steps, MIN_TIMED), warmup)
    del sets
    torch.cuda.empty_cache()
    return st


def run_decode_caches(torch, rat, w, steps, warmup, nsets=3):
    """The decode caches of a finished prefill of workload `w`: its states
    copied into the per-residue history and its last W raw tokens into the
    ring (the states come from the scan kernel, outside the timed region),
    over rotating sets.  Algorithmic bytes: the states read and the history
    written once, the ring's raw rows read and written once."""
    from dilated_sparse_attention_amd import inputs

    sets = []
    D, W = list(w.D), list(w.W)
    n_cap = rat.history_rows(w.T, D)
    w_cap = max(W)
    for i in range(nsets):
        x = inputs.make_prefill(w, seed=i, device="cuda")
        ks, vs = rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=w.modes[0])
        kc = torch.empty((w.B, w.H, n_cap, w.d), dtype=ks.dtype, device="cuda")
        kw = torch.empty((w.B, w.H, w_cap, w.d), dtype=ks.dtype, device="cuda") if w_cap > 0 else None
        sets.append((ks, vs, x["k"], x["v"], kc, torch.empty_like(kc), kw, None if kw is None else torch.empty_like(kw)))
        del x

    def call(i):
        ks, vs, k, v, kc, vc, kw, vw = sets[i % nsets]
        rat.build_decode_caches(ks, vs, k, v, D, W, n_cap=n_cap, w_cap=w_cap, kc=kc, vc=vc, kw=kw, vw=vw)

    st = time_launches(torch, call, max(steps, MIN_TIMED), warmup)
    del sets
    torch.cuda.empty_cache()
    s = 2
    nbytes = 2 * 2 * w.B * w.T * w.H * w.d * s + 2 * 2 * w.B * w.d * s * sum(min(Wh, w.T) for Wh in W)
    return st, nbytes


def run_layer_prefill(torch, rat, w, steps, warmup, mode=0, nsets=2):
    """The one-call layer prefill (recurrence with its states written into
    the per-residue decode history, attention, raw ring) against the same
    outputs from separate calls: the recurrence and the attention alone,
    and those followed by the decode-cache build.  Each timed per call."""
    from dilated_sparse_attention_amd import inputs

    D, W = list(w.D), list(w.W)
    need_raw = any(x > 0 for x in W)
    n_cap = rat.history_rows(w.T, D)
    w_cap = max(W) if need_raw else 0
    sliding = mode == 1 and w.L < w.T
    sets = []
    for i in range(nsets):
        x = inputs.make_prefill(w, seed=i, device="cuda")
        kc = torch.empty((w.B, w.H, n_cap, w.d), dtype=w.dtype, device="cuda")
        ring = (lambda: torch.zeros((w.B, w.H, w_cap, w.d), dtype=w.dtype, device="cuda")) if need_raw else (lambda: None)
        sets.append(dict(x, out=torch.empty_like(x["q"]), ks=torch.empty_like(x["k"]), vs=torch.empty_like(x["v"]),
                         kc=kc, vc=torch.empty_like(kc), kw=ring(), vw=ring(),
                         st=None if sliding else torch.empty((w.B, w.H, 2, w.d), dtype=torch.float32, device="cuda")))
        del x

    def fused(i):
        x = sets[i % nsets]
        rat.layer_prefill(x["q"], x["k"], x["v"], x["gate"], D, W, L=w.L, mode=mode, n_cap=n_cap, w_cap=w_cap,
                          final_state=False if sliding else x["st"], out=x["out"], kc=x["kc"], vc=x["vc"],
                          kw=x["kw"], vw=x["vw"])

    def two_calls(i, caches):
        x = sets[i % nsets]
        rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=mode, k_state=x["ks"], v_state=x["vs"])
        rat.dilated_attn_prefill(x["q"], x["ks"], x["vs"], x["k"] if need_raw else None,
                                 x["v"] if need_raw else None, D=D, W=W, out=x["out"])
        if caches:
            rat.build_decode_caches(x["ks"], x["vs"], x["k"], x["v"], D, W, n_cap=n_cap, w_cap=w_cap,
                                    kc=x["kc"], vc=x["vc"], kw=x["kw"], vw=x["vw"])

    n = max(steps, MIN_TIMED)
    st_f = time_launches(torch, fused, n, warmup)
    st_2 = time_launches(torch, lambda i: two_calls(i, False), n, warmup)
    st_c = time_launches(torch, lambda i: two_calls(i, True), n, warmup)
    del sets
    torch.cuda.empty_cache()
    return st_f, st_2, st_c


def run_decode_step(torch, rat, w, steps, warmup, nsets=2):
    """One decode-loop step (recurrence update, history and ring writes,
    decode attention) at context length w.T for the whole batch: the state
    history holds every position (n_cap = D ceil(T / D) rows per head)."""
    D, W = list(w.D), list(w.W)
    n_cap = max(Dh * ((w.T + Dh - 1) // Dh) for Dh in D)
    sets = []
    for i in range(nsets):
        g = torch.Generator(device="cuda")
        g.manual_seed(100 + i)
        mk = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(w.dtype)  # noqa: E731
        x = {n: mk(w.B, w.H, w.d) for n in ("q", "k", "v", "gate")}
        x["state"] = torch.randn((w.B, w.H, 2, w.d), generator=g, device="cuda")
        x["kc"], x["vc"] = mk(w.B, w.H, n_cap, w.d), mk(w.B, w.H, n_cap, w.d)
        x["kw"], x["vw"] = mk(w.B, w.H, w.w_cap, w.d), mk(w.B, w.H, w.w_cap, w.d)
        x["out"] = torch.empty_like(x["q"])
        sets.append(x)
    ws_bytes = rat.decode_workspace_bytes(w.B, w.H, w.d, w.T, D, W)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    def call(i):
        x = sets[i % nsets]
        rat.decode_step(x["q"], x["k"], x["v"], x["gate"], x["state"], x["kc"], x["vc"], x["kw"], x["vw"], w.T,
                        D, W, out=x["out"], workspace=ws if ws_bytes else None)

    st = time_launches(torch, call, max(steps, MIN_TIMED), warmup)
    # bytes: q, k, v, gate read; state read and written (fp32); the state
    # row and the raw token written; the residue's history rows and the ring
    # read; the output written
    s = 2
    E = w.B * w.H * w.d
    rows = sum((w.T - 1) // Dh + 1 + min(Wh, w.T) for Dh, Wh in zip(D, W)) * w.B * w.d
    nbytes = 4 * E * s + 2 * (2 * E * 4) + 4 * E * s + 2 * rows * s + E * s
    del sets
    torch.cuda.empty_cache()
    return st, nbytes


def run_backward_arl(torch, rat, w, steps, warmup):
    """The training step's backward of Active Recurrence Learning on the
    prefill workload `w`: half of the batch at D = 1, half at D = 64, full
    recurrence; one layer_backward call per half (the forward's states come
    from the scan kernel, outside the timed region)."""
    from dilated_sparse_attention_amd import inputs

    x = inputs.make_prefill(w, seed=7, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(w.dtype)
    half = w.B // 2
    parts = []
    for b0, Dv in ((0, 1), (half, 64)):
        xs = {n: t[b0:b0 + half].contiguous() for n, t in x.items()}
        ks, vs = rat.scan_prefill(xs["k"], xs["v"], xs["gate"])
        grads = tuple(torch.empty(xs["q"].shape, dtype=torch.float32, device="cuda") for _ in range(4))
        ws = torch.empty(rat.ops.load_library().rat_layer_backward_workspace_bytes(half, w.T, w.H, w.d),
                         dtype=torch.uint8, device="cuda")
        parts.append((xs, ks, vs, dout[b0:b0 + half].contiguous(), [Dv] * w.H, grads, ws))
    del x

    def step(_):
        for xs, ks, vs, do, D, grads, ws in parts:
            rat.layer_backward(xs["q"], xs["k"], xs["v"], xs["gate"], ks, vs, do, D, [0] * w.H, grads=grads,
                               workspace=ws)

    st = time_launches(torch, step, max(steps, MIN_TIMED), warmup)
    # algorithmic units: per visible (query, key) pair five length-d
    # contractions (scores, dout.v, and the three gradient products); bytes:
    # the seven inputs once and the four fp32 gradients once
    pairs = half * sum(attn_pairs(w.T, Dv, 0)[0] * w.H for Dv in (1, 64))
    flops = 10 * w.d * pairs
    E = w.B * w.T * w.H * w.d
    nbytes = 7 * E * 2 + 4 * E * 4
    del parts
    torch.cuda.empty_cache()
    return st, flops, nbytes


def run_backward_windowed(torch, rat, w, steps, warmup, mode):
    """The layer backward of a windowed prefill workload `w` (every head at
    its (D, W), recurrence `mode` with its L): the dilated states and the
    raw window in one softmax.  The forward's states come from the scan
    kernel, outside the timed region."""
    from dilated_sparse_attention_amd import inputs

    x = inputs.make_prefill(w, seed=9, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(10)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(w.dtype)
    ks, vs = rat.scan_prefill(x["k"], x["v"], x["gate"], L=w.L, mode=mode)
    grads = tuple(torch.empty(x["q"].shape, dtype=torch.float32, device="cuda") for _ in range(4))
    ws = torch.empty(rat.ops.load_library().rat_layer_backward_workspace_bytes(w.B, w.T, w.H, w.d),
                     dtype=torch.uint8, device="cuda")

    def step(_):
        rat.layer_backward(x["q"], x["k"], x["v"], x["gate"], ks, vs, dout, list(w.D), list(w.W), L=w.L,
                           mode=mode, grads=grads, workspace=ws)

    st = time_launches(torch, step, max(steps, MIN_TIMED), warmup)
    # the same units as the ARL backward, over the dilated and the window pairs
    pairs = w.B * sum(sum(attn_pairs(w.T, Dh, Wh)) for Dh, Wh in zip(w.D, w.W))
    flops = 10 * w.d * pairs
    E = w.B * w.T * w.H * w.d
    nbytes = 7 * E * 2 + 4 * E * 4
    del x, ks, vs, grads, ws
    torch.cuda.empty_cache()
    return st, flops, nbytes


def run_copy_reference(torch, nbytes, steps, nsets=3):
    """A plain device-to-device copy moving ``nbytes`` (half read, half
    written), over rotating buffer sets that together exceed the caches: the
    rate the HBM delivers in practice, reported beside the spec peak."""
    n = nbytes // 2
    bufs = [(torch.ones(n, dtype=torch.uint8, device="cuda"), torch.empty(n, dtype=torch.uint8, device="cuda"))
            for _ in range(nsets)]
    st = time_launches(torch, lambda i: bufs[i % nsets][1].copy_(bufs[i % nsets][0]), max(steps, MIN_TIMED),
                       2 * nsets)
    del bufs
    torch.cuda.empty_cache()
    return st


# ------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _timed(fn, min_s, max_reps):
    """Seconds per call of ``fn``: repeated until ``min_s`` seconds have
    passed (at least once, at most ``max_reps`` times)."""
    reps, total, out = 0, 0.0, None
    while (total < min_s and reps < max_reps) or reps == 0:
        t0 = time.perf_counter()
        out = fn()
        total += time.perf_counter() - t0
        reps += 1
    return total / reps, reps, out


def cpu_baseline(w, min_s=10.0, max_reps=100):
    """The fp64 oracle on the host cores, timed on the headline workload
    itself: one oracle step is the recurrence over every (batch, token, head,
    channel) followed by attention for every query row, from inputs already
    widened to float64.  Steps repeat until ``min_s`` seconds have passed
    (bounded by ``max_reps``); the value is whole-workload tokens/s."""
    import numpy as np

    from dilated_sparse_attention_amd import inputs
    from oracle import oracle

    oracle.build(force=False)
    orc = oracle.default()
    x = inputs.make_prefill(w, seed=0)
    q, k, v, g = (np.ascontiguousarray(x[n].double().numpy()) for n in ("q", "k", "v", "gate"))
    need_raw = any(wh > 0 for wh in w.W)

    def step():
        ks, vs = orc.scan(k, v, g, w.L, 0)
        orc.attn_prefill(q, ks, vs, k if need_raw else None, v if need_raw else None, w.D, w.W, w.scale)

    per_step, reps, _ = _timed(step, min_s, max_reps)
    total = per_step * reps
    return {"value": w.B * w.T / per_step, "unit": "tokens/s", "cores": orc.num_threads(),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": (f"fp64 C oracle (OpenMP), the whole {w.name} step (recurrence over all "
                       f"{w.B}x{w.T}x{w.H}x{w.d} elements, then attention for all {w.B * w.T * w.H} query "
                       f"rows) repeated {reps} times in {total:.1f} s: {per_step:.2f} s per step")}


def cpu_baseline_per_config(budget_s=4.0, sample_rows=1024):
    """The oracle per workload and per stage (recurrence, attention, decode),
    on the host cores, each stage timed by repetition for about ``budget_s``
    seconds.  The one stage whose full run would take minutes (the attention
    of the 7.6B hybrid, about 2.4 TFLOP in fp64) is timed on ``sample_rows``
    random query rows and scaled to the whole workload by visible (query,
    key) pairs; that entry says "extrapolated"."""
    import numpy as np

    from dilated_sparse_attention_amd import inputs
    from oracle import oracle

    oracle.build(force=False)
    orc = oracle.default()
    res = {"cores": orc.num_threads(), "cpu_model": _cpu_model(), "kind": "oracle", "configs": {}}
    big = {inputs.PREFILL_7P6B_HYBRID.name}
    for w in inputs.PREFILL_WORKLOADS:
        x = inputs.make_prefill(w, seed=0)
        q, k, v, g = (np.ascontiguousarray(x[n].double().numpy()) for n in ("q", "k", "v", "gate"))
        del x
        need_raw = any(wh > 0 for wh in w.W)
        kr, vr = (k, v) if need_raw else (None, None)
        entry = {"config": w.describe()}
        for mode in w.modes:
            tag = "restart" if mode == 0 else "sliding"
            t_scan, reps, (ks, vs) = _timed(lambda: orc.scan(k, v, g, w.L, mode), budget_s, 20)
            entry[f"scan_s_{tag}"] = t_scan
            if w.name in big:
                rng = np.random.default_rng(5)
                rows = np.stack([rng.integers(0, w.B, sample_rows), rng.integers(0, w.T, sample_rows),
                                 rng.integers(0, w.H, sample_rows)], 1).astype(np.int32)
                t_rows, _, _ = _timed(lambda: orc.attn_prefill_rows(q, ks, vs, kr, vr, rows, w.D, w.W, w.scale),
                                      budget_s, 50)
                pairs_rows = sum(t // w.D[h] + 1 + min(w.W[h], t + 1) for _, t, h in rows.tolist())
                pairs_all = w.B * sum(sum(attn_pairs(w.T, Dh, Wh)) for Dh, Wh in zip(w.D, w.W))
                t_attn = t_rows * pairs_all / pairs_rows
                entry["attn_timing"] = (f"extrapolated: {sample_rows} random query rows in {t_rows:.3f} s, "
                                        f"scaled by visible pairs ({pairs_all} / {pairs_rows})")
            else:
                t_attn, _, _ = _timed(lambda: orc.attn_prefill(q, ks, vs, kr, vr, w.D, w.W, w.scale), budget_s, 20)
                entry["attn_timing"] = "every query row"
            entry[f"attn_s_{tag}"] = t_attn
            entry[f"prefill_tokens_per_s_{tag}"] = w.B * w.T / (t_scan + t_attn)
            del ks, vs
        res["configs"][w.name] = entry
        del q, k, v, g
    for w in inputs.DECODE_WORKLOADS:
        x = inputs.make_decode(w, seed=0)
        a = {n: np.ascontiguousarray(t.double().numpy()) for n, t in x.items()}
        del x
        t_dec, _, _ = _timed(lambda: orc.attn_decode(a["q"], a["kd"], a["vd"], a["kw"], a["vw"], w.T, w.D, w.W,
                                                     w.scale), budget_s, 50)
        res["configs"][w.name] = {"config": w.describe(), "decode_s": t_dec, "decode_tokens_per_s": w.B / t_dec,
                                  "attn_timing": "every sequence of the batch"}
        del a
    return res


# ------------------------------------------------------------------ main
def main():
    args = parse()
    global MIN_TIMED
    MIN_TIMED = max(1, args.launches)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} / WORLD_SIZE {world} is not supported "
              "(the layer shards by (batch, head) with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dilated_sparse_attention_amd as rat
    from dilated_sparse_attention_amd import inputs, profiling

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rat.load_library()

    if args.copy_calibration:  # known-size elementwise pass: 1 GiB read, 1 GiB written
        a = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    w = inputs.PREFILL_1P5B
    if args.only is None or args.only == w.name:
        progress("prefill", w.name)
        ms, wall, scan_st, attn_st = run_prefill(torch, rat, w, args.steps, args.warmup)
    else:
        ms = wall = scan_st = attn_st = None
    scan_bytes, attn_bytes, attn_flops = prefill_units(w)

    extra = {}
    if not args.no_extra:
        for pw in (inputs.TINY_FP32, inputs.PREFILL_LONG, inputs.PREFILL_7P6B_HYBRID):
            for mode in pw.modes:
                key = pw.name + ("" if len(pw.modes) == 1 else ("_restart" if mode == 0 else "_sliding"))
                if args.only is not None and args.only != key:
                    continue
                progress("prefill", key)
                m2, _, s_st, a_st = run_prefill(torch, rat, pw, args.steps, args.warmup, mode=mode)
                sb, ab, af = prefill_units(pw)
                a_sec = a_st["median"] / 1e3
                extra[key] = {
                    "prefill_tokens_per_s": pw.B * pw.T / ((s_st["median"] + a_st["median"]) / 1e3),
                    "ms_per_step": m2,
                    **stats_fields("scan", s_st, nbytes=sb),
                    **stats_fields("attn", a_st, nbytes=ab, flops=af),
                    "attn_roofline_frac": (max(ab / HBM_PEAK_GBS / 1e9, af / MFMA_BF16_PEAK_TFLOPS / 1e12) / a_sec),
                    "scan_algorithmic_bytes": sb, "attn_algorithmic_bytes": ab, "attn_algorithmic_flops": af,
                    "config": pw.describe(), "mode": "restart" if mode == 0 else "sliding"}
        for dw in inputs.DECODE_WORKLOADS:
            if args.only is not None and args.only != dw.name:
                continue
            progress("decode", dw.name)
            dst, dbytes = run_decode(torch, rat, dw, args.steps, args.warmup)
            extra[dw.name] = {"decode_tokens_per_s": dw.B / (dst["median"] / 1e3),
                              **stats_fields("decode", dst, nbytes=dbytes), "algorithmic_bytes": dbytes,
                              "config": dw.describe()}

        cw = inputs.PREFILL_1P5B
        key = "chunk_grid_" + cw.name
        if args.only is None or args.only == key:
            progress("chunk grid", cw.name)
            cst = run_chunk(torch, rat, cw, args.steps, args.warmup)
            cb, cf = chunk_units(cw)
            extra[key] = {**stats_fields("attn", cst, nbytes=cb, flops=cf),
                          "algorithmic_bytes": cb, "algorithmic_flops": cf,
                          "config": dict(cw.describe(), attention="chunk grid: chunk-end states + own state")}
        sw = inputs.DECODE_2P6B_D64
        key = "decode_step_" + sw.name
        if args.only is None or args.only == key:
            progress("decode step", sw.name)
            sst, sbytes = run_decode_step(torch, rat, sw, args.steps, args.warmup)
            extra[key] = {"decode_tokens_per_s": sw.B / (sst["median"] / 1e3),
                          **stats_fields("step", sst, nbytes=sbytes), "algorithmic_bytes": sbytes,
                          "config": dict(sw.describe(), history_rows_per_head=max(
                              Dh * ((sw.T + Dh - 1) // Dh) for Dh in sw.D))}

        for lw in (inputs.PREFILL_1P5B, inputs.PREFILL_LONG):
            for mode in lw.modes:
                key = "layer_prefill_" + lw.name + ("" if len(lw.modes) == 1 else
                                                    ("_restart" if mode == 0 else "_sliding"))
                if args.only is not None and args.only != key:
                    continue
                progress("one-call layer prefill", key)
                st_f, st_2, st_c = run_layer_prefill(torch, rat, lw, args.steps, args.warmup, mode=mode)
                toks = lw.B * lw.T
                extra[key] = {"prefill_tokens_per_s": toks / (st_f["median"] / 1e3),
                              **stats_fields("layer", st_f), **stats_fields("two_calls", st_2),
                              **stats_fields("two_calls_and_caches", st_c),
                              "two_calls_tokens_per_s": toks / (st_2["median"] / 1e3),
                              "config": dict(lw.describe(), mode="restart" if mode == 0 else "sliding",
                                             compared="one call (states into the decode history, ring) vs "
                                                      "scan + attention, and those + the decode-cache build")}

        cw = inputs.PREFILL_LONG
        key = "decode_caches_" + cw.name
        if args.only is None or args.only == key:
            progress("decode caches from a prefill", cw.name)
            cst, cbytes = run_decode_caches(torch, rat, cw, args.steps, args.warmup)
            extra[key] = {**stats_fields("caches", cst, nbytes=cbytes), "algorithmic_bytes": cbytes,
                          "config": dict(cw.describe(), caches="per-residue state history + raw ring of the last W")}

        bw = inputs.PREFILL_1P5B
        key = "backward_arl_" + bw.name
        if args.only is None or args.only == key:
            progress("backward (ARL halves D=1 / D=64)", bw.name)
            bst, bflops, bbytes = run_backward_arl(torch, rat, bw, args.steps, 2)
            extra[key] = {"train_tokens_per_s": bw.B * bw.T / (bst["median"] / 1e3),
                          **stats_fields("backward", bst, nbytes=bbytes, flops=bflops),
                          "algorithmic_flops": bflops, "algorithmic_bytes": bbytes,
                          "config": dict(bw.describe(), D="half the batch at 1, half at 64", W=0,
                                         recurrence="full")}

        bw = inputs.PREFILL_LONG
        for mode, mname in ((rat.RESTART, "restart"), (rat.SLIDING, "sliding")):
            key = f"backward_windowed_{bw.name}_{mname}"
            if args.only is None or args.only == key:
                progress(f"backward (windowed heads, {mname})", bw.name)
                bst, bflops, bbytes = run_backward_windowed(torch, rat, bw, args.steps, 2, mode)
                extra[key] = {"train_tokens_per_s": bw.B * bw.T / (bst["median"] / 1e3),
                              **stats_fields("backward", bst, nbytes=bbytes, flops=bflops),
                              "algorithmic_flops": bflops, "algorithmic_bytes": bbytes,
                              "config": dict(bw.describe(), recurrence=mname)}

    if ms is None:  # a profiling run of one extra workload
        print(json.dumps({"extra": extra}))
        return

    scan_ms, attn_ms = scan_st["median"], attn_st["median"]
    scan_gbs = scan_bytes / (scan_ms / 1e3) / 1e9
    attn_gbs = attn_bytes / (attn_ms / 1e3) / 1e9
    if scan_ms >= attn_ms:
        dom_bytes, dom_st, dom_kernel = scan_bytes, scan_st, SCAN_KERNEL
    else:
        dom_bytes, dom_st, dom_kernel = attn_bytes, attn_st, ATTN_KERNEL
    dom_ms = dom_st["median"]
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    progress("device copy of", dom_bytes, "bytes (achievable HBM rate)")
    copy_st = run_copy_reference(torch, dom_bytes, args.steps)
    copy_ms = copy_st["median"]
    copy_gbs = dom_bytes / (copy_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(dom_kernel),
                "kernel": dom_kernel, "algorithmic_bytes_per_launch": dom_bytes,
                "kernel_ms": round(dom_ms, 4), "kernel_ms_p10": round(dom_st["p10"], 4),
                "kernel_ms_p90": round(dom_st["p90"], 4), "launches_timed": dom_st["n"],
                "timing": "median of per-launch HIP event pairs on the launch stream",
                "copy_reference": {"GBps": round(copy_gbs, 1), "ms": round(copy_ms, 4),
                                   "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                                   "kernel_frac_of_copy": round(achieved / copy_gbs, 4),
                                   "what": "torch copy_ of the same byte count (half read, half written), "
                                           "3 rotating buffer sets"}}
    line = {
        "metric": "prefill tokens/s per layer and decode tokens/s at D=16/64; % HBM / MFMA peak",
        "value": w.B * w.T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": w.describe(),
        "roofline": roofline,
        "kernels": {
            SCAN_KERNEL: {**stats_fields("scan", scan_st, nbytes=scan_bytes), "algorithmic_bytes": scan_bytes},
            ATTN_KERNEL: {**stats_fields("attn", attn_st, nbytes=attn_bytes, flops=attn_flops),
                          "algorithmic_bytes": attn_bytes, "algorithmic_flops": attn_flops},
        },
        "wall_s_timed": wall,
        "sources_hash": profiling.kernel_sources_hash(),
    }
    if extra:
        line["extra"] = extra
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle), headline step")
        line["cpu_baseline"] = cpu_baseline(w)
        if not args.no_extra:
            progress("cpu baseline (oracle), per workload and stage")
            line["cpu_baseline"]["per_config"] = cpu_baseline_per_config()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
