#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X: tokens/s per layer plus the roofline
fraction of the dominant kernel, with the CPU oracle timed beside it.

    python bench.py [--steps K] [--warmup W]
                    [--workload default|decode1|decode16|prefill|skewed|decode1_q4|prefill_q4|decode1_mix|
                                prefill_mix|decode1_q56|prefill_q56|decode1_cached|prefill_cached|tiny|all]

A step is one whole layer call (router -> top-k -> permute -> gate/up+SwiGLU ->
down -> combine [+ shared expert]) on one batch of synthetic tokens whose
inputs are already resident in HBM.  Decode workloads rotate over several
copies of the layer's packed experts and over fresh token batches so the
2.1 GB of expert weights (3.7 GB with 4-bit codes: the *_q4 workloads; 2.7 GB
with 2-bit gate/up and 4-bit down: the *_mix workloads; 5.3 GB with 5-bit
gate/up and 6-bit down, both in 6-bit units: the *_q56 workloads) stream
from HBM rather than from the 256 MB Infinity Cache.

The default prints ONE JSON line: the one-token decode workload as the
headline (value, roofline, cpu_baseline), with the 16-token decode and the
2048-token prefill workloads of the same metric nested under "workloads"
(each timed for the same --steps/--warmup).  Every HBM-bound roofline also
carries the rate of a plain streaming read of the same number of bytes on
the same GPU (read_ceiling).  --workload NAME prints NAME's line alone;
--workload all one line per workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
PCIE_PEAK_GBS = 64.0           # host link, PCIe 5.0 x16, one direction, GB/s
GRAPH_STEPS = 64               # at most this many layer calls per captured graph
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16/bf16 MFMA, TFLOP/s

DEFAULTS = {  # workload: (steps, warmup, layer copies, token batches)
    "tiny": (2000, 100, 1, 16),
    "decode1": (2000, 200, 4, 64),
    "decode16": (1000, 100, 4, 64),
    "prefill": (50, 5, 1, 4),
    "skewed": (20, 3, 1, 2),
    "decode1_q4": (2000, 200, 4, 64),
    "prefill_q4": (50, 5, 1, 4),
    "decode1_mix": (2000, 200, 4, 64),
    "prefill_mix": (50, 5, 1, 4),
    "decode1_q56": (2000, 200, 4, 64),
    "prefill_q56": (50, 5, 1, 4),
    "decode1_cached": (1000, 300, 1, 1024),
    "prefill_cached": (20, 3, 1, 8),
}
NESTED = ("decode16", "prefill")    # the metric's other two workloads, nested in the default line
NESTED_KEYS = ("value", "unit", "steps", "warmup", "ms_per_step", "config", "roofline", "layer_roofline",
               "kernel_ms", "launch", "ms_per_step_percentiles", "ms_per_step_eager")
# 80 % of the 256 experts (the pages' automatic cache budget)
CACHE_SLOTS = {"decode1_cached": 204, "prefill_cached": 204}


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "quantized_routed_moe_router_amd", "csrc")
PROFILES = os.path.join(HERE, "profiles")


def source_hash() -> str:
    """sha256 over the HIP sources and the build script (its compiler flags), so counter figures
    taken on other kernels are not reused."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    with open(os.path.join(os.path.dirname(CSRC), "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def roofline_kernel(mode_decode: bool, T: int) -> str:
    if not mode_decode:
        return "k_moe_gemm_wide"
    return "k_gateup_dec_lds" if T <= 4 else "k_gateup_dec_sh"


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None
    when there is none or the HIP sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0] in ("source_sha256", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("source_sha256") != source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def copy_calibration(mib: int, reps: int) -> dict:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters to bytes (run it under rocprofv3 --pmc)."""
    import torch
    n = mib << 20
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_calibration": True, "bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": reps,
            "source_sha256": source_hash()}


def cpu_baseline(L, budget_s: float) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    small batches are repeated over fresh token batches of the workload,
    large ones are taken in growing token prefixes, until about budget_s of
    CPU time has been spent."""
    import oracle
    import synth
    T, wl = L.T, L.wl
    done, spent, what = 0, 0.0, ""
    if T <= 16:
        b = 0
        while spent < budget_s and b < 4096:
            Lb = L if b == 0 else synth.derive(L, wl, batch=b)
            t0 = time.perf_counter()
            oracle.layer_inputs(Lb)
            spent += time.perf_counter() - t0
            done += T
            b += 1
        what = f"{b} token batches of {T} (batch 0 the benchmarked one, then fresh draws of the same recipe)"
    else:
        n = 1
        while True:
            t0 = time.perf_counter()
            oracle.layer_inputs(L, tokens=list(range(n)))
            dt = time.perf_counter() - t0
            if dt >= budget_s or n >= T:
                break
            n = min(T, max(n + 1, int(n * min(8.0, 1.2 * budget_s / max(dt, 1e-3)))))
        done, spent = n, dt
        what = f"first {n} of the {T} tokens of one batch"
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": done / spent, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{L.wl.name}: {what}, full layer (fp64 C, OpenMP), {spent:.1f} s", "cpu_model": model}


def library_gemm_reference(n: int = 8192, reps: int = 10) -> dict:
    """Context for the MFMA fraction: a dense fp16 GEMM through the vendor
    library (torch.matmul), n x n x n, on the same GPU."""
    import torch
    a = torch.randn(n, n, dtype=torch.float16, device="cuda:0")
    b = torch.randn(n, n, dtype=torch.float16, device="cuda:0")
    torch.matmul(a, b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return {"shape": f"{n}x{n}x{n} fp16", "TFLOP/s": round(2.0 * n ** 3 / dt / 1e12, 1)}


_BASE_LAYERS = {}


def base_layer(name: str, seed: int):
    """Inputs of one layer, generated once per process (the H=4096 workloads
    share one layer: router and expert weights)."""
    import synth
    if (name, seed) not in _BASE_LAYERS:
        _BASE_LAYERS[(name, seed)] = synth.make_layer(name, seed=seed)
    return _BASE_LAYERS[(name, seed)]


def read_ceiling(nbytes: int, reps: int = 24) -> dict:
    """The best rate of the library's plain streaming read (ds4moe_read_probe)
    over `nbytes`, each launch reading another slice of a pool of at least
    4 GiB so that no launch finds its bytes in the 256 MB Infinity Cache;
    kernel durations from events stamped by the kernel's own dispatch
    (the first launches of each grid size are dropped), best over a few
    grid sizes."""
    import torch
    from quantized_routed_moe_router_amd import binding as B
    nbytes = max(16, nbytes // 256 * 256)
    pool = max(4 << 30, 2 * nbytes)
    buf = torch.zeros(pool, dtype=torch.uint8, device="cuda:0")
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")
    nslot = pool // nbytes
    best = None
    for wg in (1024, 2048, 4096, 8192):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:  # torch creates the hipEvents on first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        for r in range(reps):
            off = (r % nslot) * nbytes
            B.ds4moe_read_probe(buf[off:off + nbytes], nbytes, wg, sink, evs[r])
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs[4:]]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, wg, ms)
    del buf, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "GBs": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4),
            "kernel": "k_stream_read", "workgroups": best[1], "ms": round(best[2], 5)}


def run_workload(name: str, args) -> dict:
    import torch

    import quantized_routed_moe_router_amd as q
    from quantized_routed_moe_router_amd import binding as B
    import synth

    steps, warmup, n_layers, n_batches = DEFAULTS[name]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    n_layers = args.layers if args.layers is not None else n_layers
    cached = name in CACHE_SLOTS
    wname = name[: -len("_cached")] if cached else name
    wl = synth.WORKLOADS[wname]
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    base = base_layer("prefill" if wl.layer_id == 1 else wname, args.seed)
    L = synth.derive(base, wname) if wl.layer_id == 1 else base
    dl = q.from_layer_inputs(L, dev)
    if cached:  # experts in pinned host memory, a slot cache in HBM (which also defeats the MALL)
        n_layers = 1
        S = CACHE_SLOTS[name]
        cache = q.ExpertCache(dl, S)
    layers = [dl.weights()]
    copies = []
    for i in range(1, n_layers):  # same bytes at other HBM addresses
        g, u, d = dl.gate.clone(), dl.up.clone(), dl.down.clone()
        copies.append((g, u, d))
        layers.append(dl.weights(g, u, d))
    xs = [dl.x_tensor(synth.make_x(wl, args.seed, L.T, batch=b)) for b in range(n_batches)]
    T = L.T
    mode = q.MODE_DECODE if T <= 16 else q.MODE_PREFILL
    y = torch.empty(T, wl.H, dtype=torch.float32, device=dev)
    ws = dl.workspace(T, mode)
    fwd0 = q.ds4moe_forward_decode if mode == q.MODE_DECODE else q.ds4moe_forward_prefill
    if cached and mode == q.MODE_DECODE:
        cw = cache.weights()

        def fwd(dims, w, x, T_, y_, r_, ws_, n_, st_, events=None):
            B.ds4moe_forward_decode_cached(dims, cw, S, cache.buf, cache.nbytes, x, T_, y_, r_, ws_, n_, events, st_)
    elif cached:  # no per-kernel events: fill, gate/up and down run once per batch of experts
        cw = cache.weights()

        def fwd(dims, w, x, T_, y_, r_, ws_, n_, st_, events=None):
            B.ds4moe_forward_prefill_cached(dims, cw, S, cache.buf, cache.nbytes, x, T_, y_, r_, ws_, n_, st_)
    else:
        def fwd(dims, w, x, T_, y_, r_, ws_, n_, st_, events=None):
            if events is None:
                fwd0(dims, w, x, T_, y_, r_, ws_, n_, st_)
            else:
                B.ds4moe_forward_timed(mode, dims, w, x, T_, y_, r_, ws_, n_, events, st_)
    stream = torch.cuda.current_stream(dev)
    setup_s = time.perf_counter() - t0

    # experts hit by each batch (for the algorithmic bytes of decode steps)
    distinct = []
    for b in range(n_batches):
        rt = dl.route(xs[b])
        distinct.append(int((rt["counts"] > 0).sum().item()))

    def step(i, events=None):
        w = layers[i % n_layers]
        x = xs[i % n_batches]
        fwd(dl.dims, w, x, T, y, None, ws, ws.numel(), stream, events)

    steps_eager = steps
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t1

    # The timed loop: a HIP graph holding `glen` consecutive layer calls (the
    # same rotation over layer copies and token batches), replayed; the library
    # enqueues kernels only, so a capture holds the whole layer.
    # (exactly `steps` calls: the graph length is the largest divisor of steps <= GRAPH_STEPS)
    # Through the expert cache the timed loop stays eager: a replayed graph would
    # repeat its token batches, whose experts the cache then already holds.
    glen = 0 if (args.no_graph or cached) else max(d for d in range(1, min(GRAPH_STEPS, steps) + 1)
                                                   if steps % d == 0)
    if glen:
        reps = steps // glen
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(glen):
                    w = layers[i % n_layers]
                    x = xs[i % n_batches]
                    fwd(dl.dims, w, x, T, y, None, ws, ws.numel(), cap)
        torch.cuda.current_stream(dev).wait_stream(cap)
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t1
        # spread: a second pass of the same replays with an event between
        # replays (outside the timed region); per-step time of each replay
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        marks[0].record()
        for r in range(reps):
            graph.replay()
            marks[r + 1].record()
        torch.cuda.synchronize()
        rep_ms = np.array([marks[r].elapsed_time(marks[r + 1]) / glen for r in range(reps)])
        pct = {f"p{q}": round(float(np.percentile(rep_ms, q)), 5) for q in (10, 50, 90)}
        pct["over"] = f"{reps} replays of {glen} steps"
        del graph
        if reps < 10:  # too few replays: eager steps, an event between steps
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            marks[0].record()
            for i in range(steps):
                step(i)
                marks[i + 1].record()
            torch.cuda.synchronize()
            st_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
            pct = {f"p{q}": round(float(np.percentile(st_ms, q)), 5) for q in (10, 50, 90)}
            pct["over"] = f"{steps} eager steps"
    else:
        elapsed = elapsed_eager
        pct = None
        if cached:  # spread over the eager steps (an extra pass, an event between steps)
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            marks[0].record()
            for i in range(steps):
                step(i)
                marks[i + 1].record()
            torch.cuda.synchronize()
            st_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
            pct = {f"p{q}": round(float(np.percentile(st_ms, q)), 5) for q in (10, 50, 90)}
            pct["over"] = f"{steps} eager steps"

    # second pass with per-kernel events stamped by each kernel's own dispatch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * B.N_TIMED_KERNELS)] for _ in range(steps_eager)]
    for row in ev:  # torch creates the underlying hipEvent on first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    # a marker before each step: a slot whose start event precedes it was not
    # launched in that step (its events keep the stamps of the pass above)
    pre = [torch.cuda.Event(enable_timing=True) for _ in range(steps_eager)]
    stats0 = cache.stats() if cached else None
    t2 = time.perf_counter()
    for i in range(steps_eager):
        pre[i].record(stream)
        step(i, ev[i])
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t2
    stats1 = cache.stats() if cached else None
    stage_ms = {s: 0.0 for s in B.KERNEL_SLOTS}
    stage_n = {s: 0 for s in B.KERNEL_SLOTS}
    per_step_gateup = []
    for i in range(steps_eager):
        for j, s in enumerate(B.KERNEL_SLOTS):
            if pre[i].elapsed_time(ev[i][2 * j]) < 0.0:
                continue
            dt = ev[i][2 * j].elapsed_time(ev[i][2 * j + 1])
            stage_ms[s] += dt
            stage_n[s] += 1
            if s == "gateup":
                per_step_gateup.append(dt)
    stage_ms = {s: (v / stage_n[s] if stage_n[s] else None) for s, v in stage_ms.items()}

    H, I, E, k = wl.H, wl.I, wl.E, wl.k
    gu_bytes = dl.gu_bytes
    rk = roofline_kernel(mode == q.MODE_DECODE, T)
    cache_info = None
    if cached:
        # the fill kernel is bound by the host link: expert bytes copied per launch / its duration
        misses = stats1[2] - stats0[2]
        hits = stats1[1] - stats0[1]
        fill_bytes = misses * (2 * gu_bytes + dl.d_bytes)
        if mode == q.MODE_DECODE:
            fill_s = stage_ms["cache_fill"] * steps_eager * 1e-3
            kern = "k_cache_fill"
        else:  # the whole step (fills and expert kernels in stream order): a lower bound of the fill rate
            fill_s = elapsed_ev
            kern = "k_cache_fill, over the whole step (expert kernels serialised with the fills)"
        achieved = fill_bytes / fill_s / 1e9
        roof = {"bound": "pcie", "achieved": round(achieved, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None, "kernel": kern,
                "algorithmic_bytes_per_step": fill_bytes / steps_eager}
        cache_info = {"slots": S, "experts": E, "hit_rate": round(hits / max(1, hits + misses), 4),
                      "misses_per_step": round(misses / steps_eager, 3),
                      "host_bytes": E * (2 * gu_bytes + dl.d_bytes)}
        layer = None
    elif mode == q.MODE_DECODE:
        # gate + up packed bytes of the experts each step touches
        gu_total = sum(2 * gu_bytes * distinct[i % n_batches] for i in range(steps_eager))
        achieved = gu_total / (sum(per_step_gateup) * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(rk, name),
                "kernel": rk, "algorithmic_bytes_per_launch": gu_total / steps_eager}
        if not args.no_read_ceiling:
            rc = read_ceiling(int(gu_total / steps_eager))
            roof["read_ceiling"] = rc
            roof["frac_of_read_ceiling"] = round(achieved / rc["GBs"], 4)
        layer_bytes = np.mean([d * (2 * gu_bytes + dl.d_bytes) for d in distinct]) + E * H * 2 + T * H * (2 + 4)
        layer = {"bytes_per_step": float(layer_bytes),
                 "achieved_GBs": round(layer_bytes / (elapsed / steps) / 1e9, 1),
                 "frac": round(layer_bytes / (elapsed / steps) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        flops = 2.0 * T * k * 2 * H * I
        achieved = flops / (stage_ms["gateup"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFS, 4), "traffic": measured_traffic(rk, name),
                "kernel": rk + " (gate/up + SwiGLU)", "algorithmic_flops_per_launch": flops}
        lf = 2.0 * T * k * 3 * H * I + (2.0 * T * 3 * H * wl.Is if wl.Is else 0.0)
        layer = {"flops_per_step": lf, "achieved_TFs": round(lf / (elapsed / steps) / 1e12, 2),
                 "frac": round(lf / (elapsed / steps) / 1e12 / MFMA_F16_PEAK_TFS, 4)}

    out = {
        "metric": "MoE-layer tokens/s", "value": round(T * steps / elapsed, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(elapsed / steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "operands": {"x": wl.x_dtype, "router": f"{wl.router_dtype} weights, fp64 accumulation",
                     "routed_experts": f"{wl.bits}-bit gate/up and {wl.down_width}-bit down codes in 256-weight "
                                       "super-blocks (fp16 d, dmin)",
                     "expert_products": "f16 x f16 -> f32 MFMA (exact code*scale, fp16 activations)",
                     "shared_expert": "bf16 weights as f16 operands" if wl.Is else None, "y": "f32"},
        "data": "synthetic",
        "config": {"workload": name, "T": T, "hidden": H, "inter": I, "experts": E, "top_k": k,
                   **({"expert_cache": cache_info} if cache_info else {}),
                   "shared_inter": wl.Is, "expert_bits": wl.bits, "down_bits": wl.down_width,
                   "layer_copies": n_layers,
                   "token_batches": n_batches,
                   "seed": args.seed, "distinct_experts_mean": float(np.mean(distinct))},
        "roofline": roof,
        "layer_roofline": layer,
        "kernel_ms": {s: round(v, 5) for s, v in stage_ms.items() if v is not None},
        "launch": f"hip graph of {glen} layer calls, replayed" if glen else "eager launches",
        "ms_per_step_percentiles": pct,
        "ms_per_step_eager": round(elapsed_eager / steps_eager * 1e3, 5),
        "ms_per_step_with_kernel_events": round(elapsed_ev / steps_eager * 1e3, 5),
        "setup_s": round(setup_s, 1),
    }
    if mode != q.MODE_DECODE and not args.no_gemm_reference and not cached:
        out["roofline"]["library_fp16_gemm_reference"] = library_gemm_reference()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    if cached:
        del cache, cw
    del copies, xs, dl
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="default", choices=["default", *DEFAULTS, "all"])
    ap.add_argument("--layers", type=int, default=None, help="rotated copies of the packed experts")
    ap.add_argument("--seed", type=int, default=20261203)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measured beside each HBM roofline")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the library fp16 GEMM reference run (prefill workloads)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is benchmarked on a single MI355X "
              "(no sharding, no collectives); run it without --gpus or with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration, args.steps or 10)), flush=True)
        return
    if args.workload == "default":
        head = run_workload("decode1", args)
        sub = argparse.Namespace(**{**vars(args), "no_cpu_baseline": True})
        head["workloads"] = {}
        for n in NESTED:
            r = run_workload(n, sub)
            head["workloads"][n] = {k: r[k] for k in NESTED_KEYS if k in r}
        print(json.dumps(head), flush=True)
        return
    names = [n for n in DEFAULTS if n != "tiny"] if args.workload == "all" else [args.workload]
    for n in names:
        print(json.dumps(run_workload(n, args)), flush=True)


if __name__ == "__main__":
    main()
