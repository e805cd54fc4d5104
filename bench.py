#!/usr/bin/env python3
"""Benchmark of the paged KV attention hot path on one MI355X.

Default run (``python bench.py``): one JSON line whose headline is the
Qwen3-4B-shaped decode step at batch 64 (Hq 32 / Hkv 8 / head_dim 128, bf16,
page size 16, cached lengths U{512..1024}, pages shuffled over a pool 1.25x
the pages needed), one appended token per sequence, over 36 independent layer
caches (36 x 254 MB of pools, far more than the 256 MB last-level cache, so
every layer's K/V comes from HBM).  One step = one pkv_decode_plan launch
(the cut of the step's work, shared by its layers), then for each of the 36
layers one pkv_append_decode_attn launch (append + attend); ``--no-plan``
leaves the plan out, so that every layer's launch cuts the work itself.  The
same line carries a
nested ``prefill`` object with the causal paged prefill at head_dim 256,
Hq 48 / Hkv 8: the single request q_len = kv_len = 1023 and a random batch of
8 requests (q_len U{65..4096}, kv_len = q_len + U{0..4096}), each step being
8 layers with their own pools and inputs; and a nested ``mixed`` object: a
serving step of the decode shape with 4 prompt chunks next to 64 decode rows,
one pkv_mixed_attn launch per layer against the two separate launches.

Every step is captured once in a HIP graph and replayed (``--eager`` launches
it from Python instead).  All inputs are resident in HBM before the timed
region.  W warmup steps, then exactly K timed steps between two
synchronisations; HIP events recorded between the steps on the launch stream
give the per-step median and best next to the mean.

Each workload reports a roofline object for its dominant kernel (its
per-launch duration from the HIP events of the timed region) and the CPU
oracle timed on a bounded sample of the same workload on the host cores (and
on one core).

``--workload decode|sweep|long|prefill|mixed`` with ``--batch B`` times one
workload only; ``--page-size``, ``--layout`` and ``--contiguous`` change the
pool of the decode and prefill workloads.

``--workload tune`` is the tuning sweep: for the decode step (batch 64 and
the batch-8 / batch-32 sweep shapes) it times the step with one
pkv_decode_plan, split-worker counts, page sizes, the NHD layout and
contiguous pages, and for prefill the two head_dim
256 tilings, each scored on whole-step time (all layers, HIP graph) and
timed in alternation with the library's default configuration on the same
inputs (the control), so that drift between measurements shows up in the
control's own spread.  It prints one JSON line per workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s
CPU_THREADS_MAX = 16           # host threads of one GPU's share of the box


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None, choices=["decode", "sweep", "long", "prefill", "mixed", "tune"],
                   help="time one workload only (default: decode B=64 plus the two prefill cases)")
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--layers", type=int, default=36, help="decode: layer caches per step")
    p.add_argument("--prefill-layers", type=int, default=8,
                   help="prefill: layers per step, each with its own pools and inputs")
    p.add_argument("--eager", action="store_true", help="launch from Python instead of replaying a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=6.0,
                   help="target CPU time of each oracle sample on all host threads")
    p.add_argument("--cpu-seconds-1t", type=float, default=2.0,
                   help="target CPU time of each oracle sample on one thread")
    p.add_argument("--workers", type=int, default=0, help="decode split workers (0 = library default)")
    p.add_argument("--prefill-rows", type=int, default=0,
                   help="prefill query rows per workgroup (0 = library default, 128, 192)")
    p.add_argument("--separate", action="store_true",
                   help="decode step as pkv_append + pkv_decode_attn (two launches) instead of the fused "
                        "pkv_append_decode_attn")
    p.add_argument("--decode-heads", default=None,
                   help="decode/sweep/long: HQ,HKV,D in place of the Qwen3 shape 32,8,128 (same lengths and pages)")
    p.add_argument("--no-plan", action="store_true",
                   help="decode: no pkv_decode_plan per step (every call cuts the work itself)")
    p.add_argument("--q-len", default=None,
                   help="prefill: query rows of each request (comma list; with --kv-len) instead of the "
                        "q = kv = 1023 request or a random batch")
    p.add_argument("--kv-len", default=None, help="prefill: keys of each request (comma list, kv >= q)")
    p.add_argument("--head-dim", type=int, default=256, help="prefill: head_dim (64, 128 or 256)")
    p.add_argument("--hq", type=int, default=48, help="prefill: query heads")
    p.add_argument("--hkv", type=int, default=8, help="prefill: KV heads")
    p.add_argument("--page-size", type=int, default=16, help="decode/prefill: tokens per page (16 .. 256)")
    p.add_argument("--layout", default="HND", choices=["HND", "NHD"], help="decode/prefill: pool layout")
    p.add_argument("--contiguous", action="store_true",
                   help="decode/prefill: deal every sequence a run of adjacent pages instead of shuffled pages")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


# --------------------------------------------------------------------------
# accounting
# --------------------------------------------------------------------------

def decode_bytes(spec, fused=False) -> dict:
    """Algorithmic bytes of one decode call: K and V of exactly the attended
    tokens, q and out, the table entries the rows touch, the lengths; with
    the append fused in, also the new token's K and V read and written into
    the pool and the new lengths written."""
    es = 2 if spec.dtype == "bf16" else 4
    n = [int(x) + spec.n_new for x in spec.hist_lens]
    kv = sum(n) * spec.hkv * spec.head_dim * 2 * es
    qo = 2 * spec.batch * spec.hq * spec.head_dim * es
    table = 4 * sum(-(-x // spec.page_size) for x in n) + 4 * spec.batch
    app = 2 * 2 * spec.batch * spec.hkv * spec.head_dim * es + 4 * spec.batch if fused else 0
    return {"kv": kv, "q_out": qo, "table": table, "append": app, "total": kv + qo + table + app}


def prefill_flops(spec) -> int:
    """4 * head_dim * Hq * causal pairs, pairs per request q (2 kv - q + 1) / 2."""
    pairs = sum(int(q) * (2 * int(kv) - int(q) + 1) // 2 for q, kv in zip(spec.q_lens, spec.kv_lens))
    return 4 * spec.head_dim * spec.hq * pairs


# the source files each profiled kernel is compiled from: a counter summary
# counts only while all of them are unchanged
KERNEL_SOURCES = {
    "decode": ["decode.hip", "decode_worker.hpp", "common.hpp", "internal.hpp"],
    "prefill": ["prefill.hip", "common.hpp", "internal.hpp"],
    "mixed": ["prefill.hip", "common.hpp", "internal.hpp"],
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_attention_pkv_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kind: str, name: str):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing or was taken on another version of the kernel's sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash(kind):
        return None
    return float(t.group(1))


def device_info(torch, props) -> dict:
    """The GPU the line was measured on: name, ISA, CU count, HIP runtime of
    the torch build, and the clock and L2 size where torch reports them."""
    d = {"name": props.name, "arch": getattr(props, "gcnArchName", "?"), "cus": props.multi_processor_count,
         "hip": getattr(torch.version, "hip", None)}
    for key in ("clock_rate", "L2_cache_size", "total_memory"):
        v = getattr(props, key, None)
        if v is not None:
            d[key] = v
    return d


def parity(gpu, ref, dtype: str, what: str) -> dict:
    """Element-wise |gpu - ref| <= atol + rtol |ref| of a GPU output (widened
    exactly) against the oracle's fp64 result, at the bar of the output dtype
    (bf16: 2e-2 / 2e-2, fp32: 1e-5 / 1e-5)."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_common import BF16_TOL, F32_TOL

    atol, rtol = BF16_TOL if dtype == "bf16" else F32_TOL
    g = gpu.float().double().numpy()
    r = np.asarray(ref, dtype=np.float64).reshape(g.shape)
    err = np.abs(g - r)
    return {"what": what, "elements": int(g.size), "max_abs_err": float(np.max(err)),
            "max_rel_err": float(np.max(err / np.maximum(np.abs(r), 1e-30))), "atol": atol, "rtol": rtol,
            "pass": bool(np.all(err <= atol + rtol * np.abs(r)))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------

def events_per_call(torch, calls, reps=3):
    """Mean device time of each call, bracketed by HIP events on the launch
    stream.  A GPU spin is queued first so that every launch is enqueued
    before the device reaches it (no host gaps inside the brackets)."""
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(40e6))
        except Exception:  # noqa: BLE001 - spin helper missing: brackets may include host gaps
            pass
        for (e0, e1), c in zip(ev, calls):
            e0.record(stream)
            c()
            e1.record(stream)
        torch.cuda.synchronize()
        times.extend(e0.elapsed_time(e1) for e0, e1 in ev)
    times.sort()
    return sum(times) / len(times), times[len(times) // 2]


def time_steps(torch, step, steps, warmup, use_graph):
    """Mean ms per step over exactly `steps` timed steps after `warmup`, and
    the per-step times from events recorded between the steps."""
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
    else:
        run = step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def spread(per, scale=1.0, nd=2):
    """Median and best of per-step times, scaled."""
    return {"median": round(statistics.median(per) * scale, nd), "best": round(min(per) * scale, nd),
            "rounds": len(per)}


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def bench_decode(args, torch, pkv, wl, workload):
    kw = dict(page_size=args.page_size, layout=args.layout, contiguous=args.contiguous,
              heads=tuple(int(x) for x in args.decode_heads.split(",")) if args.decode_heads else None)
    if workload == "decode":
        spec = wl.decode_spec("qwen3_decode", batch=args.batch or 64, **kw)
    elif workload == "sweep":
        spec = wl.decode_spec("qwen3_sweep", batch=args.batch or 64, **kw)
    else:
        spec = wl.decode_spec("long_ragged", batch=args.batch or 256, **kw)
    dev = torch.device("cuda:0")
    L = args.layers
    fused = not args.separate and spec.dtype == "bf16"
    acc = decode_bytes(spec, fused)
    if workload == "long":
        free = torch.cuda.mem_get_info(dev)[0]
        per_layer = 2 * spec.num_pages * spec.hkv * spec.page_size * spec.head_dim * 2
        # room for one layer's fp32 input draws on top of the pools
        spare = 4 * int(spec.hist_lens.sum()) * spec.hkv * spec.head_dim * 4 + (8 << 30)
        fit = int((free - spare) // per_layer)
        if fit < L:
            log(f"only {fit} layer caches fit in device memory; using {fit}")
            L = max(1, fit)
    log(f"[bench] {spec.name}: {L} layers, {spec.num_pages} pages/pool, KV/call {acc['kv'] / 1e6:.1f} MB")
    bt = torch.from_numpy(spec.block_table).to(dev)
    hist = torch.from_numpy(spec.hist_lens).to(dev)
    zeros = torch.zeros_like(hist)
    lens = torch.empty_like(hist)
    max_kv = int(spec.hist_lens.max()) + spec.n_new
    workspace = None
    layers = []
    # every layer's pools first, so the input draws below (freed after each
    # layer) do not split the pools' memory into unusable pieces
    pools = [(wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)) for _ in range(L)]
    for layer in range(L):
        inp = wl.decode_inputs(spec, device=dev, seed_offset=layer)
        kc, vc = pools[layer]
        if workspace is None:
            ws_bytes = pkv.decode_workspace_bytes(kc, spec.batch, spec.hq, max_kv, layout=spec.layout,
                                                  workers=args.workers)
            workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, bt, zeros, inp.hist_indptr, layout=spec.layout)
        out = torch.empty_like(inp.q)
        if layer == 0:
            out0 = out
        if fused:
            app = None
            dec = pkv.api.prepare_append_decode(inp.q, kc, vc, inp.k_new, inp.v_new, bt, hist, max_kv, spec.scale,
                                                out, workspace, seqlens_out=lens, layout=spec.layout,
                                                workers=args.workers)
        else:
            app = pkv.api.prepare_append(kc, vc, inp.k_new, inp.v_new, bt, hist, lens, layout=spec.layout)
            dec = pkv.api.prepare_decode(inp.q, kc, vc, bt, lens, max_kv, spec.scale, out, workspace,
                                         layout=spec.layout, workers=args.workers)
        layers.append((app, dec))
        del inp
    # the cut of the step's work, computed once for all its layers (the
    # lengths every decode call sees: pre-append when fused, else those the
    # first append writes)
    plan = None
    if not args.no_plan:
        plan = pkv.api.prepare_decode_plan(pools[0][0], hist if fused else lens, spec.hq, max_kv, workspace,
                                           fused=fused, layout=spec.layout, workers=args.workers)
    del pools
    torch.cuda.synchronize()

    def step():
        for n, (app, dec) in enumerate(layers):
            if app is not None:
                app()
            if n == 0 and plan is not None:
                plan()
            dec()

    ms, per = time_steps(torch, step, args.steps, args.warmup, not args.eager)
    step()  # lens is live again for the per-call brackets below
    dec_mean, _ = events_per_call(torch, [d for _, d in layers])
    app_mean = None if fused else events_per_call(torch, [a for a, _ in layers])[0]
    plan_ms = 0.0 if plan is None else events_per_call(torch, [plan])[0]
    kv_bytes_step = acc["kv"] * L
    value = kv_bytes_step / (ms * 1e-3) / 1e9
    # the kernel's average launch duration: in the fused step the timed region
    # holds exactly L launches of it and the plan launch (HIP events around
    # the graph replays, less the plan launch's own event bracket); in the
    # two-launch step, per-call event brackets of the decode launches
    launch_ms = (ms - plan_ms) / L if fused else dec_mean
    achieved = acc["total"] / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile("decode", f"decode_kernel_{spec.name}_pmc.txt") if fused else None
    result = {
        "metric": "paged decode attn: KV-read GB/s (% HBM peak) + us/call at B=64, Hq32/Hkv8/D128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "hq": spec.hq, "hkv": spec.hkv,
                   "head_dim": spec.head_dim, "page_size": spec.page_size, "layout": spec.layout,
                   "pages": "contiguous" if args.contiguous else "shuffled", "layers": L,
                   "mean_attended_len": round(float(spec.hist_lens.mean()) + spec.n_new, 1),
                   "step": ("per layer: pkv_append_decode_attn (append 1 token/seq + attend, one launch)"
                            if fused else "per layer: pkv_append(1 token/seq) + pkv_decode_attn")
                   + ("; once per step: pkv_decode_plan" if plan is not None else ""),
                   "launch": "eager" if args.eager else "hip graph", "parallelism": "none (1 GPU)"},
        "us_per_call": round(ms * 1e3 / L, 2),
        "us_per_call_over_steps": spread(per, 1e3 / L),
        "value_over_steps": {"median": round(kv_bytes_step / (statistics.median(per) * 1e-3) / 1e9, 1),
                             "best": round(kv_bytes_step / (min(per) * 1e-3) / 1e9, 1), "rounds": len(per)},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "decode_us_per_call_events": round(dec_mean * 1e3, 2),
        "append_us_per_call_events": None if app_mean is None else round(app_mean * 1e3, 2),
        "plan_us_per_step_events": None if plan is None else round(plan_ms * 1e3, 2),
        "kernel_us_per_launch": round(launch_ms * 1e3, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "decode_bf16_kernel (one launch per pkv_append_decode_attn)" if fused
                     else "decode kernel (one launch per pkv_decode_attn)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_unit": "HBM bytes per launch", "bytes_per_launch": acc["total"]},
    }
    gpu_out0 = out0.cpu()  # layer 0's output after the timed steps (every step computes the same)
    del layers, workspace, out0
    return result, spec, gpu_out0


def _timed_loop(fn, seconds, min_calls=1):
    """Call fn(i) until about `seconds` have been spent; (calls, seconds, sum of its returns)."""
    spent, calls, total = 0.0, 0, 0
    while spent < seconds or calls < min_calls:
        t0 = time.perf_counter()
        total += fn(calls)
        spent += time.perf_counter() - t0
        calls += 1
    return calls, spent, total


def cpu_baseline_decode(args, spec, gpu_out0=None):
    """The oracle (as is) on a bounded sample of the same workload: whole
    decode calls of the batch (host pools built by the oracle's own append
    from two layers' draws), on all host threads of the GPU's share, then on
    one thread.  With gpu_out0 (layer 0's output of the timed GPU step) the
    oracle's layer-0 call is also compared with it, every element."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import oracle
    from paged_kv_attention_pkv_amd import workloads as wl
    from gpu_common import host_bits, opool

    orc = oracle.load()
    threads = max(1, min(CPU_THREADS_MAX, os.cpu_count() or 1))
    pool = opool(spec)
    zeros = np.zeros(spec.batch, np.int32)
    hosts = []
    for layer in range(2):
        inp = wl.decode_inputs(spec, device="cuda:0", seed_offset=layer).to("cpu")
        kc = host_bits(wl.empty_pool(spec, "cpu")).copy()
        vc = kc.copy()
        orc.append(pool, kc, vc, host_bits(inp.k_hist), host_bits(inp.v_hist), spec.block_table, zeros,
                   inp.hist_indptr.numpy())
        lens = orc.append(pool, kc, vc, host_bits(inp.k_new), host_bits(inp.v_new), spec.block_table,
                          spec.hist_lens)
        hosts.append((host_bits(inp.q), kc, vc, lens))
    per_call = decode_bytes(spec)["kv"]

    def call(nt):
        def f(i):
            q, kc, vc, lens = hosts[i % len(hosts)]
            orc.decode(pool, q, kc, vc, spec.block_table, lens, spec.scale, nthreads=nt)
            return per_call
        return f

    calls, spent, done = _timed_loop(call(threads), args.cpu_seconds)
    calls1, spent1, done1 = _timed_loop(call(1), args.cpu_seconds_1t)
    res = {"value": round(done / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "value_1_thread": round(done1 / spent1 / 1e9, 4),
           "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
           "sample": f"{calls} decode calls of the same workload (all {spec.batch} sequences, two layers' draws "
                     f"in turn) on {threads} threads in {spent:.1f} s; {calls1} calls on 1 thread in "
                     f"{spent1:.1f} s; fp64 oracle, KV-read bytes per second"}
    if gpu_out0 is not None:
        q, kc, vc, lens = hosts[0]
        ref, _ = orc.decode(pool, q, kc, vc, spec.block_table, lens, spec.scale, nthreads=threads)
        res["parity"] = parity(gpu_out0, ref, spec.dtype, f"layer 0, all {spec.batch} x {spec.hq} output rows")
    return res


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def bench_prefill(args, torch, pkv, wl, spec):
    dev = torch.device("cuda:0")
    flops = prefill_flops(spec)
    L = max(1, args.prefill_layers)
    log(f"[bench] {spec.name}: {flops / 1e9:.2f} GFLOP per call, {L} layers per step")
    max_q, max_kv = int(spec.q_lens.max()), int(spec.kv_lens.max())
    zeros = torch.zeros(spec.batch, dtype=torch.int32, device=dev)
    calls, ws, need = [], None, 0
    for layer in range(L):
        # every layer its own pools, queries and outputs, as the layers of a model
        inp = wl.prefill_inputs(spec, device=dev, seed_offset=layer)
        kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
        lay = spec.layout
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, inp.block_table, zeros, inp.hist_indptr, layout=lay)
        kv_lens = pkv.append(kc, vc, inp.k_new, inp.v_new, inp.block_table, inp.hist_lens, inp.qo_indptr, layout=lay)
        out = torch.empty_like(inp.q)
        if layer == 0:
            out0 = out
        if ws is None:
            need = pkv.prefill_workspace_bytes(kc, spec.batch, spec.hq, int(spec.q_lens.sum()), max_q, max_kv,
                                               layout=lay)
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)  # counters start at zero
        calls.append(pkv.api.prepare_prefill(inp.q, kc, vc, inp.block_table, kv_lens, inp.qo_indptr, max_q,
                                             max_kv, spec.scale, out, ws, layout=lay,
                                             rows_per_workgroup=args.prefill_rows))
        del inp
    torch.cuda.synchronize()

    def step():
        for c in calls:
            c()

    ms, per = time_steps(torch, step, args.steps, args.warmup, not args.eager)
    mean = ms / L  # L launches per step: the timed region's HIP events give their average duration
    tfs = flops / (mean * 1e-3) / 1e12
    traffic = traffic_from_profile("prefill", f"prefill16{'' if spec.head_dim == 256 else 'r'}_kernel_{spec.name}_pmc.txt")
    # the tiling the library picks for this call, by the rule stated in
    # include/pkv.h (192 rows once ceil(total_q / 192) * Hq >= 1.5 * CUs at
    # head_dim 256, > CUs at 64 and 128), and its key splits: a workspace of
    # counters (256-byte aligned) then S records of 128 x (D + 2) fp32 per
    # (request, 128-row tile, head) workgroup
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tiling, splits = args.prefill_rows, 1
    if tiling == 0:
        units = spec.batch * (-(-max_q // 128)) * spec.hq
        wgs192 = -(-int(spec.q_lens.sum()) // 192) * spec.hq
        if need:
            tiling, splits = 128, (need - (-(-units * 4 // 256)) * 256) // (units * 128 * (spec.head_dim + 2) * 4)
        elif spec.head_dim != 256:
            tiling = 192 if wgs192 > cus else 128
        else:
            tiling = 192 if 2 * wgs192 >= 3 * cus else 128
    kname = "prefill16_kernel" if spec.head_dim == 256 else "prefill16r_kernel"
    kernel = f"{kname}<{spec.head_dim}, {tiling // 16}> ({tiling} query rows per workgroup" + (
        f", keys split in {splits} pieces)" if splits > 1 else ")")
    result = {
        "metric": f"paged causal prefill attn: TFLOP/s (% bf16 MFMA peak), D{spec.head_dim} Hq{spec.hq}/Hkv{spec.hkv}",
        "value": round(flops * L / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "hq": spec.hq, "hkv": spec.hkv,
                   "head_dim": spec.head_dim, "page_size": spec.page_size, "layout": spec.layout,
                   "pages": "contiguous" if args.contiguous else "shuffled", "q_lens_sum": int(spec.q_lens.sum()),
                   "kv_lens_sum": int(spec.kv_lens.sum()), "layers": L,
                   "step": "per layer: one pkv_prefill_attn call (own pools and inputs)",
                   "launch": "eager" if args.eager else "hip graph"},
        "us_per_call": round(ms * 1e3 / L, 2),
        "us_per_call_over_steps": spread(per, 1e3 / L),
        "value_over_steps": {"median": round(flops * L / (statistics.median(per) * 1e-3) / 1e12, 2),
                             "best": round(flops * L / (min(per) * 1e-3) / 1e12, 2), "rounds": len(per)},
        "roofline": {"bound": "mfma", "kernel": kernel + ", one launch per pkv_prefill_attn", "achieved": round(tfs, 2),
                     "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_unit": "HBM bytes per launch", "flops_per_launch": flops},
    }
    gpu_out0 = out0.cpu()
    del calls, ws, out0
    return result, gpu_out0


def bench_mixed(args, torch, pkv, wl):
    """One serving step of chunked prefill next to decode (Qwen3-4B attention
    shape: 4 prompt chunks of U{65..2048} rows continuing prompts, 64 decode
    rows of U{512..1024} cached tokens), per layer one pkv_mixed_attn launch,
    against the same work as two launches per layer (pkv_prefill_attn on the
    chunks, pkv_decode_attn on the decode rows) on the same inputs."""
    spec = wl.mixed_spec()
    dev = torch.device("cuda:0")
    P = int((spec.q_lens > 1).sum())
    npf = int(spec.q_lens[:P].sum())
    nd = spec.batch - P
    L = 16
    flops = 4 * spec.head_dim * spec.hq * sum(int(q) * (2 * int(kv) - int(q) + 1) // 2
                                              for q, kv in zip(spec.q_lens[:P], spec.kv_lens[:P]))  # chunks
    es = 2
    kv_bytes = int(spec.kv_lens[P:].sum()) * spec.hkv * spec.head_dim * 2 * es
    log(f"[bench] {spec.name}: {L} layers, {flops / 1e9:.1f} GFLOP and {kv_bytes / 1e6:.1f} MB decode KV per layer")
    max_q, max_kv = int(spec.q_lens[:P].max()), int(spec.kv_lens.max())
    zeros = torch.zeros(spec.batch, dtype=torch.int32, device=dev)
    mixed, separate, ws_m = [], [], None
    for layer in range(L):
        inp = wl.prefill_inputs(spec, device=dev, seed_offset=layer)
        kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
        if ws_m is None:
            ws_m = torch.zeros(pkv.mixed_workspace_bytes(kc, spec.batch, P, spec.hq), dtype=torch.uint8, device=dev)
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, inp.block_table, zeros, inp.hist_indptr)
        kv = pkv.append(kc, vc, inp.k_new, inp.v_new, inp.block_table, inp.hist_lens, inp.qo_indptr)
        out, out2 = torch.empty_like(inp.q), torch.empty_like(inp.q)
        mixed.append(pkv.api.prepare_mixed(inp.q, kc, vc, inp.block_table, kv, inp.qo_indptr, P, max_q, max_kv,
                                           spec.scale, out, ws_m))
        bt_d, kv_d = inp.block_table[P:].contiguous(), kv[P:].contiguous()
        ws_d = torch.zeros(pkv.decode_workspace_bytes(kc, nd, spec.hq, max_kv), dtype=torch.uint8, device=dev)
        separate.append((pkv.api.prepare_prefill(inp.q[:npf], kc, vc, inp.block_table[:P], kv[:P],
                                                 inp.qo_indptr[:P + 1], max_q, max_kv, spec.scale, out2[:npf]),
                         pkv.api.prepare_decode(inp.q[npf:], kc, vc, bt_d, kv_d, max_kv, spec.scale, out2[npf:],
                                                ws_d), bt_d, kv_d, ws_d))
        del inp
    torch.cuda.synchronize()

    def step_mixed():
        for c in mixed:
            c()

    def step_separate():
        for pf, dc, *_ in separate:
            pf()
            dc()

    ms_m, per_m = time_steps(torch, step_mixed, args.steps, args.warmup, not args.eager)
    ms_s, per_s = time_steps(torch, step_separate, args.steps, args.warmup, not args.eager)
    us_m, us_s = ms_m * 1e3 / L, ms_s * 1e3 / L
    t_ideal = flops / (BF16_MFMA_PEAK_TFS * 1e12) + kv_bytes / (HBM_PEAK_GBS * 1e9)
    result = {
        "metric": "chunked prefill + decode in one launch: us per layer (lower is better)",
        "value": round(us_m, 2), "unit": "us/layer", "higher_is_better": False,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_m, 4), "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "chunks_q": spec.q_lens[:P].tolist(), "chunks_kv": spec.kv_lens[:P].tolist(),
                   "decode_rows": nd, "decode_mean_keys": round(float(spec.kv_lens[P:].mean()), 1), "hq": spec.hq,
                   "hkv": spec.hkv, "head_dim": spec.head_dim, "layers": L,
                   "step": "per layer: one pkv_mixed_attn launch (own pools and inputs)",
                   "launch": "eager" if args.eager else "hip graph"},
        "us_per_call_over_steps": spread(per_m, 1e3 / L),
        "separate_us_per_layer": round(us_s, 2),
        "separate_us_per_call_over_steps": spread(per_s, 1e3 / L),
        "speedup_vs_separate": round(us_s / us_m, 3),
        "roofline": {"bound": "mfma+hbm",
                     "kernel": "prefill16r_kernel<128, 12> (decode rows packed by KV head, then the chunks' query tiles)",
                     "achieved": round(flops / (us_m * 1e-6) / 1e12, 2), "unit": "TFLOP/s",
                     "peak": BF16_MFMA_PEAK_TFS,
                     "frac": round(t_ideal / (us_m * 1e-6), 4),
                     "frac_definition": "(chunk flops / bf16 MFMA peak + decode KV bytes / HBM peak) / launch time",
                     "traffic": traffic_from_profile("mixed", f"prefill16r_kernel_{spec.name}_pmc.txt"),
                     "traffic_unit": "HBM bytes per launch",
                     "flops_per_launch": flops, "decode_kv_bytes_per_launch": kv_bytes},
    }
    del mixed, separate, ws_m
    return result


def cpu_baseline_prefill(args, spec, gpu_out0=None):
    """The oracle (as is) on a sample of query rows of the same request(s):
    blocks of 32 consecutive rows of request 0, from its last row backwards,
    each run as a chunked-prefill request over the keys it sees, on all host
    threads of the GPU's share, then on one thread.  With gpu_out0 (layer 0's
    output of the timed GPU step) the oracle's first and last blocks of
    request 0 are also compared with it, all heads."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import oracle
    from paged_kv_attention_pkv_amd import workloads as wl
    from gpu_common import host_bits

    orc = oracle.load()
    threads = max(1, min(CPU_THREADS_MAX, os.cpu_count() or 1))
    h = wl.prefill_inputs(spec, device="cuda:0").to("cpu")
    pool = oracle.Pool.hnd(oracle.BF16, spec.num_pages, spec.page_size, spec.hkv, spec.head_dim)
    kc = host_bits(wl.empty_pool(spec, "cpu")).copy()
    vc = kc.copy()
    orc.append(pool, kc, vc, host_bits(h.k_hist), host_bits(h.v_hist), spec.block_table,
               np.zeros(spec.batch, np.int32), h.hist_indptr.numpy())
    kv = orc.append(pool, kc, vc, host_bits(h.k_new), host_bits(h.v_new), spec.block_table, spec.hist_lens,
                    h.qo_indptr.numpy())
    r0, kvl = int(spec.q_lens[0]), int(kv[0])
    ip = h.qo_indptr.numpy()
    blk = 32

    def block(nt):
        def f(i):
            pos = (i * blk) % r0
            rows = min(blk, r0 - pos)
            a1 = r0 - pos
            a0 = a1 - rows
            kv_seen = kvl - r0 + a1
            orc.prefill(pool, host_bits(h.q[ip[0] + a0: ip[0] + a1]), kc, vc, spec.block_table[:1],
                        np.array([kv_seen], np.int32), np.array([0, rows], np.int32), spec.scale, causal=True,
                        nthreads=nt)
            return 4 * spec.head_dim * spec.hq * sum(kv_seen - rows + j + 1 for j in range(rows))
        return f

    n, spent, fl = _timed_loop(block(threads), args.cpu_seconds)
    n1, spent1, fl1 = _timed_loop(block(1), args.cpu_seconds_1t)
    res = {"value": round(fl / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "value_1_thread": round(fl1 / spent1 / 1e12, 6),
           "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
           "sample": f"{n} blocks of {blk} query rows of request 0 ({r0} rows; from its last row backwards, "
                     f"cyclically) on {threads} threads in {spent:.1f} s ({fl / 1e9:.1f} GFLOP); {n1} blocks on "
                     f"1 thread in {spent1:.1f} s; fp64 oracle"}
    if gpu_out0 is not None:
        gpu, ref = [], []
        for a0 in sorted({0, max(0, r0 - blk)}):
            a1 = min(a0 + blk, r0)
            o, _ = orc.prefill(pool, host_bits(h.q[ip[0] + a0: ip[0] + a1]), kc, vc, spec.block_table[:1],
                               np.array([kvl - r0 + a1], np.int32), np.array([0, a1 - a0], np.int32), spec.scale,
                               causal=True, nthreads=threads)
            gpu.append(gpu_out0[ip[0] + a0: ip[0] + a1])
            ref.append(o)
        import torch
        res["parity"] = parity(torch.cat(gpu), np.concatenate(ref), spec.dtype,
                               f"layer 0, request 0: its first and last {blk} query rows, all {spec.hq} heads")
    return res


# --------------------------------------------------------------------------
# tuning sweep
# --------------------------------------------------------------------------

def _median_step_ms(torch, step, args):
    _, per = time_steps(torch, step, args.steps, args.warmup, not args.eager)
    return statistics.median(per)


def _decode_setup(torch, pkv, wl, spec, L, dev):
    """L layers of pools holding the history, with each layer's q / new K/V."""
    bt = torch.from_numpy(spec.block_table).to(dev)
    hist = torch.from_numpy(spec.hist_lens).to(dev)
    zeros = torch.zeros_like(hist)
    pools = [(wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)) for _ in range(L)]
    layers = []
    for layer in range(L):
        inp = wl.decode_inputs(spec, device=dev, seed_offset=layer)
        kc, vc = pools[layer]
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, bt, zeros, inp.hist_indptr, layout=spec.layout)
        layers.append((kc, vc, inp.q, inp.k_new, inp.v_new))
        del inp
    torch.cuda.synchronize()
    return {"spec": spec, "bt": bt, "hist": hist, "layers": layers,
            "max_kv": int(spec.hist_lens.max()) + spec.n_new}


def _decode_step(torch, pkv, setup, workers, dev, plan=False):
    """One fused append + decode launch per layer with the given worker
    count (with plan: after one pkv_decode_plan for the step)."""
    spec, bt, hist, max_kv = setup["spec"], setup["bt"], setup["hist"], setup["max_kv"]
    kc0 = setup["layers"][0][0]
    ws = torch.zeros(pkv.decode_workspace_bytes(kc0, spec.batch, spec.hq, max_kv, layout=spec.layout,
                                                workers=workers), dtype=torch.uint8, device=dev)
    lens = torch.empty_like(hist)
    calls = [pkv.api.prepare_append_decode(q, kc, vc, kn, vn, bt, hist, max_kv, spec.scale, torch.empty_like(q), ws,
                                           seqlens_out=lens, layout=spec.layout, workers=workers)
             for kc, vc, q, kn, vn in setup["layers"]]
    if plan:
        calls.insert(0, pkv.api.prepare_decode_plan(kc0, hist, spec.hq, max_kv, ws, fused=True,
                                                    layout=spec.layout, workers=workers))

    def step():
        for c in calls:
            c()
    step.keep = (ws, lens, calls)
    return step


def _alternate(torch, args, control, variant, rounds):
    """Medians of `rounds` alternating measurements control, variant, ..."""
    c, v = [], []
    for _ in range(rounds):
        c.append(_median_step_ms(torch, control, args))
        v.append(_median_step_ms(torch, variant, args))
    return c, v


def bench_tune(args, torch, pkv, wl):
    dev = torch.device("cuda:0")
    L = args.layers
    rounds = 3
    lines = []

    def summarise(name, control_label, per_layer, entries, controls, unit_scale):
        all_c = [x for cs in controls for x in cs]
        med_c = statistics.median(all_c)
        rows = []
        for label, cs, vs in entries:
            mv, mc = statistics.median(vs), statistics.median(cs)
            rows.append({"config": label, "us_per_layer": round(mv * unit_scale / per_layer, 2),
                         "control_us_per_layer": round(mc * unit_scale / per_layer, 2),
                         "ratio_to_control": round(mv / mc, 4)})
        best = min(rows, key=lambda r: r["ratio_to_control"])
        return {"metric": f"tuning sweep: {name}", "unit": "us/layer", "higher_is_better": False,
                "control": control_label, "control_us_per_layer": round(med_c * unit_scale / per_layer, 2),
                "control_spread": round((max(all_c) - min(all_c)) / med_c, 4), "control_runs": len(all_c),
                "best": best["config"], "best_ratio_to_control": best["ratio_to_control"],
                "steps_per_measurement": args.steps, "rounds": rounds, "layers": per_layer, "variants": rows}

    # decode: worker counts at three batch sizes; page size, layout and page order at batch 64
    for workload, batch in (("qwen3_decode", 64), ("qwen3_sweep", 8), ("qwen3_sweep", 32)):
        base = wl.decode_spec(workload, batch=batch)
        log(f"[tune] {base.name}: {L} layers")
        ctl = _decode_setup(torch, pkv, wl, base, L, dev)
        control = _decode_step(torch, pkv, ctl, 0, dev)
        entries, controls = [], []
        c, v = _alternate(torch, args, control, _decode_step(torch, pkv, ctl, 0, dev, plan=True), rounds)
        entries.append(("pkv_decode_plan once per step", c, v))
        controls.append(c)
        for w in (128, 256, 512, 768, 1280, 2048):
            c, v = _alternate(torch, args, control, _decode_step(torch, pkv, ctl, w, dev), rounds)
            entries.append((f"workers {w}", c, v))
            controls.append(c)
        if batch == 64:
            for label, kw in (("page 64", dict(page_size=64)), ("page 256", dict(page_size=256)),
                              ("NHD layout", dict(layout="NHD")), ("contiguous pages", dict(contiguous=True)),
                              ("page 256, contiguous", dict(page_size=256, contiguous=True))):
                other = _decode_setup(torch, pkv, wl, wl.decode_spec(workload, batch=batch, **kw), L, dev)
                c, v = _alternate(torch, args, control, _decode_step(torch, pkv, other, 0, dev), rounds)
                entries.append((label, c, v))
                controls.append(c)
                del other
                torch.cuda.empty_cache()
        lines.append(dict(summarise(f"decode {base.name} (fused append + decode per layer)",
                                    "page 16, HND, shuffled pages, library worker count, no plan", L, entries,
                                    controls,
                                    1e3), workload=base.name))
        del ctl, control
        torch.cuda.empty_cache()

    # prefill: the two head_dim 256 tilings against the library's choice
    Lp = max(1, args.prefill_layers)
    for spec in (wl.prefill_spec(fixed_1023=True), wl.prefill_spec(batch=2), wl.prefill_spec(batch=4),
                 wl.prefill_spec(batch=8)):
        log(f"[tune] {spec.name}: {Lp} layers")
        max_q, max_kv = int(spec.q_lens.max()), int(spec.kv_lens.max())
        zeros = torch.zeros(spec.batch, dtype=torch.int32, device=dev)
        made = []
        for layer in range(Lp):
            inp = wl.prefill_inputs(spec, device=dev, seed_offset=layer)
            kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
            pkv.append(kc, vc, inp.k_hist, inp.v_hist, inp.block_table, zeros, inp.hist_indptr)
            kv = pkv.append(kc, vc, inp.k_new, inp.v_new, inp.block_table, inp.hist_lens, inp.qo_indptr)
            made.append((inp.q, kc, vc, inp.block_table, kv, inp.qo_indptr))
            del inp
        need = pkv.prefill_workspace_bytes(made[0][1], spec.batch, spec.hq, int(spec.q_lens.sum()), max_q, max_kv)

        def prefill_step(rows):
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            calls = [pkv.api.prepare_prefill(q, kc, vc, bt, kv, ip, max_q, max_kv, spec.scale, torch.empty_like(q), ws,
                                             rows_per_workgroup=rows) for q, kc, vc, bt, kv, ip in made]

            def step():
                for c in calls:
                    c()
            step.keep = (ws, calls)
            return step

        control = prefill_step(0)
        entries, controls = [], []
        for rows in (128, 192):
            c, v = _alternate(torch, args, control, prefill_step(rows), rounds)
            entries.append((f"{rows} query rows per workgroup", c, v))
            controls.append(c)
        lines.append(dict(summarise(f"prefill {spec.name}", "library tiling choice", Lp, entries, controls, 1e3),
                          workload=spec.name))
        del made, control
        torch.cuda.empty_cache()
    return lines


def calibrate_copy(torch):
    """A plain device copy of exactly 1 GiB (read 1 GiB, write 1 GiB), run 5
    times, for scaling the HBM byte counters."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


# --------------------------------------------------------------------------
# profile summaries (run on the host, from rocprofv3 CSV output)
# --------------------------------------------------------------------------

def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(argv):
    """Markdown table of the library's kernels from a rocprofv3
    ``--kernel-trace --stats`` kernel_stats.csv."""
    p = argparse.ArgumentParser(prog="bench.py summarize-trace")
    p.add_argument("stats_csv")
    p.add_argument("out")
    p.add_argument("--title", required=True)
    p.add_argument("--command", required=True, help="the profiled command, as run from the repository root")
    p.add_argument("--note", default="")
    p.add_argument("--bench-json", default=None, help="the JSON line the profiled bench.py run printed")
    p.add_argument("--trace-csv", default=None,
                   help="kernel_trace.csv of the same run: rows per (kernel, grid size) instead of per kernel")
    a = p.parse_args(argv)
    lines = [f"# {a.title}", "", "Command (from the repository root, on one MI355X):", "", "```", a.command, "```",
             ""]
    if a.note:
        lines += [a.note, ""]
    shorten = lambda n: n.split("(anonymous namespace)::")[-1].split("(")[0].replace("pkv::", "")
    if a.trace_csv:
        groups = {}
        for r in _csv_rows(a.trace_csv):
            if "pkv::" not in r["Kernel_Name"]:
                continue
            key = (shorten(r["Kernel_Name"]), int(r["Grid_Size_X"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines += ["| kernel | grid (work-items) | calls | average ns | min ns | max ns |", "|---|---|---|---|---|---|"]
        for (k, grid), d in sorted(groups.items()):
            lines.append(f"| {k} | {grid} | {len(d)} | {sum(d) / len(d):.0f} | {min(d)} | {max(d)} |")
    else:
        lines += ["| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
        for r in _csv_rows(a.stats_csv):
            n = r["Name"]
            if "pkv::" not in n:
                continue
            lines.append(f"| {shorten(n)} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    if a.bench_json:
        with open(a.bench_json) as f:
            d = [json.loads(x) for x in f.read().splitlines() if x.startswith('{"metric"')][-1]
        keep = {k: d[k] for k in ("value", "unit", "us_per_call") if k in d}
        keep["roofline_achieved"] = d["roofline"]["achieved"]
        keep["roofline_frac"] = d["roofline"]["frac"]
        lines += ["", "Line printed by the profiled run (HIP events over its timed region): " + json.dumps(keep)]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_pmc(argv):
    """HBM bytes per launch of one kernel from two rocprofv3 counter runs
    (FETCH_SIZE, WRITE_SIZE), each scaled by what the same counter reads for
    a 1 GiB device copy (``bench.py --calibrate-copy`` under the same passes)."""
    p = argparse.ArgumentParser(prog="bench.py summarize-pmc")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("copy_fetch_csv")
    p.add_argument("copy_write_csv")
    p.add_argument("out")
    p.add_argument("--kernel", required=True, help="substring of the kernel's name")
    p.add_argument("--kind", required=True, choices=sorted(KERNEL_SOURCES))
    p.add_argument("--command", required=True, action="append",
                   help="each profiled command, as run from the repository root")
    p.add_argument("--largest-grid", action="store_true",
                   help="only the dispatches of the kernel with the largest grid (another launch of the same "
                        "kernel in the run, with a smaller grid, is left out)")
    a = p.parse_args(argv)

    def values(path, pat, largest=False):
        rows = [r for r in _csv_rows(path) if pat in r["Kernel_Name"]]
        if largest and rows:
            top = max(int(r["Grid_Size"]) for r in rows)
            rows = [r for r in rows if int(r["Grid_Size"]) == top]
        return [float(r["Counter_Value"]) for r in rows]

    fetch = values(a.fetch_csv, a.kernel, a.largest_grid)
    write = values(a.write_csv, a.kernel, a.largest_grid)
    kib = 1 << 20  # KiB in the 1 GiB copy
    cf = [v for v in values(a.copy_fetch_csv, "copyBuffer") if v > kib / 16]
    cw = [v for v in values(a.copy_write_csv, "copyBuffer") if v > kib / 16]
    if not (fetch and write and cf and cw):
        raise SystemExit("summarize-pmc: a counter file holds no matching dispatch")
    ff, fw = kib / statistics.mean(cf), kib / statistics.mean(cw)
    medf, medw = statistics.median(fetch), statistics.median(write)
    read_b, write_b = medf * ff * 1024, medw * fw * 1024
    what = a.kernel + (" (largest grid of the run)" if a.largest_grid else "")
    lines = [f"# HBM counters: {what}", "", "Commands (from the repository root, one MI355X, one counter per run):",
             ""] + [f"    {c}" for c in a.command] + [
        "",
        "Calibration: a 1 GiB device-to-device copy reads 1 GiB and writes 1 GiB.",
        f"  FETCH_SIZE per copy: {statistics.mean(cf):.1f} KiB -> scale {ff:.4f}",
        f"  WRITE_SIZE per copy: {statistics.mean(cw):.1f} KiB -> scale {fw:.4f}",
        "",
        f"{a.kernel} dispatches: {len(fetch)} (fetch run), {len(write)} (write run)",
        f"  FETCH_SIZE KiB per dispatch: mean {statistics.mean(fetch):.1f}, median {medf:.1f}, "
        f"min {min(fetch):.1f}, max {max(fetch):.1f}",
        f"  WRITE_SIZE KiB per dispatch: mean {statistics.mean(write):.1f}, median {medw:.1f}, "
        f"min {min(write):.1f}, max {max(write):.1f}",
        f"  scaled HBM bytes per dispatch (medians): read {read_b:.0f}, write {write_b:.0f}",
        "",
        "kernel sources: " + ", ".join(f"paged_kv_attention_pkv_amd/csrc/{n}" for n in KERNEL_SOURCES[a.kind]),
        f"source_sha256_16: {source_hash(a.kind)}",
        f"hbm_bytes_per_launch: {read_b + write_b:.0f}",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_mfma(argv):
    """MFMA and LDS utilisation of one kernel from a rocprofv3 counter pass of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES, SQ_ACTIVE_INST_VALU,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT and
    GRBM_GUI_ACTIVE (the last summed over the 8 XCDs; 256 CUs, 1024 SIMDs)."""
    import collections
    p = argparse.ArgumentParser(prog="bench.py summarize-mfma")
    p.add_argument("csv")
    p.add_argument("out")
    p.add_argument("--kernel", required=True)
    p.add_argument("--kind", required=True, choices=sorted(KERNEL_SOURCES))
    p.add_argument("--command", required=True)
    p.add_argument("--flops", type=float, required=True, help="algorithmic flops per dispatch")
    p.add_argument("--largest-grid", action="store_true", help="only the dispatches with the kernel's largest grid")
    a = p.parse_args(argv)
    per = collections.defaultdict(dict)
    name = a.kernel
    rows_k = [r for r in _csv_rows(a.csv) if a.kernel in r["Kernel_Name"]]
    if a.largest_grid and rows_k:
        top = max(int(r["Grid_Size"]) for r in rows_k)
        rows_k = [r for r in rows_k if int(r["Grid_Size"]) == top]
    for r in rows_k:
        name = r["Kernel_Name"]
        per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
    ks = sorted(per, key=int)
    if not ks:
        raise SystemExit("summarize-mfma: no matching dispatch")
    rows = []
    for k in ks:
        c = per[k]
        act = c["GRBM_GUI_ACTIVE"] / 8
        rows.append({"mfma": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (act * 1024),
                     "coexec": c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / (act * 1024),
                     "valu": 4 * c.get("SQ_ACTIVE_INST_VALU", 0.0) / (act * 1024),
                     "lds": c["SQ_LDS_IDX_ACTIVE"] / (act * 256),
                     "conf": c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"]),
                     "flops": c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512, "act": act})
    med = lambda key: statistics.median(r[key] for r in rows)
    short = name.split("(anonymous namespace)::")[-1].split("(")[0].replace("pkv::", "")
    last = per[ks[-1]]
    lines = [f"# MFMA and LDS counters: {short}", "", "Command (from the repository root, one MI355X, one counter pass):",
             "", f"    {a.command}", "",
             "Per dispatch (GRBM_GUI_ACTIVE is summed over the 8 XCDs: one XCD's active cycles are the sum / 8):",
             "  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs)",
             "  MFMA and VALU at once = SQ_VALU_MFMA_COEXEC_CYCLES / (active cycles x 1024 SIMDs)",
             "  VALU issuing = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / (active cycles x 1024 SIMDs)",
             "  LDS active = SQ_LDS_IDX_ACTIVE / (active cycles x 256 CUs)",
             "  MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512", "",
             f"{short} dispatches: {len(ks)} (medians)",
             f"  MFMA busy {100 * med('mfma'):.1f}%, VALU issuing {100 * med('valu'):.1f}%, both at once "
             f"{100 * med('coexec'):.1f}%",
             f"  LDS active {100 * med('lds'):.1f}%, bank-conflict cycles {100 * med('conf'):.2f}% of LDS-active cycles",
             f"  MFMA flops per dispatch {med('flops') / 1e9:.2f} GFLOP against {a.flops / 1e9:.2f} GFLOP of causal pairs "
             f"({100 * (med('flops') / a.flops - 1):.1f}% more: the masked part of diagonal tiles)",
             f"  active cycles per XCD {med('act'):.0f}", "", "Raw counters of the last dispatch:"]
    lines += [f"  {n}: {int(last[n])}" for n in sorted(last)]
    lines += ["", "kernel sources: " + ", ".join(f"paged_kv_attention_pkv_amd/csrc/{n}" for n in KERNEL_SOURCES[a.kind]),
              f"source_sha256_16: {source_hash(a.kind)}"]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    if len(sys.argv) > 1 and sys.argv[1] in ("summarize-trace", "summarize-pmc", "summarize-mfma"):
        {"summarize-trace": summarize_trace, "summarize-pmc": summarize_pmc,
         "summarize-mfma": summarize_mfma}[sys.argv[1]](sys.argv[2:])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs each call on "
              "one GPU and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import paged_kv_attention_pkv_amd as pkv
    from paged_kv_attention_pkv_amd import workloads as wl

    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} ({getattr(props, 'gcnArchName', '?')}), CUs {props.multi_processor_count}")
    cpu = not args.no_cpu_baseline
    if args.workload == "tune":
        for line in bench_tune(args, torch, pkv, wl):
            line["device"] = device_info(torch, props)
            print(json.dumps(line), flush=True)
        return
    if args.workload == "mixed":
        result = bench_mixed(args, torch, pkv, wl)
        result.update({"n_gpus": 1, "scaling": "weak", "vs_baseline": None})
    elif args.workload == "prefill":
        kw = dict(page_size=args.page_size, layout=args.layout, contiguous=args.contiguous, head_dim=args.head_dim,
                  hq=args.hq, hkv=args.hkv)
        if args.q_len is not None or args.kv_len is not None:
            q = [int(x) for x in (args.q_len or "").split(",") if x]
            kv = [int(x) for x in (args.kv_len or "").split(",") if x]
            if not q or len(q) != len(kv) or any(a < 1 or a > b for a, b in zip(q, kv)):
                raise SystemExit("--q-len and --kv-len: equal-length lists with 1 <= q <= kv")
            spec = wl.prefill_spec(q_lens=q, kv_lens=kv, seed=9, **kw)
            spec.name = f"prefill_d{args.head_dim}_q{'-'.join(map(str, q))}_kv{'-'.join(map(str, kv))}"
        elif args.batch is None:
            spec = wl.prefill_spec(fixed_1023=True, **kw)
        else:
            spec = wl.prefill_spec(batch=args.batch, **kw)
        result, out0 = bench_prefill(args, torch, pkv, wl, spec)
        result.update({"n_gpus": 1, "scaling": "weak", "vs_baseline": None})
        if cpu:
            result["cpu_baseline"] = cpu_baseline_prefill(args, spec, out0)
    else:
        result, spec, out0 = bench_decode(args, torch, pkv, wl, args.workload or "decode")
        if cpu:
            result["cpu_baseline"] = cpu_baseline_decode(args, spec, out0)
        del out0
        if args.workload is None:
            torch.cuda.empty_cache()
            result["prefill"] = {}
            for key, pspec in (("b1_q1023", wl.prefill_spec(fixed_1023=True)),
                               ("b8_random", wl.prefill_spec(batch=8))):
                sub, out0 = bench_prefill(args, torch, pkv, wl, pspec)
                if cpu:
                    sub["cpu_baseline"] = cpu_baseline_prefill(args, pspec, out0)
                del out0
                result["prefill"][key] = sub
                torch.cuda.empty_cache()
            result["mixed"] = bench_mixed(args, torch, pkv, wl)
            torch.cuda.empty_cache()
    result["device"] = device_info(torch, props)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
