#!/usr/bin/env python3
"""Benchmark of the paged KV attention hot path on one MI355X.

Default workload: the Qwen3-4B-shaped decode step at batch 64 (Hq 32 / Hkv 8 /
head_dim 128, bf16, page size 16, cached lengths U{512..1024}, pages shuffled
over a pool 1.25x the pages needed), one appended token per sequence, over 36
independent layer caches (36 x 254 MB of pools, far more than the 256 MB
last-level cache, so every layer's K/V comes from HBM).

One step = for each of the 36 layers: pkv_append (the new token) then
pkv_decode_attn -- the whole decode hot path.  The step is captured once in a
HIP graph and replayed (``--eager`` launches it from Python instead).  All
inputs are resident in HBM before the timed region.

Printed: one JSON line with the metric (KV-read GB/s = bytes of the attended
K/V tokens read per step / step time), the per-layer call time, a roofline
object for the dominant kernel (decode; its per-launch duration measured with
HIP events on the launch stream) and the CPU oracle timed on a bounded sample
of the same workload on the host cores.

``--workload prefill`` times causal paged prefill instead (head_dim 256,
Hq 48 / Hkv 8, the B=1 q_len = kv_len = 1023 request, or ``--batch B`` random
requests) against the bf16 MFMA roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="decode", choices=["decode", "sweep", "long", "prefill"])
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--layers", type=int, default=36, help="decode: layer caches per step")
    p.add_argument("--prefill-layers", type=int, default=8,
                   help="prefill: layers per step, each with its own pools and inputs")
    p.add_argument("--eager", action="store_true", help="launch from Python instead of replaying a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    p.add_argument("--workers", type=int, default=0, help="decode split workers (0 = library default)")
    p.add_argument("--separate", action="store_true",
                   help="decode step as pkv_append + pkv_decode_attn (two launches) instead of the fused "
                        "pkv_append_decode_attn")
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


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_src: str, name: str):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing or was taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash(kernel_src):
        return None
    return float(t.group(1))


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
    """(ms per step, graph used) over `steps` timed steps after `warmup`."""
    graph = None
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, graph


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def bench_decode(args, torch, pkv, wl):
    if args.workload == "decode":
        spec = wl.decode_spec("qwen3_decode", batch=args.batch or 64)
    elif args.workload == "sweep":
        spec = wl.decode_spec("qwen3_sweep", batch=args.batch or 64)
    else:
        spec = wl.decode_spec("long_ragged", batch=args.batch or 256)
    dev = torch.device("cuda:0")
    L = args.layers
    fused = not args.separate and spec.dtype == "bf16"
    acc = decode_bytes(spec, fused)
    if args.workload == "long":
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
            ws_bytes = pkv.decode_workspace_bytes(kc, spec.batch, spec.hq, max_kv, workers=args.workers)
            workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, bt, zeros, inp.hist_indptr)
        out = torch.empty_like(inp.q)
        if fused:
            app = None
            dec = pkv.api.prepare_append_decode(inp.q, kc, vc, inp.k_new, inp.v_new, bt, hist, max_kv, spec.scale, out,
                                                workspace, seqlens_out=lens, workers=args.workers)
        else:
            app = pkv.api.prepare_append(kc, vc, inp.k_new, inp.v_new, bt, hist, lens)
            dec = pkv.api.prepare_decode(inp.q, kc, vc, bt, lens, max_kv, spec.scale, out, workspace,
                                         workers=args.workers)
        layers.append((app, dec, None))
        del inp
    del pools
    torch.cuda.synchronize()

    def step():
        for app, dec, _ in layers:
            if app is not None:
                app()
            dec()

    ms, _ = time_steps(torch, step, args.steps, args.warmup, not args.eager)
    step()  # lens is live again for the per-call brackets below
    dec_mean, dec_med = events_per_call(torch, [d for _, d, _ in layers])
    app_mean = None if fused else events_per_call(torch, [a for a, _, _ in layers])[0]
    kv_bytes_step = acc["kv"] * L
    value = kv_bytes_step / (ms * 1e-3) / 1e9
    # the kernel's average launch duration: in the fused step the timed region
    # holds exactly L launches of it (HIP events around the graph replays);
    # in the two-launch step, per-call event brackets of the decode launches
    launch_ms = ms / L if fused else dec_mean
    achieved = acc["total"] / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(os.path.join(ROOT, "paged_kv_attention_pkv_amd", "csrc", "decode.hip"),
                                   f"decode_kernel_{spec.name}_pmc.txt") if fused else None
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
                   "head_dim": spec.head_dim, "page_size": spec.page_size, "layers": L,
                   "mean_attended_len": round(float(spec.hist_lens.mean()) + spec.n_new, 1),
                   "step": ("per layer: pkv_append_decode_attn (append 1 token/seq + attend, one launch)"
                            if fused else "per layer: pkv_append(1 token/seq) + pkv_decode_attn"),
                   "launch": "eager" if args.eager else "hip graph", "parallelism": "none (1 GPU)"},
        "us_per_call": round(ms * 1e3 / L, 2),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "decode_us_per_call_events": round(dec_mean * 1e3, 2),
        "append_us_per_call_events": None if app_mean is None else round(app_mean * 1e3, 2),
        "kernel_us_per_launch": round(launch_ms * 1e3, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "decode_bf16_kernel (one launch per pkv_append_decode_attn)" if fused
                     else "decode kernel (one launch per pkv_decode_attn)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_unit": "HBM bytes per launch", "bytes_per_launch": acc["total"]},
    }
    return result, spec, layers


def cpu_baseline_decode(args, torch, spec, layers):
    """The oracle (as is) on a bounded sample of the same workload: whole
    layers of the batch (host pools built by the oracle's own append), run
    on the host cores until about --cpu-seconds have been spent."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import oracle
    from paged_kv_attention_pkv_amd import workloads as wl
    from gpu_common import host_bits, opool

    orc = oracle.load()
    threads = max(1, min(16, os.cpu_count() or 1))
    pool = opool(spec)
    zeros = np.zeros(spec.batch, np.int32)
    hosts = []
    for layer in range(min(2, len(layers))):
        inp = wl.decode_inputs(spec, device="cuda:0", seed_offset=layer).to("cpu")
        kc = host_bits(wl.empty_pool(spec, "cpu")).copy()
        vc = kc.copy()
        orc.append(pool, kc, vc, host_bits(inp.k_hist), host_bits(inp.v_hist), spec.block_table, zeros,
                   inp.hist_indptr.numpy())
        lens = orc.append(pool, kc, vc, host_bits(inp.k_new), host_bits(inp.v_new), spec.block_table,
                          spec.hist_lens)
        hosts.append((host_bits(inp.q), kc, vc, lens))
    done_bytes, spent, calls = 0, 0.0, 0
    while spent < args.cpu_seconds or calls == 0:
        q, kc, vc, lens = hosts[calls % len(hosts)]
        t0 = time.perf_counter()
        orc.decode(pool, q, kc, vc, spec.block_table, lens, spec.scale, nthreads=threads)
        spent += time.perf_counter() - t0
        done_bytes += decode_bytes(spec)["kv"]
        calls += 1
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} decode calls of the same workload (all {spec.batch} sequences, layer caches "
                      f"0..{len(hosts) - 1} in turn), fp64 oracle, {spent:.1f} s"}


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def bench_prefill(args, torch, pkv, wl):
    spec = wl.prefill_spec(fixed_1023=True) if args.batch is None else wl.prefill_spec(batch=args.batch)
    dev = torch.device("cuda:0")
    flops = prefill_flops(spec)
    L = max(1, args.prefill_layers)
    log(f"[bench] {spec.name}: {flops / 1e9:.2f} GFLOP per call, {L} layers per step")
    max_q, max_kv = int(spec.q_lens.max()), int(spec.kv_lens.max())
    zeros = torch.zeros(spec.batch, dtype=torch.int32, device=dev)
    calls, inp0, ws = [], None, None
    for layer in range(L):
        # every layer its own pools, queries and outputs, as the layers of a model
        inp = wl.prefill_inputs(spec, device=dev, seed_offset=layer)
        kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
        pkv.append(kc, vc, inp.k_hist, inp.v_hist, inp.block_table, zeros, inp.hist_indptr)
        kv_lens = pkv.append(kc, vc, inp.k_new, inp.v_new, inp.block_table, inp.hist_lens, inp.qo_indptr)
        out = torch.empty_like(inp.q)
        if ws is None:
            need = pkv.prefill_workspace_bytes(kc, spec.batch, spec.hq, int(spec.q_lens.sum()), max_q, max_kv)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        calls.append(pkv.api.prepare_prefill(inp.q, kc, vc, inp.block_table, kv_lens, inp.qo_indptr, max_q,
                                             max_kv, spec.scale, out, ws))
        if layer == 0:
            inp0 = inp
        del inp
    torch.cuda.synchronize()

    def step():
        for c in calls:
            c()

    ms, _ = time_steps(torch, step, args.steps, args.warmup, not args.eager)
    mean = ms / L  # L launches per step: the timed region's HIP events give their average duration
    tfs = flops / (mean * 1e-3) / 1e12
    traffic = traffic_from_profile(os.path.join(ROOT, "paged_kv_attention_pkv_amd", "csrc", "prefill.hip"),
                                   f"prefill16_kernel_{spec.name}_pmc.txt")
    # the workgroup size the library picks for this call, by the rule stated
    # in include/pkv.h (192 rows once ceil(total_q / 192) * Hq >= 1.5 * CUs)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    waves = 12 if 2 * (-(-int(spec.q_lens.sum()) // 192) * spec.hq) >= 3 * cus else 8
    result = {
        "metric": "paged causal prefill attn: TFLOP/s (% bf16 MFMA peak), D256 Hq48/Hkv8",
        "value": round(flops * L / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "hq": spec.hq, "hkv": spec.hkv,
                   "head_dim": spec.head_dim, "q_lens_sum": int(spec.q_lens.sum()),
                   "kv_lens_sum": int(spec.kv_lens.sum()), "layers": L,
                   "step": "per layer: one pkv_prefill_attn call (own pools and inputs)",
                   "launch": "eager" if args.eager else "hip graph", "parallelism": "none (1 GPU)"},
        "us_per_call": round(ms * 1e3 / L, 2),
        "roofline": {"bound": "mfma", "kernel": f"prefill16_kernel<256, {waves}> (one launch per pkv_prefill_attn, "
                                                  f"{16 * waves} query rows per workgroup)", "achieved": round(tfs, 2),
                     "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_unit": "HBM bytes per launch", "flops_per_launch": flops},
    }
    return result, spec, inp0


def cpu_baseline_prefill(args, torch, spec, inp):
    """Oracle on a sample of query rows of the same request(s)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import oracle
    from paged_kv_attention_pkv_amd import workloads as wl
    from gpu_common import host_bits

    orc = oracle.load()
    threads = max(1, min(16, os.cpu_count() or 1))
    h = inp.to("cpu")
    pool = oracle.Pool.hnd(oracle.BF16, spec.num_pages, spec.page_size, spec.hkv, spec.head_dim)
    kc = host_bits(wl.empty_pool(spec, "cpu")).copy()
    vc = kc.copy()
    orc.append(pool, kc, vc, host_bits(h.k_hist), host_bits(h.v_hist), spec.block_table,
               np.zeros(spec.batch, np.int32), h.hist_indptr.numpy())
    kv = orc.append(pool, kc, vc, host_bits(h.k_new), host_bits(h.v_new), spec.block_table, spec.hist_lens,
                    h.qo_indptr.numpy())
    # blocks of 32 consecutive query rows of request 0, from its last row
    # backwards (starting over at the last row once the first is reached), each
    # run as a chunked-prefill request over the keys it sees, until about
    # --cpu-seconds have been spent
    r0, kvl = int(spec.q_lens[0]), int(kv[0])
    ip = h.qo_indptr.numpy()
    fl, spent, done, blk = 0, 0.0, 0, 32
    while spent < args.cpu_seconds or done == 0:
        pos = done % r0
        rows = min(blk, r0 - pos)
        a1 = r0 - pos
        a0 = a1 - rows
        q = host_bits(h.q[ip[0] + a0: ip[0] + a1])
        kv_seen = kvl - r0 + a1
        t0 = time.perf_counter()
        orc.prefill(pool, q, kc, vc, spec.block_table[:1], np.array([kv_seen], np.int32),
                    np.array([0, rows], np.int32), spec.scale, causal=True, nthreads=threads)
        spent += time.perf_counter() - t0
        fl += 4 * spec.head_dim * spec.hq * sum(kv_seen - rows + i + 1 for i in range(rows))
        done += rows
    return {"value": round(fl / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} query rows of request 0 ({r0} rows, taken from its last row backwards, "
                      f"cyclically) in blocks of {blk} ({fl / 1e9:.2f} GFLOP), "
                      f"fp64 oracle, {spent:.1f} s"}


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU "
              "mode in this build", file=sys.stderr)
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
    if args.workload == "prefill":
        result, spec, inp = bench_prefill(args, torch, pkv, wl)
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline_prefill(args, torch, spec, inp)
    else:
        result, spec, layers = bench_decode(args, torch, pkv, wl)
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline_decode(args, torch, spec, layers)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
