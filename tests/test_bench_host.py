"""Host-side arithmetic of bench.py (no GPU): the algorithmic work per call,
the parity record of the CPU-baseline leg, and the counter summaries that
turn rocprofv3 CSV files into HBM bytes per launch."""
from __future__ import annotations

import csv
import importlib.util
import os
import sys

import numpy as np
import pytest
import torch

from paged_kv_attention_pkv_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    sys.argv = ["bench.py"]
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def test_prefill_flops_fixed_request(bench):
    """q = kv = 1023 at Hq 48, D 256: 1023 * 1024 / 2 = 523 776 causal pairs
    (the FlashInfer PR #9451 analysis's single request), 4 flops per pair,
    head dim and head: 25.74 GFLOP."""
    spec = wl.prefill_spec(fixed_1023=True)
    assert bench.prefill_flops(spec) == 4 * 256 * 48 * 523_776 == 25_744_637_952


def test_prefill_flops_counts_visible_pairs(bench):
    """Against a brute-force count of (row, key) pairs under the end-aligned
    causal mask (row i of a request sees keys 0 .. kv - q + i)."""
    rng = np.random.default_rng(5)
    q = rng.integers(1, 40, size=6)
    kv = q + rng.integers(0, 30, size=6)
    spec = wl.prefill_spec(q_lens=q.tolist(), kv_lens=kv.tolist(), hq=4, hkv=2, head_dim=64, seed=3)
    pairs = sum(1 for qq, kk in zip(q, kv) for i in range(qq) for j in range(kk) if j <= kk - qq + i)
    assert bench.prefill_flops(spec) == 4 * 64 * 4 * pairs


def test_decode_bytes_tiny(bench):
    """The tiny fp32 workload by hand: lengths 37 and 80 plus the appended
    token attend 38 and 81 keys over 2 KV heads of 64 fp32 dims (K and V);
    q and out are 2 x 4 x 64 fp32 each; 3 + 6 pages of table entries and 2
    lengths."""
    spec = wl.decode_spec("tiny_f32")
    b = bench.decode_bytes(spec)
    assert b["kv"] == (38 + 81) * 2 * 64 * 2 * 4
    assert b["q_out"] == 2 * (2 * 4 * 64 * 4)
    assert b["table"] == 4 * (3 + 6) + 4 * 2
    assert b["append"] == 0
    assert b["total"] == b["kv"] + b["q_out"] + b["table"]
    fused = bench.decode_bytes(spec, fused=True)
    assert fused["append"] == 2 * 2 * (2 * 2 * 64 * 4) + 4 * 2


def test_parity_record(bench):
    """|gpu - ref| <= atol + rtol |ref| at the bf16 bar (2e-2, 2e-2): an
    element just inside passes, one just outside fails; the record keeps the
    largest errors."""
    ref = np.array([1.0, -2.0, 0.0, 4.0])
    inside = torch.tensor([1.0 + 0.039, -2.0, 0.0, 4.0], dtype=torch.float64).to(torch.float32)
    r = bench.parity(inside, ref, "bf16", "x")
    assert r["pass"] and r["elements"] == 4 and r["atol"] == 2e-2 and r["rtol"] == 2e-2
    assert abs(r["max_abs_err"] - 0.039) < 1e-6
    outside = torch.tensor([1.0, -2.0, 0.03, 4.0])
    assert not bench.parity(outside, ref, "bf16", "x")["pass"]
    assert not bench.parity(torch.tensor([1.0 + 3e-5, -2.0, 0.0, 4.0]), ref, "f32", "x")["pass"]


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(kernel, values, counter="X", grid=1024):
    return [{"Dispatch_Id": str(i), "Kernel_Name": kernel, "Grid_Size": str(grid), "Counter_Name": counter,
             "Counter_Value": str(v)} for i, v in enumerate(values)]


def test_summarize_pmc_scales_by_the_copy(bench, tmp_path):
    """A 1 GiB copy whose FETCH_SIZE reads 512 Ki KiB and WRITE_SIZE 1 Gi KiB
    gives scale factors 2 and 1; a kernel reading a median of 1000 KiB and
    writing 300 KiB per dispatch then moves 2 * 1000 * 1024 + 300 * 1024
    bytes per launch.  Copy dispatches below 1/16 of the copy are ignored,
    and with --largest-grid only the kernel's largest grid counts."""
    d = tmp_path
    k = "void pkv::(anonymous namespace)::some_kernel<1>(Args)"
    _write_csv(d / "f.csv", _counter_rows(k, [900.0, 1000.0, 5000.0]) + _counter_rows(k, [7.0], grid=64))
    _write_csv(d / "w.csv", _counter_rows(k, [300.0, 300.0, 200.0]) + _counter_rows(k, [7.0], grid=64))
    _write_csv(d / "cf.csv", _counter_rows("copyBuffer", [524288.0, 524288.0, 10.0]))
    _write_csv(d / "cw.csv", _counter_rows("copyBuffer", [1048576.0]))
    out = d / "s.txt"
    bench.summarize_pmc([str(d / "f.csv"), str(d / "w.csv"), str(d / "cf.csv"), str(d / "cw.csv"), str(out),
                         "--kernel", "some_kernel", "--kind", "decode", "--command", "cmd", "--largest-grid"])
    text = out.read_text()
    assert "hbm_bytes_per_launch: %d" % (2 * 1000 * 1024 + 300 * 1024) in text
    assert f"source_sha256_16: {bench.source_hash('decode')}" in text


def test_traffic_needs_the_current_sources(bench, tmp_path, monkeypatch):
    """A counter summary counts only while its recorded source hash is that
    of the kernel's current sources."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    csrc = tmp_path / "paged_kv_attention_pkv_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES["decode"]:
        (csrc / name).write_text("// " + name + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    good = bench.source_hash("decode")
    (prof / "a.txt").write_text(f"source_sha256_16: {good}\nhbm_bytes_per_launch: 1234\n")
    (prof / "b.txt").write_text("source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1234\n")
    assert bench.traffic_from_profile("decode", "a.txt") == 1234.0
    assert bench.traffic_from_profile("decode", "b.txt") is None
    assert bench.traffic_from_profile("decode", "missing.txt") is None
    (csrc / "decode.hip").write_text("// changed\n")
    assert bench.traffic_from_profile("decode", "a.txt") is None
