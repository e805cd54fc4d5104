"""HIP-graph replay of the hot path: the fused decode step (append + attend)
and a prefill call, captured once and replayed several times with eager work
and synchronisations in between.  Every replay must reproduce the eager call
bit for bit (both kernels are deterministic, and neither records a memset:
the decode workspace's arrival counters are reset by the kernel itself), and
the eager result is itself checked against the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, DecodeCase, PrefillCase, compare, say, tol

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replays_match(call, outs, what):
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays; stale values must not survive
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), \
                f"{what}: replay {i} differs from the eager call"


def test_fused_decode_step_graph():
    say("[graph] fused decode step, B=48")
    rng = np.random.default_rng(41)
    hist = rng.integers(100, 1500, size=48).astype(np.int32)
    spec = wl.custom_decode_spec(hist, hq=32, hkv=8, head_dim=128, dtype="bf16", seed=41)
    case = DecodeCase(spec)
    dev = case.dev
    inp = case.inp
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    zeros = torch.zeros(spec.batch, dtype=torch.int32, device=dev)
    pkv.append(kc, vc, inp.k_hist, inp.v_hist, inp.block_table, zeros, inp.hist_indptr)
    max_kv = int(hist.max()) + 1
    ws = torch.zeros(pkv.decode_workspace_bytes(kc, spec.batch, spec.hq, max_kv), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp.q)
    lse = torch.empty((spec.batch, spec.hq), dtype=torch.float32, device=dev)
    lens = torch.empty_like(inp.hist_lens)
    call = pkv.api.prepare_append_decode(inp.q, kc, vc, inp.k_new, inp.v_new, inp.block_table, inp.hist_lens,
                                         max_kv, spec.scale, out, ws, seqlens_out=lens, lse=lse)
    call()
    torch.cuda.synchronize()
    assert lens.cpu().numpy().tolist() == (hist + 1).tolist()
    okc, ovc, olens, obt = case.oracle_pools()
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    compare(out.cpu(), ro, *tol(spec), "eager out")
    compare(lse.cpu(), rl, *tol(spec), "eager lse")
    _replays_match(call, [out, lse], "fused decode")


@pytest.mark.parametrize("rows", [128, 192])
def test_prefill_graph(rows):
    say(f"[graph] prefill, D=256, rows/wg {rows}")
    spec = wl.prefill_spec(q_lens=[300, 77, 520], kv_lens=[700, 77, 900], hq=12, hkv=2, head_dim=256, seed=43)
    case = PrefillCase(spec)
    kc, vc, kv = case.gpu_pools()
    out = torch.empty_like(case.inp.q)
    lse = torch.empty((out.shape[0], spec.hq), dtype=torch.float32, device=case.dev)
    call = pkv.api.prepare_prefill(case.inp.q, kc, vc, case.inp.block_table, kv, case.inp.qo_indptr,
                                   int(spec.q_lens.max()), int(spec.kv_lens.max()), spec.scale, out, lse=lse,
                                   rows_per_workgroup=rows)
    call()
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools(None)
    r, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs)
    compare(out.cpu()[r], ro, *BF16_TOL, "eager out")
    compare(lse.cpu()[r], rl, *BF16_TOL, "eager lse")
    _replays_match(call, [out, lse], "prefill")
