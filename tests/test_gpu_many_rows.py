"""GPU parity at wide batches of short rows: thousands of decode rows (the
length scans and plan checks run over dozens of 64-row chunks, most ranges
hold several whole rows) and hundreds of prefill requests of a few query
rows each (the grid holds hundreds of requests).  Every output row against
the oracle; pools bit-exact after the fused append."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, DecodeCase, PrefillCase, compare, host_bits, say, tol

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,d", [(3000, 128), (1500, 256)])
def test_fused_decode_thousands_of_short_rows(batch, d):
    """Fused append + attend over `batch` rows of 0..300 cached tokens (one in
    ten empty before the append), Hq 32 / Hkv 8, automatic workers; the same
    call after a pkv_decode_plan gives the same bits."""
    rng = np.random.default_rng(batch + d)
    lens = np.minimum(np.exp(rng.uniform(0, np.log(300), size=batch)).astype(np.int32), 300)
    lens[rng.random(batch) < 0.1] = 0
    say(f"[many rows decode] B={batch} D={d} fused")
    spec = wl.custom_decode_spec(lens, hq=32, hkv=8, head_dim=d, dtype="bf16", seed=7100 + batch)
    case = DecodeCase(spec)
    i = case.inp
    max_kv = int(spec.hist_lens.max()) + 1
    zeros = torch.zeros(batch, dtype=torch.int32, device=case.dev)
    pools = []
    for _ in range(2):
        kc, vc = wl.empty_pool(spec, case.dev), wl.empty_pool(spec, case.dev)
        pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, zeros, i.hist_indptr)
        pools.append((kc, vc))
    ws = torch.zeros(pkv.decode_workspace_bytes(pools[0][0], batch, spec.hq, max_kv), dtype=torch.uint8,
                     device=case.dev)
    out, lse, new_lens = pkv.append_decode_attn(i.q, *pools[0], i.k_new, i.v_new, i.block_table, i.hist_lens,
                                                max_kv, scale=spec.scale, workspace=ws, return_lse=True)
    pkv.decode_plan(pools[1][0], i.hist_lens, spec.hq, max_kv, ws, fused=True)
    out_p, lse_p, _ = pkv.append_decode_attn(i.q, *pools[1], i.k_new, i.v_new, i.block_table, i.hist_lens,
                                             max_kv, scale=spec.scale, workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    assert np.array_equal(new_lens.cpu().numpy(), olens), "seqlens_out differs"
    for kc, vc in pools:
        assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
        assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool not bit-exact"
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    say("  out:", compare(out.cpu(), ro, *tol(spec), "out"))
    compare(lse.cpu(), rl, *tol(spec), "lse")
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16)), "planned call differs"
    assert torch.equal(lse_p.view(torch.int32), lse.view(torch.int32)), "planned lse differs"


@pytest.mark.parametrize("batch,d,hq,hkv", [(400, 128, 16, 4), (200, 256, 48, 8), (300, 64, 8, 8)])
def test_prefill_hundreds_of_short_requests(batch, d, hq, hkv):
    """`batch` requests of 1..8 query rows over q..q+80 keys (chunked-prefill
    continuations), causal; every row of every request against the oracle."""
    rng = np.random.default_rng(batch + d)
    q = rng.integers(1, 9, size=batch).astype(np.int32)
    kv = (q + rng.integers(0, 81, size=batch)).astype(np.int32)
    say(f"[many rows prefill] B={batch} D={d} Hq={hq} Hkv={hkv} total_q={int(q.sum())}")
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=7200 + batch)
    case = PrefillCase(spec)
    kc, vc, kvl = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kvl)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools(None)
    r, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs)
    assert len(r) == int(q.sum())
    say("  out:", compare(out.cpu()[r], ro, *BF16_TOL, "out"))
    compare(lse.cpu()[r], rl, *BF16_TOL, "lse")
