"""GPU tests of pkv_decode_plan (the cut of a decode step computed once).

A call that takes the plan from its workspace must give the same bits as a
call that plans on its own (outputs, lse, seqlens_out and the pools), on
every call that shares the plan, and both must meet the attention bar
against the oracle.  A plan that no longer matches the call (other lengths,
mode, worker count or batch) must be ignored, so the result is again the
call's own."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import DecodeCase, compare, host_bits, say, tol

pytestmark = pytest.mark.gpu


def _ws(kc, batch, hq, max_kv, layout, workers=0):
    return torch.zeros(pkv.decode_workspace_bytes(kc, batch, hq, max_kv, layout=layout, workers=workers),
                       dtype=torch.uint8, device=kc.device)


def _history(case):
    s, i = case.spec, case.inp
    kc, vc = wl.empty_pool(s, case.dev), wl.empty_pool(s, case.dev)
    zeros = torch.zeros(s.batch, dtype=torch.int32, device=case.dev)
    pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, zeros, i.hist_indptr, layout=s.layout)
    return kc, vc


def _fused(case, kc, vc, lens, max_kv, ws, workers=0):
    s, i = case.spec, case.inp
    return pkv.append_decode_attn(i.q, kc, vc, i.k_new, i.v_new, i.block_table, lens, max_kv, scale=s.scale,
                                  workspace=ws, layout=s.layout, workers=workers, return_lse=True)


def _same(a, b, what):
    for x, y, nm in zip(a, b, ("out", "lse", "lens")):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), f"{what}: {nm} differs"


def _spec(batch, seed=11, pad=0, empty=0):
    """Qwen3-shaped rows (Hq 32 / Hkv 8 / D 128) with log-uniform lengths up
    to 4096 and `empty` rows of length 0, and the indices of `pad` further
    rows that the calls get as padding slots (length -1)."""
    rng = np.random.default_rng(seed)
    hist = np.exp(rng.uniform(np.log(1), np.log(4096), batch)).astype(np.int32)
    idx = rng.permutation(batch)
    hist[idx[:empty]] = 0
    return wl.custom_decode_spec(hist, 32, 8, 128, "bf16", seed, extra_cols=2), idx[empty:empty + pad]


@pytest.mark.parametrize("batch,pad,empty", [(1, 0, 0), (8, 0, 0), (64, 0, 0), (64, 5, 3), (100, 0, 2),
                                             (300, 7, 4)])
def test_planned_fused_calls_bit_equal_and_oracle(batch, pad, empty):
    spec, pads = _spec(batch, seed=batch + pad, pad=pad, empty=empty)
    say(f"[plan] fused B={batch} pad={pad} empty={empty}")
    case = DecodeCase(spec)
    kc, vc = _history(case)
    lens = case.inp.hist_lens.clone()
    lens[torch.from_numpy(pads).to(case.dev)] = -1
    live = np.ones(batch, bool)
    live[pads] = False
    max_kv = int(spec.hist_lens.max()) + 1
    ws_own = _ws(kc, batch, spec.hq, max_kv, spec.layout)
    ref = _fused(case, kc, vc, lens, max_kv, ws_own)
    kbits, vbits = host_bits(kc).copy(), host_bits(vc).copy()
    ws = _ws(kc, batch, spec.hq, max_kv, spec.layout)
    pkv.decode_plan(kc, lens, spec.hq, max_kv, ws, fused=True, layout=spec.layout)
    for call in range(3):  # one plan, several calls (the layers of a step)
        got = _fused(case, kc, vc, lens, max_kv, ws)
        torch.cuda.synchronize()
        _same(got, ref, f"planned call {call}")
    assert np.array_equal(host_bits(kc), kbits) and np.array_equal(host_bits(vc), vbits), "pools differ"
    assert np.all(ref[2].cpu().numpy()[~live] == -1)
    # the planned result against the oracle (padding slots: zero output and
    # -inf lse, as an oracle row of length 0; their pages belong to no live row)
    okc, ovc, olens, obt = case.oracle_pools()
    assert np.array_equal(got[2].cpu().numpy()[live], olens[live])
    ref_out, ref_lse = case.oracle_decode(okc, ovc, np.where(live, olens, 0).astype(np.int32), obt)
    atol, rtol = tol(spec)
    say("  out:", compare(got[0].cpu(), ref_out, atol, rtol, "planned out"))
    compare(got[1].cpu(), ref_lse, atol, rtol, "planned lse")


def test_planned_decode_calls_and_mode_mismatch():
    """A plan for separate decode calls is used by them; a fused plan is
    not taken by a separate call (other mode), nor the reverse."""
    spec, _ = _spec(64, seed=5, empty=2)
    say("[plan] separate decode B=64, mode mismatch")
    case = DecodeCase(spec)
    kc, vc, lens = case.gpu_pools()
    max_kv = int(spec.hist_lens.max()) + 1
    s = spec

    def call(ws):
        return pkv.decode_attn(case.inp.q, kc, vc, case.inp.block_table, lens, max_kv, scale=s.scale,
                               workspace=ws, layout=s.layout, return_lse=True)

    ref = call(_ws(kc, 64, s.hq, max_kv, s.layout))
    ws = _ws(kc, 64, s.hq, max_kv, s.layout)
    pkv.decode_plan(kc, lens, s.hq, max_kv, ws, fused=False, layout=s.layout)
    for _ in range(2):
        got = call(ws)
        torch.cuda.synchronize()
        _same(got, ref, "planned separate call")
    pkv.decode_plan(kc, lens, s.hq, max_kv, ws, fused=True, layout=s.layout)
    _same(call(ws), ref, "separate call after a fused plan")
    # a separate plan on the pre-append lengths, then the fused call
    kc2, vc2 = _history(case)
    ref_f = _fused(case, kc2, vc2, case.inp.hist_lens, max_kv, _ws(kc, 64, s.hq, max_kv, s.layout))
    ws2 = _ws(kc, 64, s.hq, max_kv, s.layout)
    pkv.decode_plan(kc2, case.inp.hist_lens, s.hq, max_kv, ws2, fused=False, layout=s.layout)
    got = _fused(case, kc2, vc2, case.inp.hist_lens, max_kv, ws2)
    torch.cuda.synchronize()
    _same(got, ref_f, "fused call after a separate plan")
    compare(ref[0].cpu(), case.oracle_decode(*case.oracle_pools())[0], *tol(s), "separate out")


def test_stale_plan_is_ignored():
    """Lengths changed after the plan (one row, or all), a different
    max_kv_len, worker count or batch: the call plans on its own."""
    spec, _ = _spec(96, seed=21, empty=1)
    say("[plan] stale plans B=96")
    case = DecodeCase(spec)
    s = spec
    max_kv = int(spec.hist_lens.max()) + 1
    lens0 = case.inp.hist_lens
    kc, vc = _history(case)
    w_auto = pkv.decode_workspace_bytes(kc, 96, s.hq, max_kv, layout=s.layout)
    w_37 = pkv.decode_workspace_bytes(kc, 96, s.hq, max_kv, layout=s.layout, workers=37)
    ws = torch.zeros(max(w_auto, w_37), dtype=torch.uint8, device=case.dev)
    ws_own = torch.zeros_like(ws)

    def both(lens, mk=max_kv, workers=0, rows=None):
        i = case.inp
        sl = slice(None) if rows is None else slice(0, rows)
        args = (i.q[sl], kc, vc, i.k_new[sl], i.v_new[sl], i.block_table[sl], lens[sl], mk)
        ref = pkv.append_decode_attn(*args, scale=s.scale, workspace=ws_own, layout=s.layout, workers=workers,
                                     return_lse=True)
        got = pkv.append_decode_attn(*args, scale=s.scale, workspace=ws, layout=s.layout, workers=workers,
                                     return_lse=True)
        torch.cuda.synchronize()
        return got, ref

    pkv.decode_plan(kc, lens0, s.hq, max_kv, ws, fused=True, layout=s.layout)
    got, ref = both(lens0)
    _same(got, ref, "matching plan")
    one = lens0.clone()
    r = int(np.flatnonzero(spec.hist_lens > 40)[0])
    one[r] -= 17
    got, ref = both(one)
    _same(got, ref, "one row shorter than planned")
    got, ref = both(torch.clamp(lens0 - 1, min=0))
    _same(got, ref, "every row shorter than planned")
    got, ref = both(lens0, mk=max_kv + 16)
    _same(got, ref, "other max_kv_len")
    got, ref = both(lens0, workers=37)
    _same(got, ref, "other worker count")
    got, ref = both(lens0, rows=48)
    _same(got, ref, "smaller batch")
    # the 48-row calls laid out their records over the counters of rows
    # 48..95: a workspace reused for another batch is reset first
    for w in (ws, ws_own):
        pkv.decode_workspace_reset(kc, 96, w, layout=s.layout)
    pkv.decode_plan(kc, lens0, s.hq, max_kv, ws, fused=True, layout=s.layout, workers=37)
    got, ref = both(lens0, workers=37)
    _same(got, ref, "matching plan, 37 workers")
    got, ref = both(lens0)
    _same(got, ref, "plan for 37 workers, automatic call")


def test_plan_in_graph_replays():
    """The plan and two layers' fused calls captured in one HIP graph;
    every replay (eager work between them) gives the eager bits."""
    spec = wl.decode_spec("qwen3_decode", batch=64)
    say("[plan] graph of plan + 2 layers, B=64")
    s = spec
    dev = torch.device("cuda")
    cases = [DecodeCase(spec, seed_offset=k) for k in range(2)]
    pools = [_history(c) for c in cases]
    max_kv = int(spec.hist_lens.max()) + 1
    lens = cases[0].inp.hist_lens
    ws_own = _ws(pools[0][0], 64, s.hq, max_kv, s.layout)
    refs = [_fused(c, kc, vc, lens, max_kv, ws_own) for c, (kc, vc) in zip(cases, pools)]
    torch.cuda.synchronize()
    refs = [tuple(t.clone() for t in r) for r in refs]
    ws = _ws(pools[0][0], 64, s.hq, max_kv, s.layout)
    outs = [(torch.empty_like(c.inp.q), torch.empty(64, s.hq, dtype=torch.float32, device=dev),
             torch.empty_like(lens)) for c in cases]
    calls = [pkv.api.prepare_decode_plan(pools[0][0], lens, s.hq, max_kv, ws, fused=True, layout=s.layout)]
    for c, (kc, vc), (o, l, so) in zip(cases, pools, outs):
        i = c.inp
        calls.append(pkv.api.prepare_append_decode(i.q, kc, vc, i.k_new, i.v_new, i.block_table, lens, max_kv,
                                                   s.scale, o, ws, seqlens_out=so, lse=l, layout=s.layout))

    def step():
        for f in calls:
            f()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:
            o[0].fill_(float("nan"))
            o[1].fill_(float("nan"))
            o[2].fill_(-7)
        _fused(cases[0], *pools[0], lens, max_kv, ws_own)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(2):
            _same(outs[k], refs[k], f"replay {rep} layer {k}")


@pytest.mark.parametrize("page,layout,d,hq,hkv", [(64, "HND", 128, 32, 8), (256, "HND", 256, 48, 8),
                                                  (16, "NHD", 128, 32, 8), (16, "HND", 64, 16, 2),
                                                  (32, "NHD", 64, 8, 8)])
def test_planned_calls_every_kernel(page, layout, d, hq, hkv):
    """Planned fused calls on the other kernel instances (head_dim 64 / 256,
    pages of 32..256 tokens, NHD) give the bits of unplanned ones."""
    rng = np.random.default_rng(page + d)
    hist = np.exp(rng.uniform(0, np.log(3000), 40)).astype(np.int32)
    spec = wl.custom_decode_spec(hist, hq, hkv, d, "bf16", page + d, layout=layout, page_size=page)
    say(f"[plan] page={page} {layout} D={d} Hq={hq} Hkv={hkv} B=40")
    case = DecodeCase(spec)
    kc, vc = _history(case)
    lens = case.inp.hist_lens
    max_kv = int(hist.max()) + 1
    ref = _fused(case, kc, vc, lens, max_kv, _ws(kc, 40, hq, max_kv, layout))
    ws = _ws(kc, 40, hq, max_kv, layout)
    pkv.decode_plan(kc, lens, hq, max_kv, ws, fused=True, layout=layout)
    for call in range(2):
        got = _fused(case, kc, vc, lens, max_kv, ws)
        torch.cuda.synchronize()
        _same(got, ref, f"planned call {call}")
