"""GPU parity on seeded random small shapes, decode and prefill, against the
oracle: head counts and GQA ratios, head dims, dtypes, layouts, page sizes,
ragged and empty rows, forced split-worker counts, planned decode steps and
prefill tilings drawn at random (fixed seeds), every output row compared.
Bar as in the other parity tests."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, DecodeCase, PrefillCase, compare, host_bits, say, tol

pytestmark = pytest.mark.gpu

HEADS = [(4, 4), (8, 2), (12, 4), (16, 1), (32, 8), (6, 1), (24, 8), (2, 2)]


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    rng = np.random.default_rng(1000 + seed)
    b = int(rng.integers(1, 41))
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128, 128, 256]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    layout = "NHD" if rng.random() < 0.3 else "HND"
    lens = np.minimum(np.exp(rng.uniform(0, np.log(3000), size=b)).astype(np.int32) - 1, 2999)
    lens[rng.random(b) < 0.1] = 0
    workers = 0 if rng.random() < 0.6 else int(rng.integers(1, 1200))
    say(f"[random decode {seed}] B={b} Hq={hq} Hkv={hkv} D={d} {dtype} {layout} workers={workers} "
        f"lens[:6]={lens[:6].tolist()}")
    spec = wl.custom_decode_spec(lens, hq=hq, hkv=hkv, head_dim=d, dtype=dtype, seed=2000 + seed, layout=layout)
    case = DecodeCase(spec)
    kc, vc, kl = case.gpu_pools()
    out, lse = case.gpu_decode(kc, vc, kl, workers=workers)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    compare(out.cpu(), ro, *tol(spec), "out")
    compare(lse.cpu(), rl, *tol(spec), "lse")


@pytest.mark.parametrize("seed", range(8))
def test_random_decode_wide(seed):
    """Batches of 65..300 rows, so that the rows' lengths span several 64-row
    chunks and ranges start and end in later chunks; empty rows; forced
    worker counts up to 3000 (many ranges then hold no page); the fused
    append + attend call on even seeds, with its pool writes bit-exact."""
    rng = np.random.default_rng(5000 + seed)
    b = int(rng.integers(65, 301))
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    fused = seed % 2 == 0
    dtype = "bf16" if fused or rng.random() < 0.7 else "f32"
    lens = np.minimum(np.exp(rng.uniform(0, np.log(3000), size=b)).astype(np.int32) - 1, 2999)
    lens[rng.random(b) < 0.15] = 0
    workers = 0 if seed < 4 else int(rng.integers(1, 3001))
    say(f"[random wide decode {seed}] B={b} Hq={hq} Hkv={hkv} D={d} {dtype} fused={fused} workers={workers}")
    spec = wl.custom_decode_spec(lens, hq=hq, hkv=hkv, head_dim=d, dtype=dtype, seed=6000 + seed)
    case = DecodeCase(spec)
    if fused:
        i = case.inp
        kc, vc = wl.empty_pool(spec, case.dev), wl.empty_pool(spec, case.dev)
        pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, torch.zeros(b, dtype=torch.int32, device=case.dev),
                   i.hist_indptr)
        out, lse, new_lens = pkv.append_decode_attn(i.q, kc, vc, i.k_new, i.v_new, i.block_table, i.hist_lens,
                                                    int(spec.hist_lens.max()) + 1, scale=spec.scale,
                                                    workers=workers, return_lse=True)
    else:
        kc, vc, kl = case.gpu_pools()
        out, lse = case.gpu_decode(kc, vc, kl, workers=workers)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    if fused:
        assert np.array_equal(new_lens.cpu().numpy(), olens), "seqlens_out differs"
        assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
        assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool not bit-exact"
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    compare(out.cpu(), ro, *tol(spec), "out")
    compare(lse.cpu(), rl, *tol(spec), "lse")


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(seed):
    rng = np.random.default_rng(3000 + seed)
    b = int(rng.integers(1, 7))
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128, 256, 256]))
    layout = "NHD" if rng.random() < 0.3 else "HND"
    q = rng.integers(1, 401, size=b).astype(np.int32)
    kv = (q + rng.integers(0, 601, size=b)).astype(np.int32)
    causal = bool(rng.random() < 0.8)
    rows = int(rng.choice([0, 128, 192]))
    page = int(rng.choice([16, 16, 32, 64, 128, 256]))
    say(f"[random prefill {seed}] B={b} Hq={hq} Hkv={hkv} D={d} {layout} page={page} causal={causal} "
        f"rows/wg={rows} q={q.tolist()} kv={kv.tolist()}")
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=4000 + seed, layout=layout,
                           page_size=page)
    case = PrefillCase(spec)
    kc, vc, kvl = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kvl, causal=causal, rows=rows)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools(None)
    r, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs, causal=causal)
    compare(out.cpu()[r], ro, *BF16_TOL, "out")
    compare(lse.cpu()[r], rl, *BF16_TOL, "lse")


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill_split(seed):
    """Few query rows over thousands of keys, so that the library splits the
    keys (asserted through the workspace size): head counts, head dims,
    layouts, page sizes, causal or full mask drawn at random, every row
    against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    b = int(rng.integers(1, 4))
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128, 256]))
    layout = "NHD" if rng.random() < 0.3 else "HND"
    q = rng.integers(1, 97, size=b).astype(np.int32)
    kv = (q + rng.integers(1000, 3001, size=b)).astype(np.int32)
    causal = bool(rng.random() < 0.7)
    page = int(rng.choice([16, 32, 64, 128, 256]))
    say(f"[random split prefill {seed}] B={b} Hq={hq} Hkv={hkv} D={d} {layout} page={page} causal={causal} "
        f"q={q.tolist()} kv={kv.tolist()}")
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=7500 + seed, layout=layout,
                           page_size=page)
    case = PrefillCase(spec)
    kc, vc, kvl = case.gpu_pools()
    need = pkv.prefill_workspace_bytes(kc, b, hq, int(q.sum()), int(q.max()), int(kv.max()), layout=layout)
    assert need > 0, "expected a key split"
    out, lse = case.gpu_prefill(kc, vc, kvl, causal=causal)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools(None)
    r, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs, causal=causal)
    compare(out.cpu()[r], ro, *BF16_TOL, "out")
    compare(lse.cpu()[r], rl, *BF16_TOL, "lse")


@pytest.mark.parametrize("seed", range(10))
def test_random_decode_planned(seed):
    """bf16 decode steps with the step's plan (pkv_decode_plan) on random
    shapes: batch 1..300, GQA ratios, head dims, pages of 16..256 tokens,
    HND or NHD, fused or separate calls, automatic or forced worker counts.
    Every row against the oracle, and bit for bit against the same call
    without a plan."""
    rng = np.random.default_rng(9000 + seed)
    b = int(rng.integers(1, 301))
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128, 256]))
    page = int(rng.choice([16, 16, 32, 64, 128, 256]))
    layout = "NHD" if rng.random() < 0.3 else "HND"
    fused = rng.random() < 0.6
    workers = 0 if rng.random() < 0.6 else int(rng.integers(1, 2000))
    lens = np.minimum(np.exp(rng.uniform(0, np.log(3000), size=b)).astype(np.int32) - 1, 2999)
    lens[rng.random(b) < 0.1] = 0
    say(f"[random planned decode {seed}] B={b} Hq={hq} Hkv={hkv} D={d} page={page} {layout} fused={fused} "
        f"workers={workers}")
    spec = wl.custom_decode_spec(lens, hq=hq, hkv=hkv, head_dim=d, dtype="bf16", seed=9500 + seed,
                                 layout=layout, page_size=page)
    case = DecodeCase(spec)
    i = case.inp
    max_kv = int(spec.hist_lens.max()) + 1
    if fused:
        kc, vc = wl.empty_pool(spec, case.dev), wl.empty_pool(spec, case.dev)
        pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, torch.zeros(b, dtype=torch.int32, device=case.dev),
                   i.hist_indptr, layout=layout)
        lens_in = i.hist_lens
    else:
        kc, vc, lens_in = case.gpu_pools()
    nbytes = pkv.decode_workspace_bytes(kc, b, hq, max_kv, layout=layout, workers=workers)
    results = []
    for planned in (False, True):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=case.dev)
        if planned:
            pkv.decode_plan(kc, lens_in, hq, max_kv, ws, fused=fused, layout=layout, workers=workers)
        if fused:
            res = pkv.append_decode_attn(i.q, kc, vc, i.k_new, i.v_new, i.block_table, lens_in, max_kv,
                                         scale=spec.scale, workspace=ws, layout=layout, workers=workers,
                                         return_lse=True)
        else:
            res = pkv.decode_attn(i.q, kc, vc, i.block_table, lens_in, max_kv, scale=spec.scale, workspace=ws,
                                  layout=layout, workers=workers, return_lse=True)
        torch.cuda.synchronize()
        results.append([t.clone() for t in res])
    for x, y in zip(*results):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), "plan changed bits"
    okc, ovc, olens, obt = case.oracle_pools()
    if fused:
        assert np.array_equal(results[1][2].cpu().numpy(), olens), "seqlens_out differs"
        assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    compare(results[1][0].cpu(), ro, *tol(spec), "out")
    compare(results[1][1].cpu(), rl, *tol(spec), "lse")
