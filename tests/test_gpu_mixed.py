"""GPU parity of pkv_mixed_attn: chunked prefill requests and decode rows of
one batch in one launch, against the oracle (every decode row, chunk rows
all or tile-edge sampled) and against the separate calls: bit for bit with
pkv_prefill_attn on the chunks (the same query tiles and key splits), within
the bf16 bar of pkv_decode_attn on the decode rows (the same sums cut
another way)."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, PrefillCase, compare, say, with_scale
from test_gpu_prefill import tile_edge_rows

pytestmark = pytest.mark.gpu


def _mixed(case, num_prefill):
    s, i = case.spec, case.inp
    kc, vc, kv = case.gpu_pools()
    max_q = int(s.q_lens[:num_prefill].max()) if num_prefill else 0
    out, lse = pkv.mixed_attn(i.q, kc, vc, i.block_table, kv, i.qo_indptr, num_prefill, max_q,
                              int(s.kv_lens.max()), s.scale, return_lse=True, layout=s.layout)
    torch.cuda.synchronize()
    return kc, vc, kv, out, lse


def _check(spec, num_prefill, sample_chunks=False):
    say(f"[mixed] {spec.name} chunks q={spec.q_lens[:num_prefill].tolist()} kv={spec.kv_lens[:num_prefill].tolist()} "
        f"decode rows {spec.batch - num_prefill} D={spec.head_dim}")
    case = PrefillCase(spec, gen_device="cuda" if sample_chunks else "cpu")
    kc, vc, kv, out, lse = _mixed(case, num_prefill)
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    if sample_chunks:
        pick = lambda r, q_len: tile_edge_rows(r, q_len) if r < num_prefill else np.arange(q_len)
        rows, ro, rl = case.oracle_row_set(okc, ovc, okv, obt, oreqs, pick)
    else:
        rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs)
    s1 = compare(out.cpu()[rows], ro, *BF16_TOL, "mixed out")
    s2 = compare(lse.cpu()[rows], rl, *BF16_TOL, "mixed lse")
    say(f"  rows checked {len(rows)} of {out.shape[0]}; out: {s1}; lse: {s2}")
    return case, kc, vc, kv, out, lse


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_small_all_rows(d):
    q = [65, 300, 129, 1, 1, 1, 1, 1, 1, 1, 1]
    kv = [200, 300, 1000, 1, 2, 16, 17, 100, 700, 1500, 2049]
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=32, hkv=8, head_dim=d, seed=d + 3)
    _check(spec, 3)


def test_mixed_equals_separate_calls():
    """Chunk rows and their lse bit for bit equal to pkv_prefill_attn on the
    chunks (the launch runs the same query tiles); decode rows within the
    bf16 bar of pkv_decode_attn (a KV head's query heads as one 16-row block
    walking the keys in 64-key tiles, against the decode kernel's split
    workers)."""
    spec = wl.mixed_spec(num_decode=40, num_chunks=3, seed=701, max_chunk=600, max_extra=900)
    case, kc, vc, kv, out, lse = _check(spec, 3)
    i, s = case.inp, spec
    P = 3
    npf = int(s.q_lens[:P].sum())
    po, pl = pkv.prefill_attn(i.q[:npf], kc, vc, i.block_table[:P], kv[:P], i.qo_indptr[:P + 1],
                              int(s.q_lens[:P].max()), int(s.kv_lens.max()), s.scale, return_lse=True)
    do, dl = pkv.decode_attn(i.q[npf:], kc, vc, i.block_table[P:].contiguous(), kv[P:].contiguous(),
                             int(s.kv_lens.max()), s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:npf].view(torch.int16), po.view(torch.int16)), "chunk rows differ from pkv_prefill_attn"
    assert torch.equal(lse[:npf], pl), "chunk lse differs"
    compare(out[npf:].cpu(), do.float().cpu().double().numpy(), *BF16_TOL, "decode rows vs pkv_decode_attn")
    compare(lse[npf:].cpu(), dl.cpu().double().numpy(), *BF16_TOL, "decode lse vs pkv_decode_attn")


def test_mixed_full_size_qwen3():
    """The mixed serving step of the benchmark (4 chunks of up to 2048 rows
    continuing prompts of up to 6144 keys, 64 decode rows of 513..1025
    keys): every decode row, tile-edge rows of every chunk."""
    _check(wl.mixed_spec(), 4, sample_chunks=True)


def test_mixed_chunks_up_to_4096():
    _check(wl.mixed_spec(num_decode=32, num_chunks=3, seed=702, max_chunk=4096), 3, sample_chunks=True)


def test_mixed_only_decode_and_only_prefill():
    spec = wl.prefill_spec(q_lens=[1] * 9, kv_lens=[1, 5, 16, 17, 33, 300, 2000, 64, 129], hq=16, hkv=4,
                           head_dim=128, seed=9)
    _check(spec, 0)
    spec = wl.prefill_spec(q_lens=[40, 1, 200], kv_lens=[40, 90, 333], hq=16, hkv=4, head_dim=128, seed=10)
    _check(spec, 3)


def test_mixed_empty_decode_rows():
    """Decode rows with no keys give out = 0, lse = -inf; the other rows are
    unchanged by them."""
    spec = wl.prefill_spec(q_lens=[100, 1, 1, 1, 1], kv_lens=[150, 40, 40, 40, 40], hq=32, hkv=8, head_dim=128,
                           seed=11)
    say("[mixed] empty decode rows")
    case = PrefillCase(spec)
    kc, vc, kv = case.gpu_pools()
    i, s = case.inp, spec
    kv0 = kv.clone()
    kv0[2] = 0
    kv0[4] = 0
    out, lse = pkv.mixed_attn(i.q, kc, vc, i.block_table, kv0, i.qo_indptr, 1, 100, 150, s.scale, return_lse=True)
    ref, rlse = pkv.mixed_attn(i.q, kc, vc, i.block_table, kv, i.qo_indptr, 1, 100, 150, s.scale, return_lse=True)
    torch.cuda.synchronize()
    o, l = out.float().cpu(), lse.cpu()
    for r in (101, 103):
        assert torch.all(o[r] == 0) and torch.all(torch.isneginf(l[r])), r
    keep = [x for x in range(104) if x not in (101, 103)]
    assert torch.equal(out[keep].view(torch.int16), ref[keep].view(torch.int16))


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_mixed_negative_and_zero_scale(scale):
    """Chunks and packed decode rows with a negative and a zero softmax
    scale (applied as the negated query, and as the smallest normal float)."""
    q = [65, 129, 1, 1, 1, 1]
    kv = [200, 1000, 1, 17, 700, 2049]
    _check(with_scale(wl.prefill_spec(q_lens=q, kv_lens=kv, hq=32, hkv=8, head_dim=128, seed=31), scale), 2)


def test_mixed_long_decode_rows_split():
    """With max_kv_len above 8192 the decode rows run as a split decode
    launch beside the chunks' prefill launch: every row against the oracle,
    chunk rows bit-equal to pkv_prefill_attn and decode rows to
    pkv_decode_attn; without a workspace the call reports PKV_EWORKSPACE."""
    rng = np.random.default_rng(41)
    q = [130, 65, 1, 1, 1, 1, 1, 1, 1, 1]
    dec = np.clip(np.rint(np.exp(rng.uniform(np.log(16), np.log(20000), size=8))), 16, 20000).astype(int) + 1
    kv = [400, 2000] + dec.tolist()
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=32, hkv=8, head_dim=128, seed=41)
    assert int(spec.kv_lens.max()) > pkv.api.MIXED_PACKED_MAX_KV
    case, kc, vc, kv_d, out, lse = _check(spec, 2)
    i, s = case.inp, spec
    P, npf = 2, int(spec.q_lens[:2].sum())
    max_kv = int(s.kv_lens.max())
    ref_p, ref_pl = pkv.prefill_attn(i.q[:npf], kc, vc, i.block_table[:P], kv_d[:P], i.qo_indptr[:P + 1],
                                     int(s.q_lens[:P].max()), max_kv, scale=s.scale, return_lse=True)
    ref_d, ref_dl = pkv.decode_attn(i.q[npf:].contiguous(), kc, vc, i.block_table[P:].contiguous(),
                                    kv_d[P:].contiguous(), max_kv, scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:npf].view(torch.int16), ref_p.view(torch.int16)), "chunk rows differ from prefill_attn"
    assert torch.equal(lse[:npf].view(torch.int32), ref_pl.view(torch.int32))
    assert torch.equal(out[npf:].view(torch.int16), ref_d.view(torch.int16)), "decode rows differ from decode_attn"
    assert torch.equal(lse[npf:].view(torch.int32), ref_dl.view(torch.int32))
    # the raw call without a workspace
    desc, args = pkv.api._mixed_args(i.q, kc, vc, i.block_table, kv_d, i.qo_indptr, P, int(s.q_lens[:P].max()),
                                     max_kv, s.scale, torch.empty_like(i.q), None, None, "HND")
    rc = pkv.api.lib().pkv_mixed_attn(*args, pkv.api._stream(kc))
    assert rc == 3, rc


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_short_chunk_over_long_keys(d):
    """A chunk of few rows continuing a long prompt next to decode rows: with
    a workspace its keys split as in pkv_prefill_attn (chunk rows bit-equal
    to pkv_prefill_attn given a workspace, every row against the oracle);
    without one (split=False) the chunk runs unsplit, bit-equal to
    pkv_prefill_attn without one."""
    rng = np.random.default_rng(50 + d)
    dec = rng.integers(512, 1025, size=48).tolist()
    spec = wl.prefill_spec(q_lens=[99] + [1] * 48, kv_lens=[3879] + dec, hq=32, hkv=8, head_dim=d, seed=51 + d)
    case, kc, vc, kv, out, lse = _check(spec, 1)
    i, s = case.inp, spec
    assert pkv.prefill_workspace_bytes(kc, 1, 32, 99, 99, int(s.kv_lens.max())) > 0, "expected a key split"
    max_kv = int(s.kv_lens.max())
    for split in (True, False):
        o, l = (out, lse) if split else pkv.mixed_attn(i.q, kc, vc, i.block_table, kv, i.qo_indptr, 1, 99, max_kv,
                                                       s.scale, return_lse=True, split=False)
        ref_p, ref_pl = pkv.prefill_attn(i.q[:99], kc, vc, i.block_table[:1], kv[:1], i.qo_indptr[:2], 99, max_kv,
                                         scale=s.scale, return_lse=True, split=split)
        torch.cuda.synchronize()
        assert torch.equal(o[:99].view(torch.int16), ref_p.view(torch.int16)), f"chunk rows, split={split}"
        assert torch.equal(l[:99].view(torch.int32), ref_pl.view(torch.int32)), f"chunk lse, split={split}"
    compare(out[:99].cpu(), o[:99].cpu().double().numpy(), *BF16_TOL, "split vs unsplit chunk rows")
    assert torch.equal(out[99:].view(torch.int16), o[99:].view(torch.int16)), "decode rows depend on the chunk split"


def test_mixed_many_decode_rows_two_launches():
    """More decode-row workgroups (rows x Hkv) than two rounds over the CUs:
    with a workspace the call runs the chunks as pkv_prefill_attn and the
    decode rows as pkv_decode_attn (both bit for bit); without one it stays
    one launch (decode rows within the bar). Every row against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_dec = 2 * cus // 8 + 16
    rng = np.random.default_rng(77)
    dec = rng.integers(16, 1025, size=n_dec).tolist()
    spec = wl.prefill_spec(q_lens=[300, 70] + [1] * n_dec, kv_lens=[900, 2500] + dec, hq=32, hkv=8, head_dim=128,
                           seed=78)
    case, kc, vc, kv, out, lse = _check(spec, 2)
    i, s = case.inp, spec
    P, npf, max_kv = 2, 370, int(s.kv_lens.max())
    ref_p, ref_pl = pkv.prefill_attn(i.q[:npf], kc, vc, i.block_table[:P], kv[:P], i.qo_indptr[:P + 1], 300, max_kv,
                                     scale=s.scale, return_lse=True)
    ref_d, ref_dl = pkv.decode_attn(i.q[npf:].contiguous(), kc, vc, i.block_table[P:].contiguous(),
                                    kv[P:].contiguous(), max_kv, scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:npf].view(torch.int16), ref_p.view(torch.int16)), "chunk rows differ from prefill_attn"
    assert torch.equal(lse[:npf].view(torch.int32), ref_pl.view(torch.int32))
    assert torch.equal(out[npf:].view(torch.int16), ref_d.view(torch.int16)), "decode rows differ from decode_attn"
    assert torch.equal(lse[npf:].view(torch.int32), ref_dl.view(torch.int32))
    # the raw call without a workspace: one launch
    o1 = torch.empty_like(i.q)
    l1 = torch.empty((o1.shape[0], s.hq), dtype=torch.float32, device=o1.device)
    desc, args = pkv.api._mixed_args(i.q, kc, vc, i.block_table, kv, i.qo_indptr, P, 300, max_kv, s.scale, o1, l1,
                                     None, "HND")
    assert pkv.api.lib().pkv_mixed_attn(*args, pkv.api._stream(kc)) == 0
    torch.cuda.synchronize()
    compare(o1[npf:].cpu(), ref_d.cpu().double().numpy(), *BF16_TOL, "one-launch decode rows")
    compare(l1[npf:].cpu(), ref_dl.cpu().double().numpy(), *BF16_TOL, "one-launch decode lse")


@pytest.mark.parametrize("seed", range(8))
def test_random_mixed(seed):
    """Random serving steps: 0-3 chunks (1-400 rows over up to 3000 more keys,
    so that some split their keys), 0-120 decode rows (enough, with 8 KV heads,
    for the two-launch route), head counts, head dims 64/128, HND or NHD,
    pages of 16-256 tokens; every row against the oracle."""
    rng = np.random.default_rng(8800 + seed)
    hq, hkv = [(32, 8), (16, 4), (8, 8), (12, 2)][int(rng.integers(4))]
    d = int(rng.choice([64, 128]))
    nc = int(rng.integers(0, 4))
    nd = int(rng.integers(0 if nc else 1, 121))
    q = rng.integers(1, 401, size=nc).tolist()
    kv = [x + int(rng.integers(0, 3001)) for x in q]
    dec = rng.integers(0, 3001, size=nd).tolist()
    layout = "NHD" if rng.random() < 0.4 else "HND"
    page = int(rng.choice([16, 16, 32, 64, 128, 256]))
    say(f"[random mixed {seed}] Hq={hq} Hkv={hkv} D={d} {layout} page={page} chunks q={q} kv={kv} decode rows {nd}")
    dec_kv = [max(x, 1) for x in dec]
    spec = wl.prefill_spec(q_lens=q + [1] * nd, kv_lens=kv + dec_kv, hq=hq, hkv=hkv, head_dim=d, seed=8900 + seed,
                           layout=layout, page_size=page)
    _check(spec, nc)
