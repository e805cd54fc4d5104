"""GPU parity of pkv_prefill_attn (bf16, MFMA) against the oracle.

Bar: |d| <= 2e-2 + 2e-2|ref| element by element on out and lse.  Large
workloads are checked on sampled rows: the first and last rows of requests,
each computed by the oracle as its own chunked-prefill request.  At head_dim
256 both workgroup tilings (128 and 192 query rows, forced through
pkv_prefill_attn_ex) are checked next to the library's own choice."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, PrefillCase, compare, say, with_scale

pytestmark = pytest.mark.gpu


def _parity(spec, causal=True, sample=None, reqs=None, gen_device="cpu", rows=0):
    say(f"[prefill parity] {spec.name} B={spec.batch} Hq={spec.hq} Hkv={spec.hkv} D={spec.head_dim} "
        f"q={spec.q_lens.tolist()[:8]} kv={spec.kv_lens.tolist()[:8]} causal={causal} seed={spec.seed} "
        f"rows/wg={rows or 'auto'}")
    case = PrefillCase(spec, gen_device=gen_device)
    kc, vc, kv = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kv, causal=causal, rows=rows)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), spec.kv_lens)
    okc, ovc, okv, obt, oreqs = case.oracle_pools(reqs)
    if sample is None:
        rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs, causal=causal)
    else:
        rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs, first=sample, last=sample, causal=causal)
    s1 = compare(out.cpu()[rows], ro, *BF16_TOL, f"{spec.name} out")
    s2 = compare(lse.cpu()[rows], rl, *BF16_TOL, f"{spec.name} lse")
    say(f"  rows checked {len(rows)}; out: {s1}; lse: {s2}")
    return case, kc, vc, kv, out, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (12, 2), (48, 8)])
def test_small_ragged(d, hq, hkv):
    q = [1, 17, 128, 129, 200, 5]
    kv = [1, 17, 300, 129, 611, 40]
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=d + hq)
    _parity(spec)


@pytest.mark.parametrize("rows", [128, 192])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (48, 8)])
def test_d256_tilings_ragged(rows, hq, hkv):
    """Both workgroup tilings of head_dim 256, with requests ending inside,
    at and just past a 192-row tile and one 128-row tile."""
    q = [1, 17, 191, 192, 193, 400, 129]
    kv = [1, 17, 300, 192, 611, 900, 129]
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=256, seed=rows + hq)
    _parity(spec, rows=rows)


@pytest.mark.parametrize("rows", [128, 192])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8)])
def test_d64_d128_tilings_ragged(d, rows, hq, hkv):
    """Both workgroup tilings of head_dim 64 and 128 (8 and 12 waves of 16
    rows), with requests ending inside, at and just past the tiles."""
    q = [1, 17, 191, 192, 193, 255, 256, 257, 400, 129]
    kv = [1, 17, 300, 192, 611, 255, 700, 257, 900, 129]
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=rows + hq + d)
    _parity(spec, rows=rows)


@pytest.mark.parametrize("d,rows", [(128, 0), (128, 128), (64, 192), (256, 128), (256, 192)])
def test_non_causal(d, rows):
    spec = wl.prefill_spec(q_lens=[3, 64, 130], kv_lens=[50, 64, 400], hq=12, hkv=4, head_dim=d, seed=7)
    _parity(spec, causal=False, rows=rows)


def test_nhd_layout():
    spec = wl.prefill_spec(q_lens=[33, 150], kv_lens=[90, 150], hq=16, hkv=4, head_dim=128, seed=8, layout="NHD")
    _parity(spec)


@pytest.mark.parametrize("rows", [128, 192])
def test_nhd_layout_d256(rows):
    """NHD pools at head_dim 256: the 16-row kernel's tile transfers step by
    the token stride Hkv*D, not D."""
    spec = wl.prefill_spec(q_lens=[33, 200, 5], kv_lens=[90, 460, 5], hq=12, hkv=2, head_dim=256, seed=9,
                           layout="NHD")
    _parity(spec, rows=rows)


@pytest.mark.parametrize("rows", [0, 192])
def test_fixed_b1_q1023(rows):
    """The single request q_len = kv_len = 1023, Hq 48 / Hkv 8, D 256, every row."""
    _parity(wl.prefill_spec(fixed_1023=True), rows=rows)


def tile_edge_rows(r, q_len):
    """Query rows whose neighbourhood a tiling bug would show in: the first
    and last row of every 128-row and every 192-row tile (both workgroup
    tilings of the head_dim 256 kernel), every 53rd row, and the last row."""
    i = np.arange(q_len)
    keep = (i % 128 == 0) | (i % 128 == 127) | (i % 192 == 0) | (i % 192 == 191) | (i % 53 == 0) | (i == q_len - 1)
    return i[keep]


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16, 32])
def test_random_batches_full_size(batch):
    """Batch 1..32, q_len U{65..4096}, kv_len = q_len + U{0..4096}, full size.
    Every request and all 48 heads are checked on the first and last row of
    every 128- and 192-row tile, every 53rd row and the last row (about 4.5%
    of the rows), each against the oracle over exactly the keys it sees."""
    spec = wl.prefill_spec(batch=batch)
    say(f"[prefill parity] random B={batch} full size, tile-edge rows of every request")
    case = PrefillCase(spec, gen_device="cuda")
    kc, vc, kv = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kv)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    rows, ro, rl = case.oracle_row_set(okc, ovc, okv, obt, oreqs, tile_edge_rows)
    s1 = compare(out.cpu()[rows], ro, *BF16_TOL, f"{spec.name} out")
    s2 = compare(lse.cpu()[rows], rl, *BF16_TOL, f"{spec.name} lse")
    say(f"  rows checked {len(rows)} of {int(spec.q_lens.sum())}; out: {s1}; lse: {s2}")


@pytest.mark.parametrize("batch,rows", [(2, 192), (8, 128)])
def test_random_batches_forced_tiling(batch, rows):
    """Full-size random batches on the tiling the library would not pick for them."""
    spec = wl.prefill_spec(batch=batch)
    rng = np.random.default_rng(batch + 100)
    reqs = sorted(rng.choice(batch, min(4, batch), replace=False).tolist())
    _parity(spec, sample=4, reqs=reqs, gen_device="cuda", rows=rows)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_tilings_give_the_same_bits(d):
    """The 128- and 192-row tilings (and the library's own unsplit choice)
    compute every row with the same operations in the same order, so their
    outputs are equal bit for bit; ragged requests, causal and full mask."""
    spec = wl.prefill_spec(q_lens=[1, 100, 300, 191], kv_lens=[500, 100, 900, 700], hq=12, hkv=4, head_dim=d,
                           seed=61 + d)
    say(f"[prefill] tilings bit-equal, D={d}")
    case = PrefillCase(spec)
    kc, vc, kv = case.gpu_pools()
    for causal in (True, False):
        ref = case.gpu_prefill(kc, vc, kv, causal=causal, split=False)
        for rows in (128, 192):
            o, l = case.gpu_prefill(kc, vc, kv, causal=causal, rows=rows)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), (causal, rows)
            assert torch.equal(l.view(torch.int32), ref[1].view(torch.int32)), (causal, rows)


@pytest.mark.parametrize("rows", [128, 192])
def test_permutation_invariance_and_determinism(rows):
    spec1 = wl.prefill_spec(q_lens=[100, 257], kv_lens=[300, 257], hq=12, hkv=2, head_dim=256, seed=21)
    spec2 = wl.prefill_spec(q_lens=[100, 257], kv_lens=[300, 257], hq=12, hkv=2, head_dim=256, seed=21)
    rng = np.random.default_rng(5)
    remap = np.concatenate([[0], rng.permutation(spec1.num_pages - 1) + 1]).astype(np.int32)
    spec2.block_table = np.where(spec1.block_table > 0, remap[spec1.block_table], 0).astype(np.int32)
    say(f"[prefill] permutation invariance, rows/wg {rows}")
    c1, c2 = PrefillCase(spec1), PrefillCase(spec2)
    o1, l1 = c1.gpu_prefill(*c1.gpu_pools(), rows=rows)
    o2, l2 = c2.gpu_prefill(*c2.gpu_pools(), rows=rows)
    k1, v1, kv1 = c1.gpu_pools()
    o3, l3 = c1.gpu_prefill(k1, v1, kv1, rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_causal_mask_closed_form():
    """Identical keys and V[j] = j: causal row i of a request (q, kv) is the
    mean of 0..kv-q+i (every weight is exactly 1 and the fp32 sums are exact).
    With kv <= 128 the means stay below 64, where one visible key more or less
    moves the mean by 0.5 = two bf16 ulps, so a 1-ulp bound pins the mask."""
    say("[prefill] causal mask closed form")
    dev = torch.device("cuda")
    q_lens, kv_lens = [1, 40, 100, 128], [1, 100, 100, 128]
    spec = wl.prefill_spec(q_lens=q_lens, kv_lens=kv_lens, hq=4, hkv=1, head_dim=128, seed=3)
    k = torch.ones((sum(kv_lens), 1, 128), dtype=torch.bfloat16, device=dev)
    v = torch.cat([torch.arange(n, dtype=torch.float32) for n in kv_lens])
    v = v[:, None, None].expand(-1, 1, 128).to(torch.bfloat16).contiguous().to(dev)
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    bt = torch.from_numpy(spec.block_table).to(dev)
    kvl = pkv.append(kc, vc, k, v, bt, torch.zeros(len(q_lens), dtype=torch.int32, device=dev),
                     torch.tensor(np.concatenate([[0], np.cumsum(kv_lens)]), dtype=torch.int32, device=dev))
    assert kvl.cpu().tolist() == kv_lens
    q = torch.ones((sum(q_lens), 4, 128), dtype=torch.bfloat16, device=dev)
    qi = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32, device=dev)
    out = pkv.prefill_attn(q, kc, vc, bt, kvl, qi, max(q_lens), max(kv_lens), causal=True, scale=0.0625)
    o = out.float().cpu()
    t = 0
    for ql, kvv in zip(q_lens, kv_lens):
        for i in range(ql):
            want = (kvv - ql + i) / 2.0  # mean of 0 .. kv-q+i
            ulp = 2.0 ** (np.floor(np.log2(want)) - 7) if want > 0 else 0.0
            assert torch.all((o[t] - want).abs() <= ulp), (ql, kvv, i, want, o[t, 0, 0].item())
            t += 1


def test_no_visible_key_rows():
    """Without the causal flag a request with kv_len 0 gives 0 and lse -inf,
    next to a request that has keys."""
    say("[prefill] empty key rows")
    dev = torch.device("cuda")
    spec = wl.custom_decode_spec([20], hq=4, hkv=2, head_dim=128, dtype="bf16", seed=4, n_new=0)
    bt1 = torch.from_numpy(spec.block_table).to(dev)
    bt = torch.cat([torch.zeros_like(bt1), bt1])
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    k = torch.randn((20, 2, 128), device=dev).to(torch.bfloat16)
    kvl = torch.tensor([0, 20], dtype=torch.int32, device=dev)
    pkv.append(kc, vc, k, k, bt1, torch.zeros(1, dtype=torch.int32, device=dev),
               torch.tensor([0, 20], dtype=torch.int32, device=dev))
    q = torch.randn((8, 4, 128), device=dev).to(torch.bfloat16)
    qi = torch.tensor([0, 3, 8], dtype=torch.int32, device=dev)
    out, lse = pkv.prefill_attn(q, kc, vc, bt, kvl, qi, 5, 20, 128 ** -0.5, causal=False, return_lse=True)
    o, l = out.float().cpu(), lse.cpu()
    assert torch.all(o[:3] == 0) and torch.all(torch.isneginf(l[:3]))
    assert torch.isfinite(o[3:]).all() and torch.isfinite(l[3:]).all()


@pytest.mark.parametrize("rows", [128, 192])
def test_long_kv_restages_table_window(rows):
    """One request of 70000 keys at D = 256: more than the 4096 page-table
    entries (65536 keys) the 16-row kernel stages in LDS at a time, so it
    restages the window during the walk.  The first and last 4 rows (the last
    see every key) are checked."""
    spec = wl.prefill_spec(q_lens=[40], kv_lens=[70000], hq=8, hkv=8, head_dim=256, seed=11)
    _parity(spec, sample=4, gen_device="cuda", rows=rows)


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 1e-3, 0.5])
@pytest.mark.parametrize("d", [128, 256])
def test_prefill_any_scale(d, scale):
    """The scale is applied inside exp2 by an fma that needs it positive:
    a negative scale runs as the negated query times |scale|, a zero scale as
    the smallest normal float.  Every row against the oracle, which takes the
    scale as given."""
    base = wl.prefill_spec(q_lens=[200, 65, 1], kv_lens=[450, 300, 90], hq=32 if d == 128 else 48, hkv=8,
                           head_dim=d, seed=17)
    spec = with_scale(base, scale)
    say(f"[prefill scale] D={d} scale={scale}")
    case = PrefillCase(spec)
    kc, vc, kv = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kv)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs)
    say("  out:", compare(out.cpu()[rows], ro, *BF16_TOL, "out"))
    compare(lse.cpu()[rows], rl, *BF16_TOL, "lse")
