"""GPU parity of pkv_append / pkv_route / pkv_decode_attn against the oracle.

Bars: append and routing bit-exact; attention within |d| <= 2e-2 + 2e-2|ref|
(bf16) or 1e-5 + 1e-5|ref| (fp32) of the fp64 oracle, element by element.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import DecodeCase, compare, host_bits, opool, say, tol

pytestmark = pytest.mark.gpu


def _run_parity(spec, workers=0, gen_device="cpu", oracle_rows=None, check_pool=True, seed_offset=0):
    say(f"[decode parity] {spec.name} B={spec.batch} Hq={spec.hq} Hkv={spec.hkv} D={spec.head_dim} "
        f"{spec.dtype} {spec.layout} seed={spec.seed} layer draw {seed_offset} workers={workers}")
    case = DecodeCase(spec, gen_device=gen_device, oracle_rows=oracle_rows, seed_offset=seed_offset)
    kc, vc, lens = case.gpu_pools()
    out, lse = case.gpu_decode(kc, vc, lens, workers=workers)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    rows = case.rows
    glens = lens.cpu().numpy()
    assert np.array_equal(glens if rows is None else glens[rows], olens), "seqlens_out differs"
    if check_pool:
        assert rows is None
        assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
        assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool not bit-exact"
    ref_out, ref_lse = case.oracle_decode(okc, ovc, olens, obt)
    atol, rtol = tol(spec)
    o = out.cpu()
    l = lse.cpu()
    if rows is not None:
        o, l = o[rows], l[rows]
    s1 = compare(o, ref_out, atol, rtol, f"{spec.name} out")
    s2 = compare(l, ref_lse, atol, rtol, f"{spec.name} lse")
    say(f"  out: {s1}; lse: {s2}")
    return case, kc, vc, lens, out, lse


def test_tiny_f32():
    _run_parity(wl.decode_spec("tiny_f32"))


def test_tiny_f32_nhd():
    _run_parity(wl.decode_spec("tiny_f32", layout="NHD"))


def test_qwen3_decode_b64():
    _run_parity(wl.decode_spec("qwen3_decode"))


@pytest.mark.parametrize("batch", [8, 16, 32, 64, 128, 256])
def test_qwen3_sweep(batch):
    _run_parity(wl.decode_spec("qwen3_sweep", batch=batch), check_pool=batch <= 64)


def test_qwen3_decode_nhd():
    _run_parity(wl.decode_spec("qwen3_decode", batch=16, layout="NHD"))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims(d, dtype):
    spec = wl.custom_decode_spec([0, 1, 15, 16, 17, 31, 33, 100, 257], hq=8, hkv=2, head_dim=d, dtype=dtype,
                                 seed=40 + d)
    _run_parity(spec)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (32, 2)])
def test_gqa_ratios(hq, hkv):
    spec = wl.custom_decode_spec([5, 40, 77, 200], hq=hq, hkv=hkv, head_dim=128, dtype="bf16", seed=hq * 7 + hkv)
    _run_parity(spec)


def test_empty_and_single_token_rows():
    # hist -1 is impossible; rows with 0 attended keys come from n_new = 0 workloads
    spec = wl.custom_decode_spec([0, 0, 3, 0, 16], hq=8, hkv=2, head_dim=128, dtype="bf16", seed=5, n_new=0)
    say("[decode] zero-length rows")
    case = DecodeCase(spec)
    kc, vc, lens = case.gpu_pools()
    out, lse = case.gpu_decode(kc, vc, lens)
    torch.cuda.synchronize()
    o, l = out.float().cpu(), lse.cpu()
    for b in (0, 1, 3):
        assert torch.all(o[b] == 0) and torch.all(torch.isneginf(l[b])), b
    assert not torch.isnan(o).any()
    okc, ovc, olens, obt = case.oracle_pools()
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    compare(o, ro, *tol(spec), "zero rows out")
    compare(l, rl, *tol(spec), "zero rows lse")


@pytest.mark.parametrize("workers", [1, 2, 3, 7, 64, 1000])
def test_split_invariance(workers):
    """Any split of the work gives the oracle's answer, and forced worker
    counts agree with the automatic split to fp32 rounding (fp32 inputs)."""
    spec = wl.custom_decode_spec([3, 16, 47, 130, 500, 1023], hq=8, hkv=2, head_dim=64, dtype="f32", seed=77)
    case, kc, vc, lens, out, lse = _run_parity(spec, workers=workers)
    auto_out, auto_lse = case.gpu_decode(kc, vc, lens, workers=0)
    compare(out.cpu(), auto_out.cpu().double().numpy(), 1e-6, 1e-6, "split vs auto")
    compare(lse.cpu(), auto_lse.cpu().double().numpy(), 1e-6, 1e-6, "split vs auto lse")


def test_bf16_split_invariance_long():
    spec = wl.custom_decode_spec([2000, 17, 4096, 1, 900], hq=32, hkv=8, head_dim=128, dtype="bf16", seed=78)
    for w in (1, 5, 13, 0):
        _run_parity(spec, workers=w)


def test_permutation_invariance_and_determinism():
    """Other physical pages, same logical content: every output bit equal;
    two runs are bitwise identical."""
    s1 = wl.decode_spec("qwen3_decode", batch=24)
    s2 = wl.decode_spec("qwen3_decode", batch=24)
    rng = np.random.default_rng(999)
    perm = rng.permutation(s1.num_pages - 1).astype(np.int32) + 1
    remap = np.concatenate([[0], perm]).astype(np.int32)
    s2.block_table = np.where(s1.block_table > 0, remap[s1.block_table], 0).astype(np.int32)
    assert not np.array_equal(s1.block_table, s2.block_table)
    say("[decode] permutation invariance")
    c1, c2 = DecodeCase(s1), DecodeCase(s2)
    k1, v1, l1 = c1.gpu_pools()
    k2, v2, l2 = c2.gpu_pools()
    o1, e1 = c1.gpu_decode(k1, v1, l1)
    o2, e2 = c2.gpu_decode(k2, v2, l2)
    o3, e3 = c1.gpu_decode(k1, v1, l1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(e1.view(torch.int32), e2.view(torch.int32))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(e1.view(torch.int32), e3.view(torch.int32))


@pytest.mark.parametrize("workers", [0, 1, 3, 50])
def test_dominant_key_bit_exact(workers):
    """K = -1 except +1 at j*, q = 16: the output is V[j*] bit for bit."""
    say(f"[decode] dominant key workers={workers}")
    dev = torch.device("cuda")
    n, hq, hkv, d = 90, 8, 2, 128
    spec = wl.custom_decode_spec([n], hq=hq, hkv=hkv, head_dim=d, dtype="bf16", seed=3, n_new=0)
    bt = torch.from_numpy(spec.block_table).to(dev)
    v = torch.randn((n, hkv, d), device=dev).to(torch.bfloat16)
    q = torch.full((1, hq, d), 16.0, device=dev, dtype=torch.bfloat16)
    for jstar in (0, 15, 16, 31, 32, 63, 64, 89):
        k = -torch.ones((n, hkv, d), device=dev, dtype=torch.bfloat16)
        k[jstar] = 1
        kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
        zeros = torch.zeros(1, dtype=torch.int32, device=dev)
        lens = pkv.append(kc, vc, k, v, bt, zeros, torch.tensor([0, n], dtype=torch.int32, device=dev))
        out = pkv.decode_attn(q, kc, vc, bt, lens, n, scale=d ** -0.5, workers=workers)
        torch.cuda.synchronize()
        for h in range(hq):
            assert torch.equal(out[0, h].view(torch.int16), v[jstar, h // (hq // hkv)].view(torch.int16)), (jstar, h)


def test_identical_keys_mean():
    say("[decode] identical keys")
    dev = torch.device("cuda")
    n, hq, hkv, d = 300, 4, 1, 128
    spec = wl.custom_decode_spec([n], hq=hq, hkv=hkv, head_dim=d, dtype="bf16", seed=4, n_new=0)
    bt = torch.from_numpy(spec.block_table).to(dev)
    k = torch.randn((1, hkv, d), device=dev).to(torch.bfloat16).expand(n, hkv, d).contiguous()
    v = torch.randn((n, hkv, d), device=dev).to(torch.bfloat16)
    q = torch.randn((1, hq, d), device=dev).to(torch.bfloat16)
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    lens = pkv.append(kc, vc, k, v, bt, torch.zeros(1, dtype=torch.int32, device=dev),
                      torch.tensor([0, n], dtype=torch.int32, device=dev))
    out = pkv.decode_attn(q, kc, vc, bt, lens, n, d ** -0.5)
    mean = v[:, 0].double().mean(0).cpu().numpy()
    compare(out[0].cpu(), np.broadcast_to(mean, (hq, d)), 2e-2, 2e-2, "identical keys")


def test_route_bit_exact():
    for layout in ("HND", "NHD"):
        spec = wl.decode_spec("qwen3_sweep", batch=32, layout=layout)
        say(f"[route] {spec.name} {layout}")
        dev = torch.device("cuda")
        lens = torch.from_numpy(spec.hist_lens + 1).to(dev)
        bt = torch.from_numpy(spec.block_table).to(dev)
        kc = wl.empty_pool(spec, dev)
        max_len = int(lens.max())
        off = pkv.route(kc, bt, lens, max_len, layout=layout)
        ref = oracle.load().route(opool(spec), spec.block_table, spec.hist_lens + 1, max_len)
        assert np.array_equal(off.cpu().numpy(), ref)


def test_append_ragged_bit_exact():
    """Ragged multi-token append (prefill-style) into a NaN pool."""
    say("[append] ragged")
    dev = torch.device("cuda")
    hist, new = [0, 5, 16, 31, 100], [1, 40, 16, 1, 0]
    total = [a + b for a, b in zip(hist, new)]
    spec = wl.custom_decode_spec(total, hq=8, hkv=8, head_dim=256, dtype="bf16", seed=9, n_new=0)
    gen = torch.Generator().manual_seed(9)
    kn = torch.randn((sum(new), 8, 256), generator=gen).to(torch.bfloat16)
    vn = torch.randn((sum(new), 8, 256), generator=gen).to(torch.bfloat16)
    indptr = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    lens = pkv.append(kc, vc, kn.to(dev), vn.to(dev), torch.from_numpy(spec.block_table).to(dev),
                      torch.tensor(hist, dtype=torch.int32, device=dev), torch.from_numpy(indptr).to(dev))
    okc = host_bits(wl.empty_pool(spec, "cpu")).copy()
    ovc = okc.copy()
    olens = oracle.load().append(opool(spec), okc, ovc, host_bits(kn), host_bits(vn), spec.block_table,
                                 np.asarray(hist, np.int32), indptr)
    assert np.array_equal(lens.cpu().numpy(), olens)
    assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8))
    assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8))


def test_long_ragged_full_size_whole_layer():
    """Batch 256, log-uniform lengths up to 32k, fully fragmented pool, at
    full size: every row of one layer cache against the oracle."""
    _run_parity(wl.decode_spec("long_ragged"), gen_device="cuda", check_pool=False)


@pytest.mark.parametrize("layer", [1, 2])
def test_long_ragged_other_layers_sampled(layer):
    """Two more layer caches of the same workload (their own K/V/q draws),
    checked on 24 seeded rows each plus the longest and the shortest."""
    spec = wl.decode_spec("long_ragged")
    n = spec.hist_lens
    rng = np.random.default_rng(4000 + layer)
    rows = set(rng.choice(spec.batch, 24, replace=False).tolist()) | {int(n.argmax()), int(n.argmin())}
    _run_parity(spec, gen_device="cuda", oracle_rows=rows, check_pool=False, seed_offset=layer)


def test_workspace_reuse_across_calls():
    """One zeroed workspace serves consecutive calls with other lengths: the
    split-row arrival counters are left at zero by every call."""
    say("[decode] workspace reuse")
    s1 = wl.custom_decode_spec([3000, 5, 700, 1500], hq=32, hkv=8, head_dim=128, dtype="bf16", seed=61)
    s2 = wl.custom_decode_spec([100, 2900, 0, 1200], hq=32, hkv=8, head_dim=128, dtype="bf16", seed=62,
                               extra_cols=2)
    c1, c2 = DecodeCase(s1), DecodeCase(s2)
    k1, v1, l1 = c1.gpu_pools()
    k2, v2, l2 = c2.gpu_pools()
    m1, m2 = 3001, 2901
    need = max(pkv.decode_workspace_bytes(k1, 4, 32, m1, workers=37),
               pkv.decode_workspace_bytes(k2, 4, 32, m2, workers=37))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = pkv.decode_attn(c1.inp.q, k1, v1, c1.inp.block_table, l1, m1, s1.scale, workspace=ws, workers=37)
    second = pkv.decode_attn(c2.inp.q, k2, v2, c2.inp.block_table, l2, m2, s2.scale, workspace=ws, workers=37)
    again = pkv.decode_attn(c1.inp.q, k1, v1, c1.inp.block_table, l1, m1, s1.scale, workspace=ws, workers=37)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    for case, out in ((c1, first), (c2, second)):
        okc, ovc, olens, obt = case.oracle_pools()
        ro, _ = case.oracle_decode(okc, ovc, olens, obt)
        compare(out.cpu(), ro, *tol(case.spec), "workspace reuse")


def test_workspace_reuse_automatic_workers_shrinking_lengths():
    """One workspace, sized once, with the library's own worker count, serves
    a batch whose lengths fall from ~2000 to ~100 (and rise again): the size
    and layout do not depend on the lengths."""
    say("[decode] workspace reuse, automatic workers, shrinking lengths")
    specs = [wl.custom_decode_spec(L, hq=32, hkv=8, head_dim=128, dtype="bf16", seed=70 + k)
             for k, L in enumerate(([1990, 2000, 1500, 1800, 1999, 1700, 1600, 1900],
                                    [90, 100, 60, 99, 80, 70, 100, 95],
                                    [5, 1, 0, 16, 17, 3, 2, 8],
                                    [1000, 2000, 30, 700, 1999, 5, 400, 1200]))]
    dev = torch.device("cuda")
    kc0 = wl.empty_pool(specs[0], dev)
    ws = torch.zeros(pkv.decode_workspace_bytes(kc0, 8, 32, 2001), dtype=torch.uint8, device=dev)
    assert ws.numel() == pkv.decode_workspace_bytes(kc0, 8, 32, 1)
    for spec in specs:
        case = DecodeCase(spec)
        kc, vc, lens = case.gpu_pools()
        max_kv = int(spec.hist_lens.max()) + 1
        out, lse = pkv.decode_attn(case.inp.q, kc, vc, case.inp.block_table, lens, max_kv, spec.scale,
                                   workspace=ws, return_lse=True)
        torch.cuda.synchronize()
        okc, ovc, olens, obt = case.oracle_pools()
        ro, rl = case.oracle_decode(okc, ovc, olens, obt)
        say(f"  max_kv {max_kv}: out " + compare(out.cpu(), ro, *tol(spec), "reuse out"))
        compare(lse.cpu(), rl, *tol(spec), "reuse lse")
    counters = ws[: 8 * 8 * 4].view(torch.int32)
    assert torch.all(counters == 0), "a call left arrival counters behind"


def test_workspace_reset_clears_counters():
    """pkv_decode_workspace_reset zeroes the arrival counters (here filled
    with junk from the host, as an aborted launch could leave them), after
    which the workspace gives the oracle's result."""
    say("[decode] workspace reset")
    spec = wl.custom_decode_spec([3000, 5, 700, 1500], hq=32, hkv=8, head_dim=128, dtype="bf16", seed=64)
    case = DecodeCase(spec)
    kc, vc, lens = case.gpu_pools()
    ws = torch.zeros(pkv.decode_workspace_bytes(kc, 4, 32, 3001), dtype=torch.uint8, device=case.dev)
    ws[:1024].fill_(0x5A)
    pkv.decode_workspace_reset(kc, 4, ws)
    torch.cuda.synchronize()
    assert torch.all(ws[: 4 * 8 * 4] == 0)
    out = pkv.decode_attn(case.inp.q, kc, vc, case.inp.block_table, lens, 3001, spec.scale, workspace=ws)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    ro, _ = case.oracle_decode(okc, ovc, olens, obt)
    compare(out.cpu(), ro, *tol(spec), "after reset")
