"""GPU parity of pkv_append_decode_attn (append + decode in one launch).

The pools it leaves must equal the oracle's append bit for bit, its lengths
must equal L + 1, and its outputs must meet the attention bar against the
oracle.  Its outputs must also equal, bit for bit, those of pkv_append
followed by pkv_decode_attn with the same worker count: the two paths read
the same keys in the same order."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import DecodeCase, compare, host_bits, say, tol

pytestmark = pytest.mark.gpu


def _fused(spec, workers=0, gen_device="cpu", check_pool=True, check_separate=True):
    say(f"[fused parity] {spec.name} B={spec.batch} Hq={spec.hq} Hkv={spec.hkv} D={spec.head_dim} "
        f"{spec.layout} seed={spec.seed} workers={workers}")
    assert spec.n_new == 1
    case = DecodeCase(spec, gen_device=gen_device)
    s, i = spec, case.inp
    dev = case.dev
    kc, vc = wl.empty_pool(s, dev), wl.empty_pool(s, dev)
    zeros = torch.zeros(s.batch, dtype=torch.int32, device=dev)
    pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, zeros, i.hist_indptr, layout=s.layout)
    max_kv = int(s.hist_lens.max()) + 1
    out, lse, lens = pkv.append_decode_attn(i.q, kc, vc, i.k_new, i.v_new, i.block_table, i.hist_lens, max_kv,
                                            scale=s.scale, layout=s.layout, workers=workers, return_lse=True)
    torch.cuda.synchronize()
    okc, ovc, olens, obt = case.oracle_pools()
    assert np.array_equal(lens.cpu().numpy(), olens), "seqlens_out differs"
    if check_pool:
        assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
        assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool not bit-exact"
    ref_out, ref_lse = case.oracle_decode(okc, ovc, olens, obt)
    atol, rtol = tol(s)
    s1 = compare(out.cpu(), ref_out, atol, rtol, f"{s.name} fused out")
    s2 = compare(lse.cpu(), ref_lse, atol, rtol, f"{s.name} fused lse")
    say(f"  out: {s1}; lse: {s2}")
    if check_separate:
        kc2, vc2, lens2 = case.gpu_pools()
        out2, lse2 = case.gpu_decode(kc2, vc2, lens2, workers=workers)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "fused and separate outputs differ"
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), "fused and separate lse differ"
    return out, lse


def test_fused_qwen3_decode_b64():
    _fused(wl.decode_spec("qwen3_decode"))


@pytest.mark.parametrize("batch", [8, 32, 128, 256])
def test_fused_qwen3_sweep(batch):
    _fused(wl.decode_spec("qwen3_sweep", batch=batch), check_pool=batch <= 64)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fused_head_dims_and_page_edges(d):
    # L = 0 (the new token is the only key), slots 15/16 (page boundaries), and
    # rows long enough to be split
    spec = wl.custom_decode_spec([0, 1, 15, 16, 17, 31, 32, 100, 257, 700], hq=8, hkv=2, head_dim=d,
                                 dtype="bf16", seed=90 + d)
    _fused(spec)


@pytest.mark.parametrize("workers", [1, 3, 7, 64, 1000])
def test_fused_split_counts(workers):
    spec = wl.custom_decode_spec([3, 16, 47, 130, 400, 911], hq=16, hkv=4, head_dim=128, dtype="bf16", seed=7)
    _fused(spec, workers=workers)


def test_fused_nhd():
    _fused(wl.decode_spec("qwen3_decode", batch=16, layout="NHD"))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (48, 8), (32, 2)])
def test_fused_gqa_ratios(hq, hkv):
    spec = wl.custom_decode_spec([5, 40, 77, 200, 1000], hq=hq, hkv=hkv, head_dim=128, dtype="bf16",
                                 seed=hq + hkv)
    _fused(spec)


def test_fused_rows_not_stored_keep_their_length():
    """A row whose L + 1 exceeds max_kv_len, and a row whose slot page is page
    0 (not a real page), attend what they can but store nothing: the pools
    stay as they were and seqlens_out reports L for them, L + 1 elsewhere."""
    say("[fused] rows whose token is not stored")
    spec = wl.custom_decode_spec([40, 63, 32, 33], hq=8, hkv=2, head_dim=128, dtype="bf16", seed=31, extra_cols=1)
    case = DecodeCase(spec)
    i, dev = case.inp, case.dev
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, torch.zeros(spec.batch, dtype=torch.int32, device=dev),
               i.hist_indptr)
    bt = i.block_table.clone()
    bt[2, 32 // 16] = 0  # row 2's new token (position 32, alone in its block) routes to page 0
    max_kv = 60          # row 1 (L = 63) is cut: 63 + 1 > 60
    k0, v0 = kc.clone(), vc.clone()
    out, lse, lens = pkv.append_decode_attn(i.q, kc, vc, i.k_new, i.v_new, bt, i.hist_lens, max_kv, spec.scale,
                                            return_lse=True)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [41, 63, 32, 34]
    hist = spec.hist_lens
    changed = (kc.view(torch.int16) != k0.view(torch.int16)).any(-1).nonzero().cpu().numpy()
    # (page, head, slot) of every changed row: only rows 0 and 3 were stored, one slot per kv head each
    want = set()
    for b in (0, 3):
        pos = int(hist[b])
        for g in range(spec.hkv):
            want.add((int(spec.block_table[b, pos // 16]), g, pos % 16))
    assert set(map(tuple, changed.tolist())) == want
    assert torch.equal((vc.view(torch.int16) != v0.view(torch.int16)).any(-1).nonzero(),
                       (kc.view(torch.int16) != k0.view(torch.int16)).any(-1).nonzero())
    assert not torch.isnan(out).any()
