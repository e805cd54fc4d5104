"""GPU parity of pkv_append_rope (append with the rotary position embedding
of the new tokens' q and k fused in) against the oracle's rotation followed
by its append.

Bars: pools, rotated q and lengths bit for bit (both sides evaluate the
rotation exactly in fp64 and round once to nearest even); attention after the
rotated append within the bf16 bar.  Both pair layouts, bf16 and fp32 pools,
head_dim 64/128/256, ragged multi-token appends with padding rows."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, compare, host_bits, opool, say

pytestmark = pytest.mark.gpu


def _case(hist, new, hq, hkv, d, dtype, seed, layout="HND", page_size=16):
    total = [max(a, 0) + b for a, b in zip(hist, new)]
    spec = wl.custom_decode_spec(total, hq=hq, hkv=hkv, head_dim=d, dtype=dtype, seed=seed, n_new=0, layout=layout,
                                 page_size=page_size)
    gen = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    nh = sum(max(a, 0) for a in hist)
    kh = torch.randn((nh, hkv, d), generator=gen).to(tdt)
    vh = torch.randn((nh, hkv, d), generator=gen).to(tdt)
    kn = torch.randn((sum(new), hkv, d), generator=gen).to(tdt)
    vn = torch.randn((sum(new), hkv, d), generator=gen).to(tdt)
    q = torch.randn((sum(new), hq, d), generator=gen).to(tdt)
    return spec, kh, vh, kn, vn, q


def _run(hist, new, hq, hkv, d, dtype, interleaved, seed, layout="HND", page_size=16):
    say(f"[rope append] hist={hist} new={new} Hq={hq} Hkv={hkv} D={d} {dtype} {layout} "
        f"{'interleaved' if interleaved else 'half-split'} page {page_size}")
    dev = torch.device("cuda")
    spec, kh, vh, kn, vn, q = _case(hist, new, hq, hkv, d, dtype, seed, layout, page_size)
    bt = spec.block_table
    hist_np = np.asarray(hist, np.int32)
    hist_ip = np.concatenate([[0], np.cumsum([max(a, 0) for a in hist])]).astype(np.int32)
    new_ip = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    rows = int(max(hist_np.max(), 0) + max(new)) + 3
    cos, sin = wl.rope_tables(rows, d)
    # device: history, then the rotated append
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    pkv.append(kc, vc, kh.to(dev), vh.to(dev), torch.from_numpy(bt).to(dev),
               torch.zeros(len(hist), dtype=torch.int32, device=dev), torch.from_numpy(hist_ip).to(dev), layout=layout)
    qd = q.to(dev)
    lens = pkv.append_rope(kc, vc, kn.to(dev), vn.to(dev), torch.from_numpy(bt).to(dev),
                           torch.from_numpy(hist_np).to(dev), cos.to(dev), sin.to(dev), interleaved=interleaved,
                           q=qd, new_indptr=torch.from_numpy(new_ip).to(dev), layout=layout)
    torch.cuda.synchronize()
    # oracle: rotate q and k of the live rows at positions L_b + t, then append
    orc = oracle.load()
    pool = opool(spec)
    odt = oracle.BF16 if dtype == "bf16" else oracle.F32
    okc = host_bits(wl.empty_pool(spec, "cpu")).copy()
    ovc = okc.copy()
    hist_live = np.maximum(hist_np, 0)
    orc.append(pool, okc, ovc, host_bits(kh), host_bits(vh), bt, np.zeros(len(hist), np.int32), hist_ip)
    live_rows = [r for b in range(len(hist)) if hist[b] >= 0 for r in range(new_ip[b], new_ip[b + 1])]
    pos = np.array([hist[b] + t for b in range(len(hist)) if hist[b] >= 0 for t in range(new[b])], np.int32)
    k_rot = host_bits(kn).copy()
    q_rot = host_bits(q).copy()
    if live_rows:
        sel = np.asarray(live_rows)
        kr = np.ascontiguousarray(k_rot[sel])
        qr = np.ascontiguousarray(q_rot[sel])
        orc.rope(odt, kr, pos, cos, sin, interleaved)
        orc.rope(odt, qr, pos, cos, sin, interleaved)
        k_rot[sel] = kr
        q_rot[sel] = qr
    live_b = [b for b in range(len(hist)) if hist[b] >= 0]
    kl = np.concatenate([k_rot[new_ip[b]:new_ip[b + 1]] for b in live_b]) if live_b else k_rot[:0]
    vl = np.concatenate([host_bits(vn)[new_ip[b]:new_ip[b + 1]] for b in live_b]) if live_b else k_rot[:0]
    ip_l = np.concatenate([[0], np.cumsum([new[b] for b in live_b])]).astype(np.int32)
    olens = orc.append(pool, okc, ovc, kl, vl, bt[live_b], hist_np[live_b], ip_l)
    glens = lens.cpu().numpy()
    assert glens[live_b].tolist() == olens.tolist()
    assert all(glens[b] == hist[b] for b in range(len(hist)) if hist[b] < 0), "padding row length changed"
    assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool not bit-exact"
    assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool not bit-exact"
    assert np.array_equal(host_bits(qd).view(np.uint8), q_rot.view(np.uint8)), "rotated q not bit-exact"
    return spec, kc, vc, qd, okc, ovc, q_rot, lens, olens, live_b


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_rope_append_bit_exact(d, dtype, interleaved):
    _run([0, 5, 16, -1, 31, 100, 3], [1, 40, 16, 7, 1, 3, 0], hq=8, hkv=2, d=d, dtype=dtype,
         interleaved=interleaved, seed=d + (7 if interleaved else 0) + (1 if dtype == "f32" else 0))


def test_rope_append_nhd():
    _run([4, 20, 0], [3, 1, 17], hq=16, hkv=4, d=128, dtype="bf16", interleaved=False, seed=5, layout="NHD")


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_then_decode_qwen3(interleaved):
    """The decode step of a Qwen3-shaped batch with its token rotated in the
    append: pkv_append_rope then pkv_decode_attn against the oracle."""
    rng = np.random.default_rng(77)
    hist = rng.integers(100, 900, size=16).tolist()
    spec, kc, vc, qd, okc, ovc, q_rot, lens, olens, live_b = _run(
        hist, [1] * 16, hq=32, hkv=8, d=128, dtype="bf16", interleaved=interleaved, seed=77)
    max_kv = int(np.max(olens))
    out, lse = pkv.decode_attn(qd, kc, vc, torch.from_numpy(spec.block_table).cuda(), lens, max_kv,
                               128 ** -0.5, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.load().decode(opool(spec), q_rot, okc, ovc, spec.block_table, olens, 128 ** -0.5)
    say("  out " + compare(out.cpu(), ro, *BF16_TOL, "rope decode out") + "; lse "
        + compare(lse.cpu(), rl, *BF16_TOL, "rope decode lse"))
