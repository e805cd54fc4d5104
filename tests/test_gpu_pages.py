"""GPU parity with pages of more than 16 tokens (32 .. 256; the flash_attn
block tensor of mini-infer 06 uses 256-token blocks, §8): every kernel walks
keys in 16-token sub-pages and finds sub-page j of a row in table column
j / (page_size / 16).  Same bars as at page size 16: pools and routes bit for
bit, attention within the bf16 / fp32 tolerance of the oracle (which walks
the table with the page size itself)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import DecodeCase, PrefillCase, host_bits, opool, say
from test_gpu_decode import _run_parity
from test_gpu_fused import _fused
from test_gpu_mixed import _check as _mixed_check
from test_gpu_prefill import _parity
from test_gpu_rope import _run as _rope_run

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 15, 16, 17, 31, 63, 64, 127, 128, 255, 256, 257, 1000]


@pytest.mark.parametrize("page", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_page_sizes(page, dtype):
    spec = wl.custom_decode_spec(EDGES, hq=8, hkv=2, head_dim=128, dtype=dtype, seed=page + 1, page_size=page)
    _run_parity(spec)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_qwen3_decode_page256(layout):
    _run_parity(wl.decode_spec("qwen3_decode", batch=64 if layout == "HND" else 16, layout=layout, page_size=256))


@pytest.mark.parametrize("workers", [1, 7, 300])
def test_split_counts_page64(workers):
    spec = wl.custom_decode_spec([3, 16, 47, 130, 500, 1023], hq=8, hkv=2, head_dim=64, dtype="bf16", seed=77,
                                 page_size=64)
    _run_parity(spec, workers=workers)


@pytest.mark.parametrize("page", [32, 256])
def test_fused_page_sizes(page):
    spec = wl.custom_decode_spec([0, 1, 15, 16, 17, 255, 256, 257, 700], hq=16, hkv=4, head_dim=128, dtype="bf16",
                                 seed=page + 5, page_size=page)
    _fused(spec)


@pytest.mark.parametrize("rows", [128, 192])
def test_prefill_d256_page256(rows):
    spec = wl.prefill_spec(q_lens=[1, 17, 191, 300, 129], kv_lens=[1, 300, 611, 900, 129], hq=12, hkv=2,
                           head_dim=256, seed=rows + 9, page_size=256)
    _parity(spec, rows=rows)


@pytest.mark.parametrize("d,page", [(128, 64), (64, 256)])
def test_prefill_page_sizes(d, page):
    spec = wl.prefill_spec(q_lens=[1, 33, 128, 250], kv_lens=[5, 90, 400, 250], hq=16, hkv=4, head_dim=d,
                           seed=d + page, page_size=page)
    _parity(spec)


def test_prefill_fixed_b1_q1023_page256():
    spec = wl.prefill_spec(q_lens=[1023], kv_lens=[1023], hq=48, hkv=8, head_dim=256, seed=599, page_size=256)
    _parity(spec, sample=64)


@pytest.mark.parametrize("page", [64, 256])
def test_mixed_page_sizes(page):
    spec = wl.prefill_spec(q_lens=[65, 300, 1, 1, 1, 1, 1], kv_lens=[600, 300, 1, 17, 257, 1500, 256], hq=32, hkv=8,
                           head_dim=128, seed=13 + page, page_size=page)
    _mixed_check(spec, 2)


@pytest.mark.parametrize("page,layout", [(32, "HND"), (256, "HND"), (128, "NHD")])
def test_rope_append_page_sizes(page, layout):
    _rope_run([0, 5, 16, -1, 31, 250, 3], [1, 40, 16, 7, 1, 300, 0], hq=8, hkv=2, d=128, dtype="bf16",
              interleaved=page == 32, seed=page, layout=layout, page_size=page)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_route_page256(layout):
    spec = wl.decode_spec("qwen3_sweep", batch=16, layout=layout, page_size=256)
    say(f"[pages] route, page 256, {layout}")
    dev = torch.device("cuda")
    lens = torch.from_numpy(spec.hist_lens + 1).to(dev)
    kc = wl.empty_pool(spec, dev)
    off = pkv.route(kc, torch.from_numpy(spec.block_table).to(dev), lens, int(lens.max()), layout=layout)
    ref = oracle.load().route(opool(spec), spec.block_table, spec.hist_lens + 1, int(lens.max()))
    assert np.array_equal(off.cpu().numpy(), ref)


def _expanded(spec):
    """The same workload on 16-token pages: page p of the spec becomes pages
    p*k .. p*k + k-1 (k = page_size / 16), every table entry expanded in place."""
    k = spec.page_size // 16
    bt = spec.block_table.astype(np.int64)
    ex = (bt[:, :, None] * k + np.arange(k)[None, None, :]).reshape(bt.shape[0], -1)
    ex = np.where(np.repeat(bt, k, axis=1) > 0, ex, 0).astype(np.int32)
    return dataclasses.replace(spec, page_size=16, num_pages=spec.num_pages * k, bt_cols=spec.bt_cols * k,
                               block_table=ex)


@pytest.mark.parametrize("page,layout,workers", [(256, "HND", 0), (64, "NHD", 0), (128, "HND", 37)])
def test_decode_bitwise_equals_expanded_16_token_pages(page, layout, workers):
    """Pages of k*16 tokens give the same bits as 16-token pages holding the
    same tokens: the kernels split work and order sums on 16-token runs."""
    spec = wl.custom_decode_spec(EDGES + [700, 2000], hq=32, hkv=8, head_dim=128, dtype="bf16", seed=page,
                                 layout=layout, page_size=page)
    say(f"[pages] decode page {page} {layout} vs 16-token pages, workers {workers or 'auto'}")
    outs = []
    for s in (spec, _expanded(spec)):
        case = DecodeCase(s)
        kc, vc, lens = case.gpu_pools()
        out, lse = case.gpu_decode(kc, vc, lens, workers=workers)
        torch.cuda.synchronize()
        outs.append((host_bits(out), host_bits(lse), lens.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("d,rows", [(256, 128), (256, 192), (128, 0)])
def test_prefill_bitwise_equals_expanded_16_token_pages(d, rows):
    spec = wl.prefill_spec(q_lens=[1, 100, 300, 513], kv_lens=[40, 100, 700, 1200], hq=16, hkv=4, head_dim=d,
                           seed=d + rows, page_size=256)
    say(f"[pages] prefill D={d} rows {rows or 'auto'} page 256 vs 16-token pages")
    outs = []
    for s in (spec, _expanded(spec)):
        case = PrefillCase(s)
        kc, vc, kv = case.gpu_pools()
        out, lse = case.gpu_prefill(kc, vc, kv, rows=rows)
        torch.cuda.synchronize()
        outs.append((host_bits(out), host_bits(lse)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
