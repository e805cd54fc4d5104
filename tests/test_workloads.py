"""CPU checks of the seeded workload generators (inputs only, no routing or
attention arithmetic): each workload has the shapes and length ranges it is
described with, page 0 is never dealt, no physical page is dealt twice, pool
sizes follow their rules, and a seed reproduces every input bit."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from paged_kv_attention_pkv_amd import workloads as wl


def _pages(lengths) -> list[int]:
    return [-(-int(n) // wl.PAGE_SIZE) for n in lengths]


def _check_table(spec, pages_per_row):
    """Rows hold distinct pages 1..num_pages-1 in their first columns and 0 after."""
    bt = spec.block_table
    assert bt.shape == (spec.batch, spec.bt_cols) and bt.dtype == np.int32
    dealt = np.concatenate([bt[b, :n] for b, n in enumerate(pages_per_row)])
    assert (dealt >= 1).all() and (dealt < spec.num_pages).all(), "page 0 dealt, or a page outside the pool"
    assert len(np.unique(dealt)) == len(dealt), "a physical page dealt twice"
    for b, n in enumerate(pages_per_row):
        assert (bt[b, n:] == 0).all()
    return dealt


def _decode_pages(spec):
    return _pages(spec.hist_lens + spec.n_new)


def test_tiny_f32():
    s = wl.decode_spec("tiny_f32")
    assert (s.batch, s.hq, s.hkv, s.head_dim, s.dtype, s.page_size) == (2, 4, 2, 64, "f32", 16)
    assert s.hist_lens.tolist() == [37, 80] and s.n_new == 1
    assert s.num_pages == 16  # page 0 plus 15 usable
    _check_table(s, _decode_pages(s))


def test_qwen3_decode_b64():
    s = wl.decode_spec("qwen3_decode")
    assert (s.batch, s.hq, s.hkv, s.head_dim, s.dtype) == (64, 32, 8, 128, "bf16")
    assert s.hist_lens.min() >= 512 and s.hist_lens.max() <= 1024
    pages = _decode_pages(s)
    assert s.num_pages == math.ceil(1.25 * sum(pages)) + 1
    dealt = _check_table(s, pages)
    assert not np.array_equal(dealt, np.sort(dealt)), "pages are not shuffled"


@pytest.mark.parametrize("batch", [8, 16, 32, 64, 128, 256])
def test_qwen3_sweep(batch):
    s = wl.decode_spec("qwen3_sweep", batch=batch)
    assert s.batch == batch and (s.hq, s.hkv, s.head_dim) == (32, 8, 128)
    # prompt U{64..512} plus generated U{0..512}
    assert s.hist_lens.min() >= 64 and s.hist_lens.max() <= 1024
    pages = _decode_pages(s)
    assert s.num_pages == math.ceil(1.25 * sum(pages)) + 1
    _check_table(s, pages)
    assert s.seed == 300 + batch  # a fresh permutation per batch


def test_long_ragged():
    s = wl.decode_spec("long_ragged")
    assert s.batch == 256 and (s.hq, s.hkv, s.head_dim) == (32, 8, 128)
    assert s.hist_lens.min() >= 16 and s.hist_lens.max() <= 32768
    # log-uniform on [ln 16, ln 32768]: mean 6.585, sd 2.2 (sample mean of 256: sd 0.14)
    assert abs(np.log(s.hist_lens).mean() - 0.5 * (math.log(16) + math.log(32768))) < 0.6
    pages = _decode_pages(s)
    assert s.num_pages == sum(pages) + 1, "the long-context pool is fully fragmented: no free page"
    _check_table(s, pages)


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16, 32])
def test_prefill_batches(batch):
    s = wl.prefill_spec(batch=batch)
    assert s.batch == batch and (s.hq, s.hkv, s.head_dim, s.dtype) == (48, 8, 256, "bf16")
    assert (s.q_lens >= 65).all() and (s.q_lens <= 4096).all()
    assert (s.kv_lens >= s.q_lens).all() and (s.kv_lens - s.q_lens <= 4096).all()
    assert (s.kv_lens <= 32768).all()
    pages = _pages(s.kv_lens)
    assert s.num_pages == sum(pages) + 1
    _check_table(s, pages)


def test_prefill_fixed_1023():
    s = wl.prefill_spec(fixed_1023=True)
    assert s.batch == 1 and s.q_lens.tolist() == [1023] and s.kv_lens.tolist() == [1023]
    _check_table(s, _pages(s.kv_lens))


def _same_inputs(a, b):
    for f in dataclasses.fields(a):
        x, y = getattr(a, f.name), getattr(b, f.name)
        if not isinstance(x, torch.Tensor) and x is not None:
            continue  # the spec it was drawn from
        if x is None or y is None:
            assert x is None and y is None, f.name
        else:
            assert x.dtype == y.dtype and torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f.name


def test_seeds_reproduce_every_bit():
    s1, s2 = wl.decode_spec("qwen3_sweep", batch=16), wl.decode_spec("qwen3_sweep", batch=16)
    assert np.array_equal(s1.block_table, s2.block_table) and np.array_equal(s1.hist_lens, s2.hist_lens)
    _same_inputs(wl.decode_inputs(s1), wl.decode_inputs(s2))
    p1, p2 = wl.prefill_spec(batch=2), wl.prefill_spec(batch=2)
    assert np.array_equal(p1.block_table, p2.block_table)
    _same_inputs(wl.prefill_inputs(p1), wl.prefill_inputs(p2))
    # another layer's inputs differ
    a, b = wl.decode_inputs(s1), wl.decode_inputs(s1, seed_offset=1)
    assert not torch.equal(a.q, b.q)


def test_contiguous_pages_are_runs_and_keep_the_draws():
    a = wl.decode_spec("qwen3_decode", batch=16)
    b = wl.decode_spec("qwen3_decode", batch=16, contiguous=True)
    assert np.array_equal(a.hist_lens, b.hist_lens) and a.num_pages == b.num_pages
    nxt = 1
    for row, L in zip(b.block_table, b.hist_lens + b.n_new):
        n = -(-int(L) // b.page_size)
        assert row[:n].tolist() == list(range(nxt, nxt + n)) and not row[n:].any()
        nxt += n
    for x, y in zip(wl.decode_inputs(a).q, wl.decode_inputs(b).q):
        assert torch.equal(x, y)


def test_decode_heads_keep_lengths_and_pages():
    """Another head shape for a named decode workload changes only the
    shape: the lengths, the pool size and the dealt pages stay."""
    for name, batch in (("qwen3_decode", 64), ("qwen3_sweep", 8), ("long_ragged", 16)):
        a = wl.decode_spec(name, batch=batch)
        b = wl.decode_spec(name, batch=batch, heads=(16, 8, 256))
        assert (b.hq, b.hkv, b.head_dim) == (16, 8, 256) and (a.hq, a.hkv, a.head_dim) == (32, 8, 128)
        assert np.array_equal(a.hist_lens, b.hist_lens) and np.array_equal(a.block_table, b.block_table)
        assert a.num_pages == b.num_pages and b.name == a.name + "_hq16_hkv8_d256"
