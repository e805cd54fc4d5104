"""Pins of the CPU oracle to facts other than its own code.

Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises (AssertionError or
an oracle error) when the oracle disagrees with what the pages and the
mathematics fix.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutants.py`` runs them against builds of the oracle with a
planted mistake and requires every mistake to be caught.

What each pin leans on:
  * layout    -- with pages dealt in order the pool, read as one token array,
                 is the dense history (the contiguous single-tensor pool of the
                 unsloth scripts page, "Why this works"; flex-vs-vLLM results,
                 "Best config" BLOCKS_ARE_CONTIGUOUS); a torch reshape is the
                 independent reader.
  * sdpa      -- torch's scaled_dot_product_attention in fp64 on the dense
                 (un-paged) K/V, GQA by enable_gqa, the causal mask by tril.
  * decimal   -- brute force at 40 significant digits on tiny inputs.
  * closed forms -- single key, identical keys, q = 0, dominant key, and the
                 per-row visible-key count kv - q + i + 1 with the per-request
                 pair count q (2 kv - q + 1) / 2 (FlashInfer PR #9451 analysis,
                 §1 work bound).
  * invariants -- physical-page permutation leaves every output bit unchanged.
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import BF16, F32, Pool

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
P = 16


# --------------------------------------------------------------------------
# helpers (data plumbing only)
# --------------------------------------------------------------------------

def _bits(t: torch.Tensor) -> np.ndarray:
    """numpy array holding the storage of a bf16 or fp32 CPU tensor."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _tdt(dtype: int):
    return torch.bfloat16 if dtype == BF16 else torch.float32


def _nan_pool(pool: Pool) -> np.ndarray:
    n = pool.num_pages * pool.num_kv_heads * pool.page_size * pool.head_dim
    t = torch.full((n,), float("nan"), dtype=_tdt(pool.dtype))
    return _bits(t)


def _indptr(lens) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int32)
    np.cumsum(np.asarray(lens, dtype=np.int64), out=out[1:])
    return out


def _deal(lens, num_pages, rng=None):
    """Block table for lens; pages 1.. in order (rng None) or shuffled."""
    pages = [-(-int(n) // P) for n in lens]
    ids = np.arange(1, num_pages, dtype=np.int32)
    if rng is not None:
        ids = rng.permutation(ids)
    cols = max(1, max(pages) if pages else 1)
    bt = np.zeros((len(lens), cols), dtype=np.int32)
    k = 0
    for b, n in enumerate(pages):
        bt[b, :n] = ids[k:k + n]
        k += n
    return bt


def _filled(orc, pool: Pool, k_dense: torch.Tensor, v_dense: torch.Tensor, lens, bt):
    """NaN pool with each sequence's dense K/V appended from position 0."""
    kc, vc = _nan_pool(pool), _nan_pool(pool)
    orc.append(pool, kc, vc, _bits(k_dense), _bits(v_dense), bt,
               np.zeros(len(lens), dtype=np.int32), _indptr(lens))
    return kc, vc


def _pool(dtype, num_pages, hkv, d, layout="HND") -> Pool:
    return (Pool.hnd if layout == "HND" else Pool.nhd)(dtype, num_pages, P, hkv, d)


def _rand(shape, dtype, gen):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(_tdt(dtype))


def _sdpa(q, k, v, scale, mask=None):
    """fp64 torch reference: q [Hq, nq, D], k/v [Hkv, nk, D]; returns out, lse."""
    q64, k64, v64 = (x.to(torch.float64) for x in (q, k, v))
    out = F.scaled_dot_product_attention(q64[None], k64[None], v64[None], attn_mask=mask,
                                         scale=scale, enable_gqa=True)[0]
    g = q.shape[0] // k.shape[0]
    kk = k64.repeat_interleave(g, dim=0)
    s = torch.matmul(q64, kk.transpose(-1, -2)) * scale
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return out, torch.logsumexp(s, dim=-1)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} vs {b.shape}")
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim) or np.isnan(a).any() != np.isnan(b).any():
        i = int(np.nanargmax(np.where(both_inf, 0, err - lim)))
        raise AssertionError(f"{what}: max excess at {i}: {a.ravel()[i]} vs {b.ravel()[i]}")


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_layout_contiguous(orc):
    """In-order pages: the pool read as [pages*P, Hkv, D] is the dense history,
    the appended token lands right after it, and nothing else is written."""
    gen = torch.Generator().manual_seed(11)
    for dtype in (F32, BF16):
        for layout in ("HND", "NHD"):
            lens, hkv, d = [21, 37, 16], 3, 8
            num_pages = 12
            pool = _pool(dtype, num_pages, hkv, d, layout)
            k = _rand((sum(lens), hkv, d), dtype, gen)
            v = _rand((sum(lens), hkv, d), dtype, gen)
            bt = _deal([n + 1 for n in lens], num_pages)  # room for one more token
            kc, vc = _filled(orc, pool, k, v, lens, bt)
            kn = _rand((len(lens), hkv, d), dtype, gen)
            vn = _rand((len(lens), hkv, d), dtype, gen)
            out_lens = orc.append(pool, kc, vc, _bits(kn), _bits(vn), bt,
                                  np.asarray(lens, dtype=np.int32))
            assert out_lens.tolist() == [n + 1 for n in lens], out_lens
            for cache, dense, new in ((kc, k, kn), (vc, v, vn)):
                t = torch.from_numpy(cache.view(np.int16) if dtype == BF16 else cache)
                if dtype == BF16:
                    t = t.view(torch.bfloat16)
                if layout == "HND":
                    tok = t.view(num_pages, hkv, P, d).permute(0, 2, 1, 3).reshape(-1, hkv, d)
                else:
                    tok = t.view(num_pages * P, hkv, d)
                ip = _indptr(lens)
                written = torch.zeros(tok.shape[0], dtype=torch.bool)
                for b, n in enumerate(lens):
                    start = int(bt[b, 0]) * P
                    assert torch.equal(_bitview(tok[start:start + n]), _bitview(dense[ip[b]:ip[b + 1]])), \
                        f"history of sequence {b} not where in-order pages put it"
                    assert torch.equal(_bitview(tok[start + n]), _bitview(new[b])), \
                        f"appended token of sequence {b} misplaced"
                    written[start:start + n + 1] = True
                assert bool(torch.isnan(tok[~written].float()).all()), "bytes outside the targets changed"


def _bitview(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def pin_sdpa_decode(orc):
    """Decode on shuffled pages equals fp64 SDPA on the dense K/V (GQA)."""
    gen = torch.Generator().manual_seed(12)
    rng = np.random.default_rng(12)
    for dtype, hq, hkv, d in ((F32, 4, 2, 16), (BF16, 8, 2, 32), (BF16, 6, 1, 8)):
        lens = [1, 15, 16, 17, 50]
        num_pages = 1 + sum(-(-n // P) for n in lens) + 3
        pool = _pool(dtype, num_pages, hkv, d)
        k = _rand((sum(lens), hkv, d), dtype, gen)
        v = _rand((sum(lens), hkv, d), dtype, gen)
        q = _rand((len(lens), hq, d), dtype, gen)
        bt = _deal(lens, num_pages, rng)
        kc, vc = _filled(orc, pool, k, v, lens, bt)
        scale = 1.0 / math.sqrt(d)
        out, lse = orc.decode(pool, _bits(q), kc, vc, bt, np.asarray(lens, np.int32), scale)
        ip = _indptr(lens)
        for b in range(len(lens)):
            kd = k[ip[b]:ip[b + 1]].transpose(0, 1)
            vd = v[ip[b]:ip[b + 1]].transpose(0, 1)
            ro, rl = _sdpa(q[b][:, None, :], kd, vd, scale)
            _close(out[b], ro[:, 0].numpy(), 1e-12, 1e-13, f"decode out b={b}")
            _close(lse[b], rl[:, 0].numpy(), 1e-12, 1e-13, f"decode lse b={b}")


def pin_sdpa_prefill(orc):
    """Causal (end-aligned) and non-causal prefill equal fp64 SDPA with a
    tril(diagonal = kv - q) mask on the dense K/V."""
    gen = torch.Generator().manual_seed(13)
    rng = np.random.default_rng(13)
    for dtype in (F32, BF16):
        hq, hkv, d = 6, 2, 16
        q_lens, kv_lens = [1, 5, 17, 20], [1, 33, 17, 40]
        num_pages = 1 + sum(-(-n // P) for n in kv_lens)
        pool = _pool(dtype, num_pages, hkv, d)
        k = _rand((sum(kv_lens), hkv, d), dtype, gen)
        v = _rand((sum(kv_lens), hkv, d), dtype, gen)
        q = _rand((sum(q_lens), hq, d), dtype, gen)
        bt = _deal(kv_lens, num_pages, rng)
        kc, vc = _filled(orc, pool, k, v, kv_lens, bt)
        scale = 0.3
        qi, ki = _indptr(q_lens), _indptr(kv_lens)
        for causal in (True, False):
            out, lse = orc.prefill(pool, _bits(q), kc, vc, bt, np.asarray(kv_lens, np.int32), qi,
                                   scale, causal=causal)
            for r, (nq, nk) in enumerate(zip(q_lens, kv_lens)):
                mask = torch.ones(nq, nk, dtype=torch.bool)
                if causal:
                    mask = mask.tril(diagonal=nk - nq)
                qd = q[qi[r]:qi[r + 1]].transpose(0, 1)
                kd = k[ki[r]:ki[r + 1]].transpose(0, 1)
                vd = v[ki[r]:ki[r + 1]].transpose(0, 1)
                ro, rl = _sdpa(qd, kd, vd, scale, mask)
                _close(out[qi[r]:qi[r + 1]], ro.transpose(0, 1).numpy(), 1e-12, 1e-13,
                       f"prefill out r={r} causal={causal}")
                _close(lse[qi[r]:qi[r + 1]], rl.transpose(0, 1).numpy(), 1e-12, 1e-13,
                       f"prefill lse r={r} causal={causal}")
        # the square causal request also matches SDPA's own is_causal flag
        r = 2
        ro = F.scaled_dot_product_attention(
            q[qi[r]:qi[r + 1]].transpose(0, 1).to(torch.float64)[None],
            k[ki[r]:ki[r + 1]].transpose(0, 1).to(torch.float64)[None],
            v[ki[r]:ki[r + 1]].transpose(0, 1).to(torch.float64)[None],
            is_causal=True, scale=scale, enable_gqa=True)[0]
        out, _ = orc.prefill(pool, _bits(q), kc, vc, bt, np.asarray(kv_lens, np.int32), qi, scale)
        _close(out[qi[r]:qi[r + 1]], ro.transpose(0, 1).numpy(), 1e-12, 1e-13, "is_causal")


def pin_decimal_bruteforce(orc):
    """Two tiny sequences against 40-digit decimal arithmetic."""
    decimal.getcontext().prec = 40
    gen = torch.Generator().manual_seed(14)
    rng = np.random.default_rng(14)
    hq, hkv, d = 2, 2, 3
    lens = [5, 19]
    num_pages = 5
    pool = _pool(F32, num_pages, hkv, d)
    k = _rand((sum(lens), hkv, d), F32, gen)
    v = _rand((sum(lens), hkv, d), F32, gen)
    q = _rand((len(lens), hq, d), F32, gen)
    bt = _deal(lens, num_pages, rng)
    kc, vc = _filled(orc, pool, k, v, lens, bt)
    scale = 0.7
    out, lse = orc.decode(pool, _bits(q), kc, vc, bt, np.asarray(lens, np.int32), scale)
    ip = _indptr(lens)
    Dm = decimal.Decimal
    for b in range(len(lens)):
        for h in range(hq):
            g = h // (hq // hkv)
            qs = [Dm(float(x)) for x in q[b, h]]
            s = []
            for j in range(ip[b], ip[b + 1]):
                s.append(Dm(scale) * sum(qs[t] * Dm(float(k[j, g, t])) for t in range(d)))
            w = [x.exp() for x in s]
            z = sum(w)
            for t in range(d):
                o = sum(w[j] * Dm(float(v[ip[b] + j, g, t])) for j in range(len(w))) / z
                _close(out[b, h, t], float(o), 1e-13, 1e-15, "decimal out")
            _close(lse[b, h], float(z.ln()), 1e-13, 1e-15, "decimal lse")


def pin_single_key(orc):
    """One visible key: the output is that key's V row, bit for bit."""
    gen = torch.Generator().manual_seed(15)
    for dtype in (F32, BF16):
        hq, hkv, d = 4, 2, 16
        pool = _pool(dtype, 4, hkv, d)
        k = _rand((1, hkv, d), dtype, gen)
        v = _rand((1, hkv, d), dtype, gen)
        q = _rand((1, hq, d), dtype, gen)
        bt = np.array([[3]], dtype=np.int32)
        kc, vc = _filled(orc, pool, k, v, [1], bt)
        out, lse = orc.decode(pool, _bits(q), kc, vc, bt, np.array([1], np.int32), 0.25)
        for h in range(hq):
            g = h // 2
            assert np.array_equal(out[0, h], v[0, g].to(torch.float64).numpy()), "single key"
            s = 0.25 * float(torch.dot(q[0, h].double(), k[0, g].double()))
            _close(lse[0, h], s, 1e-14, 1e-15, "single-key lse")


def pin_identical_keys_and_zero_query(orc):
    """All keys equal (or q = 0): weights are uniform, the output is the mean
    of the visible V rows and lse = s + ln n."""
    gen = torch.Generator().manual_seed(16)
    rng = np.random.default_rng(16)
    hq, hkv, d = 4, 1, 8
    lens = [3, 40]
    num_pages = 1 + 1 + 3 + 2
    pool = _pool(F32, num_pages, hkv, d)
    k1 = _rand((1, hkv, d), F32, gen)
    k = k1.expand(sum(lens), hkv, d).contiguous()
    v = _rand((sum(lens), hkv, d), F32, gen)
    q = _rand((len(lens), hq, d), F32, gen)
    q[1, 3] = 0
    bt = _deal(lens, num_pages, rng)
    kc, vc = _filled(orc, pool, k, v, lens, bt)
    out, lse = orc.decode(pool, _bits(q), kc, vc, bt, np.asarray(lens, np.int32), 0.5)
    ip = _indptr(lens)
    for b, n in enumerate(lens):
        mean = v[ip[b]:ip[b + 1], 0].double().mean(dim=0).numpy()
        for h in range(hq):
            _close(out[b, h], mean, 1e-13, 1e-15, "identical keys mean")
            s = 0.5 * float(torch.dot(q[b, h].double(), k1[0, 0].double()))
            _close(lse[b, h], s + math.log(n), 1e-13, 1e-15, "identical keys lse")
    # a zero query against distinct keys also weighs them uniformly
    k = _rand((sum(lens), hkv, d), F32, gen)
    kc, vc = _filled(orc, pool, k, v, lens, bt)
    q0 = torch.zeros((len(lens), hq, d))
    out, lse = orc.decode(pool, _bits(q0), kc, vc, bt, np.asarray(lens, np.int32), 0.5)
    for b, n in enumerate(lens):
        mean = v[ip[b]:ip[b + 1], 0].double().mean(dim=0).numpy()
        _close(out[b], np.broadcast_to(mean, (hq, d)), 1e-13, 1e-15, "q=0 mean")
        _close(lse[b], np.full(hq, math.log(n)), 1e-13, 1e-15, "q=0 lse")


def pin_causal_counts(orc):
    """Identical keys and V[j] = j: causal row i of a request (q, kv) is the
    mean of 0..kv-q+i, i.e. (kv - q + i) / 2; every request/head visits
    q (2 kv - q + 1) / 2 pairs; without the mask every row is (kv - 1) / 2."""
    q_lens, kv_lens = [1, 7, 16, 33], [1, 7, 40, 100]
    hq, hkv, d = 3, 1, 2
    num_pages = 1 + sum(-(-n // P) for n in kv_lens)
    pool = _pool(F32, num_pages, hkv, d)
    k = torch.ones((sum(kv_lens), hkv, d))
    v = torch.cat([torch.arange(n, dtype=torch.float32) for n in kv_lens])[:, None, None]
    v = v.expand(-1, hkv, d).contiguous()
    q = torch.full((sum(q_lens), hq, d), 0.5)
    bt = _deal(kv_lens, num_pages, np.random.default_rng(17))
    kc, vc = _filled(orc, pool, k, v, kv_lens, bt)
    qi = _indptr(q_lens)
    out, lse, pc = orc.prefill(pool, _bits(q), kc, vc, bt, np.asarray(kv_lens, np.int32), qi, 1.0,
                               causal=True, pair_counts=True)
    for r, (nq, nk) in enumerate(zip(q_lens, kv_lens)):
        for i in range(nq):
            want = (nk - nq + i) / 2.0
            _close(out[qi[r] + i], np.full((hq, d), want), 1e-13, 1e-13, f"causal row r={r} i={i}")
            _close(lse[qi[r] + i], np.full(hq, 1.0 + math.log(nk - nq + i + 1)), 1e-13, 1e-13,
                   "causal lse")
        assert pc[r].tolist() == [nq * (2 * nk - nq + 1) // 2] * hq, (r, pc[r])
    out, _ = orc.prefill(pool, _bits(q), kc, vc, bt, np.asarray(kv_lens, np.int32), qi, 1.0,
                         causal=False)
    for r, (nq, nk) in enumerate(zip(q_lens, kv_lens)):
        _close(out[qi[r]:qi[r + 1]], np.full((nq, hq, d), (nk - 1) / 2.0), 1e-13, 1e-13,
               "non-causal rows")


def pin_golden_work_bound(orc):
    """The two paged-prefill workloads quoted in the FlashInfer PR #9451
    analysis were served by the work-gated path, so their causal pair work
    reaches the page's 2^24 gate; the oracle's visit counter must say so and
    match the page's per-request formula."""
    with open(os.path.join(GOLDEN, "flashinfer_pr9451_causal_work.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        hq, hkv = case["hq"], case["hkv"]
        q_lens, kv_lens = case["q_lens"], case["kv_lens"]
        num_pages = 1 + sum(-(-n // P) for n in kv_lens)
        pool = _pool(F32, num_pages, hkv, 1)
        k = torch.zeros((sum(kv_lens), hkv, 1))
        q = torch.zeros((sum(q_lens), hq, 1))
        bt = _deal(kv_lens, num_pages)
        kc, vc = _filled(orc, pool, k, k, kv_lens, bt)
        _, _, pc = orc.prefill(pool, _bits(q), kc, vc, bt, np.asarray(kv_lens, np.int32),
                               _indptr(q_lens), 1.0, causal=True, pair_counts=True, nthreads=8)
        work = int(pc.sum())
        formula = hq * sum(qq * (2 * kk - qq + 1) // 2 for qq, kk in zip(q_lens, kv_lens))
        assert work == formula, (case["name"], work, formula)
        assert (work >= case["gate"]) == case["admitted"], (case["name"], work)


def pin_permutation_invariance(orc):
    """Moving pages to other physical slots (and remapping the table) leaves
    every output bit unchanged."""
    gen = torch.Generator().manual_seed(18)
    rng = np.random.default_rng(18)
    for dtype in (F32, BF16):
        hq, hkv, d = 4, 2, 16
        lens = [20, 47, 64]
        num_pages = 1 + sum(-(-n // P) for n in lens) + 4
        pool = _pool(dtype, num_pages, hkv, d)
        k = _rand((sum(lens), hkv, d), dtype, gen)
        v = _rand((sum(lens), hkv, d), dtype, gen)
        q = _rand((len(lens), hq, d), dtype, gen)
        bt1 = _deal(lens, num_pages, rng)
        bt2 = _deal(lens, num_pages, rng)
        assert not np.array_equal(bt1, bt2)
        a = orc.decode(pool, _bits(q), *_filled(orc, pool, k, v, lens, bt1), bt1,
                       np.asarray(lens, np.int32), 0.25)
        b = orc.decode(pool, _bits(q), *_filled(orc, pool, k, v, lens, bt2), bt2,
                       np.asarray(lens, np.int32), 0.25)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "permutation changed bits"


def pin_dominant_key(orc):
    """K = -1 except +1 at position j*, q = c: all other weights underflow
    against exp(-2 scale c D) and the output is V[j*]."""
    gen = torch.Generator().manual_seed(19)
    rng = np.random.default_rng(19)
    hq, hkv, d = 2, 1, 8
    n = 50
    num_pages = 1 + 4
    pool = _pool(BF16, num_pages, hkv, d)
    v = _rand((n, hkv, d), BF16, gen)
    q = torch.full((1, hq, d), 16.0, dtype=torch.bfloat16)
    bt = _deal([n], num_pages, rng)
    for jstar in (0, 15, 16, 31, 32, 49):
        k = -torch.ones((n, hkv, d), dtype=torch.bfloat16)
        k[jstar] = 1
        kc, vc = _filled(orc, pool, k, v, [n], bt)
        out, _ = orc.decode(pool, _bits(q), kc, vc, bt, np.array([n], np.int32), 1.0 / math.sqrt(d))
        for h in range(hq):
            _close(out[0, h], v[jstar, 0].double().numpy(), 1e-12, 0.0, f"dominant j*={jstar}")


def pin_empty_rows(orc):
    """A sequence with no keys gives out = 0 and lse = -inf, and does not
    disturb its neighbours."""
    gen = torch.Generator().manual_seed(20)
    hq, hkv, d = 2, 1, 4
    lens = [0, 5, 0]
    pool = _pool(F32, 3, hkv, d)
    k = _rand((5, hkv, d), F32, gen)
    v = _rand((5, hkv, d), F32, gen)
    q = _rand((3, hq, d), F32, gen)
    bt = np.zeros((3, 1), dtype=np.int32)
    bt[1, 0] = 2
    kc, vc = _filled(orc, pool, k, v, lens, bt)
    out, lse = orc.decode(pool, _bits(q), kc, vc, bt, np.asarray(lens, np.int32), 0.5)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))
    ro, rl = _sdpa(q[1][:, None, :], k.transpose(0, 1), v.transpose(0, 1), 0.5)
    _close(out[1], ro[:, 0].numpy(), 1e-12, 1e-13, "neighbour of empty rows")


def pin_route_matches_append(orc):
    """The routed offset of token j is where append stored token j."""
    gen = torch.Generator().manual_seed(21)
    rng = np.random.default_rng(21)
    for layout in ("HND", "NHD"):
        hkv, d = 2, 4
        lens = [3, 33, 16]
        num_pages = 1 + sum(-(-n // P) for n in lens) + 2
        pool = _pool(F32, num_pages, hkv, d, layout)
        k = _rand((sum(lens), hkv, d), F32, gen)
        bt = _deal(lens, num_pages, rng)
        kc, _ = _filled(orc, pool, k, k, lens, bt)
        off = orc.route(pool, bt, np.asarray(lens, np.int32), max(lens))
        ip = _indptr(lens)
        for b, n in enumerate(lens):
            assert np.all(off[b, n:] == -1)
            for j in range(n):
                for g in range(hkv):
                    base = off[b, j] + g * pool.s_head
                    assert np.array_equal(kc[base:base + d], k[ip[b] + j, g].numpy()), (b, j, g)


def pin_append_ragged(orc):
    """Ragged append of several tokens per sequence continues each sequence
    after its cached tokens, whatever was cached before."""
    gen = torch.Generator().manual_seed(22)
    rng = np.random.default_rng(22)
    hq, hkv, d = 2, 2, 4
    hist, new = [5, 0, 16], [3, 17, 1]
    total = [a + b for a, b in zip(hist, new)]
    num_pages = 1 + sum(-(-n // P) for n in total) + 1
    pool = _pool(F32, num_pages, hkv, d)
    kd = _rand((sum(total), hkv, d), F32, gen)
    vd = _rand((sum(total), hkv, d), F32, gen)
    bt = _deal(total, num_pages, rng)
    ti = _indptr(total)
    kh = torch.cat([kd[ti[b]:ti[b] + hist[b]] for b in range(3)])
    vh = torch.cat([vd[ti[b]:ti[b] + hist[b]] for b in range(3)])
    kn = torch.cat([kd[ti[b] + hist[b]:ti[b + 1]] for b in range(3)])
    vn = torch.cat([vd[ti[b] + hist[b]:ti[b + 1]] for b in range(3)])
    kc, vc = _filled(orc, pool, kh, vh, hist, bt)
    lens = orc.append(pool, kc, vc, _bits(kn), _bits(vn), bt, np.asarray(hist, np.int32),
                      _indptr(new))
    assert lens.tolist() == total
    kc2, vc2 = _filled(orc, pool, kd, vd, total, bt)
    assert np.array_equal(kc.view(np.uint32), kc2.view(np.uint32))
    assert np.array_equal(vc.view(np.uint32), vc2.view(np.uint32))
    q = _rand((3, hq, d), F32, gen)
    out, _ = orc.decode(pool, _bits(q), kc, vc, bt, lens, 0.5)
    for b in range(3):
        ro, _ = _sdpa(q[b][:, None, :], kd[ti[b]:ti[b + 1]].transpose(0, 1),
                      vd[ti[b]:ti[b + 1]].transpose(0, 1), 0.5)
        _close(out[b], ro[:, 0].numpy(), 1e-12, 1e-13, "after ragged append")


# --------------------------------------------------------------------------
# rotary position embedding (mini-infer 06 "True PagedAttention", §3)
# --------------------------------------------------------------------------

def _rope_tables(rows, d, base=10000.0):
    """fp32 cos/sin tables [rows, d/2] of the angles p * base^(-2i/d), the
    usual rotary frequencies, computed in fp64 and rounded to fp32."""
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _rope_np(orc, dtype, x: torch.Tensor, pos, cos, sin, interleaved):
    xb = _bits(x)
    orc.rope(dtype, xb, np.asarray(pos, np.int32), cos, sin, interleaved)
    return xb


def pin_rope_unit_vectors(orc):
    """A pair (a, b) = (1, 0) turns into (cos, sin) and (0, 1) into
    (-sin, cos): the rotation is counter-clockwise by the table's angle, in
    the slots each layout names (half-split: i and i + D/2; interleaved: 2i
    and 2i+1)."""
    d, rows = 8, 5
    cos, sin = _rope_tables(rows, d)
    half = d // 2
    for interleaved in (False, True):
        for i in range(half):
            ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
            for p in range(rows):
                for (a, b), want in (((1.0, 0.0), (cos[p, i], sin[p, i])), ((0.0, 1.0), (-sin[p, i], cos[p, i]))):
                    x = torch.zeros((1, 1, d), dtype=torch.float32)
                    x[0, 0, ia], x[0, 0, ib] = a, b
                    y = _rope_np(orc, F32, x, [p], cos, sin, interleaved)
                    assert y[0, 0, ia] == np.float32(want[0]) and y[0, 0, ib] == np.float32(want[1]), (
                        interleaved, i, p, (a, b))
                    others = np.delete(y[0, 0], [ia, ib])
                    assert np.all(others == 0)


def pin_rope_position_zero_identity(orc):
    """At position 0 (angle 0: cos 1, sin 0) every bit is unchanged, bf16 and fp32."""
    gen = torch.Generator().manual_seed(31)
    cos, sin = _rope_tables(4, 64)
    for dtype in (F32, BF16):
        x = _rand((6, 3, 64), dtype, gen)
        for interleaved in (False, True):
            y = _rope_np(orc, dtype, x, [0] * 6, cos, sin, interleaved)
            assert np.array_equal(y, _bits(x)), (dtype, interleaved)


def pin_rope_orthogonal(orc):
    """The rotation keeps every head vector's norm and the inner product of
    two vectors turned by the same positions (fp32, up to fp32 rounding)."""
    gen = torch.Generator().manual_seed(32)
    d = 128
    cos, sin = _rope_tables(5000, d)
    pos = [0, 1, 17, 999, 4095, 4999]
    x = _rand((6, 4, d), F32, gen)
    y = _rand((6, 4, d), F32, gen)
    for interleaved in (False, True):
        rx = _rope_np(orc, F32, x, pos, cos, sin, interleaved).astype(np.float64)
        ry = _rope_np(orc, F32, y, pos, cos, sin, interleaved).astype(np.float64)
        x64, y64 = x.double().numpy(), y.double().numpy()
        _close(np.linalg.norm(rx, axis=-1), np.linalg.norm(x64, axis=-1), 1e-6, 1e-6, "rope norm")
        _close((rx * ry).sum(-1), (x64 * y64).sum(-1), 1e-5, 1e-6, "rope inner product")


def pin_rope_relative_position(orc):
    """q turned by position m and k by position n have an inner product that
    depends on m - n only: shifting both positions by s leaves it unchanged
    (fp32, up to the rounding of the tables and of the rotation)."""
    gen = torch.Generator().manual_seed(33)
    d = 64
    cos, sin = _rope_tables(3000, d)
    q = _rand((1, 1, d), F32, gen)
    k = _rand((1, 1, d), F32, gen)
    for interleaved in (False, True):
        for m, n in ((5, 3), (100, 40), (700, 699)):
            dots = []
            for shift in (0, 11, 1200, 2200):
                rq = _rope_np(orc, F32, q, [m + shift], cos, sin, interleaved).astype(np.float64)
                rk = _rope_np(orc, F32, k, [n + shift], cos, sin, interleaved).astype(np.float64)
                dots.append(float((rq * rk).sum()))
            _close(np.array(dots), np.full(len(dots), dots[0]), 2e-4, 1e-5, f"relative position {m}-{n}")


def pin_rope_layouts_are_one_rotation(orc):
    """The interleaved layout is the half-split one with the dims reordered:
    moving dim 2i to i and 2i+1 to i + D/2, rotating half-split and moving
    back gives the interleaved result bit for bit."""
    gen = torch.Generator().manual_seed(34)
    d = 32
    cos, sin = _rope_tables(200, d)
    half = d // 2
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # half-split slot j holds dim perm[j]
    pos = [3, 199, 0, 42]
    for dtype in (F32, BF16):
        x = _rand((4, 2, d), dtype, gen)
        inter = _rope_np(orc, dtype, x, pos, cos, sin, True)
        split = _rope_np(orc, dtype, x[..., torch.from_numpy(perm)].contiguous(), pos, cos, sin, False)
        back = np.empty_like(split)
        back[..., perm] = split
        assert np.array_equal(inter, back), dtype
    assert half == d // 2


def pin_rope_matches_rotate_half(orc):
    """The half-split rotation equals the rotate_half form of the model code
    the pages call (apply_rotary_pos_emb: x cos + rotate_half(x) sin, with the
    half tables repeated twice), evaluated with torch in fp64; and the
    interleaved one equals the same form on interleaved pairs.  fp32 inputs:
    the fp64 results are rounded once to fp32 by torch, bit for bit equal."""
    gen = torch.Generator().manual_seed(35)
    d = 64
    cos, sin = _rope_tables(4096, d)
    pos = np.array([0, 1, 2, 77, 1023, 4095], np.int64)
    x = _rand((6, 3, d), F32, gen)
    c = torch.from_numpy(cos[pos]).double()[:, None, :]
    s = torch.from_numpy(sin[pos]).double()[:, None, :]
    x64 = x.double()
    half = d // 2
    rot = torch.cat([-x64[..., half:], x64[..., :half]], -1)
    want = (x64 * torch.cat([c, c], -1) + rot * torch.cat([s, s], -1)).float().numpy()
    got = _rope_np(orc, F32, x, pos, cos, sin, False)
    assert np.array_equal(got, want), "half-split vs rotate_half"
    x1, x2 = x64[..., 0::2], x64[..., 1::2]
    rot_i = torch.stack([-x2, x1], -1).flatten(-2)
    want_i = (x64 * c.repeat_interleave(2, -1) + rot_i * s.repeat_interleave(2, -1)).float().numpy()
    got_i = _rope_np(orc, F32, x, pos, cos, sin, True)
    assert np.array_equal(got_i, want_i), "interleaved vs pairwise rotate_half"


def _bf16_nearest_even(v: float) -> int:
    """bf16 bits of the fp64 value v rounded to nearest, ties to even, by
    exact rational arithmetic (finite, normal-range v)."""
    from fractions import Fraction

    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    f = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    q = f / Fraction(2) ** (e - 7)  # in [128, 256)
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 256:
        n, e = 128, e + 1
    return sign | ((e + 127) << 7) | (n - 128)


def pin_rope_bf16_rounding(orc):
    """bf16 storage: each rotated value is the fp64 result of the rotation
    rounded to nearest bf16 with ties to even (the fp64 value from the
    rotate_half form in torch, the rounding by exact rational arithmetic)."""
    gen = torch.Generator().manual_seed(36)
    d = 32
    cos, sin = _rope_tables(600, d)
    pos = np.array([1, 5, 99, 598, 300], np.int64)
    x = _rand((5, 4, d), BF16, gen)
    c = torch.from_numpy(cos[pos]).double()[:, None, :]
    s = torch.from_numpy(sin[pos]).double()[:, None, :]
    x64 = x.double()
    half = d // 2
    rot = torch.cat([-x64[..., half:], x64[..., :half]], -1)
    want64 = (x64 * torch.cat([c, c], -1) + rot * torch.cat([s, s], -1)).numpy()
    want = np.vectorize(_bf16_nearest_even, otypes=[np.uint16])(want64)
    got = _rope_np(orc, BF16, x, pos, cos, sin, False)
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} bf16 roundings differ"


ALL_PINS = [
    pin_layout_contiguous,
    pin_sdpa_decode,
    pin_sdpa_prefill,
    pin_decimal_bruteforce,
    pin_single_key,
    pin_identical_keys_and_zero_query,
    pin_causal_counts,
    pin_golden_work_bound,
    pin_permutation_invariance,
    pin_dominant_key,
    pin_empty_rows,
    pin_route_matches_append,
    pin_append_ragged,
    pin_rope_unit_vectors,
    pin_rope_position_zero_identity,
    pin_rope_orthogonal,
    pin_rope_relative_position,
    pin_rope_layouts_are_one_rotation,
    pin_rope_matches_rotate_half,
    pin_rope_bf16_rounding,
]
