"""Helpers for the GPU parity tests: run the same seeded inputs through the
HIP library (device) and the oracle (host) and compare.

Both sides build their own pool from the same dense history: the library
with pkv_append on the device, the oracle with its own append on the host.
Pools start NaN-filled, so page 0, free pages and the tail slots of partly
filled pages all hold NaN that must never leak into a result."""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

import oracle
import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl

BF16_TOL = (2e-2, 2e-2)   # (atol, rtol) on bf16 outputs
F32_TOL = (1e-5, 1e-5)    # (atol, rtol) on fp32 outputs


def say(*a):
    """Progress line naming the case, flushed before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def opool(spec) -> oracle.Pool:
    dt = oracle.BF16 if spec.dtype == "bf16" else oracle.F32
    ctor = oracle.Pool.hnd if spec.layout == "HND" else oracle.Pool.nhd
    return ctor(dt, spec.num_pages, spec.page_size, spec.hkv, spec.head_dim)


def tol(spec):
    return BF16_TOL if spec.dtype == "bf16" else F32_TOL


def compare(gpu, ref, atol, rtol, what):
    """|gpu - ref| <= atol + rtol |ref| elementwise, gpu widened exactly."""
    g = gpu.detach().float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    both_inf = np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r))
    # equal infinities (-inf lse of empty rows) count as exact; they are
    # masked out before the subtraction so that no inf - inf is evaluated
    err = np.abs(np.where(both_inf, 0.0, g) - np.where(both_inf, 0.0, r))
    assert not np.isnan(g).any(), f"{what}: NaN in GPU result"
    lim = atol + rtol * np.abs(r)
    bad = ~(err <= lim)
    rel = err / np.maximum(np.abs(r), 1e-30)
    stats = f"max abs err {float(np.max(err, initial=0)):.3e}, max rel err {float(np.max(np.where(both_inf, 0, rel), initial=0)):.3e}"
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at {i}: "
                             f"gpu {g.ravel()[i]!r} ref {r.ravel()[i]!r}; {stats}")
    return stats


class DecodeCase:
    """A decode workload materialised on both sides."""

    def __init__(self, spec: wl.DecodeSpec, device="cuda", gen_device="cpu", oracle_rows=None, seed_offset=0):
        self.spec = spec
        self.dev = torch.device(device)
        inp = wl.decode_inputs(spec, device=gen_device, seed_offset=seed_offset)
        self.inp_host = inp.to("cpu")
        self.inp = inp.to(self.dev)
        self.rows = None if oracle_rows is None else np.asarray(sorted(oracle_rows), dtype=np.int64)

    # -- device side -------------------------------------------------------
    def gpu_pools(self):
        s, i = self.spec, self.inp
        kc = wl.empty_pool(s, self.dev)
        vc = wl.empty_pool(s, self.dev)
        zeros = torch.zeros(s.batch, dtype=torch.int32, device=self.dev)
        pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, zeros, i.hist_indptr, layout=s.layout)
        lens = pkv.append(kc, vc, i.k_new, i.v_new, i.block_table, i.hist_lens, i.new_indptr, layout=s.layout)
        return kc, vc, lens

    def gpu_decode(self, kc, vc, lens, workers=0, q=None):
        s = self.spec
        max_kv = int(s.hist_lens.max()) + s.n_new if s.batch else 0
        return pkv.decode_attn(self.inp.q if q is None else q, kc, vc, self.inp.block_table, lens, max_kv,
                               scale=s.scale, layout=s.layout, workers=workers, return_lse=True)

    # -- oracle side -------------------------------------------------------
    def oracle_pools(self):
        """Host pools built by the oracle's append (all rows, or the sampled
        rows only when oracle_rows was given)."""
        s, h = self.spec, self.inp_host
        orc = oracle.load()
        pool = opool(s)
        kc = host_bits(wl.empty_pool(s, "cpu")).copy()
        vc = kc.copy()
        if self.rows is None:
            bt = h.block_table
            hist = h.hist_lens
            k_hist, v_hist, indptr = h.k_hist, h.v_hist, h.hist_indptr
            k_new, v_new, new_indptr = h.k_new, h.v_new, h.new_indptr
        else:
            rows = self.rows
            ip = h.hist_indptr.numpy()
            bt = h.block_table[rows]
            hist = h.hist_lens[rows]
            sel = np.concatenate([np.arange(ip[r], ip[r + 1]) for r in rows]) if len(rows) else np.zeros(0, np.int64)
            k_hist, v_hist = h.k_hist[sel], h.v_hist[sel]
            indptr = torch.from_numpy(np.concatenate([[0], np.cumsum(hist.numpy())]).astype(np.int32))
            n = s.n_new
            sel_new = np.concatenate([np.arange(r * n, (r + 1) * n) for r in rows])
            k_new, v_new = h.k_new[sel_new], h.v_new[sel_new]
            new_indptr = None if n == 1 else torch.arange(0, (len(rows) + 1) * n, n, dtype=torch.int32)
        orc.append(pool, kc, vc, host_bits(k_hist), host_bits(v_hist), bt.numpy(),
                   np.zeros(bt.shape[0], np.int32), indptr.numpy())
        lens = orc.append(pool, kc, vc, host_bits(k_new), host_bits(v_new), bt.numpy(), hist.numpy(),
                          None if new_indptr is None else new_indptr.numpy())
        return kc, vc, lens, bt

    def oracle_decode(self, kc, vc, lens, bt, q=None, nthreads=None):
        s = self.spec
        q = self.inp_host.q if q is None else q
        if self.rows is not None:
            q = q[self.rows]
        return oracle.load().decode(opool(s), host_bits(q), kc, vc, bt.numpy(), lens, s.scale,
                                    nthreads=nthreads or min(16, os.cpu_count() or 1))


def with_scale(spec, scale: float):
    """The same workload with another softmax scale (the specs derive theirs
    from head_dim)."""
    import dataclasses

    @dataclasses.dataclass
    class Scaled(type(spec)):
        scale_value: float = 0.0

        @property
        def scale(self):
            return self.scale_value

    return Scaled(**{f.name: getattr(spec, f.name) for f in dataclasses.fields(spec)}, scale_value=float(scale))


def scale_of(d):
    return float(np.float32(1.0 / math.sqrt(d)))


class PrefillCase:
    """A causal prefill workload on both sides.  The device builds its pool
    with pkv_append (history, then the chunk); the oracle does the same with
    its own append, optionally for a subset of requests only."""

    def __init__(self, spec: wl.PrefillSpec, device="cuda", gen_device="cpu"):
        self.spec = spec
        self.dev = torch.device(device)
        inp = wl.prefill_inputs(spec, device=gen_device)
        self.inp = inp.to(self.dev)
        self.inp_host = inp.to("cpu")

    def gpu_pools(self):
        s, i = self.spec, self.inp
        kc = wl.empty_pool(s, self.dev)
        vc = wl.empty_pool(s, self.dev)
        zeros = torch.zeros(s.batch, dtype=torch.int32, device=self.dev)
        pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, zeros, i.hist_indptr, layout=s.layout)
        kv = pkv.append(kc, vc, i.k_new, i.v_new, i.block_table, i.hist_lens, i.qo_indptr, layout=s.layout)
        return kc, vc, kv

    def gpu_prefill(self, kc, vc, kv, causal=True, rows=0, split=True, workspace=None):
        s = self.spec
        return pkv.prefill_attn(self.inp.q, kc, vc, self.inp.block_table, kv, self.inp.qo_indptr,
                                int(s.q_lens.max()), int(s.kv_lens.max()), causal=causal, scale=s.scale,
                                layout=s.layout, return_lse=True, rows_per_workgroup=rows, split=split,
                                workspace=workspace)

    def oracle_pools(self, requests=None):
        """Host pools holding the history and chunk of `requests` (all by default)."""
        s, h = self.spec, self.inp_host
        reqs = list(range(s.batch)) if requests is None else list(requests)
        hi = h.hist_indptr.numpy()
        qi = h.qo_indptr.numpy()
        hsel = np.concatenate([np.arange(hi[r], hi[r + 1]) for r in reqs]).astype(np.int64)
        qsel = np.concatenate([np.arange(qi[r], qi[r + 1]) for r in reqs]).astype(np.int64)
        hist = s.hist_lens[reqs]
        ql = s.q_lens[reqs]
        bt = s.block_table[reqs]
        pool = opool(s)
        kc = host_bits(wl.empty_pool(s, "cpu")).copy()
        vc = kc.copy()
        orc = oracle.load()
        orc.append(pool, kc, vc, host_bits(h.k_hist[hsel]), host_bits(h.v_hist[hsel]), bt,
                   np.zeros(len(reqs), np.int32), np.concatenate([[0], np.cumsum(hist)]).astype(np.int32))
        kv = orc.append(pool, kc, vc, host_bits(h.k_new[qsel]), host_bits(h.v_new[qsel]), bt, hist,
                        np.concatenate([[0], np.cumsum(ql)]).astype(np.int32))
        return kc, vc, kv, bt, reqs

    def oracle_rows(self, kc, vc, kv, bt, reqs, first=None, last=None, causal=True, nthreads=None):
        """Oracle output for each request of `reqs`: all rows (first = last =
        None), or its first `first` rows -- the chunk of its first `first`
        tokens over history + first keys -- and its last `last` rows -- the
        chunk of its last `last` tokens over all its keys."""
        s, h = self.spec, self.inp_host
        qi = h.qo_indptr.numpy()
        orc = oracle.load()
        nt = nthreads or min(16, os.cpu_count() or 1)
        q_parts, lens, rows = [], [], []
        for n, r in enumerate(reqs):
            q_r, kv_r = int(s.q_lens[r]), int(kv[n])
            parts = []
            if first is None and last is None:
                parts.append((0, q_r, kv_r))
            else:
                if first:
                    m = min(first, q_r)
                    parts.append((0, m, kv_r - q_r + m))
                if last:
                    m = min(last, q_r)
                    parts.append((q_r - m, q_r, kv_r))
            for a0, a1, kvp in parts:
                q_parts.append(h.q[qi[r] + a0: qi[r] + a1])
                lens.append((a1 - a0, kvp, n))
                rows.extend(range(qi[r] + a0, qi[r] + a1))
        return self._run_parts(kc, vc, bt, q_parts, lens, rows, causal, nt)

    def oracle_row_set(self, kc, vc, kv, bt, reqs, pick, causal=True, nthreads=None):
        """Oracle output for the query rows pick(r, q_r) (sorted indices) of
        each request of `reqs`.  Each run of consecutive rows [a0, a1) is its
        own chunked-prefill request over the first kv_r - q_r + a1 keys, so
        its rows see exactly the keys they see in the whole request."""
        s, h = self.spec, self.inp_host
        qi = h.qo_indptr.numpy()
        nt = nthreads or min(16, os.cpu_count() or 1)
        q_parts, lens, rows = [], [], []
        for n, r in enumerate(reqs):
            q_r, kv_r = int(s.q_lens[r]), int(kv[n])
            sel = np.asarray(sorted(set(int(i) for i in pick(r, q_r) if 0 <= i < q_r)), np.int64)
            if sel.size == 0:
                continue
            breaks = np.flatnonzero(np.diff(sel) != 1) + 1
            for run in np.split(sel, breaks):
                a0, a1 = int(run[0]), int(run[-1]) + 1
                kvp = kv_r - q_r + a1 if causal else kv_r
                q_parts.append(h.q[qi[r] + a0: qi[r] + a1])
                lens.append((a1 - a0, kvp, n))
                rows.extend(range(qi[r] + a0, qi[r] + a1))
        return self._run_parts(kc, vc, bt, q_parts, lens, rows, causal, nt)

    def _run_parts(self, kc, vc, bt, q_parts, lens, rows, causal, nt):
        s = self.spec
        orc = oracle.load()
        qcat = torch.cat(q_parts)
        ql = np.array([x[0] for x in lens], np.int32)
        kvl = np.array([x[1] for x in lens], np.int32)
        btl = bt[[x[2] for x in lens]]
        out, lse = orc.prefill(opool(s), host_bits(qcat), kc, vc, btl, kvl,
                               np.concatenate([[0], np.cumsum(ql)]).astype(np.int32), s.scale, causal=causal,
                               nthreads=nt)
        return np.asarray(rows, np.int64), out, lse
