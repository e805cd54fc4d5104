"""Seeded synthetic inputs for paged KV attention.

This module is the one piece shared by the HIP path's tests/benchmark and the
CPU oracle.  It holds none of the method's arithmetic: it draws sequence
lengths, deals physical pages to sequences, draws N(0, 1) activations and
makes NaN-filled pools.  Writing history into a pool and everything after it
is done separately by each side (the HIP library and the oracle).

Workloads (sizes from the pages' Qwen3-4B / FlashInfer settings):

* ``tiny_f32``          -- 2 sequences, Hq 4 / Hkv 2, head_dim 64, fp32,
                            cached lengths {37, 80}, a 16-page pool (page 0
                            reserved), one appended token per sequence.
* ``qwen3_decode``      -- Qwen3-4B attention shape (Hq 32 / Hkv 8 / D 128,
                            bf16), batch 64 by default, cached lengths
                            U{512..1024}, pool 1.25x the pages needed.
* ``qwen3_sweep``       -- same shape, batch 8..256, lengths U{64..512} prompt
                            + U{0..512} generated tokens, pool 1.25x.
* ``long_ragged``       -- same shape, batch 256, lengths
                            round(exp(U(ln 16, ln 32768))), a pool with no
                            free page (fully fragmented).
* ``prefill_d256``      -- causal paged prefill, Hq 48 / Hkv 8, head_dim 256,
                            bf16, per request q_len U{65..4096} and
                            kv_len = q_len + U{0..4096}; or the fixed request
                            q_len = kv_len = 1023.

Conventions: page size 16 unless a spec asks for another; page 0 is never dealt; the other pages are dealt
by a seeded permutation, sequence 0 first, logical blocks in order; unused
table entries hold 0 (the reserved page).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 16


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class DecodeSpec:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    hist_lens: np.ndarray      # int32 [batch]: tokens already cached
    n_new: int                 # tokens appended per sequence this step
    num_pages: int             # physical pages including reserved page 0
    bt_cols: int
    block_table: np.ndarray    # int32 [batch, bt_cols]
    seed: int
    page_size: int = PAGE_SIZE
    layout: str = "HND"        # pool layout: "HND" or "NHD"

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(head_dim), as a float32 value
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


@dataclass
class PrefillSpec:
    name: str
    q_lens: np.ndarray         # int32 [batch]
    kv_lens: np.ndarray        # int32 [batch], kv_len >= q_len
    num_pages: int
    bt_cols: int
    block_table: np.ndarray
    seed: int
    hq: int = 48
    hkv: int = 8
    head_dim: int = 256
    dtype: str = "bf16"
    page_size: int = PAGE_SIZE
    layout: str = "HND"

    @property
    def batch(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def hist_lens(self) -> np.ndarray:
        return (self.kv_lens - self.q_lens).astype(np.int32)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


def deal_pages(pages_per_seq: np.ndarray, usable_pages: int, bt_cols: int,
               rng: np.random.Generator, contiguous: bool = False) -> tuple[np.ndarray, int]:
    """Block table from a seeded permutation of pages 1..usable_pages (or,
    with ``contiguous``, pages 1, 2, 3, ... in order, so that every sequence
    owns a run of adjacent pages; the permutation is drawn either way, so the
    generator's state afterwards does not depend on the choice).

    Returns (block_table, num_pages) with num_pages = usable_pages + 1."""
    need = int(pages_per_seq.sum())
    if need > usable_pages:
        raise ValueError(f"pool of {usable_pages} usable pages cannot hold {need}")
    perm = rng.permutation(usable_pages).astype(np.int64) + 1
    if contiguous:
        perm = np.arange(1, usable_pages + 1, dtype=np.int64)
    bt = np.zeros((pages_per_seq.shape[0], bt_cols), dtype=np.int32)
    k = 0
    for b, n in enumerate(pages_per_seq.tolist()):
        if n > bt_cols:
            raise ValueError("block table too narrow")
        bt[b, :n] = perm[k:k + n]
        k += n
    return bt, usable_pages + 1


def _decode_from_lengths(name, hist, n_new, hq, hkv, d, dtype, max_hist, slack, seed, rng,
                         usable=None, layout="HND", page_size=PAGE_SIZE, contiguous=False) -> DecodeSpec:
    hist = np.asarray(hist, dtype=np.int32)
    pages = np.array([_ceil_div(int(L) + n_new, page_size) for L in hist], dtype=np.int64)
    bt_cols = _ceil_div(max_hist + n_new, page_size)
    if usable is None:
        usable = int(math.ceil(slack * int(pages.sum())))
    bt, num_pages = deal_pages(pages, usable, bt_cols, rng, contiguous)
    return DecodeSpec(name, len(hist), hq, hkv, d, dtype, hist, n_new, num_pages, bt_cols, bt,
                      seed, page_size=page_size, layout=layout)


def decode_spec(workload: str, batch: int | None = None, seed: int | None = None,
                layout: str = "HND", page_size: int = PAGE_SIZE, contiguous: bool = False,
                heads: tuple | None = None) -> DecodeSpec:
    """Lengths, pool size and block table of one decode workload (pages of
    `page_size` tokens, the named workloads use 16; pages dealt shuffled, or
    in order with `contiguous`).  `heads` = (Hq, Hkv, head_dim) replaces the
    Qwen3 shape (32, 8, 128) of the bf16 workloads, with the same lengths
    and pages; the name then carries the shape."""
    hq, hkv, d = (32, 8, 128) if heads is None else (int(heads[0]), int(heads[1]), int(heads[2]))
    tag = "" if heads is None else f"_hq{hq}_hkv{hkv}_d{d}"
    if workload == "tiny_f32":
        seed = 1 if seed is None else seed
        rng = np.random.default_rng(seed)
        return _decode_from_lengths("tiny_f32", [37, 80], 1, 4, 2, 64, "f32", 80, None, seed, rng,
                                    usable=15, layout=layout, page_size=page_size,
                                    contiguous=contiguous)
    if workload == "qwen3_decode":
        batch = 64 if batch is None else batch
        seed = 2 if seed is None else seed
        rng = np.random.default_rng(seed)
        hist = rng.integers(512, 1024, size=batch, endpoint=True)
        return _decode_from_lengths(f"qwen3_decode_b{batch}{tag}", hist, 1, hq, hkv, d, "bf16", 1024,
                                    1.25, seed, rng, layout=layout,
                                    page_size=page_size, contiguous=contiguous)
    if workload == "qwen3_sweep":
        if batch is None:
            raise ValueError("qwen3_sweep needs a batch size")
        seed = 300 + batch if seed is None else seed
        rng = np.random.default_rng(seed)
        prompt = rng.integers(64, 512, size=batch, endpoint=True)
        gen = rng.integers(0, 512, size=batch, endpoint=True)
        return _decode_from_lengths(f"qwen3_sweep_b{batch}{tag}", prompt + gen, 1, hq, hkv, d, "bf16",
                                    1024, 1.25, seed, rng, layout=layout,
                                    page_size=page_size, contiguous=contiguous)
    if workload == "long_ragged":
        batch = 256 if batch is None else batch
        seed = 4 if seed is None else seed
        rng = np.random.default_rng(seed)
        u = rng.uniform(math.log(16.0), math.log(32768.0), size=batch)
        hist = np.clip(np.rint(np.exp(u)), 16, 32768).astype(np.int32)
        return _decode_from_lengths(f"long_ragged_b{batch}{tag}", hist, 1, hq, hkv, d, "bf16", 32768,
                                    1.0, seed, rng, layout=layout,
                                    page_size=page_size, contiguous=contiguous)
    raise ValueError(f"unknown decode workload {workload!r}")


def custom_decode_spec(hist_lens, hq: int, hkv: int, head_dim: int, dtype: str, seed: int,
                       n_new: int = 1, slack: float = 1.25, extra_cols: int = 0,
                       layout: str = "HND", page_size: int = PAGE_SIZE, contiguous: bool = False) -> DecodeSpec:
    """Decode workload with explicit cached lengths (for edge cases)."""
    rng = np.random.default_rng(seed)
    hist = np.asarray(hist_lens, dtype=np.int32)
    max_hist = int(hist.max()) if hist.size else 0
    pages = np.array([_ceil_div(int(L) + n_new, page_size) for L in hist], dtype=np.int64)
    bt_cols = max(1, _ceil_div(max_hist + n_new, page_size) + extra_cols)
    usable = max(1, int(math.ceil(slack * int(pages.sum()))))
    bt, num_pages = deal_pages(pages, usable, bt_cols, rng, contiguous)
    return DecodeSpec("custom", len(hist), hq, hkv, head_dim, dtype, hist, n_new, num_pages,
                      bt_cols, bt, seed, page_size=page_size, layout=layout)


def prefill_spec(batch: int | None = None, seed: int | None = None, fixed_1023: bool = False,
                 q_lens=None, kv_lens=None, hq: int = 48, hkv: int = 8, head_dim: int = 256,
                 dtype: str = "bf16", layout: str = "HND", max_q: int = 4096,
                 max_extra: int = 4096, page_size: int = PAGE_SIZE, contiguous: bool = False) -> PrefillSpec:
    """Lengths, pool and block table of one causal prefill workload."""
    if fixed_1023:
        seed = 599 if seed is None else seed
        q = np.array([1023], dtype=np.int32)
        kv = np.array([1023], dtype=np.int32)
        name = f"prefill_d{head_dim}_b1_q1023"
    elif q_lens is not None:
        seed = 0 if seed is None else seed
        q = np.asarray(q_lens, dtype=np.int32)
        kv = np.asarray(kv_lens, dtype=np.int32)
        name = "prefill_custom"
    else:
        if batch is None:
            raise ValueError("prefill_spec needs a batch size")
        seed = 500 + batch if seed is None else seed
        rng0 = np.random.default_rng(seed)
        q = rng0.integers(65, max_q, size=batch, endpoint=True).astype(np.int32)
        kv = (q + rng0.integers(0, max_extra, size=batch, endpoint=True)).astype(np.int32)
        name = f"prefill_d{head_dim}_b{batch}"
    rng = np.random.default_rng(seed + 1_000_003)
    pages = np.array([_ceil_div(int(k), page_size) for k in kv], dtype=np.int64)
    bt_cols = max(1, int(pages.max()) if pages.size else 1)
    bt, num_pages = deal_pages(pages, max(1, int(pages.sum())), bt_cols, rng, contiguous)
    return PrefillSpec(name, q, kv, num_pages, bt_cols, bt, seed, hq, hkv, head_dim, dtype,
                       page_size=page_size, layout=layout)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def _indptr(lengths: np.ndarray) -> np.ndarray:
    out = np.zeros(lengths.shape[0] + 1, dtype=np.int32)
    np.cumsum(lengths, out=out[1:])
    return out


def _normal(shape, dtype, gen: torch.Generator, device) -> torch.Tensor:
    # N(0,1) drawn in fp32 then rounded to the storage type (round to nearest even)
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(dtype)


def pool_shape(spec) -> tuple[int, int, int, int]:
    if spec.layout == "HND":
        return (spec.num_pages, spec.hkv, spec.page_size, spec.head_dim)
    if spec.layout == "NHD":
        return (spec.num_pages, spec.page_size, spec.hkv, spec.head_dim)
    raise ValueError(spec.layout)


def empty_pool(spec, device="cpu", fill=float("nan")) -> torch.Tensor:
    """A pool tensor in the spec's layout with every element set to ``fill``."""
    return torch.full(pool_shape(spec), fill, dtype=spec.torch_dtype, device=device)


@dataclass
class DecodeInputs:
    spec: DecodeSpec
    q: torch.Tensor            # [B, Hq, D]
    k_hist: torch.Tensor       # [sum hist, Hkv, D]
    v_hist: torch.Tensor
    hist_indptr: torch.Tensor  # int32 [B+1]
    k_new: torch.Tensor        # [B * n_new, Hkv, D]
    v_new: torch.Tensor
    block_table: torch.Tensor  # int32 [B, bt_cols]
    hist_lens: torch.Tensor    # int32 [B]
    new_indptr: torch.Tensor | None = field(default=None)

    def to(self, device) -> "DecodeInputs":
        mv = lambda t: None if t is None else t.to(device)
        return DecodeInputs(self.spec, mv(self.q), mv(self.k_hist), mv(self.v_hist),
                            mv(self.hist_indptr), mv(self.k_new), mv(self.v_new),
                            mv(self.block_table), mv(self.hist_lens), mv(self.new_indptr))


def decode_inputs(spec: DecodeSpec, device="cpu", seed_offset: int = 0) -> DecodeInputs:
    """Seeded tensors of a decode workload, drawn on ``device``.

    On the CPU the draws are reproducible everywhere; on a GPU they are
    reproducible for the same device type and torch version."""
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed * 1_000_003 + seed_offset)
    dt = spec.torch_dtype
    B, Hq, Hkv, D = spec.batch, spec.hq, spec.hkv, spec.head_dim
    n_hist = int(spec.hist_lens.sum())
    q = _normal((B, Hq, D), dt, gen, device)
    k_new = _normal((B * spec.n_new, Hkv, D), dt, gen, device)
    v_new = _normal((B * spec.n_new, Hkv, D), dt, gen, device)
    k_hist = _normal((n_hist, Hkv, D), dt, gen, device)
    v_hist = _normal((n_hist, Hkv, D), dt, gen, device)
    hist_indptr = torch.from_numpy(_indptr(spec.hist_lens)).to(device)
    bt = torch.from_numpy(spec.block_table.copy()).to(device)
    hl = torch.from_numpy(spec.hist_lens.copy()).to(device)
    new_indptr = None
    if spec.n_new != 1:
        new_indptr = torch.from_numpy(
            _indptr(np.full(B, spec.n_new, dtype=np.int32))).to(device)
    return DecodeInputs(spec, q, k_hist, v_hist, hist_indptr, k_new, v_new, bt, hl, new_indptr)


@dataclass
class PrefillInputs:
    spec: PrefillSpec
    q: torch.Tensor            # [sum q_len, Hq, D]
    k_hist: torch.Tensor       # [sum (kv_len - q_len), Hkv, D]
    v_hist: torch.Tensor
    hist_indptr: torch.Tensor  # int32 [B+1]
    k_new: torch.Tensor        # [sum q_len, Hkv, D]: the chunk's own K/V
    v_new: torch.Tensor
    qo_indptr: torch.Tensor    # int32 [B+1]
    block_table: torch.Tensor
    hist_lens: torch.Tensor    # int32 [B]

    def to(self, device) -> "PrefillInputs":
        mv = lambda t: t.to(device)
        return PrefillInputs(self.spec, mv(self.q), mv(self.k_hist), mv(self.v_hist),
                             mv(self.hist_indptr), mv(self.k_new), mv(self.v_new),
                             mv(self.qo_indptr), mv(self.block_table), mv(self.hist_lens))


def prefill_inputs(spec: PrefillSpec, device="cpu", seed_offset: int = 0) -> PrefillInputs:
    """Seeded tensors of a prefill workload; seed_offset draws another layer's."""
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed * 1_000_003 + 7 + 1_009 * seed_offset)
    dt = spec.torch_dtype
    Hq, Hkv, D = spec.hq, spec.hkv, spec.head_dim
    total_q = int(spec.q_lens.sum())
    n_hist = int(spec.hist_lens.sum())
    q = _normal((total_q, Hq, D), dt, gen, device)
    k_new = _normal((total_q, Hkv, D), dt, gen, device)
    v_new = _normal((total_q, Hkv, D), dt, gen, device)
    k_hist = _normal((n_hist, Hkv, D), dt, gen, device)
    v_hist = _normal((n_hist, Hkv, D), dt, gen, device)
    return PrefillInputs(
        spec, q, k_hist, v_hist,
        torch.from_numpy(_indptr(spec.hist_lens)).to(device), k_new, v_new,
        torch.from_numpy(_indptr(spec.q_lens)).to(device),
        torch.from_numpy(spec.block_table.copy()).to(device),
        torch.from_numpy(spec.hist_lens.copy()).to(device))


def rope_tables(rows: int, head_dim: int, base: float = 1_000_000.0):
    """Rotary cos/sin tables as a model hands them to the attention call:
    float32 [rows, head_dim/2], entry (p, i) = cos / sin of p * base^(-2i/D)
    (angles and their cosines in fp64, rounded to fp32).  The default base
    is Qwen3's rope_theta."""
    half = head_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)), torch.from_numpy(np.sin(ang).astype(np.float32)))


def mixed_spec(num_decode: int = 64, num_chunks: int = 4, seed: int = 700, hq: int = 32, hkv: int = 8,
               head_dim: int = 128, max_chunk: int = 2048, max_extra: int = 4096) -> PrefillSpec:
    """One serving step of the Qwen3-4B attention shape with chunked prefill
    next to decode: `num_chunks` prompt chunks first (q_len U{65..max_chunk},
    kv_len = q_len + U{0..max_extra}: a chunk continues a prompt), then
    `num_decode` decode rows (one new token each over a history of
    U{512..1024} tokens, the decode workload's lengths).  A ragged prefill
    workload whose last requests have q_len 1."""
    rng = np.random.default_rng(seed)
    q = rng.integers(65, max_chunk, size=num_chunks, endpoint=True)
    kv = q + rng.integers(0, max_extra, size=num_chunks, endpoint=True)
    dec = rng.integers(512, 1024, size=num_decode, endpoint=True) + 1
    spec = prefill_spec(q_lens=np.concatenate([q, np.ones(num_decode, np.int64)]),
                        kv_lens=np.concatenate([kv, dec]), hq=hq, hkv=hkv, head_dim=head_dim, seed=seed)
    spec.name = f"mixed_c{num_chunks}_d{num_decode}"
    return spec
