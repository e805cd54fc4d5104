"""CPU fp64 oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and it shares no code
with them.

The arithmetic lives in ``pkv_oracle.c`` (plain C, fp64, a page-by-page walk
of ``block_table`` with a two-pass softmax).  This module only marshals numpy
arrays (or CPU torch tensors) into it with ctypes and builds the shared object
with gcc when it is missing or older than its sources.

bf16 data is handed over as its raw 16-bit patterns (numpy ``uint16`` /
``int16`` or a torch ``bfloat16`` tensor); the C side widens it exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SOURCES = ("pkv_oracle.c", "pkv_oracle.h")
DEFAULT_LIB = os.path.join(_HERE, "libpkvref.so")

F32, BF16 = 0, 1
_ERRORS = {
    1: "bad argument",
    2: "block maps outside 1..num_pages-1",
    3: "block table has too few columns",
    4: "bad length (negative, or q_len > kv_len when causal)",
    5: "indptr inconsistent",
    6: "host allocation failed",
}


class OracleError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"oracle {where}: {_ERRORS.get(code, 'error')} (code {code})")
        self.code = code


class _CPool(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("s_page", ctypes.c_int64),
        ("s_head", ctypes.c_int64),
        ("s_tok", ctypes.c_int64),
    ]


@dataclass(frozen=True)
class Pool:
    """Geometry of one K (or V) page pool: element strides, dim stride 1."""

    dtype: int
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    s_page: int
    s_head: int
    s_tok: int

    @staticmethod
    def hnd(dtype: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int) -> "Pool":
        """Pool stored as [num_pages, num_kv_heads, page_size, head_dim]."""
        return Pool(dtype, num_pages, page_size, num_kv_heads, head_dim,
                    num_kv_heads * page_size * head_dim, page_size * head_dim, head_dim)

    @staticmethod
    def nhd(dtype: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int) -> "Pool":
        """Pool stored as [num_pages, page_size, num_kv_heads, head_dim]."""
        return Pool(dtype, num_pages, page_size, num_kv_heads, head_dim,
                    num_kv_heads * page_size * head_dim, head_dim, num_kv_heads * head_dim)

    def _c(self) -> _CPool:
        return _CPool(self.dtype, self.num_pages, self.page_size, self.num_kv_heads,
                      self.head_dim, self.s_page, self.s_head, self.s_tok)


def _stale(lib_path: str, src_dir: str) -> bool:
    if not os.path.exists(lib_path):
        return True
    t = os.path.getmtime(lib_path)
    return any(os.path.getmtime(os.path.join(src_dir, s)) > t for s in _SOURCES)


def build(src: str | None = None, out: str | None = None) -> str:
    """Compile ``src`` (default: this directory's pkv_oracle.c) into ``out``."""
    src = src or os.path.join(_HERE, "pkv_oracle.c")
    out = out or DEFAULT_LIB
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _to_np(x, want=None):
    """numpy view of ``x`` (numpy array or CPU torch tensor); bf16 -> uint16 bits."""
    if x is None:
        return None
    if not isinstance(x, np.ndarray):
        import torch  # plumbing only

        t = x.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            x = t.view(torch.int16).numpy().view(np.uint16)
        else:
            x = t.numpy()
    if want is not None:
        x = np.ascontiguousarray(x, dtype=want)
    elif not x.flags.c_contiguous:
        raise ValueError("oracle inputs must be contiguous")
    return x


def _check_elem(x: np.ndarray, dtype: int, what: str) -> None:
    ok = x.dtype.itemsize == 2 if dtype == BF16 else x.dtype == np.float32
    if not ok:
        raise TypeError(f"{what}: element type {x.dtype} does not match the pool dtype")


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        P, I32P, I64P, DP = ctypes.POINTER(_CPool), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        V, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.pkvref_route.argtypes = [P, I32P, I, I32P, I, I, I64P]
        lib.pkvref_append.argtypes = [P, V, V, V, V, I32P, I, I32P, I32P, I, I, I32P]
        lib.pkvref_decode.argtypes = [P, DP, DP, V, I, V, V, I32P, I, I32P, I, D, I]
        lib.pkvref_prefill.argtypes = [P, DP, DP, V, I, V, V, I32P, I, I32P, I32P, I, I, D, I64P, I]
        L = ctypes.c_int64
        lib.pkvref_rope.argtypes = [I, V, L, I, I, I32P, V, V, L, I]
        for f in (lib.pkvref_route, lib.pkvref_append, lib.pkvref_decode, lib.pkvref_prefill, lib.pkvref_rope):
            f.restype = ctypes.c_int
        self._lib = lib

    # -- routing ---------------------------------------------------------
    def route(self, pool: Pool, block_table, seqlens, max_len: int) -> np.ndarray:
        bt = _to_np(block_table, np.int32)
        sl = _to_np(seqlens, np.int32)
        batch = sl.shape[0]
        out = np.empty((batch, max_len), dtype=np.int64)
        cp = pool._c()
        rc = self._lib.pkvref_route(ctypes.byref(cp), _ptr(bt), bt.shape[1] if bt.ndim == 2 else 0,
                                    _ptr(sl), batch, max_len, _ptr(out))
        if rc:
            raise OracleError(rc, "route")
        return out

    # -- append ----------------------------------------------------------
    def append(self, pool: Pool, k_cache: np.ndarray, v_cache: np.ndarray, k_new, v_new,
               block_table, cache_seqlens, new_indptr=None) -> np.ndarray:
        """Writes k_new/v_new into k_cache/v_cache (numpy, modified in place).

        Returns the new lengths cache_seqlens + tokens appended per sequence."""
        for c in (k_cache, v_cache):
            if not isinstance(c, np.ndarray) or not c.flags.c_contiguous or not c.flags.writeable:
                raise ValueError("caches must be writeable contiguous numpy arrays")
            _check_elem(c, pool.dtype, "cache")
        kn, vn = _to_np(k_new), _to_np(v_new)
        _check_elem(kn, pool.dtype, "k_new")
        _check_elem(vn, pool.dtype, "v_new")
        bt = _to_np(block_table, np.int32)
        cs = _to_np(cache_seqlens, np.int32)
        ip = _to_np(new_indptr, np.int32)
        batch = cs.shape[0]
        total_new = kn.shape[0]
        out = np.empty(batch, dtype=np.int32)
        cp = pool._c()
        rc = self._lib.pkvref_append(ctypes.byref(cp), _ptr(k_cache), _ptr(v_cache), _ptr(kn),
                                     _ptr(vn), _ptr(bt), bt.shape[1], _ptr(cs), _ptr(ip), batch,
                                     total_new, _ptr(out))
        if rc:
            raise OracleError(rc, "append")
        return out

    # -- rotary position embedding --------------------------------------
    def rope(self, dtype: int, x: np.ndarray, positions, cos_table, sin_table, interleaved: bool) -> None:
        """Rotates x [rows, heads, head_dim] (numpy; bf16 as uint16 bits or
        fp32) in place, row r by position positions[r], with fp32 tables
        [table_rows, head_dim/2]."""
        if not isinstance(x, np.ndarray) or not x.flags.c_contiguous or not x.flags.writeable or x.ndim != 3:
            raise ValueError("x must be a writeable contiguous 3-D numpy array")
        _check_elem(x, dtype, "x")
        pos = _to_np(positions, np.int32)
        c = _to_np(cos_table, np.float32)
        s = _to_np(sin_table, np.float32)
        rows, heads, d = x.shape
        if pos.shape != (rows,) or c.shape != s.shape or c.ndim != 2 or c.shape[1] * 2 != d:
            raise ValueError("positions must be [rows] and the tables [table_rows, head_dim/2]")
        rc = self._lib.pkvref_rope(int(dtype), _ptr(x), rows, heads, d, _ptr(pos), _ptr(c), _ptr(s), c.shape[0],
                                   int(bool(interleaved)))
        if rc:
            raise OracleError(rc, "rope")

    # -- attention -------------------------------------------------------
    def decode(self, pool: Pool, q, k_cache, v_cache, block_table, seqlens, scale: float,
               nthreads: int = 1):
        qn = _to_np(q)
        _check_elem(qn, pool.dtype, "q")
        batch, hq, d = qn.shape
        bt = _to_np(block_table, np.int32)
        sl = _to_np(seqlens, np.int32)
        out = np.empty((batch, hq, d), dtype=np.float64)
        lse = np.empty((batch, hq), dtype=np.float64)
        cp = pool._c()
        rc = self._lib.pkvref_decode(ctypes.byref(cp), _ptr(out), _ptr(lse), _ptr(qn), hq,
                                     _ptr(_to_np(k_cache)), _ptr(_to_np(v_cache)), _ptr(bt),
                                     bt.shape[1], _ptr(sl), batch, float(scale), int(nthreads))
        if rc:
            raise OracleError(rc, "decode")
        return out, lse

    def prefill(self, pool: Pool, q, k_cache, v_cache, block_table, kv_lens, qo_indptr,
                scale: float, causal: bool = True, nthreads: int = 1, pair_counts: bool = False):
        qn = _to_np(q)
        _check_elem(qn, pool.dtype, "q")
        total_q, hq, d = qn.shape
        bt = _to_np(block_table, np.int32)
        kl = _to_np(kv_lens, np.int32)
        ip = _to_np(qo_indptr, np.int32)
        batch = kl.shape[0]
        if ip.shape[0] != batch + 1 or int(ip[-1]) != total_q:
            raise OracleError(5, "prefill")
        out = np.empty((total_q, hq, d), dtype=np.float64)
        lse = np.empty((total_q, hq), dtype=np.float64)
        pc = np.zeros((batch, hq), dtype=np.int64) if pair_counts else None
        cp = pool._c()
        rc = self._lib.pkvref_prefill(ctypes.byref(cp), _ptr(out), _ptr(lse), _ptr(qn), hq,
                                      _ptr(_to_np(k_cache)), _ptr(_to_np(v_cache)), _ptr(bt),
                                      bt.shape[1], _ptr(kl), _ptr(ip), batch, int(bool(causal)),
                                      float(scale), _ptr(pc), int(nthreads))
        if rc:
            raise OracleError(rc, "prefill")
        return (out, lse, pc) if pair_counts else (out, lse)


_default: Oracle | None = None
_lock = threading.Lock()


def load(lib_path: str | None = None) -> Oracle:
    """The oracle built from this directory (rebuilt if stale), or ``lib_path``."""
    global _default
    if lib_path is not None:
        return Oracle(lib_path)
    with _lock:
        if _default is None:
            if _stale(DEFAULT_LIB, _HERE):
                build()
            _default = Oracle(DEFAULT_LIB)
        return _default
