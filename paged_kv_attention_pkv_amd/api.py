"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
shapes and dtypes against each other, and passes raw device pointers, sizes
and the current HIP stream to the C entry point of the same name.  All work
happens in the library's HIP kernels; nothing here computes attention and
there is no fallback: a missing library, or a non-OK status from the library,
raises.

Pool tensors are 4-D: ``layout="HND"`` is [num_pages, num_kv_heads,
page_size, head_dim] and ``layout="NHD"`` is [num_pages, page_size,
num_kv_heads, head_dim]; any strides with a unit dim stride are accepted and
K and V must share them.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build (python -m paged_kv_attention_pkv_amd.build).
_LIB_PATH = os.path.join(_HERE, "libpkv.so")
# PKV_ABI_VERSION of include/pkv.h that these bindings are written against.
ABI_VERSION = 3

PKV_F32, PKV_BF16 = 0, 1
_STATUS = {
    0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace missing or too small",
    4: "kernel launch failed", 5: "no usable HIP device", 6: "device-data precondition violated",
}


class PkvError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str = ""):
        text = _STATUS.get(code, f"status {code}")
        super().__init__(f"{fn}: {text}" + (f" ({detail})" if detail else ""))
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("s_page", ctypes.c_int64),
        ("s_head", ctypes.c_int64),
        ("s_tok", ctypes.c_int64),
    ]


_lib = None
_lock = threading.Lock()

_VP, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_DP = ctypes.POINTER(_Desc)
_SIGS = {
    "pkv_abi_version": ([], ctypes.c_int32),
    "pkv_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "pkv_append": ([_DP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _VP, _VP], ctypes.c_int),
    "pkv_append_rope": ([_DP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _VP, _I32, _VP, _VP, _I32, _I32,
                         _VP, _VP], ctypes.c_int),
    "pkv_decode_workspace_bytes": ([_DP, _I32, _I32, _I32], _SZ),
    "pkv_decode_workspace_bytes_ex": ([_DP, _I32, _I32, _I32, _I32], _SZ),
    "pkv_decode_workspace_reset": ([_DP, _I32, _VP, _SZ, _VP], ctypes.c_int),
    "pkv_decode_plan": ([_DP, _I32, _VP, _I32, _I32, _I32, _VP, _SZ, _I32, _VP], ctypes.c_int),
    "pkv_decode_attn": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP, _I32, _I32, ctypes.c_float,
                         _VP, _SZ, _VP], ctypes.c_int),
    "pkv_decode_attn_ex": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP, _I32, _I32, ctypes.c_float,
                            _VP, _SZ, _I32, _VP], ctypes.c_int),
    "pkv_append_decode_attn": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32,
                                ctypes.c_float, _VP, _SZ, _VP], ctypes.c_int),
    "pkv_append_decode_attn_ex": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32,
                                   ctypes.c_float, _VP, _SZ, _I32, _VP], ctypes.c_int),
    "pkv_append_decode_attn_noalloc": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32,
                                        _I32, ctypes.c_float, _VP], ctypes.c_int),
    "pkv_prefill_workspace_bytes": ([_DP, _I32, _I32, _I32, _I32, _I32], _SZ),
    "pkv_prefill_attn": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32,
                          _I32, ctypes.c_float, _VP, _SZ, _VP], ctypes.c_int),
    "pkv_prefill_attn_ex": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32,
                             _I32, ctypes.c_float, _VP, _SZ, _I32, _VP], ctypes.c_int),
    "pkv_mixed_workspace_bytes": ([_DP, _I32, _I32, _I32], _SZ),
    "pkv_mixed_attn": ([_DP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                        ctypes.c_float, _VP, _SZ, _VP], ctypes.c_int),
    "pkv_route": ([_DP, _VP, _I32, _VP, _I32, _I32, _VP, _VP], ctypes.c_int),
    "pkv_validate_host": ([_DP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32, ctypes.c_char_p, _SZ],
                          ctypes.c_int),
    "pkv_validate_append_host": ([_DP, _VP, _I32, _VP, _VP, _I32, _I32, ctypes.c_char_p, _SZ], ctypes.c_int),
    "pkv_validate_decode_step_host": ([_DP, _VP, _I32, _VP, _I32, _I32, ctypes.c_char_p, _SZ], ctypes.c_int),
}
EXPORTED = tuple(_SIGS)


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libpkv (ctypes.CDLL); raises if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise RuntimeError(
                        f"libpkv.so not found at {_LIB_PATH}: build it with "
                        "`python -m paged_kv_attention_pkv_amd.build` (hipcc, gfx950)")
                handle = ctypes.CDLL(_LIB_PATH)
                for name, (args, res) in _SIGS.items():
                    f = getattr(handle, name)
                    f.argtypes = args
                    f.restype = res
                got = handle.pkv_abi_version()
                if got != ABI_VERSION:
                    raise RuntimeError(f"{_LIB_PATH} has ABI version {got}; these bindings need {ABI_VERSION}")
                _lib = handle
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return PKV_BF16
    if dt == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {dt}; libpkv takes bfloat16 or float32")


def cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor | None = None, layout: str = "HND") -> _Desc:
    """pkv_cache_desc of a 4-D pool tensor in the given layout."""
    if k_cache.dim() != 4:
        raise ValueError("pool tensors are 4-D")
    if k_cache.stride(3) != 1:
        raise ValueError("pool dim stride must be 1")
    if v_cache is not None and (v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride()
                                or v_cache.dtype != k_cache.dtype):
        raise ValueError("K and V pools must have the same shape, strides and dtype")
    n, a, b, d = k_cache.shape
    s = k_cache.stride()
    if layout == "HND":
        hkv, page, s_head, s_tok = a, b, s[1], s[2]
    elif layout == "NHD":
        page, hkv, s_tok, s_head = a, b, s[1], s[2]
    else:
        raise ValueError(f"layout must be 'HND' or 'NHD', not {layout!r}")
    return _Desc(_dtype_code(k_cache.dtype), n, page, hkv, d, 0, s[0], s_head, s_tok)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn: str, rc: int, detail: str = "") -> None:
    if rc != 0:
        raise PkvError(fn, rc, detail)


def _need(t: torch.Tensor, name: str, dtype=None, dev=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scale(scale) -> None:
    """The softmax scale is the caller's (1/sqrt(head_dim) in the usual
    attention); the binding does no arithmetic of the method."""
    if scale is None:
        raise TypeError("scale must be given (a float)")


def _shape(t: torch.Tensor | None, name: str, shape) -> None:
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _decode_operands(desc: _Desc, q, out, lse, block_table, cache_seqlens, k_new=None, v_new=None,
                     seqlens_out=None) -> None:
    """Shapes of a decode call's tensors against q [B, Hq, D] and the pool
    (the library sees only pointers, so a wrong shape would be read or
    written past its end)."""
    dev = q.device
    batch, hq, d = q.shape
    if d != desc.head_dim:
        raise ValueError(f"q head_dim {d} differs from the pool's {desc.head_dim}")
    _shape(out, "out", q.shape)
    _shape(cache_seqlens, "cache_seqlens", (batch,))
    if block_table.shape[0] != batch:
        raise ValueError("block_table rows must equal batch")
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
        _shape(lse, "lse", (batch, hq))
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _shape(t, nm, (batch, desc.num_kv_heads, d))
    if seqlens_out is not None:
        _need(seqlens_out, "seqlens_out", torch.int32, dev, 1)
        _shape(seqlens_out, "seqlens_out", (batch,))


def _prefill_operands(desc: _Desc, q, out, lse, block_table, kv_lens, qo_indptr) -> None:
    """Shapes of a prefill call's tensors against q [total_q, Hq, D] and the pool."""
    dev = q.device
    total_q, hq, d = q.shape
    if d != desc.head_dim:
        raise ValueError(f"q head_dim {d} differs from the pool's {desc.head_dim}")
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(kv_lens, "kv_lens", torch.int32, dev, 1)
    _need(qo_indptr, "qo_indptr", torch.int32, dev, 1)
    batch = kv_lens.shape[0]
    if qo_indptr.shape[0] != batch + 1 or block_table.shape[0] != batch:
        raise ValueError("batch mismatch between qo_indptr, block_table and kv_lens")
    _shape(out, "out", q.shape)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
        _shape(lse, "lse", (total_q, hq))


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def append(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, new_indptr=None,
           seqlens_out=None, layout: str = "HND"):
    """pkv_append: write k_new/v_new [total_new, Hkv, D] at each sequence's
    cached length.  Returns seqlens_out (allocated when not given)."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
        _shape(t, nm, (k_new.shape[0], desc.num_kv_heads, desc.head_dim))
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch = cache_seqlens.shape[0]
    if new_indptr is not None:
        _need(new_indptr, "new_indptr", torch.int32, dev, 1)
        if new_indptr.shape[0] != batch + 1:
            raise ValueError("new_indptr must have batch+1 entries")
    if block_table.shape[0] != batch:
        raise ValueError("block_table rows must equal batch")
    if seqlens_out is None:
        seqlens_out = torch.empty_like(cache_seqlens)
    rc = lib().pkv_append(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                          _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(new_indptr),
                          batch, k_new.shape[0], _ptr(seqlens_out), _stream(k_cache))
    _check("pkv_append", rc)
    return seqlens_out


def append_rope(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, rope_cos, rope_sin,
                interleaved: bool = False, q=None, new_indptr=None, seqlens_out=None, layout: str = "HND"):
    """pkv_append_rope: pkv_append with the new tokens' k rotated before it is
    stored and q [total_new, Hq, D] (optional) rotated in place, by the
    rotary tables rope_cos / rope_sin (float32 [rows, D/2]) at positions
    cache_seqlens[b] + t.  Returns seqlens_out (allocated when not given)."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
        _shape(t, nm, (k_new.shape[0], desc.num_kv_heads, desc.head_dim))
    for t, nm in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, nm, torch.float32, dev, 2)
        _shape(t, nm, (rope_cos.shape[0], desc.head_dim // 2))
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch = cache_seqlens.shape[0]
    hq = 0
    if q is not None:
        _need(q, "q", k_cache.dtype, dev, 3)
        hq = q.shape[1]
        _shape(q, "q", (k_new.shape[0], hq, desc.head_dim))
    if new_indptr is not None:
        _need(new_indptr, "new_indptr", torch.int32, dev, 1)
        _shape(new_indptr, "new_indptr", (batch + 1,))
    if block_table.shape[0] != batch:
        raise ValueError("block_table rows must equal batch")
    if seqlens_out is None:
        seqlens_out = torch.empty_like(cache_seqlens)
    rc = lib().pkv_append_rope(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(q),
                               hq, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], int(bool(interleaved)),
                               _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(new_indptr), batch,
                               k_new.shape[0], _ptr(seqlens_out), _stream(k_cache))
    _check("pkv_append_rope", rc)
    return seqlens_out


def decode_workspace_bytes(k_cache, batch: int, num_q_heads: int, max_kv_len: int, layout: str = "HND",
                           workers: int = 0) -> int:
    desc = cache_desc(k_cache, None, layout)
    with torch.cuda.device(k_cache.device):
        n = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, num_q_heads, max_kv_len, workers)
    if n == 0:
        raise PkvError("pkv_decode_workspace_bytes", 1, "invalid sizes")
    return int(n)


def decode_workspace_reset(k_cache, batch: int, workspace, layout: str = "HND") -> None:
    """pkv_decode_workspace_reset: enqueue a zero fill of the workspace's
    arrival counters for `batch` rows on the current stream."""
    desc = cache_desc(k_cache, None, layout)
    rc = lib().pkv_decode_workspace_reset(ctypes.byref(desc), int(batch), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(workspace))
    _check("pkv_decode_workspace_reset", rc)


def _decode_plan_args(k_cache, cache_seqlens, num_q_heads: int, max_kv_len: int, workspace, fused: bool,
                      layout: str, workers: int):
    desc = cache_desc(k_cache, None, layout)
    dev = k_cache.device
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    _need(workspace, "workspace", None, dev)
    batch = cache_seqlens.shape[0]
    with torch.cuda.device(dev):
        need = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, int(num_q_heads), int(max_kv_len),
                                                   int(workers))
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise PkvError("pkv_decode_plan", 3, f"workspace {nbytes} < {need} bytes")
    args = (ctypes.byref(desc), int(num_q_heads), _ptr(cache_seqlens), batch, int(max_kv_len), int(bool(fused)),
            _ptr(workspace), nbytes, int(workers))
    return args, (k_cache, cache_seqlens, workspace, desc)


def decode_plan(k_cache, cache_seqlens, num_q_heads: int, max_kv_len: int, workspace, fused: bool,
                layout: str = "HND", workers: int = 0) -> None:
    """pkv_decode_plan: enqueue, on the current stream, the cut of the
    decode calls of one step (same lengths, shape, max_kv_len, workers and
    mode) into the workspace's plan region.  Later calls with this workspace
    use it where it matches them and give the same bits either way."""
    args, keep = _decode_plan_args(k_cache, cache_seqlens, num_q_heads, max_kv_len, workspace, fused, layout,
                                   workers)
    with torch.cuda.device(k_cache.device):
        rc = lib().pkv_decode_plan(*args, _stream(workspace))
    _check("pkv_decode_plan", rc)


def decode_attn(q, k_cache, v_cache, block_table, cache_seqlens, max_kv_len: int, scale: float,
                out=None, lse=None, workspace=None, layout: str = "HND", workers: int = 0,
                return_lse: bool = False):
    """pkv_decode_attn: q [B, Hq, D] against the first cache_seqlens[b] keys
    of each row.  Returns out (and lse when return_lse or lse is given)."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch, hq, d = q.shape
    if cache_seqlens.shape[0] != batch or block_table.shape[0] != batch:
        raise ValueError("batch mismatch between q, block_table and cache_seqlens")
    _scale(scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev, 3)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    _decode_operands(desc, q, out, lse, block_table, cache_seqlens)
    with torch.cuda.device(dev):
        need = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, hq, max_kv_len, workers)
        if workspace is None:
            # the arrival counters in the workspace must start at zero
            workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        rc = lib().pkv_decode_attn_ex(ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache),
                                      _ptr(v_cache), _ptr(block_table), block_table.shape[1],
                                      _ptr(cache_seqlens), batch, int(max_kv_len), float(scale),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      int(workers), _stream(k_cache))
    _check("pkv_decode_attn", rc)
    return (out, lse) if lse is not None else out


def append_decode_attn(q, k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, max_kv_len: int,
                       scale: float, out=None, lse=None, seqlens_out=None, workspace=None,
                       layout: str = "HND", workers: int = 0, return_lse: bool = False):
    """pkv_append_decode_attn: append k_new/v_new [B, Hkv, D] at each row's
    pre-append length cache_seqlens[b], then attend q [B, Hq, D] over the
    cache_seqlens[b] + 1 keys, in one launch.  Returns (out, seqlens_out) or
    (out, lse, seqlens_out) when return_lse or lse is given."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch, hq, d = q.shape
    if cache_seqlens.shape[0] != batch or block_table.shape[0] != batch or k_new.shape[0] != batch:
        raise ValueError("batch mismatch between q, k_new, block_table and cache_seqlens")
    _scale(scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev, 3)
    if seqlens_out is None:
        seqlens_out = torch.empty_like(cache_seqlens)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    _decode_operands(desc, q, out, lse, block_table, cache_seqlens, k_new, v_new, seqlens_out)
    with torch.cuda.device(dev):
        need = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, hq, max_kv_len, workers)
        if workspace is None:
            workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        rc = lib().pkv_append_decode_attn_ex(
            ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache), _ptr(k_new),
            _ptr(v_new), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(seqlens_out), batch,
            int(max_kv_len), float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
            int(workers), _stream(k_cache))
    _check("pkv_append_decode_attn", rc)
    return (out, lse, seqlens_out) if lse is not None else (out, seqlens_out)


def append_decode_attn_noalloc(q, k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, max_kv_len: int,
                               scale: float, out=None, lse=None, seqlens_out=None, layout: str = "HND",
                               return_lse: bool = False):
    """pkv_append_decode_attn_noalloc: the fused decode step on the library's
    fixed device workspace (no workspace argument; the library allocates
    nothing).  Output tensors are allocated here only when not given."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch, hq, d = q.shape
    if cache_seqlens.shape[0] != batch or block_table.shape[0] != batch or k_new.shape[0] != batch:
        raise ValueError("batch mismatch between q, k_new, block_table and cache_seqlens")
    _scale(scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev, 3)
    if seqlens_out is None:
        seqlens_out = torch.empty_like(cache_seqlens)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    _decode_operands(desc, q, out, lse, block_table, cache_seqlens, k_new, v_new, seqlens_out)
    with torch.cuda.device(dev):
        rc = lib().pkv_append_decode_attn_noalloc(
            ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache), _ptr(k_new),
            _ptr(v_new), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(seqlens_out), batch,
            int(max_kv_len), float(scale), _stream(k_cache))
    _check("pkv_append_decode_attn_noalloc", rc)
    return (out, lse, seqlens_out) if lse is not None else (out, seqlens_out)


def prefill_workspace_bytes(k_cache, batch, num_q_heads, total_q, max_q, max_kv_len, layout="HND") -> int:
    desc = cache_desc(k_cache, None, layout)
    with torch.cuda.device(k_cache.device):  # the size depends on the device's CU count
        return int(lib().pkv_prefill_workspace_bytes(ctypes.byref(desc), batch, num_q_heads, total_q, max_q,
                                                     max_kv_len))


def prefill_attn(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, max_q: int, max_kv_len: int,
                 scale: float, causal: bool = True, out=None, lse=None, workspace=None,
                 layout: str = "HND", return_lse: bool = False, rows_per_workgroup: int = 0,
                 split: bool = True):
    """pkv_prefill_attn: ragged queries q [total_q, Hq, D] (offsets qo_indptr)
    against kv_lens[r] keys of each request, end-aligned causal mask.
    rows_per_workgroup != 0 calls pkv_prefill_attn_ex with that tiling.
    A call that may split its keys gets a zero-filled workspace of
    pkv_prefill_workspace_bytes (allocated here unless given); split=False
    passes none, so the keys are never split."""
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    total_q, hq, d = q.shape
    batch = kv_lens.shape[0]
    _scale(scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev, 3)
    if lse is None and return_lse:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=dev)
    _prefill_operands(desc, q, out, lse, block_table, kv_lens, qo_indptr)
    with torch.cuda.device(dev):
        need = 0
        if split and not rows_per_workgroup:
            need = lib().pkv_prefill_workspace_bytes(ctypes.byref(desc), batch, hq, total_q, max_q, max_kv_len)
        if not need:
            workspace = None
        elif workspace is None:
            workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
        args = (ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache),
                _ptr(block_table), block_table.shape[1], _ptr(kv_lens), _ptr(qo_indptr), batch, total_q,
                int(max_q), int(max_kv_len), int(bool(causal)), float(scale), _ptr(workspace),
                0 if workspace is None else workspace.numel() * workspace.element_size())
        if rows_per_workgroup:
            name = "pkv_prefill_attn_ex"
            rc = lib().pkv_prefill_attn_ex(*args, int(rows_per_workgroup), _stream(k_cache))
        else:
            name = "pkv_prefill_attn"
            rc = lib().pkv_prefill_attn(*args, _stream(k_cache))
    _check(name, rc)
    return (out, lse) if lse is not None else out


# max_kv_len above which pkv_mixed_attn runs its decode rows as a split
# decode launch (and needs its workspace); include/pkv.h states the same.
MIXED_PACKED_MAX_KV = 8192


def mixed_workspace_bytes(k_cache, batch: int, num_prefill: int, num_q_heads: int, layout: str = "HND") -> int:
    desc = cache_desc(k_cache, None, layout)
    with torch.cuda.device(k_cache.device):
        n = lib().pkv_mixed_workspace_bytes(ctypes.byref(desc), batch, num_prefill, num_q_heads)
    if n == 0:
        raise PkvError("pkv_mixed_workspace_bytes", 1, "invalid sizes")
    return int(n)


def _mixed_args(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, num_prefill, max_q, max_kv_len, scale, out,
                lse, workspace, layout):
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", q.dtype, dev, 3)
    _prefill_operands(desc, q, out, lse, block_table, kv_lens, qo_indptr)
    _scale(scale)
    total_q, hq, _ = q.shape
    batch = kv_lens.shape[0]
    if not 0 <= num_prefill <= batch or total_q < batch - num_prefill:
        raise ValueError("num_prefill must be in 0..batch and each decode row needs a query row")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return desc, (ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache),
                  _ptr(block_table), block_table.shape[1], _ptr(kv_lens), _ptr(qo_indptr), batch, int(num_prefill),
                  total_q, int(max_q), int(max_kv_len), float(scale), _ptr(workspace), nbytes)


def mixed_attn(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, num_prefill: int, max_q: int, max_kv_len: int,
               scale: float, out=None, lse=None, workspace=None, layout: str = "HND", return_lse: bool = False,
               split: bool = True):
    """pkv_mixed_attn: requests 0..num_prefill-1 are causal prefill chunks,
    the others decode rows (one query row each, the last query rows), in one
    launch (two for decode rows over more than 8192 keys or more than 2 x CUs
    of them per KV head).  A zeroed workspace of pkv_mixed_workspace_bytes is
    allocated here when none is given and the call uses one: in those two
    cases, or for chunks that split their keys (split=False passes none where
    it can).  Returns out (and lse when return_lse or lse is given)."""
    if out is None:
        out = torch.empty_like(q)
    total_q, hq, _ = q.shape
    batch = kv_lens.shape[0]
    if lse is None and return_lse:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        n_dec = batch - num_prefill
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        use = n_dec > 0 and (max_kv_len > MIXED_PACKED_MAX_KV or n_dec * k_cache.shape[1 if layout == "HND" else 2]
                             > 2 * cus)
        if split and not use and num_prefill > 0 and max_q > 0:
            use = prefill_workspace_bytes(k_cache, num_prefill, hq, total_q - (batch - num_prefill), max_q,
                                          max_kv_len, layout=layout) > 0
        if use:
            workspace = torch.zeros(mixed_workspace_bytes(k_cache, batch, num_prefill, hq, layout=layout),
                                    dtype=torch.uint8, device=q.device)
    _, args = _mixed_args(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, num_prefill, max_q, max_kv_len,
                          scale, out, lse, workspace, layout)
    with torch.cuda.device(q.device):
        rc = lib().pkv_mixed_attn(*args, _stream(k_cache))
    _check("pkv_mixed_attn", rc)
    return (out, lse) if lse is not None else out


def prepare_mixed(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, num_prefill: int, max_q: int,
                  max_kv_len: int, scale: float, out, workspace=None, lse=None, layout: str = "HND") -> "PreparedCall":
    desc, args = _mixed_args(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, num_prefill, max_q, max_kv_len,
                             scale, out, lse, workspace, layout)
    # a workspace is needed for decode rows over more than 8192 keys, and
    # optional otherwise (with one, the chunks may split their keys)
    if workspace is not None or (max_kv_len > MIXED_PACKED_MAX_KV and num_prefill < kv_lens.shape[0]):
        need = mixed_workspace_bytes(k_cache, kv_lens.shape[0], num_prefill, q.shape[1], layout=layout)
        have = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if have < need:
            raise PkvError("pkv_mixed_attn", 3, f"workspace {have} < {need} bytes")
    return PreparedCall("pkv_mixed_attn", args, (k_cache, v_cache, q, out, block_table, kv_lens, qo_indptr,
                                                 workspace, lse, desc))


def route(k_cache, block_table, seqlens, max_len: int, layout: str = "HND"):
    """pkv_route: int64 [B, max_len] element offsets of every logical token."""
    desc = cache_desc(k_cache, None, layout)
    dev = k_cache.device
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seqlens, "seqlens", torch.int32, dev, 1)
    batch = seqlens.shape[0]
    offsets = torch.empty((batch, max_len), dtype=torch.int64, device=dev)
    rc = lib().pkv_route(ctypes.byref(desc), _ptr(block_table), block_table.shape[1], _ptr(seqlens), batch,
                         max_len, _ptr(offsets), _stream(k_cache))
    _check("pkv_route", rc)
    return offsets


def validate_host(k_cache, block_table, kv_lens, qo_indptr=None, max_q: int = 0, max_kv_len: int | None = None,
                  causal: bool = True, layout: str = "HND") -> None:
    """pkv_validate_host on host copies of the metadata; raises PkvError
    naming the first violated precondition."""
    desc = cache_desc(k_cache, None, layout)
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    kl = kv_lens.detach().to("cpu", torch.int32).contiguous()
    ip = None if qo_indptr is None else qo_indptr.detach().to("cpu", torch.int32).contiguous()
    batch = kl.shape[0]
    total_q = int(ip[-1]) if ip is not None else 0
    if max_kv_len is None:
        max_kv_len = int(kl.max()) if batch else 0
    msg = ctypes.create_string_buffer(256)
    rc = lib().pkv_validate_host(ctypes.byref(desc), _ptr(bt), bt.shape[1], _ptr(kl), _ptr(ip), batch, total_q,
                                 int(max_q), int(max_kv_len), int(bool(causal)), msg, 256)
    _check("pkv_validate_host", rc, msg.value.decode())


def validate_append_host(k_cache, block_table, cache_seqlens, new_indptr=None, total_new: int | None = None,
                         layout: str = "HND") -> None:
    desc = cache_desc(k_cache, None, layout)
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    cs = cache_seqlens.detach().to("cpu", torch.int32).contiguous()
    ip = None if new_indptr is None else new_indptr.detach().to("cpu", torch.int32).contiguous()
    batch = cs.shape[0]
    if total_new is None:
        total_new = int(ip[-1]) if ip is not None else batch
    msg = ctypes.create_string_buffer(256)
    rc = lib().pkv_validate_append_host(ctypes.byref(desc), _ptr(bt), bt.shape[1], _ptr(cs), _ptr(ip), batch,
                                        int(total_new), msg, 256)
    _check("pkv_validate_append_host", rc, msg.value.decode())


def validate_decode_step_host(k_cache, block_table, cache_seqlens, max_kv_len: int, layout: str = "HND") -> None:
    """pkv_validate_decode_step_host: the preconditions of
    pkv_append_decode_attn on host copies; raises PkvError naming the first
    violated one."""
    desc = cache_desc(k_cache, None, layout)
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    cs = cache_seqlens.detach().to("cpu", torch.int32).contiguous()
    msg = ctypes.create_string_buffer(256)
    rc = lib().pkv_validate_decode_step_host(ctypes.byref(desc), _ptr(bt), bt.shape[1], _ptr(cs), cs.shape[0],
                                             int(max_kv_len), msg, 256)
    _check("pkv_validate_decode_step_host", rc, msg.value.decode())


# --------------------------------------------------------------------------
# prepared calls: validate once, then launch with stored ctypes arguments
# --------------------------------------------------------------------------

class PreparedCall:
    """A library entry point with every argument already marshalled.

    Calling it enqueues the kernels on the current torch stream (so it can be
    recorded into a HIP graph) and raises on a non-OK status.  The tensors it
    was prepared from must stay alive and keep their storage."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self._fn = getattr(lib(), name)
        self._name = name
        self._args = args
        self._keep = keep  # tensors whose storage the pointers refer to
        self._dev = keep[0].device

    def __call__(self) -> None:
        rc = self._fn(*self._args, ctypes.c_void_p(torch.cuda.current_stream(self._dev).cuda_stream))
        if rc != 0:
            raise PkvError(self._name, rc)


def prepare_append(k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, seqlens_out, new_indptr=None,
                   layout: str = "HND") -> PreparedCall:
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
        _shape(t, nm, (k_new.shape[0], desc.num_kv_heads, desc.head_dim))
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    _need(seqlens_out, "seqlens_out", torch.int32, dev, 1)
    batch = cache_seqlens.shape[0]
    _shape(seqlens_out, "seqlens_out", (batch,))
    if block_table.shape[0] != batch:
        raise ValueError("block_table rows must equal batch")
    if new_indptr is not None:
        _need(new_indptr, "new_indptr", torch.int32, dev, 1)
        _shape(new_indptr, "new_indptr", (batch + 1,))
    args = (ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_table),
            block_table.shape[1], _ptr(cache_seqlens), _ptr(new_indptr), batch, k_new.shape[0], _ptr(seqlens_out))
    return PreparedCall("pkv_append", args, (k_cache, v_cache, k_new, v_new, block_table, cache_seqlens,
                                             seqlens_out, new_indptr, desc))


def prepare_decode(q, k_cache, v_cache, block_table, cache_seqlens, max_kv_len: int, scale: float, out,
                   workspace, lse=None, layout: str = "HND", workers: int = 0) -> PreparedCall:
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", q.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch, hq, d = q.shape
    _decode_operands(desc, q, out, lse, block_table, cache_seqlens)
    _scale(scale)
    with torch.cuda.device(dev):
        need = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, hq, max_kv_len, workers)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise PkvError("pkv_decode_attn", 3, f"workspace {nbytes} < {need} bytes")
    args = (ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            block_table.shape[1], _ptr(cache_seqlens), batch, int(max_kv_len), float(scale), _ptr(workspace),
            nbytes, int(workers))
    return PreparedCall("pkv_decode_attn_ex", args, (k_cache, v_cache, q, out, block_table, cache_seqlens,
                                                     workspace, lse, desc))


def prepare_append_decode(q, k_cache, v_cache, k_new, v_new, block_table, cache_seqlens, max_kv_len: int,
                          scale: float, out, workspace, seqlens_out=None, lse=None, layout: str = "HND",
                          workers: int = 0) -> PreparedCall:
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", q.dtype, dev, 3)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, k_cache.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    batch, hq, d = q.shape
    _decode_operands(desc, q, out, lse, block_table, cache_seqlens, k_new, v_new, seqlens_out)
    _scale(scale)
    with torch.cuda.device(dev):
        need = lib().pkv_decode_workspace_bytes_ex(ctypes.byref(desc), batch, hq, max_kv_len, workers)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise PkvError("pkv_append_decode_attn", 3, f"workspace {nbytes} < {need} bytes")
    args = (ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache), _ptr(k_new),
            _ptr(v_new), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(seqlens_out), batch,
            int(max_kv_len), float(scale), _ptr(workspace), nbytes, int(workers))
    return PreparedCall("pkv_append_decode_attn_ex", args, (k_cache, v_cache, q, out, k_new, v_new, block_table,
                                                            cache_seqlens, seqlens_out, workspace, lse, desc))


def prepare_decode_plan(k_cache, cache_seqlens, num_q_heads: int, max_kv_len: int, workspace, fused: bool,
                        layout: str = "HND", workers: int = 0) -> PreparedCall:
    args, keep = _decode_plan_args(k_cache, cache_seqlens, num_q_heads, max_kv_len, workspace, fused, layout,
                                   workers)
    return PreparedCall("pkv_decode_plan", args, keep)


def prepare_prefill(q, k_cache, v_cache, block_table, kv_lens, qo_indptr, max_q: int, max_kv_len: int,
                    scale: float, out, workspace=None, lse=None, causal: bool = True,
                    layout: str = "HND", rows_per_workgroup: int = 0) -> PreparedCall:
    desc = cache_desc(k_cache, v_cache, layout)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", q.dtype, dev, 3)
    _prefill_operands(desc, q, out, lse, block_table, kv_lens, qo_indptr)
    total_q, hq, d = q.shape
    batch = kv_lens.shape[0]
    _scale(scale)
    # without a workspace (or with a tiling fixed by the caller) the keys are never split
    need = 0
    if workspace is not None and not rows_per_workgroup:
        with torch.cuda.device(dev):
            need = lib().pkv_prefill_workspace_bytes(ctypes.byref(desc), batch, hq, total_q, max_q, max_kv_len)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise PkvError("pkv_prefill_attn", 3, f"workspace {nbytes} < {need} bytes")
    args = (ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(q), hq, _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            block_table.shape[1], _ptr(kv_lens), _ptr(qo_indptr), batch, total_q, int(max_q), int(max_kv_len),
            int(bool(causal)), float(scale), _ptr(workspace), nbytes)
    name = "pkv_prefill_attn"
    if rows_per_workgroup:
        name, args = "pkv_prefill_attn_ex", args + (int(rows_per_workgroup),)
    return PreparedCall(name, args, (k_cache, v_cache, q, out, block_table, kv_lens, qo_indptr, workspace, lse,
                                     desc))
