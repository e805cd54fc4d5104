"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad host scalars before launching anything."""
import ctypes
import os
import re

import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ELAUNCH, EDEVICE, EVALIDATE = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for required in ("pkv_append", "pkv_decode_attn", "pkv_prefill_attn"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = api.lib()
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(api.EXPORTED) == names, "binding signatures out of sync with the header"
    header_version = int(re.search(r"#define PKV_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.pkv_abi_version() == header_version == api.ABI_VERSION
    for code in range(7):
        assert lib.pkv_status_string(code)


def _desc(**kw):
    base = dict(dtype=api.PKV_BF16, num_pages=10, page_size=16, num_kv_heads=8, head_dim=128, reserved=0,
                s_page=8 * 16 * 128, s_head=16 * 128, s_tok=128)
    base.update(kw)
    return api._Desc(*[base[f] for f, _ in api._Desc._fields_])


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails its host checks


def _decode(desc, hq=32, batch=4, max_kv=64, bt_cols=4, out=FAKE, ws=FAKE, ws_bytes=1 << 30, scale=0.1):
    return api.lib().pkv_decode_attn(ctypes.byref(desc), out, None, FAKE, hq, FAKE, FAKE, FAKE, bt_cols, FAKE,
                                     batch, max_kv, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), EUNSUPPORTED),
    (dict(page_size=48), EUNSUPPORTED),
    (dict(dtype=7), EUNSUPPORTED),
    (dict(s_tok=127), EUNSUPPORTED),
    (dict(reserved=1), EINVAL),
    (dict(num_kv_heads=0), EINVAL),
    (dict(s_page=-8), EINVAL),
])
def test_decode_rejects_descriptor(kw, code):
    assert _decode(_desc(**kw)) == code


def test_decode_rejects_scalars():
    d = _desc()
    assert _decode(d, hq=30) == EINVAL            # Hq % Hkv != 0
    assert _decode(d, hq=8 * 17) == EUNSUPPORTED  # GQA ratio 17 > 16 MFMA columns
    assert _decode(d, batch=-1) == EINVAL
    assert _decode(d, batch=0) == OK              # nothing to do
    assert _decode(d, max_kv=65, bt_cols=4) == EINVAL  # table too narrow for max_kv_len
    assert _decode(d, max_kv=(1 << 28) + 1, bt_cols=1 << 25) == EUNSUPPORTED  # beyond the 32-bit page sums
    assert _decode(d, out=None) == EINVAL
    assert _decode(d, out=ctypes.c_void_p((1 << 20) + 2)) == EUNSUPPORTED  # misaligned
    assert _decode(d, scale=float("nan")) == EINVAL


def test_append_rejects_scalars():
    d = _desc()
    lib = api.lib()
    call = lambda **kw: lib.pkv_append(ctypes.byref(kw.get("desc", d)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                       kw.get("bt_cols", 4), kw.get("seqlens", FAKE), kw.get("indptr", None),
                                       kw.get("batch", 4), kw.get("total", 4), kw.get("out", None), None)
    assert call(total=5) == EINVAL                   # no indptr => one token per sequence
    assert call(batch=-1) == EINVAL
    assert call(batch=0, total=0) == OK
    assert call(seqlens=None) == EINVAL
    assert call(out=FAKE) == EINVAL                  # seqlens_out aliases cache_seqlens
    assert call(desc=_desc(head_dim=32)) == EUNSUPPORTED


def test_fused_decode_rejects_scalars():
    d = _desc()
    lib = api.lib()
    SEQ = ctypes.c_void_p((1 << 20) + 4096)
    call = lambda **kw: lib.pkv_append_decode_attn(
        ctypes.byref(kw.get("desc", d)), FAKE, None, FAKE, 32, FAKE, FAKE, kw.get("k_new", FAKE),
        kw.get("v_new", FAKE), FAKE, 4, SEQ, kw.get("out", None), kw.get("batch", 4), 64, 0.1, FAKE, 1 << 30, None)
    assert call(k_new=None) == EINVAL
    assert call(v_new=None) == EINVAL
    assert call(out=SEQ) == EINVAL                   # seqlens_out aliases cache_seqlens
    assert call(batch=0) == OK
    assert call(k_new=ctypes.c_void_p((1 << 20) + 8)) == EUNSUPPORTED  # misaligned
    f32 = _desc(dtype=api.PKV_F32)
    assert call(desc=f32) == EUNSUPPORTED            # fused append is bf16 only


def test_prefill_rejects_scalars():
    lib = api.lib()
    call = lambda desc, **kw: lib.pkv_prefill_attn(
        ctypes.byref(desc), FAKE, None, FAKE, kw.get("hq", 48), FAKE, FAKE, FAKE, 300, FAKE, FAKE,
        kw.get("batch", 2), kw.get("total_q", 10), 8, kw.get("max_kv", 4096), 1, 0.0625, FAKE, 1 << 30, None)
    assert call(_desc(dtype=api.PKV_F32, head_dim=256, s_page=8 * 16 * 256, s_head=16 * 256, s_tok=256)) == EUNSUPPORTED
    d = _desc(head_dim=256, s_page=8 * 16 * 256, s_head=16 * 256, s_tok=256)
    assert call(d, hq=44) == EINVAL
    assert call(d, batch=0, total_q=3) == EINVAL
    assert call(d, max_kv=300 * 16 + 1) == EINVAL


def test_prefill_workspace_sizes():
    """Invalid sizes need no workspace; without a device (CU count unknown)
    no call splits its keys, so none needs one either."""
    lib = api.lib()
    d = _desc(head_dim=256, s_page=8 * 16 * 256, s_head=16 * 256, s_tok=256)
    size = lambda *a: lib.pkv_prefill_workspace_bytes(ctypes.byref(d), *a)
    for args in ((0, 48, 64, 64, 4096), (1, 0, 64, 64, 4096), (1, 48, 64, 0, 4096), (1, 48, 64, 64, 0)):
        assert size(*args) == 0, args
    if not torch.cuda.is_available():
        assert size(1, 48, 64, 64, 32768) == 0


def test_prefill_ex_rejects_tilings():
    """rows_per_workgroup is 0, 128 or 192 (any head_dim)."""
    lib = api.lib()
    call = lambda desc, rows: lib.pkv_prefill_attn_ex(
        ctypes.byref(desc), FAKE, None, FAKE, 48, FAKE, FAKE, FAKE, 300, FAKE, FAKE, 2, 10, 8, 4096, 1, 0.0625,
        FAKE, 1 << 30, rows, None)
    d256 = _desc(head_dim=256, s_page=8 * 16 * 256, s_head=16 * 256, s_tok=256)
    d128 = _desc(head_dim=128, s_page=8 * 16 * 128, s_head=16 * 128, s_tok=128)
    for rows in (-1, 1, 64, 127, 256, 384):
        assert call(d256, rows) == EINVAL, rows
        assert call(d128, rows) == EINVAL, rows


def _cpu_pool(num_pages=10):
    return torch.empty((num_pages, 2, 16, 64), dtype=torch.bfloat16)


def test_validate_host_paths():
    kc = _cpu_pool()
    bt = torch.tensor([[1, 2, 0], [3, 4, 5]], dtype=torch.int32)
    pkv.validate_host(kc, bt, torch.tensor([20, 40], dtype=torch.int32), max_kv_len=48)
    with pytest.raises(pkv.PkvError, match="page 0"):
        pkv.validate_host(kc, bt, torch.tensor([40, 40], dtype=torch.int32), max_kv_len=48)
    with pytest.raises(pkv.PkvError, match="kv_len"):
        pkv.validate_host(kc, bt, torch.tensor([20, 49], dtype=torch.int32), max_kv_len=48)
    bad = torch.tensor([[1, 2, 0], [3, 10, 5]], dtype=torch.int32)
    with pytest.raises(pkv.PkvError, match="page 10"):
        pkv.validate_host(kc, bad, torch.tensor([20, 40], dtype=torch.int32), max_kv_len=48)
    kv = torch.tensor([20, 40], dtype=torch.int32)
    pkv.validate_host(kc, bt, kv, torch.tensor([0, 5, 45], dtype=torch.int32), max_q=40, max_kv_len=48)
    for ip, pat in (([0, 21, 30], "q_len"), ([1, 5, 30], "qo_indptr"), ([0, 0, 30], "q_len"),
                    ([0, 5, 4], "q_len")):
        with pytest.raises(pkv.PkvError, match=pat):
            pkv.validate_host(kc, bt, kv, torch.tensor(ip, dtype=torch.int32), max_q=64, max_kv_len=48)
    # non-causal allows an empty request
    pkv.validate_host(kc, bt, kv, torch.tensor([0, 0, 30], dtype=torch.int32), max_q=64, max_kv_len=48,
                      causal=False)


def test_validate_append_paths():
    kc = _cpu_pool()
    bt = torch.tensor([[1, 2, 0], [3, 4, 5]], dtype=torch.int32)
    pkv.validate_append_host(kc, bt, torch.tensor([16, 40], dtype=torch.int32))
    with pytest.raises(pkv.PkvError, match="page 0"):
        pkv.validate_append_host(kc, bt, torch.tensor([32, 40], dtype=torch.int32))
    with pytest.raises(pkv.PkvError, match="beyond the table"):
        pkv.validate_append_host(kc, bt, torch.tensor([16, 48], dtype=torch.int32))
    shared = torch.tensor([[1, 2, 0], [1, 4, 5]], dtype=torch.int32)
    with pytest.raises(pkv.PkvError, match="written twice"):
        pkv.validate_append_host(kc, shared, torch.tensor([3, 3], dtype=torch.int32))
    pkv.validate_append_host(kc, bt, torch.tensor([10, 40], dtype=torch.int32),
                             torch.tensor([0, 6, 14], dtype=torch.int32))
    with pytest.raises(pkv.PkvError, match="new_indptr"):
        pkv.validate_append_host(kc, bt, torch.tensor([10, 40], dtype=torch.int32),
                                 torch.tensor([0, 6, 14], dtype=torch.int32), total_new=13)


def test_workspace_query_rejects_bad_sizes():
    lib = api.lib()
    d = _desc()
    assert lib.pkv_decode_workspace_bytes_ex(ctypes.byref(d), 0, 32, 100, 10) == 0
    assert lib.pkv_decode_workspace_bytes_ex(ctypes.byref(d), 4, 30, 100, 10) == 0
    # an explicit worker count needs no device: (workers + B*Hkv) records of G*D fp32 + (m, l) + meta
    n = lib.pkv_decode_workspace_bytes_ex(ctypes.byref(d), 4, 32, 100, 10)
    recs = 10 + 4 * 8
    assert n >= recs * 4 * 128 * 4 + recs * 4 * 2 * 4 + 4 * 8 * 2 * 4


def test_binding_refuses_missing_library(monkeypatch):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "_LIB_PATH", "/nonexistent/libpkv.so")
    with pytest.raises(RuntimeError, match="libpkv.so not found"):
        api.lib()


def test_binding_refuses_other_abi_version(monkeypatch):
    api.lib()  # the real library loads
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "ABI_VERSION", api.ABI_VERSION + 1)
    with pytest.raises(RuntimeError, match="ABI version"):
        api.lib()


def test_binding_checks_operand_shapes():
    """The library sees only pointers, so the binding rejects tensors whose
    shapes disagree with the pool or with each other before any call."""
    kc = _cpu_pool()  # [10, 2, 16, 64] bf16: Hkv 2, D 64
    bt = torch.ones((3, 4), dtype=torch.int32)
    lens = torch.full((3,), 5, dtype=torch.int32)
    q = torch.zeros((3, 4, 64), dtype=torch.bfloat16)
    kn = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.decode_attn(torch.zeros((3, 4, 32), dtype=torch.bfloat16), kc, kc, bt, lens, 16, 0.125)
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.decode_attn(q, kc, kc, bt, lens, 16, 0.125, out=torch.zeros((3, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must have shape"):
        pkv.decode_attn(q, kc, kc, bt, lens, 16, 0.125, lse=torch.zeros((3, 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="k_new must have shape"):
        pkv.append_decode_attn(q, kc, kc, torch.zeros((3, 1, 64), dtype=torch.bfloat16), kn, bt, lens, 16, 0.125)
    with pytest.raises(ValueError, match="v_new must have shape"):
        pkv.append(kc, kc, kn, torch.zeros((3, 2, 32), dtype=torch.bfloat16), bt, lens)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="seqlens_out must have shape"):
        api.prepare_append_decode(q, kc, kc, kn, kn, bt, lens, 16, 0.125, torch.empty_like(q), ws,
                                  seqlens_out=torch.zeros(2, dtype=torch.int32))
    ip = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.prefill_attn(torch.zeros((3, 4, 128), dtype=torch.bfloat16), kc, kc, bt, lens, ip, 1, 16, 0.125)
    with pytest.raises(ValueError, match="batch mismatch"):
        api.prepare_prefill(q, kc, kc, bt, lens, ip[:3], 1, 16, 0.125, torch.empty_like(q))
    with pytest.raises(ValueError, match="lse must have shape"):
        pkv.prefill_attn(q, kc, kc, bt, lens, ip, 1, 16, 0.125, lse=torch.zeros((3, 5), dtype=torch.float32))


def test_workspace_size_ignores_lengths():
    """With an explicit worker count (no device query) the decode workspace
    size depends on the batch shape only: the same for every max_kv_len, and
    the arrival counters sit at a fixed place (the start)."""
    lib = api.lib()
    d = _desc()
    sizes = {lib.pkv_decode_workspace_bytes_ex(ctypes.byref(d), 8, 32, m, 37) for m in (0, 1, 16, 100, 2000, 1 << 20)}
    assert len(sizes) == 1 and sizes.pop() > 0


def test_validate_decode_step_paths():
    """pkv_validate_decode_step_host: L + 1 within max_kv_len, attended blocks
    on real pages, append slots distinct."""
    kc = _cpu_pool()
    bt = torch.tensor([[1, 2, 0], [3, 4, 5]], dtype=torch.int32)
    pkv.validate_decode_step_host(kc, bt, torch.tensor([15, 40], dtype=torch.int32), 48)
    with pytest.raises(pkv.PkvError, match="max_kv_len"):
        pkv.validate_decode_step_host(kc, bt, torch.tensor([15, 40], dtype=torch.int32), 40)
    with pytest.raises(pkv.PkvError, match="max_kv_len"):
        pkv.validate_decode_step_host(kc, bt, torch.tensor([-3, 40], dtype=torch.int32), 48)
    # row 0's token at position 32 opens block 2, which routes to page 0
    with pytest.raises(pkv.PkvError, match="page 0"):
        pkv.validate_decode_step_host(kc, bt, torch.tensor([32, 40], dtype=torch.int32), 48)
    shared = torch.tensor([[1, 2, 0], [1, 4, 5]], dtype=torch.int32)
    with pytest.raises(pkv.PkvError, match="written twice"):
        pkv.validate_decode_step_host(kc, shared, torch.tensor([3, 3], dtype=torch.int32), 48)
    with pytest.raises(pkv.PkvError, match="max_kv_len"):
        pkv.validate_decode_step_host(kc, bt, torch.tensor([3, 3], dtype=torch.int32), 49)


def test_workspace_reset_rejects_bad_buffers():
    lib = api.lib()
    d = _desc()
    reset = lambda batch, ws, n: lib.pkv_decode_workspace_reset(ctypes.byref(d), batch, ws, n, None)
    assert reset(-1, FAKE, 1 << 20) == EINVAL
    assert reset(0, None, 0) == OK  # nothing to clear
    assert reset(4, None, 1 << 20) == EWORKSPACE
    assert reset(4, FAKE, 4 * 8 * 4 - 1) == EWORKSPACE  # 4 rows x 8 kv heads of int32 counters
    assert reset(4, ctypes.c_void_p((1 << 20) + 4), 1 << 20) == EWORKSPACE  # misaligned


def test_decode_plan_rejects_scalars():
    lib = api.lib()
    d = _desc()
    plan = lambda **kw: lib.pkv_decode_plan(ctypes.byref(kw.get("desc", d)), kw.get("hq", 32),
                                            kw.get("seqlens", FAKE), kw.get("batch", 4), kw.get("max_kv", 64),
                                            kw.get("fused", 1), FAKE, 1 << 30, kw.get("workers", 0), None)
    assert plan(fused=2) == EINVAL
    assert plan(batch=-1) == EINVAL
    assert plan(batch=0) == OK                       # nothing to plan
    assert plan(seqlens=None) == EINVAL
    assert plan(hq=30) == EINVAL                     # Hq % Hkv != 0
    assert plan(workers=-1) == EINVAL
    assert plan(max_kv=-1) == EINVAL
    assert plan(max_kv=(1 << 28) + 1) == EUNSUPPORTED
    assert plan(desc=_desc(dtype=api.PKV_F32)) == EUNSUPPORTED  # fused calls are bf16 only
    assert plan(desc=_desc(head_dim=96)) == EUNSUPPORTED


def test_binding_requires_scale():
    """The softmax scale is the caller's: the binding computes no default."""
    kc = _cpu_pool()
    bt = torch.ones((3, 4), dtype=torch.int32)
    lens = torch.full((3,), 5, dtype=torch.int32)
    q = torch.zeros((3, 4, 64), dtype=torch.bfloat16)
    ip = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    with pytest.raises(TypeError):
        pkv.decode_attn(q, kc, kc, bt, lens, 16)
    with pytest.raises(TypeError, match="scale"):
        pkv.decode_attn(q, kc, kc, bt, lens, 16, None)
    with pytest.raises(TypeError):
        pkv.prefill_attn(q, kc, kc, bt, lens, ip, 1, 16)
    with pytest.raises(TypeError, match="scale"):
        pkv.prefill_attn(q, kc, kc, bt, lens, ip, 1, 16, None)


def test_validators_accept_padding_rows():
    """cache length -1 marks a padding slot: it writes nothing, so the append
    and decode-step validators skip it (other negative lengths stay errors)."""
    kc = _cpu_pool()
    bt = torch.tensor([[1, 2, 0], [0, 0, 0], [3, 4, 5]], dtype=torch.int32)
    pad = torch.tensor([16, -1, 40], dtype=torch.int32)
    pkv.validate_append_host(kc, bt, pad)
    pkv.validate_decode_step_host(kc, bt, pad, 48)
    with pytest.raises(pkv.PkvError, match="negative"):
        pkv.validate_append_host(kc, bt, torch.tensor([16, -2, 40], dtype=torch.int32))
    with pytest.raises(pkv.PkvError, match="max_kv_len"):
        pkv.validate_decode_step_host(kc, bt, torch.tensor([16, -2, 40], dtype=torch.int32), 48)


def test_page_sizes_accepted():
    """Pages of 16, 32, 64, 128 or 256 tokens; anything else is refused before
    any launch (a zero-batch append reaches the descriptor checks only)."""
    lib = api.lib()
    for page, want in ((16, OK), (32, OK), (64, OK), (128, OK), (256, OK), (8, EUNSUPPORTED), (24, EUNSUPPORTED),
                       (512, EUNSUPPORTED)):
        d = _desc(page_size=page, s_page=8 * page * 128, s_head=page * 128, s_tok=128)
        rc = lib.pkv_append(ctypes.byref(d), None, None, None, None, None, 0, None, None, 0, 0, None, None)
        assert rc == want, (page, rc)
