"""GPU test of pkv_append_decode_attn_noalloc, the fused decode step on the
library's fixed device workspace (for callers that cannot allocate).

Two calls in a row, the second with a smaller batch and other lengths: each
is checked against pkv_append_decode_attn with a caller workspace on an
identical copy of the pools (pools and lengths bit for bit, outputs within
the attention bar and in fact bit for bit: the same kernel, the same split)
and against the oracle.  A batch whose workspace would exceed the array is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import DecodeCase, compare, host_bits, say, tol

pytestmark = pytest.mark.gpu


def _pools(case):
    s, i = case.spec, case.inp
    kc, vc = wl.empty_pool(s, case.dev), wl.empty_pool(s, case.dev)
    pkv.append(kc, vc, i.k_hist, i.v_hist, i.block_table, torch.zeros(s.batch, dtype=torch.int32, device=case.dev),
               i.hist_indptr)
    return kc, vc


def _one_step(spec):
    say(f"[no-alloc] {spec.name} B={spec.batch} seed={spec.seed}")
    case = DecodeCase(spec)
    i = case.inp
    max_kv = int(spec.hist_lens.max()) + 1
    ka, va = _pools(case)
    kb, vb = ka.clone(), va.clone()
    ws = torch.zeros(pkv.decode_workspace_bytes(ka, spec.batch, spec.hq, max_kv), dtype=torch.uint8,
                     device=case.dev)
    ref_out, ref_lse, ref_lens = pkv.append_decode_attn(i.q, ka, va, i.k_new, i.v_new, i.block_table, i.hist_lens,
                                                        max_kv, spec.scale, workspace=ws, return_lse=True)
    out, lse, lens = pkv.append_decode_attn_noalloc(i.q, kb, vb, i.k_new, i.v_new, i.block_table, i.hist_lens,
                                                    max_kv, spec.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(lens, ref_lens), "seqlens_out differs from the workspace entry point"
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16)), "K pool differs"
    assert torch.equal(va.view(torch.int16), vb.view(torch.int16)), "V pool differs"
    atol, rtol = tol(spec)
    say("  vs workspace entry point: out " + compare(out.cpu(), ref_out.cpu().double().numpy(), atol, rtol, "out")
        + "; lse " + compare(lse.cpu(), ref_lse.cpu().double().numpy(), atol, rtol, "lse"))
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out not bit-identical"
    assert torch.equal(lse, ref_lse), "lse not bit-identical"
    okc, ovc, olens, obt = case.oracle_pools()
    assert np.array_equal(lens.cpu().numpy(), olens)
    assert np.array_equal(host_bits(kb).view(np.uint8), okc.view(np.uint8)), "K pool vs oracle"
    ro, rl = case.oracle_decode(okc, ovc, olens, obt)
    say("  vs oracle: out " + compare(out.cpu(), ro, atol, rtol, "out") + "; lse "
        + compare(lse.cpu(), rl, atol, rtol, "lse"))


def test_noalloc_two_calls_second_smaller():
    _one_step(wl.decode_spec("qwen3_decode"))           # B = 64, lengths U{512..1024}
    _one_step(wl.decode_spec("qwen3_sweep", batch=8))   # B = 8, other lengths


def test_noalloc_refuses_batches_beyond_the_array():
    say("[no-alloc] oversized batch refused")
    dev = torch.device("cuda")
    b, hq, hkv, d = 4096, 32, 8, 128  # (1024 + 4096*8) records of 2 KB > 32 MiB
    kc = torch.zeros((4, hkv, 16, d), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((b, hq, d), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((b, hkv, d), dtype=torch.bfloat16, device=dev)
    bt = torch.ones((b, 1), dtype=torch.int32, device=dev)
    lens = torch.zeros(b, dtype=torch.int32, device=dev)
    out = torch.full_like(q, 7.0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.append_decode_attn_noalloc(q, kc, kc, kn, kn, bt, lens, 1, d ** -0.5, out=out)
    assert e.value.code == 3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "a refused call wrote its output"
