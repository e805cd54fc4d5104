"""GPU test of batch-bucket graph capture of the fused decode step with
padding rows (paged_kv_attention_pkv_amd.graphs).

One HIP graph per bucket {1, 2, 4, ..., 64} over two layer caches, all
captured before any replay.  Each bucket then replays two decode steps with
fewer live rows than slots.  The spare slots are poisoned: NaN q / k_new /
v_new and a table row that routes to live pages of another sequence.  After
each replay: live rows match the oracle (which appends and attends the live
rows only), padding slots give out = 0, lse = -inf and keep length -1, and
both layers' pools equal the oracle's byte for byte (so a padding slot wrote
nothing).  Eager work and synchronisations run between the replays."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from paged_kv_attention_pkv_amd.graphs import DecodeStepGraphs
from gpu_common import BF16_TOL, compare, host_bits, opool, say

pytestmark = pytest.mark.gpu

BUCKETS = (1, 2, 4, 8, 16, 32, 64)
LIVE = {1: 1, 2: 1, 4: 3, 8: 5, 16: 11, 32: 23, 64: 37}
STEPS = 2


def test_bucket_graphs_with_padding_rows():
    say("[buckets] one graph per bucket 1..64, two layers, padding rows poisoned")
    dev = torch.device("cuda")
    rng = np.random.default_rng(123)
    nseq, layers = 64, 2
    hist = rng.integers(0, 300, size=nseq)
    # table room for every token the test appends (at most one per bucket and step)
    spec = wl.custom_decode_spec(hist.tolist(), hq=32, hkv=8, head_dim=128, dtype="bf16", seed=123,
                                 n_new=len(BUCKETS) * STEPS)
    pool = opool(spec)
    orc = oracle.load()
    bt_all = spec.block_table
    gpu_pools, host_pools = [], []
    for layer in range(layers):
        inp = wl.decode_inputs(spec, device="cpu", seed_offset=layer)
        kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
        pkv.append(kc, vc, inp.k_hist.to(dev), inp.v_hist.to(dev), torch.from_numpy(bt_all).to(dev),
                   torch.zeros(nseq, dtype=torch.int32, device=dev), inp.hist_indptr.to(dev))
        okc = host_bits(wl.empty_pool(spec, "cpu")).copy()
        ovc = okc.copy()
        orc.append(pool, okc, ovc, host_bits(inp.k_hist), host_bits(inp.v_hist), bt_all,
                   np.zeros(nseq, np.int32), inp.hist_indptr.numpy())
        gpu_pools.append((kc, vc))
        host_pools.append((okc, ovc))
    max_kv = int(hist.max()) + len(BUCKETS) * STEPS
    graphs = DecodeStepGraphs(gpu_pools, 32, spec.bt_cols, max_kv, spec.scale, buckets=BUCKETS)
    lens = hist.astype(np.int32).copy()  # current length of every sequence (both sides)
    gen = torch.Generator().manual_seed(321)
    for b in BUCKETS:
        n = LIVE[b]
        live = np.sort(rng.choice(nseq, n, replace=False))
        for step in range(STEPS):
            say(f"  bucket {b}: {n} live rows, step {step}")
            q = [torch.randn((n, 32, 128), generator=gen).to(torch.bfloat16) for _ in range(layers)]
            kn = [torch.randn((n, 8, 128), generator=gen).to(torch.bfloat16) for _ in range(layers)]
            vn = [torch.randn((n, 8, 128), generator=gen).to(torch.bfloat16) for _ in range(layers)]
            buf = graphs.buffers(b)
            # poison the spare slots: NaN activations, a table row routing to live pages
            for i in range(layers):
                buf["q"][i].fill_(float("nan"))
                buf["k_new"][i].fill_(float("nan"))
                buf["v_new"][i].fill_(float("nan"))
                buf["out"][i].fill_(7.0)
            buf["block_table"].copy_(torch.from_numpy(bt_all[live[0]]).to(dev).expand(b, -1))
            got = graphs.stage(torch.from_numpy(bt_all[live]).to(dev), torch.from_numpy(lens[live]).to(dev),
                               [x.to(dev) for x in q], [x.to(dev) for x in kn], [x.to(dev) for x in vn], bucket=b)
            assert got == b
            torch.cuda.synchronize()
            graphs.replay(b)
            torch.cuda.synchronize()
            _ = torch.ones(1024, device=dev).sum()  # eager work between replays
            new_lens = buf["seqlens_out"].cpu().numpy()
            assert new_lens[:n].tolist() == (lens[live] + 1).tolist()
            assert np.all(new_lens[n:] == -1)
            for i in range(layers):
                okc, ovc = host_pools[i]
                olens = orc.append(pool, okc, ovc, host_bits(kn[i]), host_bits(vn[i]), bt_all[live], lens[live])
                ro, rl = orc.decode(pool, host_bits(q[i]), okc, ovc, bt_all[live], olens, spec.scale)
                out, lse = buf["out"][i].cpu(), buf["lse"][i].cpu()
                compare(out[:n], ro, *BF16_TOL, f"bucket {b} layer {i} out")
                compare(lse[:n], rl, *BF16_TOL, f"bucket {b} layer {i} lse")
                assert torch.all(out[n:] == 0) and torch.all(torch.isneginf(lse[n:])), "padding slot output"
                kc, vc = gpu_pools[i]
                assert np.array_equal(host_bits(kc).view(np.uint8), okc.view(np.uint8)), "K pool differs"
                assert np.array_equal(host_bits(vc).view(np.uint8), ovc.view(np.uint8)), "V pool differs"
            lens[live] += 1
