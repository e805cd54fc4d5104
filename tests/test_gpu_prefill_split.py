"""GPU parity of pkv_prefill_attn's key splits against the oracle.

A call whose (request, 128-row query tile, head) workgroups number at most
the CUs, over more than 960 keys, may run with each workgroup's keys cut
into pieces that are merged through the workspace.  The cases below take every
path of that: each head_dim's kernel, pieces with no key tiles at all (short
requests beside long ones), waves past a request's last row, requests with
no rows or no keys, the page-table window past 65536 keys (head_dim 256),
the causal and the full mask, and reuse of one workspace.  Bar: |d| <= 2e-2
+ 2e-2|ref| on out and lse, every row; split results are deterministic."""
import numpy as np
import pytest
import torch

import paged_kv_attention_pkv_amd as pkv
from paged_kv_attention_pkv_amd import workloads as wl
from gpu_common import BF16_TOL, PrefillCase, compare, say

pytestmark = pytest.mark.gpu


def _need(case):
    s = case.spec
    kc = wl.empty_pool(s, case.dev)
    return pkv.prefill_workspace_bytes(kc, s.batch, s.hq, int(s.q_lens.sum()), int(s.q_lens.max()),
                                       int(s.kv_lens.max()), layout=s.layout)


def _parity(spec, causal=True):
    say(f"[prefill split] B={spec.batch} Hq={spec.hq} Hkv={spec.hkv} D={spec.head_dim} q={spec.q_lens.tolist()} "
        f"kv={spec.kv_lens.tolist()} causal={causal} seed={spec.seed}")
    case = PrefillCase(spec)
    need = _need(case)
    assert need > 0, "this shape is expected to split its keys"
    kc, vc, kv = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kv, causal=causal)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs, causal=causal)
    s1 = compare(out.cpu()[rows], ro, *BF16_TOL, "split out")
    s2 = compare(lse.cpu()[rows], rl, *BF16_TOL, "split lse")
    say(f"  workspace {need} B; rows checked {len(rows)}; out: {s1}; lse: {s2}")
    return case, kc, vc, kv, out, lse


@pytest.mark.parametrize("d,hq,hkv,q,kv", [
    (256, 48, 8, [64], [4000]),             # one query tile per head, 7 pieces
    (256, 8, 2, [5, 300], [70, 3000]),      # the short request's workgroups get empty pieces
    (128, 32, 8, [1, 200], [3000, 2500]),   # one-row request: 7 of 8 waves past its rows
    (128, 8, 1, [130], [9000]),             # 16 pieces (the cap)
    (64, 8, 1, [5, 64], [70, 5000]),        # empty pieces at head_dim 64
    (64, 16, 4, [0, 40, 129], [50, 2000, 2100]),  # a request with no rows
])
def test_split_parity(d, hq, hkv, q, kv):
    spec = wl.prefill_spec(q_lens=q, kv_lens=kv, hq=hq, hkv=hkv, head_dim=d, seed=d + hq + len(q))
    _parity(spec)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_split_full_mask(d):
    """causal = 0: every row sees every key."""
    spec = wl.prefill_spec(q_lens=[3, 70], kv_lens=[2500, 1800], hq=8, hkv=2, head_dim=d, seed=7 + d)
    _parity(spec, causal=False)


def test_split_rows_without_keys():
    """causal = 0, a request with 3 rows and no keys beside one of 3000 keys:
    the first gives zero rows and lse -inf from every piece, the second
    matches the unsplit call within the bar."""
    say("[prefill split] rows without keys")
    dev = torch.device("cuda")
    spec = wl.custom_decode_spec([3000], hq=4, hkv=2, head_dim=128, dtype="bf16", seed=4, n_new=0)
    bt1 = torch.from_numpy(spec.block_table).to(dev)
    bt = torch.cat([torch.zeros_like(bt1), bt1])
    kc, vc = wl.empty_pool(spec, dev), wl.empty_pool(spec, dev)
    g = torch.Generator(device="cpu").manual_seed(4)
    k = torch.randn((3000, 2, 128), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((3000, 2, 128), generator=g).to(torch.bfloat16).to(dev)
    kvl = torch.tensor([0, 3000], dtype=torch.int32, device=dev)
    pkv.append(kc, vc, k, v, bt1, torch.zeros(1, dtype=torch.int32, device=dev),
               torch.tensor([0, 3000], dtype=torch.int32, device=dev))
    q = torch.randn((8, 4, 128), generator=g).to(torch.bfloat16).to(dev)
    qi = torch.tensor([0, 3, 8], dtype=torch.int32, device=dev)
    assert pkv.prefill_workspace_bytes(kc, 2, 4, 8, 5, 3000) > 0
    args = (q, kc, vc, bt, kvl, qi, 5, 3000, 128 ** -0.5)
    out, lse = pkv.prefill_attn(*args, causal=False, return_lse=True)
    o2, l2 = pkv.prefill_attn(*args, causal=False, return_lse=True, split=False)
    o, l = out.float().cpu(), lse.cpu()
    assert torch.all(o[:3] == 0) and torch.all(torch.isneginf(l[:3]))
    compare(out[3:], o2[3:].cpu().double(), *BF16_TOL, "split vs unsplit out")
    compare(lse[3:], l2[3:].cpu().double(), *BF16_TOL, "split vs unsplit lse")


def test_split_past_first_table_window():
    """head_dim 256 stages page-table entries 4096 16-token blocks at a time;
    with 70000 keys the later pieces start in the second window."""
    spec = wl.prefill_spec(q_lens=[16], kv_lens=[70000], hq=2, hkv=1, head_dim=256, seed=99)
    _parity(spec)


@pytest.mark.parametrize("d", [128, 256])
def test_split_deterministic_and_reusable(d):
    """The same call twice on one workspace gives the same bits (the merge
    order is fixed and the counters are left at zero), and a smaller call on
    that workspace after it still matches the oracle."""
    spec = wl.prefill_spec(q_lens=[64, 17], kv_lens=[4000, 2048], hq=16, hkv=4, head_dim=d, seed=31 + d)
    case = PrefillCase(spec)
    need = _need(case)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=case.dev)
    kc, vc, kv = case.gpu_pools()
    o1, l1 = case.gpu_prefill(kc, vc, kv, workspace=ws)
    o2, l2 = case.gpu_prefill(kc, vc, kv, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    # a smaller call: fewer workgroups, key tiles and pieces
    small = wl.prefill_spec(q_lens=[8], kv_lens=[1500], hq=16, hkv=4, head_dim=d, seed=5 + d)
    c2 = PrefillCase(small)
    assert _need(c2) <= need
    k2, v2, kv2 = c2.gpu_pools()
    o3, l3 = c2.gpu_prefill(k2, v2, kv2, workspace=ws)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = c2.oracle_pools()
    rows, ro, rl = c2.oracle_rows(okc, ovc, okv, obt, oreqs)
    compare(o3.cpu()[rows], ro, *BF16_TOL, "reused workspace out")
    compare(l3.cpu()[rows], rl, *BF16_TOL, "reused workspace lse")
    assert torch.all(ws[:256] == 0), "arrival counters left non-zero"


@pytest.mark.parametrize("d", [128, 256])
def test_unsplit_without_workspace(d):
    """Without a workspace the call runs unsplit on the library's tiling (128
    rows here), which gives the bits of either forced tiling; the split call
    agrees with it within the bar (and with the oracle)."""
    spec = wl.prefill_spec(q_lens=[64, 100], kv_lens=[3000, 1500], hq=16, hkv=2, head_dim=d, seed=77 + d)
    case, kc, vc, kv, out, lse = _parity(spec)
    o_ns, l_ns = case.gpu_prefill(kc, vc, kv, split=False)
    for rows in (128, 192):
        o_f, l_f = case.gpu_prefill(kc, vc, kv, rows=rows)
        torch.cuda.synchronize()
        assert torch.equal(o_ns.view(torch.int16), o_f.view(torch.int16)), rows
        assert torch.equal(l_ns.view(torch.int32), l_f.view(torch.int32)), rows
    compare(out, o_ns.cpu().double(), *BF16_TOL, "split vs unsplit out")
    compare(lse, l_ns.cpu().double(), *BF16_TOL, "split vs unsplit lse")


def test_short_workspace_rejected():
    spec = wl.prefill_spec(q_lens=[64], kv_lens=[4000], hq=8, hkv=8, head_dim=128, seed=3)
    case = PrefillCase(spec)
    need = _need(case)
    assert need > 256
    kc, vc, kv = case.gpu_pools()
    ws = torch.zeros(need - 256, dtype=torch.uint8, device=case.dev)
    with pytest.raises(pkv.PkvError):
        case.gpu_prefill(kc, vc, kv, workspace=ws)


def test_split_graph_replays():
    """A split call recorded in a HIP graph: every replay (the counters are
    reset by the kernel itself, nothing is cleared by the graph) gives the
    eager call's bits."""
    spec = wl.prefill_spec(q_lens=[64, 30], kv_lens=[3000, 2000], hq=16, hkv=2, head_dim=256, seed=12)
    case = PrefillCase(spec)
    need = _need(case)
    assert need > 0
    kc, vc, kv = case.gpu_pools()
    out = torch.empty_like(case.inp.q)
    lse = torch.empty((out.shape[0], spec.hq), dtype=torch.float32, device=case.dev)
    ws = torch.zeros(need, dtype=torch.uint8, device=case.dev)
    call = pkv.api.prepare_prefill(case.inp.q, kc, vc, case.inp.block_table, kv, case.inp.qo_indptr,
                                   int(spec.q_lens.max()), int(spec.kv_lens.max()), spec.scale, out, ws, lse=lse)
    call()
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"replay {rep} out"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), f"replay {rep} lse"
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    rows, ro, rl = case.oracle_rows(okc, ovc, okv, obt, oreqs)
    compare(out.cpu()[rows], ro, *BF16_TOL, "graph out")


@pytest.mark.parametrize("d,hq,q,kv,pieces", [(128, 32, 600, 4096, 3), (64, 32, 700, 16384, 4), (256, 48, 256, 32768, 8)])
def test_split_over_several_rounds(d, hq, q, kv, pieces):
    """Splits whose pieces take two or three rounds over the CUs (the cost
    model's choice on 256 CUs), checked on the tile-edge rows, every 53rd and
    the last row, each against the oracle over exactly the keys it sees."""
    from test_gpu_prefill import tile_edge_rows
    spec = wl.prefill_spec(q_lens=[q], kv_lens=[kv], hq=hq, hkv=8, head_dim=d, seed=90 + d)
    say(f"[prefill split] several rounds D={d} Hq={hq} q={q} kv={kv}")
    case = PrefillCase(spec, gen_device="cuda")
    need = _need(case)
    units = -(-q // 128) * hq
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert need == -(-units * 4 // 256) * 256 + units * pieces * 128 * (d + 2) * 4, need
    assert need > 0
    kc, vc, kv_t = case.gpu_pools()
    out, lse = case.gpu_prefill(kc, vc, kv_t)
    torch.cuda.synchronize()
    okc, ovc, okv, obt, oreqs = case.oracle_pools()
    rows, ro, rl = case.oracle_row_set(okc, ovc, okv, obt, oreqs, lambda r, q_len: tile_edge_rows(r, q_len))
    compare(out.cpu()[rows], ro, *BF16_TOL, "out")
    compare(lse.cpu()[rows], rl, *BF16_TOL, "lse")
