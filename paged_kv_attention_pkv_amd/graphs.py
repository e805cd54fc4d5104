"""Batch-bucket HIP graphs of the fused decode step (plumbing, no arithmetic).

A serving loop replays one captured graph per step instead of launching from
the host: the unsloth scripts commit page ("Why this works", item 3) captures
one CUDA graph per batch-size bucket and pads the live batch up to the
bucket.  ``DecodeStepGraphs`` does the same over this library: for every
bucket size it owns static buffers (per layer q, k_new, v_new, out, lse; per
step the block table, cache lengths and new lengths) and one graph holding
one ``pkv_decode_plan`` launch (the cut of the step's work, shared by its
layers) and the ``pkv_append_decode_attn`` launch of every layer.  ``stage`` copies the
live rows of a step into the bucket's buffers and marks the other slots as
padding rows (cache length -1: nothing is read or written for them, their
output is 0 / -inf and their new length stays -1), ``replay`` runs the graph.

Graph-safety of the captured calls: they allocate nothing, never synchronise
and record no memset node; each bucket has its own decode workspace, zeroed
once at construction and left zeroed by every replay.
"""
from __future__ import annotations

import torch

from . import api

PADDING_ROW = -1  # cache length that marks a padding slot


class DecodeStepGraphs:
    def __init__(self, layers, num_q_heads: int, bt_cols: int, max_kv_len: int, scale: float,
                 buckets=(1, 2, 4, 8, 16, 32, 64), layout: str = "HND"):
        """layers: [(k_cache, v_cache)] pools of the layers a step runs over
        (one shared block table and one set of lengths, as the layers of one
        model); the graphs read and write them in place."""
        if not layers:
            raise ValueError("at least one layer")
        self.layers = list(layers)
        self.layout = layout
        self.hq = int(num_q_heads)
        self.bt_cols = int(bt_cols)
        self.max_kv_len = int(max_kv_len)
        self.scale = float(scale)
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        k0 = self.layers[0][0]
        self.dev = k0.device
        desc = api.cache_desc(k0, self.layers[0][1], layout)
        self.hkv, self.d = desc.num_kv_heads, desc.head_dim
        dt = k0.dtype
        self._buf = {}
        self._graph = {}
        for b in self.buckets:
            buf = {
                "q": [torch.zeros((b, self.hq, self.d), dtype=dt, device=self.dev) for _ in self.layers],
                "k_new": [torch.zeros((b, self.hkv, self.d), dtype=dt, device=self.dev) for _ in self.layers],
                "v_new": [torch.zeros((b, self.hkv, self.d), dtype=dt, device=self.dev) for _ in self.layers],
                "out": [torch.zeros((b, self.hq, self.d), dtype=dt, device=self.dev) for _ in self.layers],
                "lse": [torch.zeros((b, self.hq), dtype=torch.float32, device=self.dev) for _ in self.layers],
                "block_table": torch.zeros((b, self.bt_cols), dtype=torch.int32, device=self.dev),
                "cache_seqlens": torch.full((b,), PADDING_ROW, dtype=torch.int32, device=self.dev),
                "seqlens_out": torch.full((b,), PADDING_ROW, dtype=torch.int32, device=self.dev),
            }
            nbytes = api.decode_workspace_bytes(k0, b, self.hq, self.max_kv_len, layout=layout)
            buf["workspace"] = torch.zeros(nbytes, dtype=torch.uint8, device=self.dev)
            buf["calls"] = [
                api.prepare_append_decode(buf["q"][i], kc, vc, buf["k_new"][i], buf["v_new"][i],
                                          buf["block_table"], buf["cache_seqlens"], self.max_kv_len, self.scale,
                                          buf["out"][i], buf["workspace"], seqlens_out=buf["seqlens_out"],
                                          lse=buf["lse"][i], layout=layout)
                for i, (kc, vc) in enumerate(self.layers)]
            if len(self.layers) > 1:
                buf["calls"].insert(0, api.prepare_decode_plan(k0, buf["cache_seqlens"], self.hq, self.max_kv_len,
                                                               buf["workspace"], fused=True, layout=layout))
            self._buf[b] = buf
        torch.cuda.synchronize(self.dev)
        for b in self.buckets:
            self._capture(b)

    def _capture(self, b: int) -> None:
        calls = self._buf[b]["calls"]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(self.dev)
        s.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for c in calls:
                    c()
        torch.cuda.current_stream(self.dev).wait_stream(s)
        torch.cuda.synchronize(self.dev)
        self._graph[b] = g

    def bucket_for(self, n: int) -> int:
        for b in self.buckets:
            if b >= n:
                return b
        raise ValueError(f"{n} rows exceed the largest bucket {self.buckets[-1]}")

    def buffers(self, bucket: int) -> dict:
        """The static tensors of a bucket (per-layer lists for q, k_new,
        v_new, out and lse)."""
        return self._buf[bucket]

    def stage(self, block_table, cache_seqlens, q, k_new, v_new, bucket: int | None = None) -> int:
        """Copy a step's live rows (n of them) into `bucket` (default: the
        smallest that holds them) and mark the remaining slots as padding
        rows.  q, k_new, v_new are per-layer lists of [n, ...] device tensors.
        Returns the bucket.  The padding slots' other inputs keep whatever
        they held."""
        n = int(cache_seqlens.shape[0])
        b = self.bucket_for(n) if bucket is None else int(bucket)
        if b not in self._buf or b < n:
            raise ValueError(f"bucket {b} cannot hold {n} rows")
        buf = self._buf[b]
        buf["block_table"][:n].copy_(block_table)
        buf["cache_seqlens"][:n].copy_(cache_seqlens)
        buf["cache_seqlens"][n:].fill_(PADDING_ROW)
        for i in range(len(self.layers)):
            buf["q"][i][:n].copy_(q[i])
            buf["k_new"][i][:n].copy_(k_new[i])
            buf["v_new"][i][:n].copy_(v_new[i])
        return b

    def replay(self, bucket: int) -> None:
        self._graph[bucket].replay()
