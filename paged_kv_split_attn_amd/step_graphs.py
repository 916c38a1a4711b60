"""Whole-step hipGraph harness: one captured graph per power-of-two batch size.

A decode step of an N-layer model's attention is one launch per layer: the
first layer's pkv_decode_plan builds the step's plan and kv_indptr (what
pkv_build_metadata does) in the same launch as its fused append + decode, and
every later layer's pkv_decode_append runs on that plan (each layer's new K/V
token is written into its pool and attended in the same launch).  The pages capture
such steps once per power-of-two batch size at start-up and replay them with
every input at a fixed workspace address (AstrAI commit 05739629,
astrai/inference: the _warmup_cuda_graphs and CudaGraphContext bullets).

Here a bucket of size B owns fixed device buffers -- seq_lens [B],
kv_indices [capacity], kv_indptr [B + 1], the workspace of a descriptor with
max_batch B, and per layer q / k_new / v_new / out [B, ...] -- and one graph
that runs the step on them.  A live batch of n <= B requests is padded with
zero-length requests: before each replay, outside the graph, its lengths are
copied into seq_lens with zeros after them and its page table into
kv_indices.  A zero-length request owns no page, so it adds no work to the
plan and gets a zero output row; the live rows are bitwise those of the
unpadded step, because the plan depends only on the pages of the requests.

This module only moves data between torch tensors and replays graphs; every
step of the computation runs in the library's kernels.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import Desc, Pool, pkv_build_metadata, pkv_decode_append, pkv_decode_plan, \
    pkv_workspace_bytes


def buckets_up_to(max_batch: int) -> List[int]:
    """Powers of two 1, 2, 4, ... up to the first one that holds max_batch."""
    out, b = [], 1
    while True:
        out.append(b)
        if b >= max_batch:
            return out
        b *= 2


class _Bucket:
    def __init__(self, B: int, template: Desc, layers: int, max_pages: int, device):
        self.B = B
        self.desc = Desc(max_batch=B, num_q_heads=template.num_q_heads,
                         num_kv_heads=template.num_kv_heads, head_dim=template.head_dim,
                         page_size=template.page_size, num_workgroups=template.num_workgroups,
                         min_tiles_per_group=template.min_tiles_per_group)
        Hq, Hkv, D = template.num_q_heads, template.num_kv_heads, template.head_dim
        i32 = dict(dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros(B, **i32)
        self.kv_indices = torch.zeros(max(1, max_pages), **i32)
        self.kv_indptr = torch.zeros(B + 1, **i32)
        self.ws = torch.zeros(pkv_workspace_bytes(self.desc), dtype=torch.uint8, device=device)
        # one metadata build: every arrival counter starts at zero (the planning
        # launch relies on it, and every decode leaves them so)
        pkv_build_metadata(self.desc, self.seq_lens, 0, self.kv_indptr, self.ws)
        bf = dict(dtype=torch.int16, device=device)
        self.q = torch.zeros((layers, B, Hq, D), **bf)
        self.k_new = torch.zeros((layers, B, Hkv, D), **bf)
        self.v_new = torch.zeros((layers, B, Hkv, D), **bf)
        self.out = torch.zeros((layers, B, Hq, D), **bf)
        self.graph: Optional[torch.cuda.CUDAGraph] = None


class StepGraphs:
    """Captured decode steps, one per power-of-two batch size up to max_batch.

    pools: one Pool per layer (shared by every bucket: the page table decides
    which pages a step touches).  sm_scale: the softmax scale.  max_pages:
    capacity of the page table (entries of kv_indices).
    """

    def __init__(self, template: Desc, pools: Sequence[Pool], sm_scale: float, max_batch: int,
                 max_pages: int, device="cuda:0"):
        self.template = template
        self.pools = list(pools)
        self.sm_scale = float(sm_scale)
        self.max_pages = int(max_pages)
        self.device = torch.device(device)
        self.buckets = {B: _Bucket(B, template, len(self.pools), self.max_pages, self.device)
                        for B in buckets_up_to(max_batch)}

    def bucket_for(self, n: int) -> int:
        for B in sorted(self.buckets):
            if B >= n:
                return B
        raise ValueError(f"batch {n} above the largest bucket {max(self.buckets)}")

    def _step_on(self, bk: _Bucket, stream) -> None:
        for layer, pool in enumerate(self.pools):
            if layer == 0:
                pkv_decode_plan(pool, bk.desc, bk.q[0], bk.k_new[0], bk.v_new[0], bk.seq_lens, 0,
                                bk.kv_indptr, bk.kv_indices, self.sm_scale, bk.ws, bk.out[0],
                                stream)
            else:
                pkv_decode_append(pool, bk.desc, bk.q[layer], bk.k_new[layer], bk.v_new[layer],
                                  bk.kv_indptr, bk.kv_indices, bk.seq_lens, self.sm_scale, bk.ws,
                                  bk.out[layer], stream)

    def capture(self) -> None:
        """Capture every bucket's step (after one eager run of it on a side stream).

        The buffers hold zero-length requests while this runs, so capturing
        writes nothing into the pools."""
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        for bk in self.buckets.values():
            bk.seq_lens.zero_()
            with torch.cuda.stream(side):
                self._step_on(bk, side)
            side.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    self._step_on(bk, side)
            bk.graph = g
        torch.cuda.current_stream(self.device).wait_stream(side)
        torch.cuda.synchronize(self.device)

    def load(self, seq_lens: torch.Tensor, kv_indices: torch.Tensor, q: torch.Tensor,
             k_new: torch.Tensor, v_new: torch.Tensor) -> _Bucket:
        """Copy a live batch into its bucket's fixed buffers (zero-length padding).

        seq_lens int32 [n] and kv_indices int32 [m] on the device; q [layers, n,
        Hq, D], k_new / v_new [layers, n, Hkv, D] (bf16 bits)."""
        n = seq_lens.numel()
        bk = self.buckets[self.bucket_for(n)]
        if kv_indices.numel() > bk.kv_indices.numel():
            raise ValueError("page table above the harness capacity")
        bk.seq_lens[:n].copy_(seq_lens)
        bk.seq_lens[n:].zero_()
        bk.kv_indices[: kv_indices.numel()].copy_(kv_indices)
        bk.q[:, :n].copy_(q)
        bk.k_new[:, :n].copy_(k_new)
        bk.v_new[:, :n].copy_(v_new)
        return bk

    def replay(self, bk: _Bucket) -> torch.Tensor:
        bk.graph.replay()
        return bk.out

    def eager(self, bk: _Bucket, stream=None) -> torch.Tensor:
        """The same step issued launch by launch (for comparison)."""
        self._step_on(bk, stream if stream is not None else torch.cuda.current_stream(self.device))
        return bk.out
