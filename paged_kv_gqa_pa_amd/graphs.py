"""Attention steps captured once per batch-size bucket and replayed.

The engine of "From 183 ms to 19 ms per decode step" replays one captured
decode step per batch size, over buffers that outlive the capture, and pads a
batch to its size with rows that attend to a spare block (section "Four
changes, one profile at a time", change 4; the verify step's own graph set,
section "Then speculative decoding got slower").  `StepGraphs` does that for
this library's calls: one HIP graph per bucket of batch sizes, each holding a
whole step over every layer's cache -- a work plan for the step's tables and
lengths, then per layer the cache write of the new tokens and the attention
call (or the fused write + decode call).

A batch of n sequences runs on the smallest bucket B >= n: its rows are copied
into the first n rows of the bucket's static buffers and rows n .. B-1 are
padding: a table row holding only the spare block, T positions, and slots
spare * 16 + t (t < T), so each padding row writes and reads the spare block
only.  Several padding rows write the same spare slots, so the spare block's
contents are unspecified; padding outputs are not returned.  Every real row's
result depends on its own inputs only (the kernels fix their piece length per
shape, never per batch), so the rows returned are bit-identical to eager calls
on the unpadded batch.

This module only allocates buffers, copies inputs into them and replays graphs
of the library's calls; every step of the attention runs in those calls.
"""
from typing import List, Optional, Sequence

import torch

from . import _lib as pa


class StepGraphs:
    """Captured attention steps for batch sizes up to max(buckets).

    k_caches / v_caches: one [kv_heads, num_blocks, 16, head_dim] tensor per layer (bf16,
    fp32 or int8; an int8 cache takes k_scales / v_scales, one float32 [kv_heads,
    num_blocks] tensor per layer, bf16 queries and bf16 new rows, written with
    requantization of their blocks).  spare_block: a block index no sequence uses, in
    every layer's cache.  num_query_tokens: 1 for decode, T = k + 1 (<= 16) for
    speculative verify.  fused: use pa_decode_append (pa_decode_append_quant for int8;
    decode only).  use_plan: one work plan per step (pa_plan) in every
    bucket (True), in none (False), or (None, the default) in the buckets whose
    (sequence, KV head, piece) units outnumber the GPU's compute units.  With no more
    units than compute units every unit starts on a CU of its own, so the order changes
    nothing and the plan's launch is pure cost (batch-64 workload, 28 layers: 218.2 ->
    210.3 us per step at batch 1, 333.9 -> 325.7 at batch 32; at batch 64, 512 units,
    the plan saves 6.8 us).  A plan never changes a result bit.
    """

    def __init__(self, k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
                 q_heads: int, max_blocks_per_seq: int, spare_block: int, scale: float,
                 buckets=(1, 2, 4, 8, 16, 32, 64), num_query_tokens: int = 1,
                 fused: bool = False, split_tokens: int = 0,
                 use_plan: Optional[bool] = None,
                 k_scales: Optional[Sequence[torch.Tensor]] = None,
                 v_scales: Optional[Sequence[torch.Tensor]] = None):
        if len(k_caches) == 0 or len(k_caches) != len(v_caches):
            raise ValueError("one K and one V cache per layer")
        kv_heads, num_blocks, bs, head_dim = k_caches[0].shape
        for k, v in zip(k_caches, v_caches):
            if k.shape != k_caches[0].shape or v.shape != k.shape or k.dtype != k_caches[0].dtype:
                raise ValueError("every layer's caches need the same shape and dtype")
        if bs != 16:
            raise ValueError("block_size must be 16")
        if not 0 <= spare_block < num_blocks:
            raise ValueError("spare_block outside the cache")
        T = int(num_query_tokens)
        if not 1 <= T <= 16:
            raise ValueError("num_query_tokens must be in [1, 16]")
        if fused and T != 1:
            raise ValueError("the fused write + decode call takes one token per sequence")
        self.int8 = k_caches[0].dtype == torch.int8
        if self.int8:
            if (k_scales is None or v_scales is None or len(k_scales) != len(k_caches) or
                    len(v_scales) != len(k_caches)):
                raise ValueError("an int8 cache needs k_scales / v_scales, one per layer")
            for ks, vs in zip(k_scales, v_scales):
                if (ks.dtype != torch.float32 or vs.dtype != torch.float32 or
                        tuple(ks.shape) != (kv_heads, num_blocks) or ks.shape != vs.shape):
                    raise ValueError("scales must be float32 [kv_heads, num_blocks]")
        self.k_scales = list(k_scales) if self.int8 else [None] * len(k_caches)
        self.v_scales = list(v_scales) if self.int8 else [None] * len(k_caches)
        self.k_caches, self.v_caches = list(k_caches), list(v_caches)
        self.layers = len(k_caches)
        self.q_heads, self.kv_heads, self.head_dim = q_heads, kv_heads, head_dim
        self.num_blocks, self.max_blocks = num_blocks, int(max_blocks_per_seq)
        self.max_len = self.max_blocks * 16
        self.spare, self.scale, self.T = int(spare_block), float(scale), T
        self.fused, self.split, self.use_plan = fused, int(split_tokens), use_plan
        self.dtype = k_caches[0].dtype
        # queries and new rows: the cache's dtype, bf16 for an int8 cache
        self.row_dtype = torch.bfloat16 if self.int8 else self.dtype
        self.device = k_caches[0].device
        self.buckets = sorted(set(int(b) for b in buckets))
        self._graphs = {}
        self._bufs = {}
        for B in self.buckets:
            self._capture(B)

    def _plan_pays(self, B: int) -> bool:
        if self.use_plan is not None:
            return bool(self.use_plan)
        split = self.split or pa.default_split_tokens(self.q_heads, self.kv_heads, self.head_dim,
                                                      self.dtype, num_query_tokens=self.T)
        pieces = -(-self.max_len // split)
        cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        return B * self.kv_heads * pieces > cus

    def bucket_for(self, n: int) -> int:
        for B in self.buckets:
            if n <= B:
                return B
        raise ValueError(f"batch of {n} exceeds the largest bucket {self.buckets[-1]}")

    # -- capture ---------------------------------------------------------------
    def _alloc(self, B: int):
        T, dev = self.T, self.device
        qshape = (B, self.q_heads, self.head_dim) if T == 1 else (B, T, self.q_heads, self.head_dim)
        z = lambda *s: torch.zeros(s, dtype=self.row_dtype, device=dev)
        b = {
            "q": [torch.zeros(qshape, dtype=self.row_dtype, device=dev) for _ in range(self.layers)],
            "out": [torch.zeros(qshape, dtype=self.row_dtype, device=dev) for _ in range(self.layers)],
            "k_new": [z(B * T, self.kv_heads, self.head_dim) for _ in range(self.layers)],
            "v_new": [z(B * T, self.kv_heads, self.head_dim) for _ in range(self.layers)],
            "tables": torch.full((B, self.max_blocks), -1, dtype=torch.int32, device=dev),
            "lens": torch.zeros(B, dtype=torch.int32, device=dev),
            "slots": torch.zeros(B * T, dtype=torch.int64, device=dev),
        }
        ws = pa.workspace_size(B, T, self.q_heads, self.kv_heads, self.head_dim, self.max_len,
                               self.dtype, self.split)
        b["ws"] = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        b["plan"] = None
        if self._plan_pays(B):
            n = pa.plan_size(B, T, self.q_heads, self.kv_heads, self.head_dim, self.max_len,
                             self.dtype, self.split)
            b["plan"] = torch.zeros(n, dtype=torch.uint8, device=dev)
        self._pad(b, 0, B)
        return b

    def _pad(self, b, n: int, B: int):
        """Rows n .. B-1 attend to the spare block only."""
        if n >= B:
            return
        T = self.T
        b["tables"][n:].fill_(-1)
        b["tables"][n:, 0] = self.spare
        b["lens"][n:] = T
        b["slots"][n * T:] = (self.spare * 16 +
                              torch.arange(T, device=self.device, dtype=torch.int64).repeat(B - n))

    def _step(self, b):
        T = self.T
        if b["plan"] is not None:
            pa.make_plan(b["tables"], b["lens"], self.q_heads, self.kv_heads, self.head_dim,
                         self.max_len, self.dtype, num_query_tokens=T, split_tokens=self.split,
                         plan=b["plan"])
        for l in range(self.layers):
            kc, vc = self.k_caches[l], self.v_caches[l]
            ks, vs = self.k_scales[l], self.v_scales[l]
            if self.fused and self.int8:
                pa.decode_append_quant(b["out"][l], b["q"][l], b["k_new"][l], b["v_new"][l], kc,
                                       vc, ks, vs, b["slots"], b["tables"], b["lens"], self.scale,
                                       self.max_len, split_tokens=self.split, workspace=b["ws"],
                                       plan=b["plan"])
                continue
            if self.fused:
                pa.decode_append(b["out"][l], b["q"][l], b["k_new"][l], b["v_new"][l], kc, vc,
                                 b["slots"], b["tables"], b["lens"], self.scale, self.max_len,
                                 split_tokens=self.split, workspace=b["ws"], plan=b["plan"])
                continue
            if self.int8:
                pa.reshape_and_cache_quant(b["k_new"][l], b["v_new"][l], kc, vc, ks, vs,
                                           b["slots"])
            else:
                pa.reshape_and_cache(b["k_new"][l], b["v_new"][l], kc, vc, b["slots"])
            if T == 1:
                pa.decode(b["out"][l], b["q"][l], kc, vc, b["tables"], b["lens"], self.scale,
                          self.max_len, ks, vs, split_tokens=self.split, workspace=b["ws"],
                          plan=b["plan"])
            else:
                pa.verify(b["out"][l], b["q"][l], kc, vc, b["tables"], b["lens"], self.scale,
                          self.max_len, ks, vs, split_tokens=self.split, workspace=b["ws"],
                          plan=b["plan"])

    def _capture(self, B: int):
        b = self._alloc(B)
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self._step(b)       # warm-up outside the capture
        torch.cuda.current_stream(self.device).wait_stream(side)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self._step(b)
        self._graphs[B], self._bufs[B] = g, b

    def replay(self, B: int):
        """Replay bucket B's step on the inputs last copied into it (timing)."""
        self._graphs[B].replay()

    # -- run -------------------------------------------------------------------
    def step(self, q: Sequence[torch.Tensor], k_new: Sequence[torch.Tensor],
             v_new: Sequence[torch.Tensor], block_tables: torch.Tensor,
             context_lens: torch.Tensor, slot_mapping: torch.Tensor) -> List[torch.Tensor]:
        """One step for n sequences.  Per layer: q [n, (T,) q_heads, head_dim], k_new / v_new
        [n*T, kv_heads, head_dim]; shared: block_tables int32 [n, <= max_blocks_per_seq],
        context_lens int32 [n] (the new tokens included), slot_mapping int64 [n*T].  Returns
        one [n, (T,) q_heads, head_dim] view per layer into the bucket's output buffers (valid
        until the next step on the same bucket)."""
        n = int(context_lens.shape[0])
        T = self.T
        if len(q) != self.layers or len(k_new) != self.layers or len(v_new) != self.layers:
            raise ValueError("one q, k_new and v_new per layer")
        if block_tables.shape[0] != n or slot_mapping.shape[0] != n * T:
            raise ValueError("block_tables / slot_mapping do not match context_lens")
        if block_tables.shape[1] > self.max_blocks:
            raise ValueError("block_tables wider than max_blocks_per_seq")
        qshape = (n, self.q_heads, self.head_dim) if T == 1 else (n, T, self.q_heads, self.head_dim)
        kvshape = (n * T, self.kv_heads, self.head_dim)
        for l in range(self.layers):
            if tuple(q[l].shape) != qshape or q[l].dtype != self.row_dtype:
                raise ValueError(f"layer {l}: q must be {self.row_dtype} {qshape}")
            if (tuple(k_new[l].shape) != kvshape or tuple(v_new[l].shape) != kvshape or
                    k_new[l].dtype != self.row_dtype or v_new[l].dtype != self.row_dtype):
                raise ValueError(f"layer {l}: k_new / v_new must be {self.row_dtype} {kvshape}")
        if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or
                slot_mapping.dtype != torch.int64):
            raise ValueError("block_tables / context_lens int32, slot_mapping int64")
        B = self.bucket_for(n)
        b = self._bufs[B]
        w = block_tables.shape[1]
        b["tables"][:n, :w].copy_(block_tables)
        b["tables"][:n, w:].fill_(-1)
        b["lens"][:n].copy_(context_lens)
        b["slots"][:n * T].copy_(slot_mapping)
        self._pad(b, n, B)
        for l in range(self.layers):
            b["q"][l][:n].copy_(q[l])
            b["k_new"][l][:n * T].copy_(k_new[l])
            b["v_new"][l][:n * T].copy_(v_new[l])
        self._graphs[B].replay()
        return [o[:n] for o in b["out"]]
