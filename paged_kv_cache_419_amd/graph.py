"""Decode steps captured as HIP graphs, one per padded batch bucket.

The Nano-vLLM write-up replays the decode step from graphs captured for batch
sizes 1, 2, 4, 8, 16, ... up to 512 so that launch overhead does not dominate
small decode batches ("Nano-vLLM part 1", section 5.3).  The store and decode
calls of this library allocate nothing, synchronise nothing and read no device
memory from the host, so a step (store the new tokens, then decode) can be
captured as it is.  A batch of B sequences runs in the smallest bucket >= B;
the padding rows carry slot -1 (the store skips them) and context length 0
(decode writes zeros), so they touch no cache slot.

With ``fused=True`` a step is the single store_and_decode kernel instead of
the store and decode kernels.  This module only arranges static buffers and
graph capture with torch; every step still runs in the HIP kernels of
libpagedkv.so.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from . import binding

DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


class _Bucket:
    def __init__(self, size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_blocks_per_seq: int, device: torch.device):
        bf = dict(dtype=torch.bfloat16, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.size = size
        self.q = torch.zeros((size, num_q_heads, head_dim), **bf)
        self.k = torch.zeros((size, num_kv_heads, head_dim), **bf)
        self.v = torch.zeros((size, num_kv_heads, head_dim), **bf)
        self.out = torch.zeros((size, num_q_heads, head_dim), **bf)
        self.slot_mapping = torch.full((size,), -1, **i32)
        self.block_tables = torch.full((size, max_blocks_per_seq), -1, **i32)
        self.context_lens = torch.zeros((size,), **i32)
        self.workspace: Optional[torch.Tensor] = None
        self.graph: Optional[torch.cuda.CUDAGraph] = None


class DecodeGraphs:
    """Captured store + decode steps over one paged K/V cache.

    ``max_context_len`` bounds every context length passed to :meth:`run`
    (it sizes the captured launch).  ``buckets`` are the padded batch sizes.
    """

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, num_q_heads: int,
                 block_size: int, max_blocks_per_seq: int, max_context_len: int, scale: float,
                 buckets: Sequence[int] = DEFAULT_BUCKETS, split_tokens: int = 0,
                 fused: bool = False):
        if k_cache.shape != v_cache.shape or k_cache.dim() != 3:
            raise ValueError("k_cache and v_cache must both be [num_slots, num_kv_heads, head_dim]")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.num_q_heads = num_q_heads
        self.num_kv_heads, self.head_dim = k_cache.shape[1], k_cache.shape[2]
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.max_context_len = max_context_len
        self.scale = scale
        self.split_tokens = split_tokens
        self.fused = fused  # one kernel per step (store_and_decode) instead of two
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        self._b: Dict[int, _Bucket] = {}
        dev = k_cache.device
        for size in self.buckets:
            bk = _Bucket(size, num_q_heads, self.num_kv_heads, self.head_dim, max_blocks_per_seq, dev)
            need = binding.decode_workspace_bytes(size, num_q_heads, self.num_kv_heads,
                                                  self.head_dim, max_context_len, split_tokens)
            bk.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            self._b[size] = bk
        self._capture_all()

    def _step(self, bk: _Bucket) -> None:
        if self.fused:
            binding.store_and_decode(bk.out, bk.q, bk.k, bk.v, self.k_cache, self.v_cache,
                                     bk.slot_mapping, bk.block_tables, bk.context_lens,
                                     self.block_size, self.max_context_len, self.scale,
                                     self.split_tokens, bk.workspace)
            return
        binding.store_kvcache(bk.k, bk.v, self.k_cache, self.v_cache, bk.slot_mapping)
        binding.paged_decode_attention(bk.out, bk.q, self.k_cache, self.v_cache, bk.block_tables,
                                       bk.context_lens, self.block_size, self.max_context_len,
                                       self.scale, self.split_tokens, bk.workspace)

    def _capture_all(self) -> None:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for bk in self._b.values():  # all padding: touches no cache slot
                self._step(bk)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for bk in self._b.values():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._step(bk)
            bk.graph = g
        torch.cuda.synchronize()

    def bucket_for(self, batch: int) -> int:
        for size in self.buckets:
            if size >= batch:
                return size
        raise ValueError(f"batch {batch} exceeds the largest bucket {self.buckets[-1]}")

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor) -> torch.Tensor:
        """Store this step's tokens and decode; returns ``out[:batch]`` (a view)."""
        batch = q.shape[0]
        if block_tables.shape[1] > self.max_blocks_per_seq:
            raise ValueError("block table wider than the captured one")
        if context_lens.device.type == "cpu" and batch and int(context_lens.max()) > self.max_context_len:
            # the captured launch covers max_context_len positions: a longer context
            # would be cut short (and the fused step would not store its new token)
            raise ValueError(f"context length {int(context_lens.max())} exceeds the captured "
                             f"bound {self.max_context_len}")
        bk = self._b[self.bucket_for(batch)]
        bk.q[:batch].copy_(q)
        bk.k[:batch].copy_(k)
        bk.v[:batch].copy_(v)
        bk.slot_mapping[:batch].copy_(slot_mapping)
        bk.slot_mapping[batch:].fill_(-1)
        bk.block_tables[:batch, :block_tables.shape[1]].copy_(block_tables)
        bk.block_tables[:batch, block_tables.shape[1]:].fill_(-1)
        bk.block_tables[batch:].fill_(-1)
        bk.context_lens[:batch].copy_(context_lens)
        bk.context_lens[batch:].fill_(0)
        bk.graph.replay()
        return bk.out[:batch]
