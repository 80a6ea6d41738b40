"""A paged KV cache that lives across decode steps.

`PagedKVCache` keeps the host block pool and the device K/V caches of one
attention layer and runs one step at a time: every listed sequence appends
its new tokens (a whole prompt, a decode token, or a few speculative tokens),
and the step returns the attention output of each sequence's last new token
over its whole context ([VLLBC] paper sections 4.2 and 4.4; [PUFANYI]
"按 Block 分配" and "共享前缀，分叉时 Copy-on-write").  Sequences can fork
(sharing every block, copy-on-write on the next append) and be freed; with a
sliding window each step first releases the blocks the window has left
([CSDN] sections 3.1.1 and 3.3.1).

Host bookkeeping runs in the C++ allocator; every device computation is one
`pa_decode_step` launch (copy-on-write of the old slots, scatter of the new
rows, planned attention; plus the merge launch with partitions).  With
``cascade`` > 0 a step runs over a cascade plan instead
(`pa_decode_step_cascade`): sequences that share leading blocks, such as the
forks of one prompt, read them once per group of at most ``cascade``.  With
``cascade`` None (the default) each step chooses: a cascade plan as wide as
the matrix cores allow when the allocator reports shared blocks, one query
per sequence is asked for and the shape has a cascade kernel; 0 never builds
one.
"""

from __future__ import annotations

import numpy as np
import torch

from . import ops
from .host import Pool
from .step import auto_cascade_group

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


class PagedKVCache:
    """K/V caches [num_blocks, num_kv_heads, block_size, head_size] of one
    layer plus the host allocator that hands out their blocks."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_size: int,
                 dtype: str = "f16", device="cuda", free_order=None, sliding_window: int = 0,
                 partition_size: int = 0, cascade=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_kv_heads, self.head_size = int(num_kv_heads), int(head_size)
        self.dtype = _TORCH[dtype]
        self.device = torch.device(device)
        self.sliding_window = int(sliding_window)
        self.partition_size = int(partition_size)
        self.cascade = None if cascade is None else int(cascade)
        if self.cascade and (self.sliding_window or dtype == "f32" or self.head_size != 128):
            raise ValueError("cascade plans need 16-bit storage, head_size 128 and no window")
        self.pool = Pool(self.num_blocks, self.block_size, free_order)
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_size)
        self.key_cache = torch.zeros(shape, dtype=self.dtype, device=self.device)
        self.value_cache = torch.zeros(shape, dtype=self.dtype, device=self.device)
        self._seqs: set = set()

    # ---- sequences ------------------------------------------------------
    def add(self, seq: int) -> None:
        """A new, empty sequence (its prompt arrives with the next step)."""
        self.pool.add_seq(seq)
        self._seqs.add(seq)

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares all of ``parent``'s blocks."""
        self.pool.fork(parent, child)
        self._seqs.add(child)

    def free(self, seq: int) -> None:
        self.pool.free_seq(seq)
        self._seqs.discard(seq)

    def length(self, seq: int) -> int:
        return self.pool.seq_len(seq)

    # ---- one step ---------------------------------------------------------
    def step(self, seqs, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
             new_tokens, scale: float, all_queries: bool = False) -> torch.Tensor:
        """Append new_tokens[i] tokens to seqs[i] (their K/V rows are the
        consecutive rows of ``key`` / ``value``, [T, num_kv_heads, head_size])
        and attend with query[i] ([S, num_heads, head_size], the last new
        token of each sequence).  Returns out [S, num_heads, head_size].

        ``all_queries``: every new token is a query (query/out [T, num_heads,
        head_size] in the order of ``key``), causal over its sequence's new
        tokens: speculative drafts, or prompts and prefill chunks.  A sequence
        with more new tokens than one workgroup holds as query vectors is
        attended as query blocks: in one launch on the prefill kernel (16-bit
        storage, head_size 128, no partitions), else after the step's cache
        writes on the decode kernels."""
        seqs = [int(s) for s in seqs]
        n = [int(x) for x in new_tokens]
        T = sum(n)
        if len(n) != len(seqs) or query.shape[0] != (T if all_queries else len(seqs)):
            raise ValueError("one query per sequence, or per new token with all_queries, and "
                             "one new-token count per sequence")
        if all_queries and self.cascade:
            raise ValueError("cascade plans take one query per sequence")
        if key.shape[0] != T or value.shape[0] != T:
            raise ValueError("key/value must hold the new tokens of every sequence in order")
        for name, t in (("key", key), ("value", value)):
            if tuple(t.shape[1:]) != (self.num_kv_heads, self.head_size) or t.dtype != self.dtype:
                raise ValueError(f"{name} must be [T, num_kv_heads, head_size] of the cache dtype")
        if (query.dim() != 3 or query.shape[2] != self.head_size or query.dtype != self.dtype
                or query.shape[1] % self.num_kv_heads):
            raise ValueError("query must be [rows, num_heads, head_size] of the cache dtype, "
                             "num_heads a multiple of num_kv_heads")
        # host: every row releases what its window left behind, then
        # allocates; the batch fits as a whole or leaves the pool unchanged
        batch = self.pool.append_batch(seqs, n, self.sliding_window)
        qsl, cow_src, cow_pairs = batch.query_start_loc, batch.cow_src, batch.cow_pairs
        positions = batch.positions
        width = max(self.pool.seq_num_blocks(s) for s in seqs)
        tables, lens = self.pool.block_tables(seqs, width)
        shared = batch.shared_blocks
        dev = self.device
        # readers of one shared prefix run together (a key per prefix)
        groups = batch.group_keys
        widest = 0  # members of the widest cascade group of the step
        cascade = self.cascade
        if cascade is None:  # chosen per step
            cascade = (auto_cascade_group(query.shape[1], self.num_kv_heads, self.head_size,
                                          self.dtype)
                       if shared.any() and not all_queries and not self.sliding_window else 0)
        if all_queries:
            H, D = query.shape[1], query.shape[2]
            G = H // self.num_kv_heads
            matrix = self.dtype != torch.float32 and D == 128
            if max(n) * G > (16 if matrix else 8):  # more than one workgroup's query vectors
                out = self._query_blocks(query, key, value, tables, lens, qsl, cow_src,
                                         cow_pairs, positions, scale, shared, matrix)
                self.last_tables, self.last_lens, self.last_group = tables, lens, 0
                return out
        chunk = 0  # a chunked cascade plan's piece size (the step's own choice)
        if cascade and not self.partition_size:
            chunk = ops.cascade_auto_chunk(tables, lens, self.block_size, cascade,
                                           self.num_kv_heads, n)
        if cascade:
            plan, num_items, widest = ops.decode_plan_cascade(
                tables, lens, self.block_size, self.partition_size, cascade, n,
                chunk_tokens=chunk)
        else:
            plan = ops.decode_plan(lens, self.partition_size, self.sliding_window,
                                   n if all_queries else None, groups)
        t = {name: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for name, a in (
            ("tables", tables), ("lens", lens), ("qsl", qsl), ("cow_src", cow_src),
            ("plan", plan))}
        out = torch.empty_like(query)
        workspace = None
        if self.partition_size or chunk:
            # the one-launch step sizes multi-query rows as num_seqs x max_query_len
            rows = len(seqs) * max(n) if all_queries else len(seqs)
            workspace = ops.alloc_split_workspace(max(rows, query.shape[0]), query.shape[1],
                                                  self.head_size, int(lens.max()),
                                                  self.partition_size or chunk, dev)
        shared_dev = torch.from_numpy(shared).to(dev) if shared.any() else None
        if cascade:
            ops.decode_step_cascade(out, query, self.key_cache, self.value_cache, t["tables"],
                                    t["lens"], scale, int(lens.max()),
                                    self.partition_size or chunk, t["plan"], num_items, widest,
                                    t["qsl"], key, value, t["cow_src"], None, workspace,
                                    shared_dev, chunked=bool(chunk))
        else:
            ops.decode_step(out, query, self.key_cache, self.value_cache, t["tables"],
                            t["lens"], scale, int(lens.max()), self.partition_size, t["plan"],
                            t["qsl"], key, value, t["cow_src"], None, workspace, shared_dev,
                            max(n) if all_queries else 0, self.sliding_window)
        self.last_tables, self.last_lens, self.last_group = tables, lens, widest
        return out

    def _query_blocks(self, query, key, value, tables, lens, qsl, cow_src, cow_pairs, positions,
                      scale, shared, matrix):
        """A step whose sequences bring more new tokens than a workgroup holds,
        attended over query blocks (pa_query_blocks): on the prefill kernel
        with the cache writes in the same launch (pa_prefill_step), else the
        cache writes (copy-on-write, slot mapping, scatter) first, then the
        split prefill kernel (partitions, on the matrix cores) or the decode
        kernels."""
        dev = self.device
        T = len(positions)
        tab = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
        qsl_host = qsl
        out = torch.empty_like(query)
        H = query.shape[1]
        max_len = int(lens.max())
        part = self.partition_size
        if matrix and not part:
            row_seq, row_lens, row_qsl = ops.query_blocks(
                lens, qsl_host, ops.prefill_block_tokens(H, self.num_kv_heads))
            # a long context under few rows goes to the split kernel by itself
            keys = int(row_lens.max())
            if self.sliding_window:
                keys = min(keys, self.sliding_window + int(np.diff(row_qsl).max()))
            part = ops.prefill_auto_partition(len(row_seq), self.num_kv_heads, keys,
                                              self.block_size)
        if matrix and not part:
            items = ops.prefill_plan(row_seq, row_lens, np.diff(row_qsl), self.sliding_window)
            ops.prefill_step(out, query, self.key_cache, self.value_cache, tab,
                             torch.from_numpy(row_seq).to(dev), torch.from_numpy(row_lens).to(dev),
                             torch.from_numpy(row_qsl).to(dev), scale, max_len,
                             torch.from_numpy(qsl_host).to(dev), key, value,
                             torch.from_numpy(cow_src).to(dev), None,
                             torch.from_numpy(items).to(dev), self.sliding_window)
            return out
        if len(cow_pairs):
            ops.copy_blocks(self.key_cache, self.value_cache, torch.from_numpy(cow_pairs).to(dev))
        slots = torch.empty(T, dtype=torch.int64, device=dev)
        ops.compute_slot_mapping(torch.from_numpy(qsl_host).to(dev),
                                 torch.from_numpy(positions).to(dev), tab, self.block_size, slots,
                                 T)
        ops.reshape_and_cache(key, value, self.key_cache, self.value_cache, slots)
        if matrix:
            # partitions on the matrix cores: the split prefill kernel and its merge
            row_seq, row_lens, row_qsl = ops.query_blocks(
                lens, qsl_host, ops.prefill_block_tokens(H, self.num_kv_heads))
            items = ops.prefill_plan_split(row_seq, row_lens, np.diff(row_qsl),
                                           self.sliding_window, part)
            workspace = ops.alloc_split_workspace(T, H, self.head_size, max_len, part, dev)
            ops.paged_attention_prefill_split(
                out, query, self.key_cache, self.value_cache, tab,
                torch.from_numpy(row_seq).to(dev), torch.from_numpy(row_lens).to(dev),
                torch.from_numpy(row_qsl).to(dev), scale, max_len,
                torch.from_numpy(items).to(dev), part, workspace, self.sliding_window)
            return out
        block = (16 if matrix else 8) // (H // self.num_kv_heads)
        row_seq, row_lens, row_qsl = ops.query_blocks(lens, qsl_host, block)
        # a sequence cut into several rows has all of its blocks read by each
        row_shared = ops.query_block_hints(row_seq, row_lens, shared, self.block_size)
        plan = ops.decode_plan(row_lens, self.partition_size, self.sliding_window,
                               np.diff(row_qsl), row_seq)
        workspace = None
        if self.partition_size:
            workspace = ops.alloc_split_workspace(T, H, self.head_size, max_len,
                                                  self.partition_size, dev)
        ops.paged_attention_multi(out, query, self.key_cache, self.value_cache,
                                  torch.from_numpy(np.ascontiguousarray(tables[row_seq])).to(dev),
                                  torch.from_numpy(row_lens).to(dev),
                                  torch.from_numpy(row_qsl).to(dev), int(np.diff(row_qsl).max()),
                                  scale, max_len, self.partition_size,
                                  torch.from_numpy(plan).to(dev), workspace,
                                  torch.from_numpy(row_shared).to(dev), self.sliding_window)
        return out
