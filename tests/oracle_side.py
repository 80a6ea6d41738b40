"""Oracle side of the GPU parity tests: replays a workload's allocator history
through the oracle pool and applies the oracle's cache writes and attention
to host copies of the inputs.  Imports nothing from the product package."""

from __future__ import annotations

import numpy as np

from oracle.allocator import OraclePool
from oracle.attention import (merge_rank_partials, paged_attention, paged_attention_multi,
                              paged_attention_partials, paged_attention_split)
from oracle.cache_ops import copy_blocks, reshape_and_cache
from oracle.prefix_cache import OraclePrefixPool
from oracle.slots import (compute_slot_mapping, compute_slot_mapping_cp, cp_local_length,
                          map_to_kernel_blocks)


def to_host(t):
    """Raw storage array of a torch tensor: float32 / float16 / uint16 (bf16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class OracleStep:
    """Under context parallelism (w.extra["cp_world"] > 1) the pool hands out
    virtual blocks of block_size * cp_world positions shared by the ranks.
    With w.extra["sliding_window"] each row releases the blocks outside its
    next query's window before the step appends; with
    w.extra["kernel_block_size"] the pool's blocks are split into kernel
    blocks for the tables, copies and cache accesses."""

    def __init__(self, w):
        self.world = int(w.extra.get("cp_world", 1))
        self.interleave = int(w.extra.get("cp_interleave", 1))
        self.window = int(w.extra.get("sliding_window", 0))
        self.kb = int(w.extra.get("kernel_block_size", 0)) or w.block_size
        k = w.block_size // self.kb
        caching = any(op[0] == "request" for op in w.prefill)
        pool = (OraclePrefixPool if caching else OraclePool)(
            w.num_blocks, w.block_size * self.world, w.free_order)
        for op in w.prefill:
            if op[0] == "add":
                pool.add_seq(op[1])
            elif op[0] == "append":
                pool.append(op[1], op[2])
            elif op[0] == "fork":
                pool.fork(op[1], op[2])
            elif op[0] == "free":
                pool.free_seq(op[1])
            else:  # a request through the prefix cache
                _, s, prompt, extra = op
                done = pool.add_seq_cached(s, prompt, extra)
                pool.append_tokens(s, prompt[done:])
                pool.cache_full_blocks(s)
        positions, qsl, cow, slots = [], [0], [], []
        for s, n in w.step:
            start = pool.seq_len(s)
            pool.remove_skipped(s, start, self.window)
            sl, c = pool.append(s, n)
            slots += sl
            cow += c
            positions += list(range(start, start + n))
            qsl.append(qsl[-1] + n)
        self.pool = pool
        self.seqs = [s for s, _ in w.step]
        width = max(len(pool.block_table(s)) for s in self.seqs) * k
        self.tables = np.full((len(self.seqs), width), -1, dtype=np.int64)
        for r, s in enumerate(self.seqs):
            t = []
            for b in pool.block_table(s):  # released blocks stay holes
                t += [-1] * k if b is None else map_to_kernel_blocks([b], k)
            self.tables[r, :len(t)] = t
        cow = [(a * k + j, b * k + j) for a, b in cow for j in range(k)]
        self.context_lens = np.array([pool.seq_len(s) for s in self.seqs], dtype=np.int64)
        self.positions = positions
        self.query_start_loc = qsl
        self.cow_pairs = cow
        self.alloc_slots = slots
        self.w = w

    def slot_mapping(self, max_num_tokens=None):
        T = self.query_start_loc[-1]
        return compute_slot_mapping(self.query_start_loc, self.positions, self.tables,
                                    self.kb, max_num_tokens or T)

    def apply_copies(self, kc, vc):
        copy_blocks(kc, vc, self.cow_pairs)

    def apply_scatter(self, kc, vc, new_key, new_value):
        reshape_and_cache(kc, vc, new_key, new_value, self.slot_mapping(), self.kb)

    def attention(self, query, kc, vc, pairs=None, tables=None):
        t = self.tables if tables is None else tables
        return paged_attention(query, kc, vc, t, self.context_lens, self.w.scale, self.w.dtype,
                               pairs=pairs, window=self.window)

    def attention_split(self, query, kc, vc, partition_size, pairs=None):
        assert self.window == 0, "the split oracle has no window"
        return paged_attention_split(query, kc, vc, self.tables, self.context_lens, self.w.scale,
                                     self.w.dtype, partition_size, pairs=pairs)

    def attention_multi(self, query, kc, vc):
        return paged_attention_multi(query, kc, vc, self.tables, self.context_lens,
                                     self.query_start_loc, self.w.scale, self.w.dtype,
                                     window=self.window)

    # ---- context parallelism: one rank's share ----------------------------
    def cp_slot_mapping(self, rank, max_num_tokens=None):
        T = self.query_start_loc[-1]
        return compute_slot_mapping_cp(self.query_start_loc, self.positions, self.tables,
                                       self.w.block_size, max_num_tokens or T, self.world, rank,
                                       self.interleave)

    def cp_local_lens(self, rank):
        return np.array([cp_local_length(int(L), self.w.block_size, self.world, rank,
                                         self.interleave) for L in self.context_lens])

    def apply_cp_scatter(self, rank, kc, vc, new_key, new_value):
        reshape_and_cache(kc, vc, new_key, new_value, self.cp_slot_mapping(rank),
                          self.w.block_size)

    def cp_partials(self, rank, query, kc, vc, tables=None, rows=None):
        """(m, l, o) of the rank's share; ``rows`` restricts it to some sequences
        (the other rows are left empty)."""
        t = self.tables if tables is None else tables
        lens = self.cp_local_lens(rank)
        if rows is not None:
            lens = np.where(np.isin(np.arange(len(lens)), rows), lens, 0)
        return paged_attention_partials(query, kc, vc, t, lens, self.w.scale, self.w.dtype)

    @staticmethod
    def cp_merge(m, l, o):
        return merge_rank_partials(np.asarray(m), np.asarray(l), np.asarray(o))
