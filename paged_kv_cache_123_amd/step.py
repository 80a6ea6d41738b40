"""One decode step of the paged-KV path on the device.

Host side: the C++ block allocator replays a batch's history (sequences
added, prompts appended, samples forked) and then the step's own appends,
which yields the block tables, context lengths, token positions and
copy-on-write pairs.  Device side, in order on one stream:

  copy_blocks            copy-on-write of shared partial tails
  compute_slot_mapping   physical slot of every new token
  reshape_and_cache      new tokens' K/V into their slots
  paged attention        single pass or split-K (partition + reduce), launched
                         from a host work plan (largest pieces first) unless
                         ``planned=False``

or all four in one launch (``run(fused=True)``, pa_decode_step).

([VLLBC] paper sections 4.2 and 4.4 / Fig. 8; [PUFANYI] "按 Block 分配" and
"共享前缀，分叉时 Copy-on-write"; [CSDN] section 2.3.)
"""

from __future__ import annotations

import numpy as np
import torch

from . import ops
from .host import Pool


def replay(pool: Pool, history, appends):
    """Run a batch's history and then the step's appends through ``pool``.

    Returns (seqs, positions, query_start_loc, cow_pairs, cow_src): the batch
    rows, the position of every new token, the row boundaries of the new
    tokens, the (src, dst) copy-on-write pairs, and per row the source block
    of its copy-on-write (-1 for none)."""
    for op in history:
        if op[0] == "add":
            pool.add_seq(op[1])
        elif op[0] == "append":
            pool.append(op[1], op[2])
        elif op[0] == "fork":
            pool.fork(op[1], op[2])
        else:
            raise ValueError(f"unknown operation {op!r}")
    seqs, positions, qsl, cow, cow_src = [], [], [0], [], []
    for s, n in appends:
        start = pool.seq_len(s)
        _, pair = pool.append(s, n)
        seqs.append(s)
        positions.extend(range(start, start + n))
        qsl.append(qsl[-1] + n)
        cow_src.append(-1 if pair is None else pair[0])
        if pair is not None:
            cow.append(pair)
    return seqs, positions, qsl, cow, cow_src


class DecodeStep:
    """Allocator replay plus device tensors of one decode step.

    ``history``: list of ("add", s) / ("append", s, n) / ("fork", parent, child);
    ``appends``: list of (s, n) appended by the step, one per batch row, in
    batch order; ``values``: dict with key_cache, value_cache, query, new_key,
    new_value device tensors (caches [NB, H_kv, B, D]).  ``all_queries``:
    every new token is a query (query/out [num_tokens, H, D], causal over each
    sequence's new tokens) instead of one query per sequence.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order, history, appends,
                 values: dict, scale: float, partition_size: int = 0, planned: bool = True,
                 all_queries: bool = False):
        self.pool = Pool(num_blocks, block_size, free_order)
        seqs, positions, qsl, cow, cow_src = replay(self.pool, history, appends)
        self.seqs = seqs
        self.block_size = block_size
        width = max(self.pool.seq_num_blocks(s) for s in seqs)
        tables, lens = self.pool.block_tables(seqs, width)
        self.tables_host = tables
        self.context_lens_host = lens
        self.cow_pairs_host = np.asarray(cow, dtype=np.int64).reshape(-1, 2)
        self.cow_src_host = np.asarray(cow_src, dtype=np.int64)
        self.shared_blocks_host = self.pool.shared_prefix_blocks(seqs)
        self.positions_host = np.asarray(positions, dtype=np.int64)
        self.query_start_loc_host = np.asarray(qsl, dtype=np.int32)
        self.num_tokens = int(qsl[-1])
        self.max_context_len = int(lens.max())
        self.scale = float(scale)
        self.partition_size = int(partition_size)

        dev = values["key_cache"].device
        self.key_cache = values["key_cache"]
        self.value_cache = values["value_cache"]
        self.query = values["query"]
        self.new_key = values["new_key"]
        self.new_value = values["new_value"]
        self.block_tables = torch.from_numpy(tables).to(dev)
        self.context_lens = torch.from_numpy(lens).to(dev)
        self.cow_pairs = torch.from_numpy(self.cow_pairs_host).to(dev)
        self.cow_src = torch.from_numpy(self.cow_src_host).to(dev)
        self.shared_blocks = (torch.from_numpy(self.shared_blocks_host).to(dev)
                              if self.shared_blocks_host.any() else None)
        self.positions = torch.from_numpy(self.positions_host).to(dev)
        self.query_start_loc = torch.from_numpy(self.query_start_loc_host).to(dev)
        self.slot_mapping = torch.empty(self.num_tokens, dtype=torch.int64, device=dev)
        self.out = torch.empty_like(self.query)
        self.planned = planned
        self.all_queries = bool(all_queries)
        self.max_query_len = int(max(n for _, n in appends)) if all_queries else 0
        if all_queries and not planned:
            raise ValueError("every-token queries use the planned launch")
        self.plan_host = ops.decode_plan(lens, self.partition_size)
        self.plan = torch.from_numpy(self.plan_host).to(dev)
        self.workspace = None
        if self.partition_size:
            rows, H, D = self.query.shape
            if all_queries:  # the one-launch step sizes rows as num_seqs x max_query_len
                rows = max(rows, len(seqs) * self.max_query_len)
            self.workspace = ops.alloc_split_workspace(rows, H, D, self.max_context_len,
                                                       self.partition_size, dev)

    # ---- the step, kernel by kernel --------------------------------------
    def copy_blocks(self):
        ops.copy_blocks(self.key_cache, self.value_cache, self.cow_pairs)

    def slot_mapping_kernel(self):
        ops.compute_slot_mapping(self.query_start_loc, self.positions, self.block_tables,
                                 self.block_size, self.slot_mapping, self.num_tokens)

    def scatter(self):
        ops.reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                              self.slot_mapping)

    def attention(self):
        if self.all_queries:
            ops.paged_attention_multi(self.out, self.query, self.key_cache, self.value_cache,
                                      self.block_tables, self.context_lens,
                                      self.query_start_loc, self.max_query_len, self.scale,
                                      self.max_context_len, self.partition_size, self.plan,
                                      self.workspace, self.shared_blocks)
        elif self.planned:
            ops.paged_attention_decode_planned(self.out, self.query, self.key_cache,
                                               self.value_cache, self.block_tables,
                                               self.context_lens, self.scale,
                                               self.max_context_len, self.partition_size,
                                               self.plan, self.workspace, self.shared_blocks)
        elif self.partition_size:
            ops.paged_attention_decode_split(self.out, self.query, self.key_cache,
                                             self.value_cache, self.block_tables,
                                             self.context_lens, self.scale,
                                             self.max_context_len, self.partition_size,
                                             self.workspace)
        else:
            ops.paged_attention_decode(self.out, self.query, self.key_cache, self.value_cache,
                                       self.block_tables, self.context_lens, self.scale,
                                       self.max_context_len)

    def fused(self):
        """The whole step as one launch (pa_decode_step)."""
        ops.decode_step(self.out, self.query, self.key_cache, self.value_cache,
                        self.block_tables, self.context_lens, self.scale, self.max_context_len,
                        self.partition_size, self.plan, self.query_start_loc, self.new_key,
                        self.new_value, self.cow_src, self.slot_mapping, self.workspace,
                        self.shared_blocks, self.max_query_len)

    def run(self, fused: bool = False):
        """The whole step; returns ``out`` [num_seqs, num_heads, head_size].
        ``fused``: one launch instead of copy, slot mapping, scatter, attention."""
        if fused:
            self.fused()
            return self.out
        self.copy_blocks()
        self.slot_mapping_kernel()
        self.scatter()
        self.attention()
        return self.out
