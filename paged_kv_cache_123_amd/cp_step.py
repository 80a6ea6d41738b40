"""One rank's share of a decode step under context parallelism.

A context-parallel group of ``world`` ranks spreads every sequence's
positions over the ranks ([CSDN] section 2.3: the slot-mapping kernel with a
world size above one).  The ranks share one block table whose entries name
virtual blocks of ``block_size * world`` positions, so the host allocator
works in virtual blocks; each rank's cache holds ``block_size`` slots of every
virtual block.  One rank's step, in order on one stream:

  copy_blocks                    copy-on-write of shared partial tails (every
                                 rank copies its own part of the block)
  compute_slot_mapping_cp        this rank's slot of every new token (-1 for
                                 the tokens other ranks store)
  reshape_and_cache              the rank's new tokens into its cache
  paged_attention_partials       (m, l, o) over the rank's tokens, written
                                 into this rank's slice of the gathered buffer
  [all-gather of the slices]     between GPUs; not part of one GPU's step
  merge_attention_partials       the attention output from all ranks' slices
"""

from __future__ import annotations

import torch

from . import ops
from .host import Pool
from .step import replay


def alloc_gathered(world: int, num_seqs: int, num_heads: int, head_size: int, device):
    """Rank-major fp32 buffers for the gathered (m, l, o) of a group."""
    return {
        "m": torch.empty((world, num_seqs, num_heads), dtype=torch.float32, device=device),
        "l": torch.empty((world, num_seqs, num_heads), dtype=torch.float32, device=device),
        "o": torch.empty((world, num_seqs, num_heads, head_size), dtype=torch.float32,
                         device=device),
    }


class CPRankStep:
    """Allocator replay (virtual blocks) plus one rank's device tensors.

    ``values``: dict with this rank's key_cache / value_cache [NB, H_kv, B, D]
    and the step's query [S, H, D], new_key / new_value [T, H_kv, D].
    ``gathered``: the group's buffers from ``alloc_gathered`` (this rank
    writes slice ``rank``); allocated here when None.
    """

    def __init__(self, num_blocks: int, block_size: int, world: int, rank: int, interleave: int,
                 free_order, history, appends, values: dict, scale: float,
                 partition_size: int, gathered=None, planned: bool = True):
        if partition_size <= 0:
            raise ValueError("rank partials use split partitions (partition_size > 0)")
        self.world, self.rank, self.interleave = int(world), int(rank), int(interleave)
        self.block_size = int(block_size)
        self.pool = Pool(num_blocks, block_size * world, free_order)
        batch = replay(self.pool, history, appends)
        seqs = [s for s, _ in appends]
        width = max(max(self.pool.seq_num_blocks(s) for s in seqs), 1)
        tables, lens = self.pool.block_tables(seqs, width)
        self.seqs = seqs
        self.tables_host = tables
        self.context_lens_host = lens            # whole sequences
        self.local_lens_host = ops.cp_local_context_lens(lens, block_size, world, rank,
                                                         interleave)
        self.cow_pairs_host = batch.cow_pairs
        self.positions_host = batch.positions
        self.query_start_loc_host = batch.query_start_loc
        self.num_tokens = int(batch.query_start_loc[-1])
        self.max_local_len = int(self.local_lens_host.max())
        self.scale = float(scale)
        self.partition_size = int(partition_size)

        dev = values["key_cache"].device
        self.key_cache = values["key_cache"]
        self.value_cache = values["value_cache"]
        self.query = values["query"]
        self.new_key = values["new_key"]
        self.new_value = values["new_value"]
        S, H, D = self.query.shape
        self.block_tables = torch.from_numpy(tables).to(dev)
        self.local_lens = torch.from_numpy(self.local_lens_host).to(dev)
        self.cow_pairs = torch.from_numpy(self.cow_pairs_host).to(dev)
        self.positions = torch.from_numpy(self.positions_host).to(dev)
        self.query_start_loc = torch.from_numpy(self.query_start_loc_host).to(dev)
        self.slot_mapping = torch.empty(self.num_tokens, dtype=torch.int64, device=dev)
        self.gathered = gathered if gathered is not None else alloc_gathered(world, S, H, D, dev)
        self.m = self.gathered["m"][rank]
        self.l = self.gathered["l"][rank]
        self.o = self.gathered["o"][rank]
        self.out = torch.empty_like(self.query)
        self.plan = None
        if planned:
            self.plan_host = ops.decode_plan(self.local_lens_host, self.partition_size)
            self.plan = torch.from_numpy(self.plan_host).to(dev)
        self.workspace = ops.alloc_split_workspace(S, H, D, max(self.max_local_len, 1),
                                                   self.partition_size, dev)

    # ---- the step, kernel by kernel --------------------------------------
    def copy_blocks(self):
        ops.copy_blocks(self.key_cache, self.value_cache, self.cow_pairs)

    def slot_mapping_kernel(self):
        ops.compute_slot_mapping_cp(self.query_start_loc, self.positions, self.block_tables,
                                    self.block_size, self.slot_mapping, self.num_tokens,
                                    self.world, self.rank, self.interleave)

    def scatter(self):
        ops.reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                              self.slot_mapping)

    def partials(self):
        ops.paged_attention_partials(self.m, self.l, self.o, self.query, self.key_cache,
                                     self.value_cache, self.block_tables, self.local_lens,
                                     self.scale, self.max_local_len, self.partition_size,
                                     self.workspace, self.plan)

    def merge(self):
        """The attention output from every rank's slice of the gathered buffers."""
        ops.merge_attention_partials(self.out, self.gathered["m"], self.gathered["l"],
                                     self.gathered["o"])
        return self.out

    def run(self, merge: bool = True):
        """The rank's whole step; returns ``out`` when ``merge``, else None
        (the partials are in this rank's slice of the gathered buffers)."""
        if len(self.cow_pairs_host):
            self.copy_blocks()
        self.slot_mapping_kernel()
        self.scatter()
        self.partials()
        return self.merge() if merge else None
