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


def replay(pool: Pool, history, appends, sliding_window: int = 0,
           blocks_per_kv_block: int = 1):
    """Run a batch's history and then the step's appends through ``pool``.
    History operations: ("add", s), ("append", s, n), ("fork", parent, child),
    ("free", s), and ("request", s, prompt_token_ids, extra_key_bytes): a
    request served through the prefix cache (its longest cached prefix is
    taken over, the rest of the prompt appended, and its full blocks cached).
    The step's appends, (s, n) per batch row, go through the allocator as one
    batch (pa_pool_append_batch): with a sliding window each row first
    releases the blocks its next query can no longer see ([CSDN] sections
    3.1.1 and 3.3.1), and the batch fits as a whole or changes nothing.

    Returns the batch's StepAppends (positions, row boundaries, slots, copy
    sources and kernel-block copy pairs, shared-prefix hints and group keys)."""
    for op in history:
        if op[0] == "add":
            pool.add_seq(op[1])
        elif op[0] == "append":
            pool.append(op[1], op[2])
        elif op[0] == "fork":
            pool.fork(op[1], op[2])
        elif op[0] == "free":
            pool.free_seq(op[1])
        elif op[0] == "request":
            _, s, prompt, extra = op
            done = pool.add_seq_cached(s, prompt, extra)
            pool.append_tokens(s, prompt[done:])
            pool.cache_full_blocks(s)
        else:
            raise ValueError(f"unknown operation {op!r}")
    return pool.append_batch([s for s, _ in appends], [n for _, n in appends], sliding_window,
                             blocks_per_kv_block)


def auto_cascade_group(num_heads: int, num_kv_heads: int, head_size: int, dtype) -> int:
    """Group width of the cascade plan a step takes on its own when sequences
    share blocks: members x query heads per KV head fill the matrix cores' 16
    columns, at most 8 members (pa_cascade_max_group).  0, i.e. per-sequence
    work, where the group would hold fewer than 4 members (8 query heads per
    KV head) or the shape has no cascade kernel (fp32, head_size 64)."""
    group = ops.cascade_max_group(num_heads, num_kv_heads, head_size, dtype)
    return group if group >= 4 else 0


class DecodeStep:
    """Allocator replay plus device tensors of one decode step.

    ``history``: list of ("add", s) / ("append", s, n) / ("fork", parent, child);
    ``appends``: list of (s, n) appended by the step, one per batch row, in
    batch order; ``values``: dict with key_cache, value_cache, query, new_key,
    new_value device tensors (caches [NB, H_kv, B, D]).  ``all_queries``:
    every new token is a query (query/out [num_tokens, H, D], causal over each
    sequence's new tokens) instead of one query per sequence; a sequence with
    more new tokens than one workgroup holds as query vectors (a prefill
    chunk) is attended as several query blocks (pa_query_blocks): with 16-bit
    storage, head_size 128 and no partitions the blocks hold 128 query vectors
    and run on the prefill kernel (pa_paged_attention_prefill, or
    pa_prefill_step with the cache writes in the same launch) unless
    ``prefill_kernel`` is False; otherwise on the decode kernels after the
    step's cache writes (separate launches).
    ``sliding_window``: attention sees the last W tokens only, and blocks
    outside every query's window are released before the step's appends.
    ``kernel_block_size``: the allocator hands out blocks of ``block_size``
    tokens that the kernels see as block_size / kernel_block_size blocks of
    kernel_block_size tokens ([CSDN] section 3.4): tables and copy-on-write
    pairs are mapped, and the caches hold num_blocks * k kernel blocks.
    ``cascade``: build a cascade plan with groups of at most ``cascade``
    members, for the one-launch step: with partitions, those inside a prefix
    several sequences share run once per group of sharers; without, one
    workgroup per group and KV head reads the prefix once and then every
    member's own tokens.  Needs one query per sequence and no window.
    None (the default) chooses: a cascade plan as wide as the matrix-core
    columns allow (``auto_cascade_group``) when the allocator reports blocks
    several sequences share and the shape allows one; 0 never builds one.
    ``cascade_chunk``: with a cascade plan and no partitions, cut each shared
    prefix into pieces of this many tokens, each read once for the group by a
    workgroup of its own, plus one item for the rest of the prefix and the
    members' own tokens; partials merged as in split-K (0: one workgroup per
    group and KV head; None: the step's choice, pa_cascade_auto_chunk).
    """

    def __init__(self, num_blocks: int, block_size: int, free_order, history, appends,
                 values: dict, scale: float, partition_size: int = 0, planned: bool = True,
                 all_queries: bool = False, sliding_window: int = 0,
                 kernel_block_size: int = 0, cascade=None, prefill_kernel: bool = True,
                 cascade_chunk=None):
        self.pool = Pool(num_blocks, block_size, free_order)
        if any(op[0] == "request" for op in history):
            self.pool.enable_prefix_caching()
        self.sliding_window = int(sliding_window)
        kb = int(kernel_block_size) or block_size
        if block_size % kb:
            raise ValueError("kernel_block_size must divide block_size")
        k = block_size // kb
        batch = replay(self.pool, history, appends, self.sliding_window, k)
        seqs = [s for s, _ in appends]
        self.seqs = seqs
        self.block_size = kb
        self.kernel_blocks_per_block = k
        width = max(self.pool.seq_num_blocks(s) for s in seqs)
        tables, lens = self.pool.block_tables(seqs, width)
        self.manager_tables_host = tables
        if k > 1:
            tables = ops.map_to_kernel_blocks(tables, k)
        self.tables_host = tables
        self.context_lens_host = lens
        self.cow_pairs_host = batch.cow_pairs
        # the one-launch step copies a row's tail from one source block: a
        # manager block of several kernel blocks needs pa_copy_blocks
        self.fused_ok = k == 1 or not (batch.cow_src >= 0).any()
        self.cow_src_host = batch.cow_src if k == 1 else np.full(len(seqs), -1, dtype=np.int64)
        self.shared_blocks_host = batch.shared_blocks  # in kernel blocks
        self.positions_host = batch.positions
        self.query_start_loc_host = batch.query_start_loc
        self.num_tokens = int(batch.query_start_loc[-1])
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
        if self.sliding_window and not planned:
            raise ValueError("a sliding window uses the planned launch")
        query_lens = [n for _, n in appends] if all_queries else None
        # readers of one shared prefix run together (a key per prefix)
        groups = batch.group_keys
        if cascade is None:
            cascade = (auto_cascade_group(self.query.shape[1], self.key_cache.shape[1],
                                          self.query.shape[2], self.query.dtype)
                       if (self.shared_blocks_host.any() and planned and not all_queries
                           and not self.sliding_window and k == 1) else 0)
        self.cascade = int(cascade)
        if self.cascade and not self.partition_size and cascade_chunk is None:
            cascade_chunk = ops.cascade_auto_chunk(tables, lens, kb, self.cascade,
                                                   self.key_cache.shape[1],
                                                   [n for _, n in appends])
        self.cascade_chunk = (int(cascade_chunk or 0) if self.cascade and not self.partition_size
                              else 0)
        self.num_items, self.max_group = 0, 0
        if self.cascade:
            if all_queries or self.sliding_window or k > 1:
                raise ValueError("a cascade plan needs one query per sequence, no window and "
                                 "kernel blocks equal to the allocator's")
            self.plan_host, self.num_items, self.max_group = ops.decode_plan_cascade(
                tables, lens, kb, self.partition_size, self.cascade, [n for _, n in appends],
                chunk_tokens=self.cascade_chunk)
        else:
            self.plan_host = ops.decode_plan(lens, self.partition_size, self.sliding_window,
                                             query_lens, groups)
        # the rows the multi-query attention runs over: the sequences, or their
        # query blocks when a sequence brings more tokens than a workgroup holds
        self.attn_tables, self.attn_lens = self.block_tables, self.context_lens
        self.attn_qsl, self.attn_max_query_len = self.query_start_loc, self.max_query_len
        self.attn_shared = self.shared_blocks
        self.query_blocks = False
        self.prefill_rows = False
        if all_queries:
            H, D = self.query.shape[1], self.query.shape[2]
            G = H // values["key_cache"].shape[1]
            matrix = self.query.dtype != torch.float32 and D == 128
            block = (16 if matrix else 8) // G
            if block < 1:
                raise ValueError("one new token's query heads exceed a workgroup's query vectors")
            if self.max_query_len > block:
                self.query_blocks = True
                # on the matrix cores: the prefill kernel's larger blocks, each
                # K/V tile staged once in LDS for the whole block; in a single
                # pass it reads the step's new rows from their inputs, so the
                # step can run as one launch (with partitions: the cache
                # writes first, then the split kernel and its merge).  On the
                # decode kernels, blocks of one sequence read each other's new
                # rows from the cache.
                self.prefill_rows = prefill_kernel and matrix
                self.fused_ok = self.fused_ok and self.prefill_rows and not self.partition_size
                if self.prefill_rows:
                    block = ops.prefill_block_tokens(H, values["key_cache"].shape[1])
                row_seq, row_lens, row_qsl = ops.query_blocks(lens, self.query_start_loc_host,
                                                              block)
                row_tables = np.ascontiguousarray(tables[row_seq])
                row_shared = ops.query_block_hints(row_seq, row_lens, self.shared_blocks_host,
                                                   kb)
                self.plan_host = ops.decode_plan(row_lens, self.partition_size,
                                                 self.sliding_window, np.diff(row_qsl), row_seq)
                self.attn_tables = torch.from_numpy(row_tables).to(dev)
                self.attn_lens = torch.from_numpy(row_lens).to(dev)
                self.attn_qsl = torch.from_numpy(row_qsl).to(dev)
                self.attn_max_query_len = int(np.diff(row_qsl).max())
                self.attn_shared = torch.from_numpy(row_shared).to(dev)
                self.row_seq = torch.from_numpy(row_seq).to(dev)
                if self.prefill_rows and self.partition_size:
                    # (row, partition) items, a sequence's together
                    self.prefill_items = torch.from_numpy(ops.prefill_plan_split(
                        row_seq, row_lens, np.diff(row_qsl), self.sliding_window,
                        self.partition_size)).to(dev)
                elif self.prefill_rows:
                    # launch order: a sequence's rows together, the largest
                    # sequences first
                    self.prefill_items = torch.from_numpy(ops.prefill_plan(
                        row_seq, row_lens, np.diff(row_qsl), self.sliding_window)).to(dev)
        self.plan = torch.from_numpy(self.plan_host).to(dev)
        self._fused_call = None  # the one-launch step's marshalled arguments
        self.workspace = None
        if self.partition_size or self.cascade_chunk:
            rows, H, D = self.query.shape
            if all_queries:  # the one-launch step sizes rows as num_seqs x max_query_len
                rows = max(rows, len(seqs) * self.max_query_len)
            self.workspace = ops.alloc_split_workspace(rows, H, D, self.max_context_len,
                                                       self.partition_size or self.cascade_chunk,
                                                       dev)

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
        if self.cascade:
            ops.paged_attention_cascade(self.out, self.query, self.key_cache, self.value_cache,
                                        self.block_tables, self.context_lens, self.scale,
                                        self.max_context_len,
                                        self.partition_size or self.cascade_chunk, self.plan,
                                        self.num_items, self.max_group, self.workspace,
                                        chunked=bool(self.cascade_chunk))
        elif self.prefill_rows and self.partition_size:
            ops.paged_attention_prefill_split(self.out, self.query, self.key_cache,
                                              self.value_cache, self.block_tables, self.row_seq,
                                              self.attn_lens, self.attn_qsl, self.scale,
                                              self.max_context_len, self.prefill_items,
                                              self.partition_size, self.workspace,
                                              self.sliding_window)
        elif self.prefill_rows:
            ops.paged_attention_prefill(self.out, self.query, self.key_cache, self.value_cache,
                                        self.block_tables, self.row_seq, self.attn_lens,
                                        self.attn_qsl, self.scale, self.max_context_len,
                                        self.prefill_items, self.sliding_window)
        elif self.all_queries:
            ops.paged_attention_multi(self.out, self.query, self.key_cache, self.value_cache,
                                      self.attn_tables, self.attn_lens, self.attn_qsl,
                                      self.attn_max_query_len, self.scale,
                                      self.max_context_len, self.partition_size, self.plan,
                                      self.workspace, self.attn_shared, self.sliding_window)
        elif self.planned:
            ops.paged_attention_decode_planned(self.out, self.query, self.key_cache,
                                               self.value_cache, self.block_tables,
                                               self.context_lens, self.scale,
                                               self.max_context_len, self.partition_size,
                                               self.plan, self.workspace, self.shared_blocks,
                                               self.sliding_window)
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
        """The whole step as one launch (pa_decode_step, or pa_prefill_step for
        query blocks on the prefill kernel).  The arguments are
        checked and marshalled on the first call (or by prepare_fused); later
        calls launch them on the current stream."""
        self.prepare_fused()
        ops.launch_prepared(self._fused_call)

    def prepare_fused(self):
        """The one-launch step's checks and argument marshalling, without a
        launch (host only; done once)."""
        if not self.fused_ok:
            raise ValueError("a copy-on-write of a block of several kernel blocks, query "
                             "blocks on the decode kernels (they read each other's new rows "
                             "from the cache) or split query blocks need the separate calls: "
                             "run the step unfused")
        if self._fused_call is None:
            if self.prefill_rows:
                self._fused_call = ops.prepare_prefill_step(
                    self.out, self.query, self.key_cache, self.value_cache, self.block_tables,
                    self.row_seq, self.attn_lens, self.attn_qsl, self.scale,
                    self.max_context_len, self.query_start_loc, self.new_key, self.new_value,
                    self.cow_src, self.slot_mapping, self.prefill_items, self.sliding_window)
            elif self.cascade:
                self._fused_call = ops.prepare_decode_step_cascade(
                    self.out, self.query, self.key_cache, self.value_cache, self.block_tables,
                    self.context_lens, self.scale, self.max_context_len,
                    self.partition_size or self.cascade_chunk, self.plan, self.num_items,
                    self.max_group, self.query_start_loc, self.new_key, self.new_value,
                    self.cow_src, self.slot_mapping, self.workspace, self.shared_blocks,
                    chunked=bool(self.cascade_chunk))
            else:
                self._fused_call = ops.prepare_decode_step(
                    self.out, self.query, self.key_cache, self.value_cache, self.block_tables,
                    self.context_lens, self.scale, self.max_context_len, self.partition_size,
                    self.plan, self.query_start_loc, self.new_key, self.new_value,
                    self.cow_src, self.slot_mapping, self.workspace, self.shared_blocks,
                    self.max_query_len, self.sliding_window)

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
