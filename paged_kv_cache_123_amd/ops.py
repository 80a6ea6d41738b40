"""Torch-tensor front end of the device entry points of pagedkv.h.

Argument marshalling only: shapes, dtypes and devices are checked here, sizes
are read off the tensors, and the call goes to the HIP library on the current
torch stream.  Every computation happens in the library's kernels.

Tensor shapes (see include/pagedkv.h for the semantics):
  key_cache, value_cache  [num_blocks, num_kv_heads, block_size, head_size]
  query, out              [num_seqs, num_heads, head_size]
  block_tables            int32 [num_seqs, width]
  context_lens            int32 [num_seqs]
  key, value (new tokens) [num_tokens, num_kv_heads, head_size] (token stride free)
  slot_mapping            int64 [>= num_tokens]
  block_mapping           int64 [num_pairs, 2]
"""

from __future__ import annotations

import torch

import ctypes

import numpy as np

from ._lib import PA_BF16, PA_F16, PA_F32, check, lib

_DTYPES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported storage dtype {t.dtype}") from None


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("pagedkv kernels take device tensors")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _contig(name: str, t: torch.Tensor) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _cache_shape(key_cache: torch.Tensor, value_cache: torch.Tensor):
    if key_cache.dim() != 4 or key_cache.shape != value_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_size]")
    if key_cache.dtype != value_cache.dtype:
        raise ValueError("key and value caches differ in dtype")
    _contig("key_cache", key_cache)
    _contig("value_cache", value_cache)
    return tuple(int(x) for x in key_cache.shape)


def compute_slot_mapping(query_start_loc: torch.Tensor, positions: torch.Tensor,
                         block_tables: torch.Tensor, block_size: int,
                         slot_mapping: torch.Tensor, num_tokens: int) -> None:
    """slot_mapping[i] = block_tables[r, pos_i // B] * B + pos_i % B; tail -> -1."""
    _dev(query_start_loc, positions, block_tables, slot_mapping)
    if query_start_loc.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise TypeError("query_start_loc and block_tables must be int32")
    if positions.dtype != torch.int64 or slot_mapping.dtype != torch.int64:
        raise TypeError("positions and slot_mapping must be int64")
    for n, t in (("query_start_loc", query_start_loc), ("positions", positions),
                 ("block_tables", block_tables), ("slot_mapping", slot_mapping)):
        _contig(n, t)
    num_reqs = query_start_loc.numel() - 1
    if block_tables.dim() != 2 or block_tables.shape[0] < num_reqs:
        raise ValueError("block_tables must be [>= num_reqs, width]")
    if positions.numel() < num_tokens:
        raise ValueError("positions shorter than num_tokens")
    check(lib().pa_compute_slot_mapping(
        query_start_loc.data_ptr(), positions.data_ptr(), block_tables.data_ptr(),
        block_tables.stride(0), num_reqs, num_tokens, slot_mapping.numel(), block_size,
        slot_mapping.data_ptr(), _stream()))


def compute_slot_mapping_cp(query_start_loc: torch.Tensor, positions: torch.Tensor,
                            block_tables: torch.Tensor, block_size: int,
                            slot_mapping: torch.Tensor, num_tokens: int, cp_world: int,
                            cp_rank: int, interleave: int = 1) -> None:
    """Rank ``cp_rank``'s slots under context parallelism (-1 for the tokens
    other ranks store, and for the padding tail)."""
    _dev(query_start_loc, positions, block_tables, slot_mapping)
    if query_start_loc.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise TypeError("query_start_loc and block_tables must be int32")
    if positions.dtype != torch.int64 or slot_mapping.dtype != torch.int64:
        raise TypeError("positions and slot_mapping must be int64")
    for n, t in (("query_start_loc", query_start_loc), ("positions", positions),
                 ("block_tables", block_tables), ("slot_mapping", slot_mapping)):
        _contig(n, t)
    num_reqs = query_start_loc.numel() - 1
    if block_tables.dim() != 2 or block_tables.shape[0] < num_reqs:
        raise ValueError("block_tables must be [>= num_reqs, width]")
    if positions.numel() < num_tokens:
        raise ValueError("positions shorter than num_tokens")
    check(lib().pa_compute_slot_mapping_cp(
        query_start_loc.data_ptr(), positions.data_ptr(), block_tables.data_ptr(),
        block_tables.stride(0), num_reqs, num_tokens, slot_mapping.numel(), block_size,
        cp_world, cp_rank, interleave, slot_mapping.data_ptr(), _stream()))


def cp_local_context_lens(context_lens, block_size: int, cp_world: int, cp_rank: int,
                          interleave: int = 1) -> np.ndarray:
    """Host int32: how many positions of each sequence rank ``cp_rank`` stores."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    out = np.empty_like(lens)
    p32 = ctypes.POINTER(ctypes.c_int32)
    check(lib().pa_cp_local_context_lens(lens.ctypes.data_as(p32), lens.size, block_size,
                                         cp_world, cp_rank, interleave,
                                         out.ctypes.data_as(p32)))
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Store each new token's K/V rows at its slot (slots < 0 are skipped)."""
    _dev(key, value, key_cache, value_cache, slot_mapping)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise TypeError("new K/V must have the cache dtype")
    if key.dim() != 3 or tuple(key.shape[1:]) != (hkv, D) or value.shape != key.shape:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_size]")
    for n, t in (("key", key), ("value", value)):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{n} rows must be contiguous [num_kv_heads, head_size]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() < key.shape[0]:
        raise ValueError("slot_mapping must be int64 with an entry per token")
    check(lib().pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0), key_cache.data_ptr(),
        value_cache.data_ptr(), slot_mapping.data_ptr(), key.shape[0], hkv, D, B,
        _dtype(key_cache), _stream()))


def validate_tables(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                    num_blocks: int, sliding_window: int = 0, result=None):
    """Device check of tables and lengths; returns (invalid sequences, the
    smallest invalid sequence or None).  Synchronises the stream."""
    _dev(block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    _contig("context_lens", context_lens)
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [num_seqs, width] with unit column stride")
    S = context_lens.numel()
    if block_tables.shape[0] < S:
        raise ValueError("block_tables has fewer rows than context_lens")
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=block_tables.device)
    check(lib().pa_validate_tables(block_tables.data_ptr(), block_tables.stride(0),
                                   context_lens.data_ptr(), S, block_size, num_blocks,
                                   sliding_window, result.data_ptr(), _stream()))
    bad, first = (int(x) for x in result.cpu())
    return bad, (None if bad == 0 else first)


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                block_mapping: torch.Tensor) -> None:
    """cache[dst] = cache[src] for every (src, dst) row, key and value."""
    _dev(key_cache, value_cache, block_mapping)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if block_mapping.dtype != torch.int64 or (block_mapping.numel() and
                                              tuple(block_mapping.shape[1:]) != (2,)):
        raise ValueError("block_mapping must be int64 [num_pairs, 2]")
    _contig("block_mapping", block_mapping)
    n = block_mapping.shape[0] if block_mapping.numel() else 0
    check(lib().pa_copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(),
                               block_mapping.data_ptr(), n, hkv, D, B, _dtype(key_cache),
                               _stream()))


def _attn_common(out, query, key_cache, value_cache, block_tables, context_lens,
                 check_out_dtype=True):
    _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != D or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if query.dtype != key_cache.dtype or (check_out_dtype and out.dtype != key_cache.dtype):
        raise TypeError("query/out must have the cache dtype")
    for n, t in (("query", query), ("out", out), ("block_tables", block_tables),
                 ("context_lens", context_lens)):
        _contig(n, t)
    S = query.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] < S:
        raise ValueError("block_tables must be int32 [num_seqs, width]")
    if context_lens.dtype != torch.int32 or context_lens.numel() < S:
        raise ValueError("context_lens must be int32 [num_seqs]")
    return S, query.shape[1], hkv, D, B


def paged_attention_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float,
                           max_context_len: int) -> None:
    """Single-pass paged decode attention into ``out``."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables, context_lens)
    check(lib().pa_paged_attention_decode(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), _stream()))


DECODE_KERNELS = {"auto": 0, "valu": 1, "mfma": 2}


def set_decode_kernel(mode: str) -> str:
    """Select the attention kernel ("auto", "valu" or "mfma"); returns the
    previous choice.  Process-wide."""
    prev = lib().pa_set_decode_kernel(DECODE_KERNELS[mode])
    return {v: k for k, v in DECODE_KERNELS.items()}[prev]


def split_workspace_bytes(num_seqs: int, num_heads: int, head_size: int,
                          max_context_len: int, partition_size: int) -> int:
    return int(lib().pa_split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len,
                                              partition_size))


def alloc_split_workspace(num_seqs: int, num_heads: int, head_size: int, max_context_len: int,
                          partition_size: int, device) -> torch.Tensor:
    """A byte tensor large enough for the split-K workspace (256-byte aligned)."""
    n = split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len, partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def paged_attention_decode_split(out: torch.Tensor, query: torch.Tensor,
                                 key_cache: torch.Tensor, value_cache: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                                 scale: float, max_context_len: int, partition_size: int,
                                 workspace: torch.Tensor) -> None:
    """Split-K paged decode attention (partition kernel + reduce kernel)."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables, context_lens)
    _dev(workspace)
    check(lib().pa_paged_attention_decode_split(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), partition_size, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))


def paged_attention_decode_split_noalloc(out: torch.Tensor, query: torch.Tensor,
                                         key_cache: torch.Tensor, value_cache: torch.Tensor,
                                         block_tables: torch.Tensor, context_lens: torch.Tensor,
                                         scale: float, max_context_len: int,
                                         partition_size: int) -> None:
    """Split-K decode whose workspace is the library's static device array
    (pa_paged_attention_decode_split_noalloc): nothing is allocated."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables,
                                   context_lens)
    check(lib().pa_paged_attention_decode_split_noalloc(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), partition_size, _stream()))


def workspace_views(workspace: torch.Tensor, num_seqs: int, num_heads: int, head_size: int,
                    max_context_len: int, partition_size: int):
    """(max_logits [S,H,NP], exp_sums [S,H,NP], tmp_out [S,H,NP,D]) views of a
    split workspace, in the layout pagedkv.h documents."""
    offs = np.zeros(3, dtype=np.int64)
    nparts = ctypes.c_int32(0)
    check(lib().pa_split_workspace_layout(num_seqs, num_heads, head_size, max_context_len,
                                          partition_size,
                                          offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          ctypes.byref(nparts)))
    shape = (num_seqs, num_heads, nparts.value)
    f = workspace.view(torch.uint8)

    def section(i, per_part):
        n = int(np.prod(shape)) * per_part * 4
        return f[int(offs[i]):int(offs[i]) + n].view(torch.float32)

    return (section(0, 1).view(shape), section(1, 1).view(shape),
            section(2, head_size).view(*shape, head_size))


def _shared_ptr(shared_prefix_blocks, S):
    if shared_prefix_blocks is None:
        return None
    _dev(shared_prefix_blocks)
    if shared_prefix_blocks.dtype != torch.int32 or shared_prefix_blocks.numel() < S:
        raise ValueError("shared_prefix_blocks must be int32 [num_seqs]")
    return shared_prefix_blocks.data_ptr()


def decode_plan(context_lens, partition_size: int, sliding_window: int = 0,
                query_lens=None, group_keys=None) -> np.ndarray:
    """Host work plan: int32 [num_items, 2] of (sequence, partition), every
    non-empty item once, largest first (partition_size 0: one per sequence).
    With a sliding window, only the items inside each sequence's window;
    ``query_lens`` (new tokens per sequence) place its first query.
    ``group_keys``: items of one size bucket run in key order (readers of a
    shared prefix together)."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    n = ctypes.c_int64(0)
    p32 = ctypes.POINTER(ctypes.c_int32)

    def opt(x):
        if x is None:
            return None, None
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
        if a.size != lens.size:
            raise ValueError("per-sequence arrays must have one entry per sequence")
        return a, a.ctypes.data_as(p32)

    qlens, qp = opt(query_lens)
    gkeys, gp = opt(group_keys)
    check(lib().pa_decode_plan_window(lens.ctypes.data_as(p32), qp, gp, lens.size,
                                      partition_size, sliding_window, None, 0, ctypes.byref(n)))
    items = np.empty((n.value, 2), dtype=np.int32)
    check(lib().pa_decode_plan_window(lens.ctypes.data_as(p32), qp, gp, lens.size,
                                      partition_size, sliding_window,
                                      items.ctypes.data_as(p32), n.value, ctypes.byref(n)))
    return items


def decode_plan_cascade(block_tables, context_lens, block_size: int, partition_size: int,
                        max_group_size: int, new_tokens=None, chunk_tokens: int = 0):
    """Host cascade plan (pa_decode_plan_cascade): partitions wholly inside a
    prefix several sequences share become one group item per chunk of at most
    ``max_group_size`` sharers; with ``partition_size`` 0, one single-pass item
    per chunk (prefix once, then each member's own tokens).  With
    ``chunk_tokens`` > 0 (``partition_size`` ignored) the chunked plan
    (pa_decode_plan_cascade_chunked): each prefix in pieces of chunk_tokens
    plus one item for the rest and the members' own tokens, all writing
    partials.  Returns (plan int32 1-D: items then the group section,
    num_items, max_members)."""
    tables = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if tables.ndim != 2 or tables.shape[0] != lens.size:
        raise ValueError("block_tables must be [num_seqs, width]")
    p32 = ctypes.POINTER(ctypes.c_int32)
    newp = None
    if new_tokens is not None:
        new = np.ascontiguousarray(np.asarray(new_tokens, dtype=np.int32))
        if new.size != lens.size:
            raise ValueError("new_tokens must have one entry per sequence")
        newp = new.ctypes.data_as(p32)
    n, plen, widest = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    fn = lib().pa_decode_plan_cascade_chunked if chunk_tokens else lib().pa_decode_plan_cascade
    args = (lens.ctypes.data_as(p32), tables.ctypes.data_as(p32), tables.shape[1], newp,
            lens.size, block_size, chunk_tokens or partition_size, max_group_size)
    check(fn(*args, None, 0, ctypes.byref(n), ctypes.byref(plen), ctypes.byref(widest)))
    plan = np.empty(plen.value, dtype=np.int32)
    check(fn(*args, plan.ctypes.data_as(p32), plan.size, ctypes.byref(n), ctypes.byref(plen),
             ctypes.byref(widest)))
    return plan, n.value, widest.value


def cascade_auto_chunk(block_tables, context_lens, block_size: int, max_group_size: int,
                       num_kv_heads: int, new_tokens=None) -> int:
    """The chunk_tokens a cascade step takes on its own (pa_cascade_auto_chunk):
    0 for the single-pass plan."""
    tables = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if tables.ndim != 2 or tables.shape[0] != lens.size:
        raise ValueError("block_tables must be [num_seqs, width]")
    p32 = ctypes.POINTER(ctypes.c_int32)
    newp = None
    if new_tokens is not None:
        new = np.ascontiguousarray(np.asarray(new_tokens, dtype=np.int32))
        newp = new.ctypes.data_as(p32)
    out = ctypes.c_int32(0)
    check(lib().pa_cascade_auto_chunk(lens.ctypes.data_as(p32), tables.ctypes.data_as(p32),
                                      tables.shape[1], newp, lens.size, block_size,
                                      max_group_size, num_kv_heads, ctypes.byref(out)))
    return out.value


def query_blocks(context_lens, query_start_loc, max_block: int):
    """Host query blocks (pa_query_blocks): each sequence's new tokens cut into
    rows of at most ``max_block`` tokens.  Returns (row_seq, row_lens, row_qsl)
    as int32 arrays."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    qsl = np.ascontiguousarray(np.asarray(query_start_loc, dtype=np.int32))
    if qsl.size != lens.size + 1:
        raise ValueError("query_start_loc must have num_seqs + 1 entries")
    p32 = ctypes.POINTER(ctypes.c_int32)
    rows = ctypes.c_int64(0)
    check(lib().pa_query_blocks(lens.ctypes.data_as(p32), qsl.ctypes.data_as(p32), lens.size,
                                max_block, None, None, None, 0, ctypes.byref(rows)))
    n = rows.value
    row_seq = np.empty(n, np.int32)
    row_lens = np.empty(n, np.int32)
    row_qsl = np.empty(n + 1, np.int32)
    check(lib().pa_query_blocks(lens.ctypes.data_as(p32), qsl.ctypes.data_as(p32), lens.size,
                                max_block, row_seq.ctypes.data_as(p32),
                                row_lens.ctypes.data_as(p32), row_qsl.ctypes.data_as(p32), n,
                                ctypes.byref(rows)))
    return row_seq, row_lens, row_qsl


def cascade_max_group(num_heads: int, num_kv_heads: int, head_size: int, dtype) -> int:
    """Widest group a cascade plan may take for this shape (pa_cascade_max_group);
    ``dtype`` is a torch dtype or "f32" / "f16" / "bf16"."""
    code = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16}.get(dtype) if isinstance(
        dtype, str) else {torch.float32: PA_F32, torch.float16: PA_F16,
                          torch.bfloat16: PA_BF16}[dtype]
    g = ctypes.c_int32(0)
    check(lib().pa_cascade_max_group(num_heads, num_kv_heads, head_size, code, ctypes.byref(g)))
    return g.value


def query_block_hints(row_seq, row_lens, seq_shared_blocks, block_size: int) -> np.ndarray:
    """Shared-block cache hints of query-block rows (pa_query_block_hints):
    int32 [num_rows]."""
    rs = np.ascontiguousarray(np.asarray(row_seq, dtype=np.int32))
    rl = np.ascontiguousarray(np.asarray(row_lens, dtype=np.int32))
    sh = np.ascontiguousarray(np.asarray(seq_shared_blocks, dtype=np.int32))
    out = np.empty(rs.size, dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    check(lib().pa_query_block_hints(rs.ctypes.data_as(p32), rl.ctypes.data_as(p32), rs.size,
                                     sh.ctypes.data_as(p32), sh.size, block_size,
                                     out.ctypes.data_as(p32)))
    return out


def prefill_plan(row_seq, row_lens, row_qlens=None, sliding_window: int = 0) -> np.ndarray:
    """Launch order of the prefill kernel's rows (pa_prefill_plan): host
    int32 [num_rows, 2] of (row, 0), for work_items."""
    rs = np.ascontiguousarray(np.asarray(row_seq, dtype=np.int32))
    rl = np.ascontiguousarray(np.asarray(row_lens, dtype=np.int32))
    p32 = ctypes.POINTER(ctypes.c_int32)
    qp = None
    if row_qlens is not None:
        rq = np.ascontiguousarray(np.asarray(row_qlens, dtype=np.int32))
        if rq.size != rs.size:
            raise ValueError("row_qlens must have one entry per row")
        qp = rq.ctypes.data_as(p32)
    if rl.size != rs.size:
        raise ValueError("row_lens must have one entry per row")
    out = np.empty((rs.size, 2), dtype=np.int32)
    check(lib().pa_prefill_plan(rs.ctypes.data_as(p32), rl.ctypes.data_as(p32), qp, rs.size,
                                sliding_window, out.ctypes.data_as(p32)))
    return out


def prefill_plan_split(row_seq, row_lens, row_qlens, sliding_window: int,
                       partition_size: int) -> np.ndarray:
    """Work list of the split prefill kernel (pa_prefill_plan_split): host
    int32 [num_items, 2] of (row, partition)."""
    rs = np.ascontiguousarray(np.asarray(row_seq, dtype=np.int32))
    rl = np.ascontiguousarray(np.asarray(row_lens, dtype=np.int32))
    rq = np.ascontiguousarray(np.asarray(row_qlens, dtype=np.int32))
    if rl.size != rs.size or rq.size != rs.size:
        raise ValueError("row_lens and row_qlens must have one entry per row")
    p32 = ctypes.POINTER(ctypes.c_int32)
    n = ctypes.c_int64(0)
    args = (rs.ctypes.data_as(p32), rl.ctypes.data_as(p32), rq.ctypes.data_as(p32), rs.size,
            sliding_window, partition_size)
    check(lib().pa_prefill_plan_split(*args, None, 0, ctypes.byref(n)))
    out = np.empty((max(n.value, 1), 2), dtype=np.int32)
    check(lib().pa_prefill_plan_split(*args, out.ctypes.data_as(p32), n.value, ctypes.byref(n)))
    return out[:n.value]


def prefill_auto_partition(num_rows: int, num_kv_heads: int, max_row_len: int,
                           block_size: int) -> int:
    """Partition size for the split prefill when one pass would leave the GPU
    mostly idle, else 0 (pa_prefill_auto_partition)."""
    p = ctypes.c_int32(0)
    check(lib().pa_prefill_auto_partition(num_rows, num_kv_heads, max_row_len, block_size,
                                          ctypes.byref(p)))
    return p.value


def prefill_block_tokens(num_heads: int, num_kv_heads: int) -> int:
    """New tokens per query block of the prefill kernel (pa_prefill_block_tokens)."""
    t = ctypes.c_int32(0)
    check(lib().pa_prefill_block_tokens(num_heads, num_kv_heads, ctypes.byref(t)))
    return t.value


def map_to_kernel_blocks(manager_ids, blocks_per_kv_block: int) -> np.ndarray:
    """Host int32 kernel block ids of manager block ids (any shape; the last
    axis grows by ``blocks_per_kv_block``); -1 entries stay -1."""
    ids = np.ascontiguousarray(np.asarray(manager_ids, dtype=np.int32))
    out = np.empty(ids.shape[:-1] + (ids.shape[-1] * blocks_per_kv_block,) if ids.ndim else
                   (blocks_per_kv_block,), dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    check(lib().pa_map_to_kernel_blocks(ids.ctypes.data_as(p32), ids.size, blocks_per_kv_block,
                                        out.ctypes.data_as(p32)))
    return out


def paged_attention_decode_planned(out: torch.Tensor, query: torch.Tensor,
                                   key_cache: torch.Tensor, value_cache: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   scale: float, max_context_len: int, partition_size: int,
                                   work_items: torch.Tensor, workspace=None,
                                   shared_prefix_blocks=None, sliding_window: int = 0) -> None:
    """Attention driven by a work plan (device int32 [num_items, 2]).
    ``shared_prefix_blocks``: optional device int32 [num_seqs] cache hint;
    ``sliding_window``: attend to the last W tokens only (0: all)."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables, context_lens)
    _dev(work_items)
    if work_items.dtype != torch.int32 or work_items.dim() != 2 or work_items.shape[1] != 2:
        raise ValueError("work_items must be int32 [num_items, 2]")
    _contig("work_items", work_items)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().pa_paged_attention_decode_planned(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), partition_size, work_items.data_ptr(),
        work_items.shape[0], _shared_ptr(shared_prefix_blocks, S), ws_ptr or None, ws_bytes,
        sliding_window, _stream()))


def paged_attention_partials(max_logits: torch.Tensor, exp_sums: torch.Tensor,
                             partial_out: torch.Tensor, query: torch.Tensor,
                             key_cache: torch.Tensor, value_cache: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor,
                             scale: float, max_context_len: int, partition_size: int,
                             workspace=None, work_items=None, shared_prefix_blocks=None) -> None:
    """Rank-local attention partials: fp32 max_logits / exp_sums [S, H] and
    partial_out [S, H, D] over the tokens of this rank's cache."""
    S, H, hkv, D, B = _attn_common(partial_out, query, key_cache, value_cache, block_tables,
                                   context_lens, check_out_dtype=False)
    _dev(max_logits, exp_sums)
    for n, t in (("max_logits", max_logits), ("exp_sums", exp_sums),
                 ("partial_out", partial_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
        _contig(n, t)
    if max_logits.shape != (S, H) or exp_sums.shape != (S, H):
        raise ValueError("max_logits and exp_sums must be [num_seqs, num_heads]")
    items_ptr, n_items = None, 0
    if work_items is not None:
        _dev(work_items)
        if work_items.dtype != torch.int32 or work_items.dim() != 2 or work_items.shape[1] != 2:
            raise ValueError("work_items must be int32 [num_items, 2]")
        _contig("work_items", work_items)
        items_ptr, n_items = work_items.data_ptr() or None, work_items.shape[0]
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().pa_paged_attention_partials(
        max_logits.data_ptr(), exp_sums.data_ptr(), partial_out.data_ptr(), query.data_ptr(),
        key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D, B, max_context_len,
        scale, _dtype(key_cache), partition_size, items_ptr, n_items,
        _shared_ptr(shared_prefix_blocks, S), ws_ptr or None, ws_bytes, _stream()))


def merge_attention_partials(out: torch.Tensor, max_logits: torch.Tensor,
                             exp_sums: torch.Tensor, partial_out: torch.Tensor) -> None:
    """out [S, H, D] from gathered rank partials: max_logits / exp_sums
    [N, S, H], partial_out [N, S, H, D] (fp32)."""
    _dev(out, max_logits, exp_sums, partial_out)
    if partial_out.dim() != 4:
        raise ValueError("partial_out must be [num_parts, num_seqs, num_heads, head_size]")
    N, S, H, D = (int(x) for x in partial_out.shape)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [num_seqs, num_heads, head_size]")
    for n, t in (("max_logits", max_logits), ("exp_sums", exp_sums),
                 ("partial_out", partial_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
        _contig(n, t)
    if tuple(max_logits.shape) != (N, S, H) or tuple(exp_sums.shape) != (N, S, H):
        raise ValueError("max_logits and exp_sums must be [num_parts, num_seqs, num_heads]")
    _contig("out", out)
    check(lib().pa_merge_attention_partials(
        out.data_ptr(), max_logits.data_ptr(), exp_sums.data_ptr(), partial_out.data_ptr(), N, S,
        H, D, _dtype(out), _stream()))


def probe_read_blocks(buffer: torch.Tensor, block_order: torch.Tensor, sink: torch.Tensor,
                      grid: int = 16384, non_temporal: bool = False) -> None:
    """Diagnostic: read ``buffer`` as whole 4 KiB blocks in ``block_order``."""
    _dev(buffer, block_order, sink)
    if block_order.dtype != torch.int32:
        raise TypeError("block_order must be int32")
    _contig("block_order", block_order)
    check(lib().pa_probe_read_blocks(buffer.data_ptr(), block_order.data_ptr(),
                                     block_order.numel(), sink.data_ptr(), grid,
                                     int(non_temporal), _stream()))


def timeline_reset() -> None:
    """Diagnostic: clear the cascade kernel's per-workgroup timeline (a
    library built with PA_TIMELINE=1 only; raises otherwise)."""
    check(lib().pa_timeline_reset(_stream()))


def timeline_read(capacity: int = 8192) -> np.ndarray:
    """Diagnostic: the timeline records of the last cascade launch, uint64
    [n, 4] (entry, tiles described, exit: 100 MHz counter; hardware ids)."""
    rec = np.zeros((capacity, 4), dtype=np.uint64)
    n = ctypes.c_int64(0)
    check(lib().pa_timeline_read(rec.ctypes.data, capacity, ctypes.byref(n)))
    return rec[:n.value].copy()


def decode_step(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                value_cache: torch.Tensor, block_tables: torch.Tensor,
                context_lens: torch.Tensor, scale: float, max_context_len: int,
                partition_size: int, work_items: torch.Tensor, query_start_loc: torch.Tensor,
                key: torch.Tensor, value: torch.Tensor, cow_src=None, slot_mapping=None,
                workspace=None, shared_prefix_blocks=None, max_query_len: int = 0,
                sliding_window: int = 0) -> None:
    """The whole decode step in one launch: copy-on-write of the old slots of
    fresh tail blocks (``cow_src`` int64 [num_seqs], -1 for none), the new
    tokens' K/V (rows of ``key``/``value`` per ``query_start_loc``) into their
    slots, and planned attention over the updated caches.  ``max_query_len``
    > 0 makes every new token a query (query/out [num_tokens, H, D])."""
    launch_prepared(prepare_decode_step(
        out, query, key_cache, value_cache, block_tables, context_lens, scale,
        max_context_len, partition_size, work_items, query_start_loc, key, value, cow_src,
        slot_mapping, workspace, shared_prefix_blocks, max_query_len, sliding_window))


def launch_prepared(prepared) -> None:
    """Launch a call prepared by prepare_decode_step or
    prepare_decode_step_cascade on the current stream: the tensors it names
    must still be alive and unchanged in shape."""
    fn, args = prepared
    check(fn(*args, _stream()))


def prepare_decode_step(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                        value_cache: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        partition_size: int, work_items: torch.Tensor,
                        query_start_loc: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                        cow_src=None, slot_mapping=None, workspace=None,
                        shared_prefix_blocks=None, max_query_len: int = 0,
                        sliding_window: int = 0):
    """decode_step's checks and argument marshalling, done once: returns what
    launch_prepared takes (the C function and its arguments but the stream),
    for a step launched repeatedly on the same tensors."""
    if max_query_len > 0:
        S = block_tables.shape[0]
        _dev(out, query, key_cache, value_cache, block_tables, context_lens)
        nb, hkv, B, D = _cache_shape(key_cache, value_cache)
        if out.shape != query.shape or query.dim() != 3 or query.shape[2] != D:
            raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
        H = query.shape[1]
    else:
        S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables,
                                       context_lens)
    _dev(work_items, query_start_loc, key, value)
    if query_start_loc.dtype != torch.int32 or query_start_loc.numel() < S + 1:
        raise ValueError("query_start_loc must be int32 [num_seqs + 1]")
    for n, t in (("key", key), ("value", value)):
        if t.dtype != key_cache.dtype or t.dim() != 3 or tuple(t.shape[1:]) != (hkv, D):
            raise ValueError(f"{n} must be [num_tokens, num_kv_heads, head_size] in cache dtype")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{n} rows must be contiguous [num_kv_heads, head_size]")
    cow_ptr = 0
    if cow_src is not None:
        _dev(cow_src)
        if cow_src.dtype != torch.int64 or cow_src.numel() < S:
            raise ValueError("cow_src must be int64 [num_seqs]")
        cow_ptr = cow_src.data_ptr()
    slot_ptr = 0
    if slot_mapping is not None:
        _dev(slot_mapping)
        if slot_mapping.dtype != torch.int64 or slot_mapping.numel() < key.shape[0]:
            raise ValueError("slot_mapping must be int64 [num_tokens]")
        slot_ptr = slot_mapping.data_ptr()
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return lib().pa_decode_step, (
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), partition_size, work_items.data_ptr(),
        work_items.shape[0], _shared_ptr(shared_prefix_blocks, S), ws_ptr or None, ws_bytes,
        query_start_loc.data_ptr(),
        key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0), cow_ptr or None,
        slot_ptr or None, max_query_len, sliding_window)


def decode_step_cascade(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                        value_cache: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        partition_size: int, plan: torch.Tensor, num_items: int,
                        max_group_size: int, query_start_loc: torch.Tensor, key: torch.Tensor,
                        value: torch.Tensor, cow_src=None, slot_mapping=None, workspace=None,
                        shared_prefix_blocks=None, chunked: bool = False) -> None:
    """decode_step over a cascade plan (decode_plan_cascade, uploaded as a
    device int32 tensor): the prefix of each group of sharers is read once
    for all of them (per shared partition, or in one single-pass item when
    ``partition_size`` is 0).  ``chunked``: a chunked plan, whose chunk_tokens
    is ``partition_size`` (pa_decode_step_cascade_chunked)."""
    launch_prepared(prepare_decode_step_cascade(
        out, query, key_cache, value_cache, block_tables, context_lens, scale,
        max_context_len, partition_size, plan, num_items, max_group_size, query_start_loc,
        key, value, cow_src, slot_mapping, workspace, shared_prefix_blocks, chunked))


def prepare_decode_step_cascade(out: torch.Tensor, query: torch.Tensor,
                                key_cache: torch.Tensor, value_cache: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                scale: float, max_context_len: int, partition_size: int,
                                plan: torch.Tensor, num_items: int, max_group_size: int,
                                query_start_loc: torch.Tensor, key: torch.Tensor,
                                value: torch.Tensor, cow_src=None, slot_mapping=None,
                                workspace=None, shared_prefix_blocks=None,
                                chunked: bool = False):
    """decode_step_cascade's checks and argument marshalling, done once (see
    prepare_decode_step)."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables,
                                   context_lens)
    _dev(plan, query_start_loc, key, value)
    if plan.dtype != torch.int32 or plan.dim() != 1 or plan.numel() < 2 * num_items + 2:
        raise ValueError("plan must be the int32 cascade plan")
    _contig("plan", plan)
    if query_start_loc.dtype != torch.int32 or query_start_loc.numel() < S + 1:
        raise ValueError("query_start_loc must be int32 [num_seqs + 1]")
    for n, t in (("key", key), ("value", value)):
        if t.dtype != key_cache.dtype or t.dim() != 3 or tuple(t.shape[1:]) != (hkv, D):
            raise ValueError(f"{n} must be [num_tokens, num_kv_heads, head_size] in cache dtype")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{n} rows must be contiguous [num_kv_heads, head_size]")
    cow_ptr = 0
    if cow_src is not None:
        _dev(cow_src)
        if cow_src.dtype != torch.int64 or cow_src.numel() < S:
            raise ValueError("cow_src must be int64 [num_seqs]")
        cow_ptr = cow_src.data_ptr()
    slot_ptr = 0
    if slot_mapping is not None:
        _dev(slot_mapping)
        if slot_mapping.dtype != torch.int64 or slot_mapping.numel() < key.shape[0]:
            raise ValueError("slot_mapping must be int64 [num_tokens]")
        slot_ptr = slot_mapping.data_ptr()
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    common = (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
              block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H,
              hkv, D, B, max_context_len, scale, _dtype(key_cache), partition_size,
              plan.data_ptr(), num_items, max_group_size)
    rest = (ws_ptr or None, ws_bytes, query_start_loc.data_ptr(), key.data_ptr(),
            value.data_ptr(), key.stride(0), value.stride(0), cow_ptr or None, slot_ptr or None)
    if chunked:
        return lib().pa_decode_step_cascade_chunked, common + rest
    return lib().pa_decode_step_cascade, common + (_shared_ptr(shared_prefix_blocks, S),) + rest


def paged_attention_cascade(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                            value_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, max_context_len: int,
                            partition_size: int, plan: torch.Tensor, num_items: int,
                            max_group_size: int, workspace=None, chunked: bool = False) -> None:
    """Attention alone over a cascade plan (pa_paged_attention_cascade, or
    pa_paged_attention_cascade_chunked with ``chunked``, ``partition_size``
    then being the plan's chunk_tokens), on caches that already hold the
    step's rows."""
    S, H, hkv, D, B = _attn_common(out, query, key_cache, value_cache, block_tables,
                                   context_lens)
    _dev(plan)
    if plan.dtype != torch.int32 or plan.dim() != 1 or plan.numel() < 2 * num_items + 2:
        raise ValueError("plan must be the int32 cascade plan")
    _contig("plan", plan)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    fn = lib().pa_paged_attention_cascade_chunked if chunked else lib().pa_paged_attention_cascade
    check(fn(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(), S, H, hkv, D,
        B, max_context_len, scale, _dtype(key_cache), partition_size, plan.data_ptr(),
        num_items, max_group_size, ws_ptr or None, ws_bytes, _stream()))


def paged_attention_prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                            value_cache: torch.Tensor, block_tables: torch.Tensor,
                            row_seq: torch.Tensor, row_lens: torch.Tensor, row_qsl: torch.Tensor,
                            scale: float, max_context_len: int, work_items=None,
                            sliding_window: int = 0) -> None:
    """Attention of every new token over query blocks (pa_paged_attention_prefill):
    row_seq/row_lens/row_qsl as from query_blocks with prefill_block_tokens;
    the step's cache writes must have run."""
    _dev(out, query, key_cache, value_cache, block_tables, row_seq, row_lens, row_qsl)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != D or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    if query.dtype != key_cache.dtype or out.dtype != key_cache.dtype:
        raise TypeError("query/out must have the cache dtype")
    for n, t in (("query", query), ("out", out), ("block_tables", block_tables),
                 ("row_seq", row_seq), ("row_lens", row_lens), ("row_qsl", row_qsl)):
        _contig(n, t)
    R = row_seq.numel()
    for n, t, size in (("row_seq", row_seq, R), ("row_lens", row_lens, R),
                       ("row_qsl", row_qsl, R + 1)):
        if t.dtype != torch.int32 or t.numel() != size:
            raise ValueError(f"{n} must be int32 with {size} entries")
    items = 0
    if work_items is not None:
        _dev(work_items)
        _contig("work_items", work_items)
        if work_items.dtype != torch.int32 or work_items.shape != (R, 2):
            raise ValueError("work_items must be int32 [num_rows, 2]")
        items = work_items.data_ptr()
    check(lib().pa_paged_attention_prefill(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), row_seq.data_ptr(), row_lens.data_ptr(),
        row_qsl.data_ptr(), R, query.shape[1], hkv, D, B, max_context_len, scale,
        _dtype(key_cache), items or None, sliding_window, _stream()))


def paged_attention_prefill_split(out: torch.Tensor, query: torch.Tensor,
                                  key_cache: torch.Tensor, value_cache: torch.Tensor,
                                  block_tables: torch.Tensor, row_seq: torch.Tensor,
                                  row_lens: torch.Tensor, row_qsl: torch.Tensor, scale: float,
                                  max_context_len: int, work_items: torch.Tensor,
                                  partition_size: int, workspace: torch.Tensor,
                                  sliding_window: int = 0) -> None:
    """pa_paged_attention_prefill_split: the prefill kernel over (row,
    partition) work items (prefill_plan_split) and the merge; workspace from
    alloc_split_workspace(num_tokens, ...)."""
    _dev(out, query, key_cache, value_cache, block_tables, row_seq, row_lens, row_qsl,
         work_items, workspace)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != D or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    if query.dtype != key_cache.dtype or out.dtype != key_cache.dtype:
        raise TypeError("query/out must have the cache dtype")
    for n, t in (("query", query), ("out", out), ("block_tables", block_tables),
                 ("row_seq", row_seq), ("row_lens", row_lens), ("row_qsl", row_qsl),
                 ("work_items", work_items), ("workspace", workspace)):
        _contig(n, t)
    R = row_seq.numel()
    for n, t, size in (("row_seq", row_seq, R), ("row_lens", row_lens, R),
                       ("row_qsl", row_qsl, R + 1)):
        if t.dtype != torch.int32 or t.numel() != size:
            raise ValueError(f"{n} must be int32 with {size} entries")
    if work_items.dtype != torch.int32 or work_items.dim() != 2 or work_items.shape[1] != 2:
        raise ValueError("work_items must be int32 [num_items, 2]")
    check(lib().pa_paged_attention_prefill_split(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), row_seq.data_ptr(), row_lens.data_ptr(),
        row_qsl.data_ptr(), R, query.shape[1], hkv, D, B, max_context_len, scale,
        _dtype(key_cache), work_items.data_ptr(), work_items.shape[0], partition_size,
        sliding_window, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        query.shape[0], _stream()))


def prepare_prefill_step(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, block_tables: torch.Tensor,
                         row_seq: torch.Tensor, row_lens: torch.Tensor, row_qsl: torch.Tensor,
                         scale: float, max_context_len: int, query_start_loc: torch.Tensor,
                         key: torch.Tensor, value: torch.Tensor, cow_src=None,
                         slot_mapping=None, work_items=None, sliding_window: int = 0):
    """Check and marshal a pa_prefill_step call (prefill attention over query
    blocks with the step's copy-on-write and scatter in the same launch);
    launch it with launch_prepared."""
    _dev(out, query, key_cache, value_cache, block_tables, row_seq, row_lens, row_qsl,
         query_start_loc, key, value)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != D or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    for n, t in (("query", query), ("out", out), ("key", key), ("value", value)):
        if t.dtype != key_cache.dtype:
            raise TypeError(f"{n} must have the cache dtype")
    for n, t in (("query", query), ("out", out), ("block_tables", block_tables),
                 ("row_seq", row_seq), ("row_lens", row_lens), ("row_qsl", row_qsl),
                 ("query_start_loc", query_start_loc)):
        _contig(n, t)
    R = row_seq.numel()
    for n, t, size in (("row_seq", row_seq, R), ("row_lens", row_lens, R),
                       ("row_qsl", row_qsl, R + 1),
                       ("query_start_loc", query_start_loc, block_tables.shape[0] + 1)):
        if t.dtype != torch.int32 or t.numel() != size:
            raise ValueError(f"{n} must be int32 with {size} entries")
    T = query.shape[0]
    if key.shape != (T, hkv, D) or value.shape != (T, hkv, D):
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_size]")
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("key/value rows must be dense [num_kv_heads, head_size]")
    cow = 0
    if cow_src is not None:
        _dev(cow_src)
        if cow_src.dtype != torch.int64 or cow_src.numel() != block_tables.shape[0]:
            raise ValueError("cow_src must be int64 [num_seqs]")
        cow = cow_src.data_ptr()
    slots = 0
    if slot_mapping is not None:
        _dev(slot_mapping)
        if slot_mapping.dtype != torch.int64 or slot_mapping.numel() < T:
            raise ValueError("slot_mapping must be int64 [num_tokens]")
        slots = slot_mapping.data_ptr()
    items = 0
    if work_items is not None:
        _dev(work_items)
        _contig("work_items", work_items)
        if work_items.dtype != torch.int32 or work_items.shape != (R, 2):
            raise ValueError("work_items must be int32 [num_rows, 2]")
        items = work_items.data_ptr()
    return lib().pa_prefill_step, (
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), row_seq.data_ptr(), row_lens.data_ptr(),
        row_qsl.data_ptr(), R, query.shape[1], hkv, D, B, max_context_len, scale,
        _dtype(key_cache), items or None, sliding_window, query_start_loc.data_ptr(),
        key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0), cow or None,
        slots or None)


def prefill_step(*args, **kw) -> None:
    """pa_prefill_step on the current stream (arguments as prepare_prefill_step)."""
    launch_prepared(prepare_prefill_step(*args, **kw))


def paged_attention_multi(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                          max_query_len: int, scale: float, max_context_len: int,
                          partition_size: int, work_items: torch.Tensor, workspace=None,
                          shared_prefix_blocks=None, sliding_window: int = 0) -> None:
    """Attention of every new token (query/out [num_tokens, H, D]), causal over
    each sequence's new tokens."""
    _dev(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
         work_items)
    nb, hkv, B, D = _cache_shape(key_cache, value_cache)
    if query.dim() != 3 or query.shape[2] != D or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    if query.dtype != key_cache.dtype or out.dtype != key_cache.dtype:
        raise TypeError("query/out must have the cache dtype")
    for n, t in (("query", query), ("out", out), ("block_tables", block_tables),
                 ("context_lens", context_lens), ("query_start_loc", query_start_loc),
                 ("work_items", work_items)):
        _contig(n, t)
    S = block_tables.shape[0]
    if query_start_loc.dtype != torch.int32 or query_start_loc.numel() < S + 1:
        raise ValueError("query_start_loc must be int32 [num_seqs + 1]")
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().pa_paged_attention_multi(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(),
        query_start_loc.data_ptr(), S, max_query_len, query.shape[1], hkv, D, B,
        max_context_len, scale, _dtype(key_cache), partition_size, work_items.data_ptr(),
        work_items.shape[0], _shared_ptr(shared_prefix_blocks, S), ws_ptr or None, ws_bytes,
        query.shape[0], sliding_window, _stream()))
