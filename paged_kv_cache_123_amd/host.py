"""Python handle on the C++ host block allocator (pa_pool_* in pagedkv.h)."""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._lib import PA_ENOMEM, PagedKVError, check, lib


class PoolExhausted(PagedKVError):
    """pa_pool_append returned PA_ENOMEM (the pool is unchanged)."""


def _p32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _p64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


@dataclass
class StepAppends:
    """What pa_pool_append_batch hands back for one step (host arrays)."""
    positions: np.ndarray        # int64 [T]
    query_start_loc: np.ndarray  # int32 [S + 1]
    slots: np.ndarray            # int64 [T]
    cow_src: np.ndarray          # int64 [S], -1: no copy
    cow_pairs: np.ndarray        # int64 [P, 2], kernel blocks
    shared_blocks: np.ndarray    # int32 [S], kernel blocks
    group_keys: np.ndarray       # int32 [S]


class Pool:
    """A pool of ``num_blocks`` physical blocks of ``block_size`` slots."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        handle = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.size != self.num_blocks:
                raise ValueError("free_order must hold num_blocks entries")
        check(lib().pa_pool_create(self.num_blocks, self.block_size,
                                   None if order is None else _p32(order),
                                   ctypes.byref(handle)))
        self._h = handle
        # kept here: at interpreter exit the module's globals may already be
        # gone when the last pools are collected
        self._destroy = lib().pa_pool_destroy

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    def add_seq(self, seq: int) -> None:
        check(lib().pa_pool_add_seq(self._h, seq))

    def fork(self, parent: int, child: int) -> None:
        check(lib().pa_pool_fork(self._h, parent, child))

    def append(self, seq: int, n: int):
        """Returns (slots int64 [n], cow pair (src, dst) or None)."""
        slots = np.empty(n, dtype=np.int64)
        cow = np.empty(2, dtype=np.int64)
        n_cow = ctypes.c_int32(0)
        st = lib().pa_pool_append(self._h, seq, n, _p64(slots), _p64(cow), ctypes.byref(n_cow))
        if st == PA_ENOMEM:
            raise PoolExhausted(st, lib().pa_last_error().decode())
        check(st)
        return slots, ((int(cow[0]), int(cow[1])) if n_cow.value else None)

    def append_batch(self, seqs, num_new, sliding_window: int = 0,
                     blocks_per_kv_block: int = 1) -> "StepAppends":
        """The appends of one step, all or nothing (pa_pool_append_batch):
        row r releases what its window left (sliding_window > 0), then appends
        num_new[r] tokens to seqs[r].  Raises PoolExhausted (or PagedKVError
        for an unknown or repeated sequence, or a count < 1) with the pool
        unchanged."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = np.ascontiguousarray(np.asarray(num_new, dtype=np.int32))
        if ids.ndim != 1 or n.shape != ids.shape or ids.size < 1:
            raise ValueError("one new-token count per sequence, at least one sequence")
        k = int(blocks_per_kv_block)
        total = int(n.astype(np.int64).sum()) if (n >= 1).all() else 0
        out = StepAppends(
            positions=np.empty(max(total, 1), dtype=np.int64),
            query_start_loc=np.empty(ids.size + 1, dtype=np.int32),
            slots=np.empty(max(total, 1), dtype=np.int64),
            cow_src=np.empty(ids.size, dtype=np.int64),
            cow_pairs=np.empty((ids.size * max(k, 1), 2), dtype=np.int64),
            shared_blocks=np.empty(ids.size, dtype=np.int32),
            group_keys=np.empty(ids.size, dtype=np.int32))
        n_pairs = ctypes.c_int32(0)
        st = lib().pa_pool_append_batch(
            self._h, _p64(ids), _p32(n), ids.size, int(sliding_window), k,
            _p64(out.positions), _p32(out.query_start_loc), _p64(out.slots), _p64(out.cow_src),
            _p64(out.cow_pairs), ctypes.byref(n_pairs), _p32(out.shared_blocks),
            _p32(out.group_keys))
        if st == PA_ENOMEM:
            raise PoolExhausted(st, lib().pa_last_error().decode())
        check(st)
        out.positions = out.positions[:total]
        out.slots = out.slots[:total]
        out.cow_pairs = out.cow_pairs[:n_pairs.value]
        return out

    def free_seq(self, seq: int) -> None:
        check(lib().pa_pool_free_seq(self._h, seq))

    def remove_skipped(self, seq: int, num_computed_tokens: int, sliding_window: int) -> int:
        """Release the blocks of ``seq`` wholly before its next query's
        window; returns how many were released (their entries become -1)."""
        n = ctypes.c_int32(0)
        check(lib().pa_pool_remove_skipped(self._h, seq, num_computed_tokens, sliding_window,
                                           ctypes.byref(n)))
        return n.value

    def seq_len(self, seq: int) -> int:
        out = ctypes.c_int64()
        check(lib().pa_pool_seq_len(self._h, seq, ctypes.byref(out)))
        return out.value

    def seq_num_blocks(self, seq: int) -> int:
        out = ctypes.c_int32()
        check(lib().pa_pool_seq_num_blocks(self._h, seq, ctypes.byref(out)))
        return out.value

    def block_tables(self, seqs, width: int):
        """(tables int32 [len(seqs), width] padded with -1, lengths int32)."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        out = np.empty((ids.size, width), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        check(lib().pa_pool_block_tables(self._h, _p64(ids), ids.size, _p32(out), width,
                                         _p32(lens)))
        return out, lens

    def block_table(self, seq: int) -> list:
        """Physical blocks of ``seq`` in logical order; released ones are -1."""
        n = self.seq_num_blocks(seq)
        t, _ = self.block_tables([seq], max(n, 1))
        return [int(b) for b in t[0, :n]]

    def shared_prefix_blocks(self, seqs) -> np.ndarray:
        """int32 [len(seqs)]: leading blocks of each table with reference count > 1."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        out = np.empty(ids.size, dtype=np.int32)
        check(lib().pa_pool_shared_prefix_blocks(self._h, _p64(ids), ids.size, _p32(out)))
        return out

    def num_free(self) -> int:
        return int(lib().pa_pool_num_free(self._h))

    def ref(self, block: int) -> int:
        return int(lib().pa_pool_ref(self._h, block))

    def free_queue(self) -> list:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = lib().pa_pool_free_queue(self._h, _p32(out), self.num_blocks)
        return [int(b) for b in out[:n]]

    def num_cow(self) -> int:
        return int(lib().pa_pool_num_cow(self._h))

    # ---- prefix caching ----------------------------------------------------
    def enable_prefix_caching(self) -> None:
        check(lib().pa_pool_enable_prefix_caching(self._h))

    def add_seq_cached(self, seq: int, prompt, extra: bytes = b"") -> int:
        """New sequence for ``prompt`` (token ids); returns how many of its
        tokens were taken over from the cache."""
        toks = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
        done = ctypes.c_int64(0)
        check(lib().pa_pool_add_seq_cached(self._h, seq, _p32(toks), toks.size,
                                           extra if extra else None, len(extra),
                                           ctypes.byref(done)))
        return done.value

    def append_tokens(self, seq: int, tokens):
        """append() that records the token ids for later caching."""
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = toks.size
        slots = np.empty(n, dtype=np.int64)
        cow = np.empty(2, dtype=np.int64)
        n_cow = ctypes.c_int32(0)
        st = lib().pa_pool_append_tokens(self._h, seq, _p32(toks), n, _p64(slots), _p64(cow),
                                         ctypes.byref(n_cow))
        if st == PA_ENOMEM:
            raise PoolExhausted(st, lib().pa_last_error().decode())
        check(st)
        return slots, ((int(cow[0]), int(cow[1])) if n_cow.value else None)

    def cache_full_blocks(self, seq: int) -> int:
        n = ctypes.c_int32(0)
        check(lib().pa_pool_cache_full_blocks(self._h, seq, ctypes.byref(n)))
        return n.value

    def num_cached_blocks(self) -> int:
        return int(lib().pa_pool_num_cached_blocks(self._h))

    def num_evicted(self) -> int:
        return int(lib().pa_pool_num_evicted(self._h))


def block_keys(tokens, block_size: int, extra: bytes = b"") -> list:
    """Chained keys (32 bytes each) of the full blocks of a token sequence."""
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    nk = toks.size // block_size
    out = np.zeros((max(nk, 1), 32), dtype=np.uint8)
    check(lib().pa_block_keys(_p32(toks), toks.size, block_size, extra if extra else None,
                              len(extra), out.ctypes.data))
    return [bytes(out[j]) for j in range(nk)]
