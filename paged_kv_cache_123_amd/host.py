"""Python handle on the C++ host block allocator (pa_pool_* in pagedkv.h)."""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import PA_ENOMEM, PagedKVError, check, lib


class PoolExhausted(PagedKVError):
    """pa_pool_append returned PA_ENOMEM (the pool is unchanged)."""


def _p32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _p64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


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

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib().pa_pool_destroy(h)
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
