"""Planted mistakes in the oracle (CPU only): each one must break a pin.

Every case patches one oracle function with a plausible slip (a swapped
index, a dropped term, a wrong sign, a wrong queue end) and re-runs the pin
tests that should notice; the case passes when at least one of them fails.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle.allocator as alloc_mod
import oracle.attention as attn_mod
import oracle.prefix_cache as pc_mod
import oracle.slots as slots_mod
import test_oracle_allocator as TA
import test_oracle_attention as TT
import test_oracle_cp as TC
import test_oracle_slots as TS
import test_oracle_prefix_cache as TP
import test_oracle_window as TW


def _gather_swapped(cache, table_row, length, kv_head, block_size, start=0):
    t = np.arange(start, length)
    blocks = np.asarray(table_row, dtype=np.int64)[t % len(table_row)]
    return cache[blocks, kv_head, t % block_size, :]


def _attend_no_max(q, K, V, scale):
    x = scale * (K @ q)
    w = np.exp(x)
    return (w @ V) / w.sum()


def _attend_no_scale(q, K, V, scale):
    x = K @ q
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()


def _attend_unnormalised(q, K, V, scale):
    x = scale * (K @ q)
    w = np.exp(x - x.max())
    return w @ V


def _merge_wrong_sign(m, l, o):
    M = m.max()
    a = l * np.exp(M - m)
    return (a @ o) / a.sum()


def _merge_ignores_mass(m, l, o):
    a = np.exp(m - m.max())
    return (a @ o) / a.sum()


def _cp_owner_ignores_interleave(o, world, interleave):
    return o % world, (o // (world * interleave)) * interleave + o % interleave


def _cp_local_drops_run_offset(o, world, interleave):
    return (o // interleave) % world, (o // (world * interleave)) * interleave


def _partial_unnormalised(q, K, V, scale):
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    x = scale * (K @ q)
    m = x.max()
    w = np.exp(x - m)
    return m, w.sum(), w @ V


class _PrefixSkipsMisses(pc_mod.OraclePrefixPool):
    def longest_hit(self, keys, max_length):
        return [self.cached[k] for k in keys[:max_length // self.block_size] if k in self.cached]


class _PrefixNoLastTokenCap(pc_mod.OraclePrefixPool):
    def longest_hit(self, keys, max_length):
        return super().longest_hit(keys, max_length + 1)


class _PrefixNoEviction(pc_mod.OraclePrefixPool):
    def _take(self):
        return alloc_mod.OraclePool._take(self)


_block_key = pc_mod.block_key


def _key_without_parent(parent, tokens, extra=b""):
    return _block_key(pc_mod.ROOT_KEY, tokens, extra)


def _kernel_blocks_strided(ids, k):
    return [int(b) + j * len(ids) for b in ids for j in range(int(k))]


def _slot_transposed(table_row, pos, block_size):
    return (pos % block_size) * block_size + int(table_row[pos // block_size])


class _PoolFreeToHead(alloc_mod.OraclePool):
    def free_seq(self, seq):
        table = self.tables.pop(seq)
        del self.lens[seq]
        for blk in reversed(table):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.appendleft(blk)


class _PoolCowKeepsRef(alloc_mod.OraclePool):
    def append(self, seq, n):
        B = self.block_size
        table = self.tables[seq]
        slots, cow = [], []
        for _ in range(n):
            length = self.lens[seq]
            if length % B == 0:
                table.append(self._take())
            elif self.ref[table[-1]] > 1:
                new = self._take()
                cow.append((table[-1], new))
                table[-1] = new
            slots.append(table[length // B] * B + length % B)
            self.lens[seq] = length + 1
        return slots, cow


class _PoolNoCow(alloc_mod.OraclePool):
    def append(self, seq, n):
        B = self.block_size
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            length = self.lens[seq]
            if length % B == 0:
                table.append(self._take())
            slots.append(table[length // B] * B + length % B)
            self.lens[seq] = length + 1
        return slots, []


def _all(module):
    tests = []
    for name in dir(module):
        fn = getattr(module, name)
        if name.startswith("test_") and callable(fn):
            tests.append(fn)
    return tests


def _run(fn):
    marks = getattr(fn, "pytestmark", [])
    params = [m for m in marks if m.name == "parametrize"]
    if not params:
        fn()
        return
    # expand (at most two) parametrize marks
    combos = [{}]
    for m in params:
        argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) \
            else list(m.args[0])
        new = []
        for c in combos:
            for val in m.args[1]:
                vals = val if len(argnames) > 1 else (val,)
                d = dict(c)
                d.update(zip(argnames, vals))
                new.append(d)
        combos = new
    for c in combos:
        fn(**c)


def _some_pin_fails(tests):
    for fn in tests:
        try:
            _run(fn)
        except (AssertionError, ValueError, FloatingPointError, IndexError, KeyError):
            return True
    return False


MUTATIONS = [
    ("gather block index uses mod", attn_mod, "gather_tokens", _gather_swapped, TT),
    ("softmax without max shift", attn_mod, "attend", _attend_no_max, TT),
    ("scale dropped", attn_mod, "attend", _attend_no_scale, TT),
    ("softmax not normalised", attn_mod, "attend", _attend_unnormalised, TT),
    ("GQA head map h mod G", attn_mod, "kv_head_of", lambda h, g: h % g, TT),
    ("merge exponent sign flipped", attn_mod, "merge_partials", _merge_wrong_sign, TT),
    ("merge ignores partition mass", attn_mod, "merge_partials", _merge_ignores_mass, TT),
    ("causal bound off by one", attn_mod, "visible_tokens", lambda L, n, i: L - n + i, TT),
    ("causal bound ignores the position", attn_mod, "visible_tokens", lambda L, n, i: L, TT),
    ("slot block/offset transposed", slots_mod, "slot_of", _slot_transposed, TS),
    ("CP owner ignores the interleave", slots_mod, "cp_owner_and_offset",
     _cp_owner_ignores_interleave, TC),
    ("CP local offset drops the offset inside a run", slots_mod, "cp_owner_and_offset",
     _cp_local_drops_run_offset, TC),
    ("CP partial output not divided by its sum", attn_mod, "attention_partial",
     _partial_unnormalised, TC),
    ("kernel blocks strided instead of consecutive", slots_mod, "map_to_kernel_blocks",
     _kernel_blocks_strided, TS),
    ("window start off by one", attn_mod, "window_start",
     lambda p, w: max(0, p - w) if w > 0 else 0, TW),
    ("window ignored", attn_mod, "window_start", lambda p, w: 0, TW),
    ("skipped tokens off by one", alloc_mod, "num_skipped_tokens",
     lambda n, w: max(0, n - w) if w > 0 else 0, TW),
    ("block key ignores the parent key", pc_mod, "block_key", _key_without_parent, TP),
    ("prefix lookup skips misses", pc_mod, "OraclePrefixPool", _PrefixSkipsMisses, TP),
    ("prefix lookup may cover the last token", pc_mod, "OraclePrefixPool",
     _PrefixNoLastTokenCap, TP),
    ("reused blocks keep their cache key", pc_mod, "OraclePrefixPool", _PrefixNoEviction, TP),
    ("free returns blocks to the queue head", alloc_mod, "OraclePool", _PoolFreeToHead, TA),
    ("COW keeps the old reference", alloc_mod, "OraclePool", _PoolCowKeepsRef, TA),
    ("no copy-on-write", alloc_mod, "OraclePool", _PoolNoCow, TA),
]


@pytest.mark.parametrize("label,module,name,replacement,pins", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, label, module, name, replacement, pins):
    monkeypatch.setattr(module, name, replacement)
    # test modules bound some names at import time: patch those bindings too
    for mod in (TA, TT, TS, TC, TW, TP):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, replacement)
    with np.errstate(all="ignore"):
        assert _some_pin_fails(_all(pins)), f"no pin noticed: {label}"


@pytest.mark.parametrize("pins", [TA, TT, TS, TC, TW, TP],
                         ids=["allocator", "attention", "slots", "context_parallel", "window",
                              "prefix_cache"])
def test_unmutated_oracle_passes_every_pin(pins):
    """Control: the harness above reports no failure for the real oracle."""
    assert not _some_pin_fails(_all(pins))
