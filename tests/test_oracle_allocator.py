"""Pins of the oracle block pool against the pages' worked examples."""

from __future__ import annotations

import random

import pytest

from conftest import ints, load_golden, refs
from oracle.allocator import OraclePool, PoolExhausted, sharing_saving, tail_fragmentation
from oracle.slots import slot_of


def _pool(g):
    return OraclePool(int(g["num_blocks"][0]), int(g["block_size"][0]), ints(g["free_order"]))


def test_growth_example():
    g = load_golden("t_grow")
    pool = _pool(g)
    pool.add_seq(0)
    slots, cow = pool.append(0, int(g["prompt_len"][0]))
    assert pool.block_table(0) == ints(g["table_after_prompt"])
    assert slots == ints(g["prompt_slots"]) and cow == []
    slots, cow = pool.append(0, 1)
    assert slots == ints(g["decode1_slot"]) and cow == []
    assert pool.block_table(0) == ints(g["table_after_decode1"])
    slots, cow = pool.append(0, 1)
    assert slots == ints(g["decode2_slot"]) and cow == []
    assert pool.block_table(0) == ints(g["table_after_decode2"])
    pool.check_invariants()


def test_sharing_fig8_and_simulator():
    g = load_golden("t_sharing")
    pool = _pool(g)
    pool.add_seq(0)  # A
    pool.append(0, int(g["prompt_len"][0]))
    pool.fork(0, 1)  # B shares A's prompt
    assert pool.block_table(0) == pool.block_table(1) == ints(g["shared_table"])
    assert [pool.ref[b] for b in ints(g["shared_table"])] == ints(g["shared_refs"])
    assert round(sharing_saving([pool.block_table(0), pool.block_table(1)]), 3) == \
        float(g["saving_shared"][0])

    _, cow_a = pool.append(0, 1)
    assert cow_a == [tuple(ints(g["A_cow_first"]))]
    _, cow_b = pool.append(1, 1)
    assert cow_b == [tuple(ints(g["B_cow_first"]))] if g["B_cow_first"] else cow_b == []
    assert pool.block_table(0) == ints(g["A_after_first"])
    assert pool.block_table(1) == ints(g["B_after_first"])
    for blk, r in refs(g["refs_after_first"]).items():
        assert pool.ref[blk] == r
    assert round(sharing_saving([pool.block_table(0), pool.block_table(1)]), 3) == \
        float(g["saving_after_first"][0])

    pool.append(0, 1)
    pool.append(1, 1)
    assert pool.block_table(0) == ints(g["A_after_second"])
    assert pool.block_table(1) == ints(g["B_after_second"])
    assert round(sharing_saving([pool.block_table(0), pool.block_table(1)]), 3) == \
        float(g["saving_after_second"][0])
    assert pool.num_cow == 1
    pool.check_invariants()


def test_table_lookup_example():
    g = load_golden("t_table")
    pool = _pool(g)
    pool.add_seq(0)
    pool.add_seq(1)
    pool.append(0, int(g["A_len"][0]))
    pool.append(1, int(g["B_len"][0]))
    assert pool.block_table(0) == ints(g["A_table"])
    assert pool.block_table(1) == ints(g["B_table"])
    assert list(pool.free) == ints(g["free_after"])
    B = int(g["block_size"][0])
    pos = int(g["query_pos"][0])
    table = pool.block_table(0)
    assert pos // B == int(g["query_logical_block"][0])
    assert table[pos // B] == int(g["query_physical_block"][0])
    assert pos % B == int(g["query_offset"][0])
    assert slot_of(table, pos, B) == int(g["query_slot"][0])
    blocks, slots, empty, _ = tail_fragmentation([int(g["A_len"][0])], B)
    assert (blocks, slots, empty) == (int(g["A_blocks"][0]), int(g["A_slots"][0]),
                                      int(g["A_empty"][0]))


def test_cow_partial_tail_example():
    g = load_golden("t_cow4")
    pool = _pool(g)
    pool.add_seq(0)
    pool.append(0, int(g["prompt_len"][0]))
    pool.fork(0, 1)
    assert pool.block_table(0) == ints(g["shared_table"])
    _, cow = pool.append(0, 1)
    assert cow == [tuple(ints(g["A_cow"]))]
    _, cow = pool.append(1, 1)
    assert cow == []
    assert pool.block_table(0) == ints(g["A_after"])
    assert pool.block_table(1) == ints(g["B_after"])
    for blk, r in refs(g["refs_after"]).items():
        assert pool.ref[blk] == r


@pytest.mark.parametrize("B", [16, 64])
def test_fragmentation_example(B):
    g = load_golden("t_frag")
    lengths = ints(g["lengths"])
    blocks, slots, empty, frac = tail_fragmentation(lengths, B)
    p = f"b{B}_"
    assert blocks == int(g[p + "blocks"][0])
    assert slots == int(g[p + "slots"][0])
    assert empty == int(g[p + "empty"][0])
    assert round(frac, 3) == float(g[p + "frac"][0])
    # the same counts from the pool itself
    pool = OraclePool(64, B)
    per_seq_blocks, per_seq_empty = [], []
    for s, L in enumerate(lengths):
        pool.add_seq(s)
        pool.append(s, L)
        per_seq_blocks.append(len(pool.block_table(s)))
        per_seq_empty.append(len(pool.block_table(s)) * B - L)
    assert per_seq_blocks == ints(g[p + "per_seq_blocks"])
    assert per_seq_empty == ints(g[p + "per_seq_empty"])


def test_ceil_blocks_closed_form():
    for B in (1, 2, 3, 4, 16, 64):
        for T in range(1, 3 * B + 2):
            pool = OraclePool(16, B)
            pool.add_seq(0)
            pool.append(0, T)
            n = len(pool.block_table(0))
            assert (n - 1) * B < T <= n * B  # n = ceil(T / B)
            assert n * B - T <= B - 1


def test_exhaustion_is_all_or_nothing():
    pool = OraclePool(3, 4, [2, 0, 1])
    pool.add_seq(0)
    pool.append(0, 10)  # 3 blocks
    before = (pool.block_table(0), list(pool.free), list(pool.ref), pool.seq_len(0))
    with pytest.raises(PoolExhausted):
        pool.append(0, 3)
    assert (pool.block_table(0), list(pool.free), list(pool.ref), pool.seq_len(0)) == before
    pool.append(0, 2)  # still fits in the tail
    assert pool.seq_len(0) == 12


def test_exhaustion_counts_the_cow_block():
    pool = OraclePool(2, 4)
    pool.add_seq(0)
    pool.append(0, 3)
    pool.fork(0, 1)
    pool.add_seq(2)
    pool.append(2, 1)  # pool now empty
    with pytest.raises(PoolExhausted):
        pool.append(1, 1)  # needs a copy of the shared tail
    pool.check_invariants()


def test_free_releases_tail_first_to_queue_tail():
    pool = OraclePool(6, 2, [5, 4, 3, 2, 1, 0])
    pool.add_seq(0)
    pool.append(0, 5)  # blocks 5 4 3
    pool.free_seq(0)
    assert list(pool.free) == [2, 1, 0, 3, 4, 5]
    pool.check_invariants()


def test_shared_blocks_survive_until_last_holder():
    pool = OraclePool(4, 4)
    pool.add_seq(0)
    pool.append(0, 8)
    pool.fork(0, 1)
    pool.free_seq(0)
    assert pool.num_free() == 2 and pool.block_table(1) == [0, 1]
    pool.free_seq(1)
    assert pool.num_free() == 4
    pool.check_invariants()


def test_random_operations_keep_invariants():
    rng = random.Random(7)
    for trial in range(20):
        B = rng.choice([1, 2, 4, 16])
        nb = rng.randint(4, 40)
        order = list(range(nb))
        rng.shuffle(order)
        pool = OraclePool(nb, B, order)
        live, next_id = [], 0
        for _ in range(200):
            op = rng.random()
            if op < 0.2 or not live:
                pool.add_seq(next_id)
                live.append(next_id)
                next_id += 1
            elif op < 0.35:
                pool.fork(rng.choice(live), next_id)
                live.append(next_id)
                next_id += 1
            elif op < 0.5:
                s = rng.choice(live)
                pool.free_seq(s)
                live.remove(s)
            else:
                s = rng.choice(live)
                n = rng.randint(1, 3 * B)
                try:
                    slots, _ = pool.append(s, n)
                except PoolExhausted:
                    continue
                L = pool.seq_len(s)
                table = pool.block_table(s)
                assert slots == [slot_of(table, p, B) for p in range(L - n, L)]
            pool.check_invariants()
