"""Pins of the oracle prefix cache (CPU only)."""

from __future__ import annotations

import hashlib

import pytest

from oracle.prefix_cache import ROOT_KEY, OraclePrefixPool, block_key, key_chain


def test_sha256_matches_the_fips_examples():
    # FIPS 180-2 appendix B examples (also the hashlib documentation's)
    assert hashlib.sha256(b"abc").hexdigest() == (
        "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad")
    assert hashlib.sha256(b"").hexdigest() == (
        "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855")


def test_key_message_layout():
    # parent || int32 LE tokens || extra
    msg = ROOT_KEY + bytes([1, 0, 0, 0, 0xFF, 0xFF, 0xFF, 0xFF]) + b"lora7"
    assert block_key(ROOT_KEY, [1, -1], b"lora7") == hashlib.sha256(msg).digest()


def test_chain_changes_from_the_first_differing_block_on():
    B = 4
    a = list(range(20))
    b = list(a)
    b[9] = 999  # block 2
    ka, kb = key_chain(a, B), key_chain(b, B)
    assert len(ka) == 5  # full blocks only
    assert ka[:2] == kb[:2]
    assert all(x != y for x, y in zip(ka[2:], kb[2:]))
    # the same block content after a different prefix has a different key
    c = [7] * 4 + a[4:8]
    assert key_chain(c, B)[1] != ka[1]
    # extra keys separate otherwise equal prompts
    assert key_chain(a, B, b"x")[0] != ka[0]
    assert key_chain(a[:7], B) == ka[:1]


def _run_prompt(pool, seq, prompt, extra=b""):
    done = pool.add_seq_cached(seq, prompt, extra)
    pool.append_tokens(seq, prompt[done:])
    pool.cache_full_blocks(seq)
    return done


def test_hit_reuses_full_blocks_and_recomputes_the_last_token():
    B = 4
    pool = OraclePrefixPool(16, B, list(range(16)))
    prompt = list(range(100, 112))  # 3 full blocks
    assert _run_prompt(pool, 0, prompt) == 0
    assert pool.block_table(0) == [0, 1, 2]
    # the same prompt again: at most 11 tokens may come from the cache
    assert pool.add_seq_cached(1, prompt) == 8
    assert pool.block_table(1) == [0, 1]
    assert [pool.ref[b] for b in (0, 1, 2)] == [2, 2, 1]
    slots, _ = pool.append_tokens(1, prompt[8:])
    assert [s // B for s in slots] == [3] * 4  # the last block is computed again
    # a longer prompt with the same start hits all three blocks
    assert pool.add_seq_cached(2, prompt + [5]) == 12
    pool.check_invariants()


def test_lookup_stops_at_the_first_miss():
    B = 2
    pool = OraclePrefixPool(8, B, list(range(8)))
    prompt = [1, 2, 3, 4, 5, 6, 7]
    _run_prompt(pool, 0, prompt)  # caches blocks 0..2 (keys k0 k1 k2)
    keys = key_chain(prompt, B)
    # drop k1 from the cache: k2 is still cached but unreachable
    del pool.cached[keys[1]]
    pool.key_of[pool.block_table(0)[1]] = None
    assert pool.longest_hit(keys, 100) == [pool.block_table(0)[0]]
    assert pool.add_seq_cached(1, prompt) == 2


def test_partial_blocks_are_never_cached():
    pool = OraclePrefixPool(8, 4, list(range(8)))
    _run_prompt(pool, 0, list(range(10)))  # blocks: full, full, 2 tokens
    assert pool.key_of[pool.block_table(0)[2]] is None
    assert len(pool.cached) == 2


def test_freed_cached_blocks_are_evicted_in_lru_order():
    B = 2
    pool = OraclePrefixPool(6, B, list(range(6)))
    a = [1, 2, 3, 4, 5]  # blocks 0, 1 cached, block 2 partial
    _run_prompt(pool, 0, a)
    pool.free_seq(0)  # tail first: 2, 1, 0 join the queue tail
    assert list(pool.free) == [3, 4, 5, 2, 1, 0]
    assert len(pool.cached) == 2
    # a different 8-token prompt takes 4 blocks from the head: 3, 4, 5, 2
    _run_prompt(pool, 1, [9, 9, 8, 8, 7, 7, 6, 6])
    assert pool.num_evicted == 0 and len(pool.cached) == 2 + 4
    pool.free_seq(1)  # 2, 5, 4, 3 to the tail -> queue 1 0 2 5 4 3
    assert list(pool.free) == [1, 0, 2, 5, 4, 3]
    # a third prompt takes the two oldest cached blocks (1 then 0): both evicted
    _run_prompt(pool, 2, [4, 4, 4])
    assert pool.num_evicted == 2
    assert pool.add_seq_cached(3, a) == 0  # a's first block is gone: nothing hits
    pool.check_invariants()


def test_touch_takes_a_freed_cached_block_out_of_the_queue():
    pool = OraclePrefixPool(6, 2, list(range(6)))
    _run_prompt(pool, 0, [1, 2, 3, 4, 5])
    pool.free_seq(0)
    free_before = pool.num_free()
    assert pool.add_seq_cached(1, [1, 2, 3, 4, 9]) == 4
    assert pool.num_free() == free_before - 2
    assert 0 not in pool.free and 1 not in pool.free
    assert pool.ref[0] == pool.ref[1] == 1
    pool.check_invariants()


@pytest.mark.parametrize("B", [1, 3, 16])
def test_equal_prompts_share_every_full_block_but_the_last_token(B):
    pool = OraclePrefixPool(64, B, list(range(64)))
    prompt = [t % 11 for t in range(5 * B + 2)]
    _run_prompt(pool, 0, prompt)
    done = pool.add_seq_cached(1, prompt)
    assert done == ((len(prompt) - 1) // B) * B
    assert pool.block_table(1) == pool.block_table(0)[:done // B]
