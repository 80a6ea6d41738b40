"""Pins of the oracle's sliding window (CPU only): attention over the last W
keys against a dense banded softmax, closed forms, and the allocator's
release of the blocks the window leaves behind."""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax

from oracle.allocator import OraclePool, num_skipped_tokens
from oracle.attention import paged_attention, paged_attention_multi
from test_oracle_attention import _dense, _random_case


def _banded(q, Klog, Vlog, scale, G, positions, window):
    """Dense softmax of query rows over the keys p - W + 1 .. p."""
    out = np.zeros(q.shape)
    for r, (s, p) in enumerate(positions):
        for h in range(q.shape[1]):
            g = h // G
            t = np.arange(Klog[s].shape[1])
            mask = (t <= p) & (t >= p - window + 1)
            x = np.where(mask, scale * (Klog[s][g] @ q[r, h]), -np.inf)
            out[r, h] = softmax(x) @ Vlog[s][g]
    return out


@pytest.mark.parametrize("B", [1, 3, 4])
@pytest.mark.parametrize("W", [1, 2, 5, 17])
@pytest.mark.parametrize("G", [1, 2])
def test_window_decode_equals_banded_dense_softmax(B, W, G):
    rng = np.random.default_rng(1000 * B + 10 * W + G)
    hkv, D = 2, 8
    lens = list(range(1, 31, 2))
    q, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), hkv * G, hkv, D, B, lens)
    scale = 0.41
    got = paged_attention(q, kc, vc, bt, lens, scale, "f64", window=W)
    want = _banded(q, Klog, Vlog, float(np.float32(scale)), G,
                   [(s, L - 1) for s, L in enumerate(lens)], W)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_window_covering_the_context_is_full_attention():
    rng = np.random.default_rng(5)
    lens = [1, 4, 9, 16]
    q, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), 2, 2, 8, 4, lens)
    full = paged_attention(q, kc, vc, bt, lens, 0.3, "f64")
    for W in (16, 17, 1000):
        np.testing.assert_array_equal(paged_attention(q, kc, vc, bt, lens, 0.3, "f64", window=W),
                                      full)


def test_window_of_one_returns_the_last_value():
    rng = np.random.default_rng(6)
    lens = [3, 8, 11]
    q, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), 4, 2, 8, 4, lens)
    got = paged_attention(q, kc, vc, bt, lens, 0.3, "f64", window=1)
    for s, L in enumerate(lens):
        for h in range(4):
            np.testing.assert_array_equal(got[s, h], Vlog[s][h // 2][L - 1])


@pytest.mark.parametrize("W", [1, 3, 6, 40])
def test_window_multi_query_equals_banded_dense_softmax(W):
    rng = np.random.default_rng(W)
    B, hkv, G, D = 4, 2, 2, 8
    lens = [5, 12, 20, 33]
    news = [1, 3, 4, 5]
    q0, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), hkv * G, hkv, D, B, lens)
    qsl = np.concatenate([[0], np.cumsum(news)])
    q = rng.standard_normal((int(qsl[-1]), hkv * G, D))
    got = paged_attention_multi(q, kc, vc, bt, lens, qsl, 0.37, "f64", window=W)
    rows = [(s, L - n + i) for s, (L, n) in enumerate(zip(lens, news)) for i in range(n)]
    want = _banded(q, Klog, Vlog, float(np.float32(0.37)), G, rows, W)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---- the allocator ------------------------------------------------------------

def test_skipped_tokens_closed_form():
    assert num_skipped_tokens(10, 0) == 0
    assert num_skipped_tokens(10, 4) == 7  # next query at 10 sees 7 .. 10
    assert num_skipped_tokens(3, 4) == 0
    assert num_skipped_tokens(4, 4) == 1
    assert num_skipped_tokens(8, 1) == 8


def _table(pool, s):
    return [-1 if b is None else b for b in pool.block_table(s)]


@pytest.mark.parametrize("N,W,B", [(30, 7, 4), (32, 1, 4), (17, 17, 4), (40, 9, 3), (5, 8, 2)])
def test_release_of_skipped_blocks(N, W, B):
    pool = OraclePool(32, B, list(range(32)))
    pool.add_seq(0)
    pool.append(0, N)
    before = pool.block_table(0)
    released = pool.remove_skipped(0, N, W)
    k = num_skipped_tokens(N, W) // B
    assert released == list(reversed(before[:k]))  # tail first
    assert pool.block_table(0) == [None] * k + before[k:]
    assert list(pool.free)[-len(released):] == released if released else True
    pool.check_invariants()
    assert pool.remove_skipped(0, N, W) == []  # nothing left to release
    # the next token still gets a slot; the holes are never read
    slots, _ = pool.append(0, 1)
    assert slots[0] // B == pool.block_table(0)[N // B]


def test_windowed_attention_reads_no_released_block():
    """Attention with the window after the release equals attention with
    the window before it: the released blocks are never read."""
    rng = np.random.default_rng(9)
    B, W, N = 4, 6, 23
    pool = OraclePool(16, B, rng.permutation(16))
    pool.add_seq(0)
    slots, _ = pool.append(0, N)
    kc = rng.standard_normal((16, 1, B, 8))
    vc = rng.standard_normal((16, 1, B, 8))
    q = rng.standard_normal((1, 1, 8))
    before = paged_attention(q, kc, vc, [pool.block_table(0)], [N], 0.5, "f64", window=W)
    pool.remove_skipped(0, N - 1, W)  # the last token's query starts at N - W
    table = _table(pool, 0)
    assert table[0] == -1 and table[(N - W) // B] >= 0
    after = paged_attention(q, kc, vc, [table], [N], 0.5, "f64", window=W)
    np.testing.assert_array_equal(before, after)
    with pytest.raises(ValueError):  # the full context would read a hole
        paged_attention(q, kc, vc, [table], [N], 0.5, "f64")


def test_fork_after_release_shares_only_live_blocks():
    pool = OraclePool(16, 4, list(range(16)))
    pool.add_seq(0)
    pool.append(0, 13)
    pool.remove_skipped(0, 13, 5)  # 9 skipped tokens -> 2 blocks
    pool.fork(0, 1)
    assert pool.block_table(1) == [None, None, 2, 3]
    assert [pool.ref[b] for b in (0, 1, 2, 3)] == [0, 0, 2, 2]
    pool.check_invariants()
    pool.free_seq(0)
    pool.free_seq(1)
    pool.check_invariants()
    assert pool.num_free() == 16
