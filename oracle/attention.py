"""Oracle paged decode attention (float64), single pass and split-K.

TEST INFRASTRUCTURE (see the package header).

What it follows:
  * [VLLBC] walk-through of paper §4.1-4.2: the KV cache of a sequence is cut
    into blocks of B tokens; attention reads it block by block through the
    block table instead of from one contiguous array.  (The block-wise
    formula itself is lost from the extracted page.)
  * [PUFANYI] "按 Block 分配" (the kernel reads through the table, no copy to
    a contiguous buffer) and its closing remark that paging keeps the dense
    attention semantics: the result equals attention over the same tokens
    laid out contiguously.
  * [DEEPSONAR] §2.1: grouped-query attention, where 64 query heads share
    8 KV heads.

Readings where the pages are silent:
  * The decode step scores the one new query vector of each (sequence, query
    head) against the keys of all context_len cached tokens with
    x_t = scale * <q, k_t>, applies a softmax over t and returns
    sum_t softmax(x)_t v_t.  context_len >= 1.  ``scale`` is the fp32 value the
    kernel receives, widened exactly.
  * Query head h reads KV head floor(h / G), G = H / H_kv (contiguous groups).
  * Split-K: the context is cut at logical positions into partitions of P
    tokens; partition p yields m_p = max x, l_p = sum exp(x - m_p) and
    o_p = sum exp(x - m_p) v / l_p; the merge takes M = max m_p,
    a_p = l_p exp(m_p - M) and returns sum a_p o_p / sum a_p.  Only the
    ceil(L / P) non-empty partitions exist.

  * Several new tokens per sequence (chunked prefill, speculative drafts):
    the query tokens of sequence s are rows query_start_loc[s] ..
    query_start_loc[s+1]-1, the last n_s of its L_s tokens; query token i
    (position L_s - n_s + i) scores the keys at positions 0 .. L_s - n_s + i
    (causal over the new tokens, the whole cached context before them).

  * Sliding window ([CSDN] §3.1.1 and §3.3.1 release the blocks a sliding
    window leaves behind, without giving the window's rule): with window W, a
    query at position p scores only the keys at positions p - W + 1 .. p
    (the W most recent tokens, itself included); W = 0 means no window.

  * Context parallelism ([CSDN] §2.3 spreads a sequence's positions over the
    ranks of a context-parallel group): every rank attends over the tokens
    it stores and keeps (m, l, o) as for a split partition; merging the
    ranks' triples with the split-K merge gives attention over the whole
    context.  A rank with no token of a sequence contributes m = -inf,
    l = 0, o = 0 and no weight.

Pinned by tests/test_oracle_attention.py: brute force against a dense
softmax attention built from scipy.special.softmax on contiguous K/V, closed
forms (one token -> its value; equal keys or scale 0 -> mean of V), invariance
under any permutation of physical blocks, shared-prefix identity, GQA equal to
MHA with repeated KV heads, and split-K merge equal to the single pass.
The context-parallel functions are pinned by tests/test_oracle_cp.py: the
ranks' partials, built from rank-local caches written through the
context-parallel slot mapping, merge to the single pass over the whole
cache, and each rank's partial equals the one over the positions it owns.
"""

from __future__ import annotations

import numpy as np

from .dtypes import decode


def widen_scale(scale: float) -> float:
    """The fp32 softmax scale as the kernel sees it, as a float64."""
    return float(np.float32(scale))


def gather_tokens(cache: np.ndarray, table_row, length: int, kv_head: int,
                  block_size: int, start: int = 0) -> np.ndarray:
    """Rows [length - start, head_size] of one KV head of one sequence,
    positions start .. length - 1, read through its block table: position t
    is (table_row[t div B], kv_head, t mod B)."""
    t = np.arange(start, length)
    blocks = np.asarray(table_row, dtype=np.int64)[t // block_size]
    if (blocks < 0).any():
        raise ValueError("a position to read lies in a released block")
    return cache[blocks, kv_head, t % block_size, :]


def window_start(position: int, window: int) -> int:
    """First key position a query at ``position`` sees (0 without a window)."""
    return max(0, position - window + 1) if window > 0 else 0


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head ``h`` when ``group`` query heads share one."""
    return h // group


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q)^T V for one query vector (float64)."""
    x = scale * (K @ q)
    m = x.max()
    w = np.exp(x - m)
    return (w @ V) / w.sum()


def paged_attention(query, key_cache, value_cache, block_tables, context_lens,
                    scale: float, dtype: str, pairs=None, window: int = 0) -> np.ndarray:
    """Decode attention of every (sequence, query head), or of ``pairs``.

    query: raw [S, H, D]; caches: raw [NB, H_kv, B, D]; block_tables: [S, W]
    ints; context_lens: [S].  The query is the token at position L - 1 and
    sees keys from window_start(L - 1, window).  Returns float64 [S, H, D]
    (rows not in ``pairs`` are left zero).
    """
    S, H, D = query.shape
    H_kv, B = key_cache.shape[1], key_cache.shape[2]
    if H % H_kv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // H_kv
    sc = widen_scale(scale)
    out = np.zeros((S, H, D), dtype=np.float64)
    wanted = None if pairs is None else {(int(s), int(h)) for s, h in pairs}
    for s in range(S):
        L = int(context_lens[s])
        if L < 1:
            raise ValueError("context_len must be >= 1")
        for g in range(H_kv):
            heads = [h for h in range(H) if kv_head_of(h, G) == g
                     and (wanted is None or (s, h) in wanted)]
            if not heads:
                continue
            lo = window_start(L - 1, window)
            K = decode(gather_tokens(key_cache, block_tables[s], L, g, B, lo), dtype)
            V = decode(gather_tokens(value_cache, block_tables[s], L, g, B, lo), dtype)
            for h in heads:
                out[s, h] = attend(decode(query[s, h], dtype), K, V, sc)
    return out


def split_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                   partition_size: int):
    """(m, l, o) of every non-empty partition of one query's context."""
    L = K.shape[0]
    num_parts = -(-L // partition_size)
    m = np.empty(num_parts)
    l = np.empty(num_parts)
    o = np.empty((num_parts, K.shape[1]))
    for p in range(num_parts):
        lo, hi = p * partition_size, min((p + 1) * partition_size, L)
        x = scale * (K[lo:hi] @ q)
        m[p] = x.max()
        w = np.exp(x - m[p])
        l[p] = w.sum()
        o[p] = (w @ V[lo:hi]) / l[p]
    return m, l, o


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine partition results into the softmax-weighted output."""
    M = m.max()
    a = l * np.exp(m - M)
    return (a @ o) / a.sum()


def paged_attention_split(query, key_cache, value_cache, block_tables, context_lens,
                          scale: float, dtype: str, partition_size: int, pairs=None):
    """Same result as ``paged_attention`` computed partition by partition.

    Returns (out [S, H, D], partials) where partials[(s, h)] = (m, l, o).
    """
    S, H, D = query.shape
    H_kv, B = key_cache.shape[1], key_cache.shape[2]
    G = H // H_kv
    sc = widen_scale(scale)
    out = np.zeros((S, H, D), dtype=np.float64)
    partials = {}
    wanted = None if pairs is None else {(int(s), int(h)) for s, h in pairs}
    for s in range(S):
        L = int(context_lens[s])
        if L < 1:
            raise ValueError("context_len must be >= 1")
        for g in range(H_kv):
            heads = [h for h in range(H) if kv_head_of(h, G) == g
                     and (wanted is None or (s, h) in wanted)]
            if not heads:
                continue
            K = decode(gather_tokens(key_cache, block_tables[s], L, g, B), dtype)
            V = decode(gather_tokens(value_cache, block_tables[s], L, g, B), dtype)
            for h in heads:
                m, l, o = split_partials(decode(query[s, h], dtype), K, V, sc, partition_size)
                partials[(s, h)] = (m, l, o)
                out[s, h] = merge_partials(m, l, o)
    return out, partials


def visible_tokens(L: int, n: int, i: int) -> int:
    """Keys seen by new token i of n in a context of L tokens: positions
    0 .. L - n + i, i.e. the cached context and the new tokens up to itself."""
    return L - n + i + 1


def paged_attention_multi(query, key_cache, value_cache, block_tables, context_lens,
                          query_start_loc, scale: float, dtype: str,
                          window: int = 0) -> np.ndarray:
    """Attention of every new token of every sequence, causal over the new
    tokens ([CSDN] section 2.3 lays out a step's tokens by query_start_loc;
    [DEEPSONAR] section 2.5 schedules prefill chunks and speculative tokens
    the same way as decode tokens).

    query: raw [T, H, D]; returns float64 [T, H, D].  With a window, query
    token i sees keys from window_start(L - n + i, window) on."""
    T, H, D = query.shape
    H_kv, B = key_cache.shape[1], key_cache.shape[2]
    G = H // H_kv
    sc = widen_scale(scale)
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        q0, q1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n = q1 - q0
        if n > L:
            raise ValueError("more new tokens than the context holds")
        lo0 = window_start(L - n, window)  # no query of the row reads keys before it
        for g in range(H_kv):
            K = decode(gather_tokens(key_cache, block_tables[s], L, g, B, lo0), dtype)
            V = decode(gather_tokens(value_cache, block_tables[s], L, g, B, lo0), dtype)
            for i in range(n):
                visible = visible_tokens(L, n, i)
                lo = window_start(visible - 1, window)
                for h in range(H):
                    if kv_head_of(h, G) == g:
                        out[q0 + i, h] = attend(decode(query[q0 + i, h], dtype),
                                                K[lo - lo0:visible - lo0],
                                                V[lo - lo0:visible - lo0], sc)
    return out


def attention_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """(m, l, o) of one query over a set of keys; an empty set gives
    (-inf, 0, zeros)."""
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    x = scale * (K @ q)
    m = x.max()
    w = np.exp(x - m)
    l = w.sum()
    return m, l, (w @ V) / l


def paged_attention_partials(query, key_cache, value_cache, block_tables, context_lens,
                             scale: float, dtype: str):
    """Rank-local (m [S, H], l [S, H], o [S, H, D]) over the first
    context_lens[s] tokens of each sequence in this rank's cache (0 allowed)."""
    S, H, D = query.shape
    H_kv, B = key_cache.shape[1], key_cache.shape[2]
    G = H // H_kv
    sc = widen_scale(scale)
    m = np.full((S, H), -np.inf)
    l = np.zeros((S, H))
    o = np.zeros((S, H, D))
    for s in range(S):
        L = int(context_lens[s])
        for g in range(H_kv):
            K = decode(gather_tokens(key_cache, block_tables[s], L, g, B), dtype)
            V = decode(gather_tokens(value_cache, block_tables[s], L, g, B), dtype)
            for h in range(H):
                if kv_head_of(h, G) == g:
                    m[s, h], l[s, h], o[s, h] = attention_partial(decode(query[s, h], dtype),
                                                                  K, V, sc)
    return m, l, o


def merge_rank_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """out [S, H, D] from the ranks' m, l [N, S, H] and o [N, S, H, D]; parts
    with l = 0 carry no weight and a row without any key is 0."""
    N, S, H, D = o.shape
    out = np.zeros((S, H, D))
    for s in range(S):
        for h in range(H):
            keep = l[:, s, h] > 0
            if keep.any():
                out[s, h] = merge_partials(m[keep, s, h], l[keep, s, h], o[keep, s, h])
    return out
