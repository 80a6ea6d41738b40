"""Host logic of bench.py's algorithmic byte count (CPU only): the distinct
cache rows a batch attends, checked by brute force over slots."""

from __future__ import annotations

import numpy as np

import bench


class _W:
    """The few workload fields the byte count reads."""

    def __init__(self, window=0, B=4, H=4, Hkv=2, D=8, e=2, S=3):
        self.extra = {"sliding_window": window} if window else {}
        self.block_size = B
        self.num_heads, self.num_kv_heads, self.head_size, self.elem_bytes = H, Hkv, D, e
        self.num_seqs = S


def _brute_rows(tables, lens, B, window=0):
    seen = set()
    for s, L in enumerate(lens):
        lo = max(0, L - window) if window else 0
        for t in range(lo, L):
            seen.add(int(tables[s][t // B]) * B + t % B)
    return len(seen)


def test_distinct_rows_count_shared_blocks_once():
    rng = np.random.default_rng(0)
    for trial in range(50):
        B = int(rng.choice([1, 2, 4, 16]))
        S = int(rng.integers(1, 6))
        lens = rng.integers(1, 70, size=S)
        width = int(-(-lens.max() // B))
        # a common prefix of random length, then private blocks
        shared = rng.permutation(10_000)[:width]
        tables = np.tile(shared, (S, 1)).astype(np.int32)
        k = int(rng.integers(0, width + 1))
        for s in range(S):
            tables[s, k:] = 20_000 + 100 * s + np.arange(width - k)
        window = int(rng.choice([0, 1, 5, 33]))
        spans = bench.attended(_W(window, B), lens)
        assert bench.attended_rows(spans, tables, B) == _brute_rows(tables, lens, B, window)


def test_without_sharing_distinct_rows_are_the_attended_tokens():
    rng = np.random.default_rng(1)
    lens = rng.integers(1, 300, size=12)
    B = 16
    width = int(-(-lens.max() // B))
    tables = rng.permutation(12 * width).astype(np.int32).reshape(12, width)
    spans = bench.attended(_W(B=B, S=12), lens)
    assert bench.attended_rows(spans, tables, B) == int(lens.sum())
    w = _W(B=B, S=12)
    with_tables = bench.attention_bytes(w, lens, tables=tables)
    assert with_tables == bench.attention_bytes(w, lens)


def test_attention_bytes_formula():
    """KV rows x 2*Hkv*D*e, q and out rows, table entries, lengths."""
    w = _W(B=4, H=4, Hkv=2, D=8, e=2, S=2)
    lens = [5, 4]
    tables = np.array([[7, 3], [7, 9]], dtype=np.int32)  # block 7 shared
    # rows: seq 0 -> 7:0..3, 3:0 ; seq 1 -> 7:0..3 : distinct 5
    got = bench.attention_bytes(w, lens, tables=tables)
    kv = 5 * 2 * 2 * 8 * 2
    qo = 2 * 2 * 4 * 8 * 2
    entries = 4 * (2 + 1)
    assert got == kv + qo + entries + 4 * 2


def test_bench_refuses_more_than_one_gpu():
    """Only one GPU's share is measured: --gpus N > 1 exits with a message,
    before anything touches a GPU."""
    import subprocess
    import sys

    from conftest import REPO
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=REPO,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
