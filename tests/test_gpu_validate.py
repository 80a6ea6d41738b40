"""Device check of tables and lengths (pa_validate_tables)."""

from __future__ import annotations

import pytest
import torch

import workloads as W
from test_gpu_parity import _require_gpu, _step

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("make", [
    lambda: W.llama7b_fp16(num_seqs=16),
    lambda: W.custom_decode("v_win", 31, [1, 17, 100, 1030], dtype="f16", H=2, Hkv=2, D=128,
                            B=16, sliding_window=40),
    lambda: W.custom_decode("v_kb", 41, [1, 33, 257], dtype="bf16", H=4, Hkv=2, D=128, B=32,
                            kernel_block_size=8),
], ids=["llama", "window", "kernel_blocks"])
def test_step_tables_are_valid(make):
    _require_gpu()
    from paged_kv_cache_123_amd import ops
    w = make()
    step = _step(w, W.make_values(w, DEV))
    nb = step.key_cache.shape[0]
    assert ops.validate_tables(step.block_tables, step.context_lens, step.block_size, nb,
                               step.sliding_window) == (0, None)
    if step.sliding_window:  # the released entries are -1: checked without the window, they fail
        bad, first = ops.validate_tables(step.block_tables, step.context_lens, step.block_size, nb)
        assert bad > 0


def test_planted_errors_are_reported():
    _require_gpu()
    from paged_kv_cache_123_amd import ops
    tables = torch.tensor([[0, 1, 2, -1], [3, 4, -1, -1], [5, 6, 7, 8], [9, -1, -1, -1]],
                          dtype=torch.int32, device=DEV)
    lens = torch.tensor([9, 5, 16, 4], dtype=torch.int32, device=DEV)
    assert ops.validate_tables(tables, lens, 4, 10) == (0, None)
    t = tables.clone()
    t[2, 3] = 10  # outside the pool
    assert ops.validate_tables(t, lens, 4, 10) == (1, 2)
    t = tables.clone()
    t[1, 1] = -3
    t[3, 0] = 99
    assert ops.validate_tables(t, lens, 4, 10) == (2, 1)
    bad_len = lens.clone()
    bad_len[0] = 17  # needs 5 entries, the row holds 4: reported, not followed
    assert ops.validate_tables(tables, bad_len, 4, 10) == (1, 0)
    bad_len[3] = -1
    assert ops.validate_tables(tables, bad_len, 4, 10) == (2, 0)
    # a window hides entries before length - W
    t = tables.clone()
    t[2, 0] = -1
    assert ops.validate_tables(t, lens, 4, 10) == (1, 2)
    assert ops.validate_tables(t, lens, 4, 10, sliding_window=8) == (0, None)
