"""GPU parity of decode over tables built through the host prefix cache:
tables bit for bit against the oracle's cache, then the whole step.

Attention within the attention tolerances (fp32 storage 1e-5 max-abs;
16-bit storage 2e-2 max-abs and 5e-3 relative L2).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import OracleStep, to_host
from test_gpu_parity import (BOTH, _require_gpu, _step, check_attention,  # noqa: F401
                             decode_kernel, full_parity)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_prefix_cache_batch_full_size():
    """128 requests over 16 cached system prompts, one decode token each."""
    w = W.prefix_cache_bf16()
    step, ora, _ = full_parity(w)
    shared = (step.shared_blocks_host > 0).sum()
    assert shared >= 112  # every request after the first of its prompt hits
    assert len(ora.pool.cached) > 0


@BOTH
@pytest.mark.parametrize("dtype,G,B,part", [("bf16", 8, 16, 0), ("f16", 2, 4, 32),
                                            ("f32", 1, 8, 0), ("bf16", 4, 32, 64)])
def test_prefix_hits_and_evictions(dtype, G, B, part, decode_kernel):
    """A pool just large enough that finished requests' cached blocks are
    evicted while others are still hit."""
    systems = [3 * B + 5, 5 * B, 2 * B + 1]
    requests = [(0, 7), (1, 3), (0, 2 * B), (2, 1), (-1, 4 * B), (1, B), (0, 9), (2, 3 * B),
                (1, 2), (0, 1)]
    w = W.custom_prefix(f"prefix_{dtype}_{B}", 51, systems, requests, dtype=dtype, H=2 * G,
                        Hkv=2, D=128, B=B, finished={0, 3, 4, 6}, partition_size=part,
                        num_blocks=24)
    ora = OracleStep(w)
    assert ora.pool.num_evicted > 0, "the case should reach eviction"
    full_parity(w)


@BOTH
def test_prefix_fused_step(decode_kernel):
    _require_gpu()
    w = W.custom_prefix("prefix_fused", 52, [40, 75], [(0, 5), (1, 9), (0, 30), (1, 2), (0, 1)],
                        dtype="bf16", H=8, Hkv=2, D=128, B=16)
    vals = W.make_values(w, DEV)
    host = {k: to_host(v) for k, v in vals.items()}
    ora = OracleStep(w)
    sep_vals = {k: v.clone() for k, v in vals.items()}
    sep = _step(w, sep_vals)
    sep.run()
    step = _step(w, vals)
    out = step.run(fused=True)
    torch.cuda.synchronize()
    assert np.array_equal(step.tables_host.astype(np.int64), ora.tables)
    kc, vc = host["key_cache"], host["value_cache"]
    ora.apply_copies(kc, vc)
    ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
    assert np.array_equal(to_host(step.key_cache), kc) and np.array_equal(to_host(step.value_cache), vc)
    want = ora.attention(host["query"], kc, vc)
    check_attention(to_host(out), want, w.dtype, "prefix fused")
    assert torch.equal(out.view(torch.int16), sep.out.view(torch.int16))
