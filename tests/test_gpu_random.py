"""Seeded random configurations through the whole step, against the oracle.

Each case draws a storage dtype, head size, block size, GQA group, KV head
count, partition size, sliding window, kernel block size and attention kernel,
then either a parallel-sampling batch (prompts forked into samples that
append several tokens each, with copy-on-write of shared tails) or a batch
whose every new token is a query.  The separate calls and the one-launch step
are both checked: tables, slots and caches bit-exact, attention within the
stated tolerances, and the two paths' outputs bit-identical.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import OracleStep, to_host
from test_gpu_parity import _dead_cow_slots, _require_gpu, _step, check_attention

pytestmark = pytest.mark.gpu

DEV = "cuda"
NUM_CASES = 64


def draw_case(seed: int) -> dict:
    """A random configuration within the library's documented limits."""
    rng = np.random.default_rng(5000 + seed)
    c = {"seed": seed}
    c["dtype"] = str(rng.choice(["f32", "f16", "bf16"]))
    c["D"] = int(rng.choice([64, 128]))
    c["B"] = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    c["G"] = int(rng.choice([1, 2, 4, 8]))
    c["Hkv"] = int(rng.choice([1, 2, 3]))
    c["part"] = 0 if rng.random() < 0.4 else math.lcm(16, c["B"]) * int(rng.integers(1, 5))
    c["window"] = 0 if rng.random() < 0.6 else int(rng.integers(1, 400))
    c["kind"] = "forks" if rng.random() < 0.6 else "multi"
    matrix = c["dtype"] != "f32" and c["D"] == 128
    c["kernel"] = "mfma" if matrix and rng.random() < 0.75 else "valu"
    kb = 0
    if c["kind"] == "forks" and c["B"] > 1 and rng.random() < 0.3:
        kb = c["B"] // int(rng.choice([2, 4])) or 1
    c["kernel_block"] = kb
    if c["kind"] == "forks":
        groups = int(rng.integers(1, 5))
        c["samples"] = int(rng.integers(1, 5))
        c["prompts"] = [int(x) for x in rng.integers(1, 400, size=groups)]
        c["appends"] = [[int(x) for x in rng.integers(1, min(2 * c["B"], 40) + 1,
                                                          size=c["samples"])]
                        for _ in range(groups)]
    else:
        cap = (16 if c["kernel"] == "mfma" else 8) // c["G"]
        n = int(rng.integers(3, 9))
        c["lens"] = [int(x) for x in rng.integers(1, 400, size=n)]
        c["new"] = [min(L, int(x)) for L, x in zip(c["lens"], rng.integers(1, cap + 1, size=n))]
    return c


def _workload(c):
    H = c["Hkv"] * c["G"]
    common = dict(dtype=c["dtype"], H=H, Hkv=c["Hkv"], D=c["D"], B=c["B"],
                  partition_size=c["part"], sliding_window=c["window"])
    if c["kind"] == "forks":
        return W.custom_forks(f"rand{c['seed']}", c["seed"], c["prompts"], c["samples"],
                              c["appends"], kernel_block_size=c["kernel_block"], **common)
    return W.custom_multi(f"rand{c['seed']}", c["seed"], c["lens"], c["new"], **common)


@pytest.mark.parametrize("seed", range(NUM_CASES))
def test_random_configuration(seed):
    _require_gpu()
    from paged_kv_cache_123_amd import ops
    c = draw_case(seed)
    print(f"[random] {c}", flush=True)
    prev = ops.set_decode_kernel(c["kernel"])
    try:
        w = _workload(c)
        vals = W.make_values(w, DEV)
        host = {k: to_host(v) for k, v in vals.items()}
        ora = OracleStep(w)
        sep = _step(w, {k: v.clone() for k, v in vals.items()})
        assert np.array_equal(sep.tables_host.astype(np.int64), ora.tables)
        assert [tuple(p) for p in sep.cow_pairs_host.tolist()] == ora.cow_pairs
        sep.run()
        torch.cuda.synchronize()
        kc, vc = host["key_cache"], host["value_cache"]
        ora.apply_copies(kc, vc)
        ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
        assert to_host(sep.slot_mapping).tolist() == ora.slot_mapping()
        assert np.array_equal(to_host(sep.key_cache), kc)
        assert np.array_equal(to_host(sep.value_cache), vc)
        multi = c["kind"] == "multi"
        want = (ora.attention_multi(host["query"], kc, vc) if multi
                else ora.attention(host["query"], kc, vc))
        check_attention(to_host(sep.out), want, w.dtype, f"separate calls, case {seed}")
        step = _step(w, vals)
        if not step.fused_ok:
            return  # copy-on-write of a block of several kernel blocks: no one-launch form
        out = step.run(fused=True)
        torch.cuda.synchronize()
        gk, gv = to_host(step.key_cache), to_host(step.value_cache)
        if not multi:
            for blk, off in _dead_cow_slots(ora, w):
                gk[blk, :, off, :] = kc[blk, :, off, :]
                gv[blk, :, off, :] = vc[blk, :, off, :]
        assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
        check_attention(to_host(out), want, w.dtype, f"one launch, case {seed}")
        raw = (lambda t: t) if out.dtype == torch.float32 else (lambda t: t.view(torch.int16))
        assert torch.equal(raw(out), raw(sep.out)), f"case {seed}: paths differ"
    finally:
        ops.set_decode_kernel(prev)
