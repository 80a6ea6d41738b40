"""GPU parity of the cascade step: a prefix several sequences share is read
once per group of sharers, per shared partition (split plans) or in one
single-pass item per group that then reads every member's own tokens.

Checked against the oracle (tables, slots and every readable cache slot
bit-exact; attention within the stated tolerances).  A split cascade step is
also checked against the ordinary split step on the matrix-core kernel with
the same partition size, which must give identical bits: a group item
computes each member's column with the same arithmetic as that member's own
item would.  A single-pass cascade step accumulates the prefix and the
member's own tokens in another order than a plain single pass, so there the
oracle alone decides; running it again must give identical bits.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import OracleStep, to_host
from test_gpu_parity import _dead_cow_slots, _require_gpu, check_attention

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _steps(w, part, group, fused=True, chunk=0):
    from paged_kv_cache_123_amd import ops
    from paged_kv_cache_123_amd.step import DecodeStep
    vals = W.make_values(w, DEV)
    host = {k: to_host(v) for k, v in vals.items()}
    plain_vals = {k: v.clone() for k, v in vals.items()}
    casc = DecodeStep(w.num_blocks, w.block_size, w.free_order, w.prefill, w.step, vals, w.scale,
                      part, cascade=group, cascade_chunk=chunk)
    assert casc.cascade_chunk == chunk
    prev = ops.set_decode_kernel("mfma")
    try:
        plain = DecodeStep(w.num_blocks, w.block_size, w.free_order, w.prefill, w.step,
                           plain_vals, w.scale, part)
        plain.run(fused=True)
    finally:
        ops.set_decode_kernel(prev)
    casc.slot_mapping.fill_(-7)
    out = casc.run(fused=fused)
    torch.cuda.synchronize()
    return casc, plain, out, host


def _check(w, part, group, expect_groups=True, fused=True, chunk=0):
    """``fused``: the one-launch step; else copy_blocks, slot mapping, scatter
    and the cascade attention as separate launches.  ``chunk``: a chunked
    single-pass plan with pieces of that many tokens (partials and a merge)."""
    casc, plain, out, host = _steps(w, part, group, fused, chunk)
    if expect_groups:
        assert casc.max_group >= 2, "the batch should form groups"
    ora = OracleStep(w)
    assert np.array_equal(casc.tables_host.astype(np.int64), ora.tables)
    assert to_host(casc.slot_mapping).tolist() == ora.slot_mapping()
    kc, vc = host["key_cache"], host["value_cache"]
    ora.apply_copies(kc, vc)
    ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
    gk, gv = to_host(casc.key_cache), to_host(casc.value_cache)
    for blk, off in _dead_cow_slots(ora, w):
        gk[blk, :, off, :] = kc[blk, :, off, :]
        gv[blk, :, off, :] = vc[blk, :, off, :]
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    want = ora.attention(host["query"], kc, vc)
    check_attention(to_host(out), want, w.dtype, f"cascade P={part} group={group} chunk={chunk}")
    if part:
        assert torch.equal(out.view(torch.int16), plain.out.view(torch.int16)), \
            "cascade and plain split steps differ"
    else:
        first = out.clone()
        casc.run(fused=not fused)  # writes the same rows again, the other way
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), casc.out.view(torch.int16)), \
            "single-pass cascade: one launch and separate calls differ"


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "calls"])
@pytest.mark.parametrize("chunk,group", [(256, 8), (512, 8), (1024, 8), (128, 3), (32, 16)])
def test_shared_prefix_batch_chunked(chunk, group, fused):
    """The shared-prefix configuration on a chunked plan: each 1024-token
    prefix in pieces of ``chunk`` tokens, one workgroup per piece and KV head,
    the rest of the prefix and the samples' own tokens in the group's last
    item, partials merged."""
    _require_gpu()
    print(f"[cascade] shared prefix chunked chunk={chunk} group={group} fused={fused}",
          flush=True)
    _check(W.shared_prefix_bf16(), 0, group, fused=fused, chunk=chunk)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "calls"])
@pytest.mark.parametrize("part,group", [(256, 8), (512, 8), (256, 3), (1024, 16), (0, 8),
                                        (0, 3), (0, 16)])
def test_shared_prefix_batch_full_size(part, group, fused):
    """16 prompts x 8 samples sharing 1024-token prefixes (the shared-prefix
    configuration)."""
    _require_gpu()
    print(f"[cascade] shared prefix P={part} group={group} fused={fused}", flush=True)
    _check(W.shared_prefix_bf16(), part, group, fused=fused)


FORK_CASES = [
    # dtype, B, G, partition, group, prompts, samples, appends (per sample, cycled)
    ("bf16", 16, 1, 64, 8, [300, 77, 129], 5, [1, 3, 17, 2, 40]),
    ("f16", 16, 2, 32, 8, [200, 33], 4, [1, 1, 9, 16]),
    ("bf16", 32, 4, 64, 4, [500, 64, 65], 3, [2, 31, 1]),
    ("bf16", 64, 8, 128, 2, [700], 6, [1, 5, 64, 3, 2, 9]),
    ("f16", 128, 1, 256, 16, [1000, 257], 8, [1, 2, 3, 4, 5, 6, 7, 130]),
    ("bf16", 16, 1, 16, 2, [48, 49, 15], 3, [1, 16, 2]),
]


@pytest.mark.parametrize("mode", ["split", "single", "chunked"])
@pytest.mark.parametrize("dtype,B,G,part,group,prompts,samples,appends", FORK_CASES,
                         ids=[f"{c[0]}-B{c[1]}-G{c[2]}-P{c[3]}-g{c[4]}" for c in FORK_CASES])
def test_forks(dtype, B, G, part, group, prompts, samples, appends, mode):
    """Forked samples of several prompts, several new tokens per sample,
    copy-on-write tails, prefixes that end inside a partition; chunked plans
    use pieces of the case's partition size, so own tokens reach past the
    group's last slot (marked empty for the merge)."""
    _require_gpu()
    chunk = part if mode == "chunked" else 0
    part = part if mode == "split" else 0
    print(f"[cascade] forks {dtype} B={B} G={G} P={part} chunk={chunk} group={group}",
          flush=True)
    rows = [[appends[(g + j) % len(appends)] for j in range(samples)]
            for g in range(len(prompts))]
    w = W.custom_forks("cascade", 41, prompts, samples, rows, dtype=dtype, H=2 * G, Hkv=2,
                       D=128, B=B, partition_size=part)
    _check(w, part, group, fused=mode != "single", chunk=chunk)


@pytest.mark.parametrize("part,chunk", [(64, 0), (0, 0), (0, 64)])
def test_no_sharing_runs_as_the_plain_step(part, chunk):
    _require_gpu()
    w = W.custom_decode("cascade_none", 43, [1, 17, 300, 1025, 64], dtype="bf16", H=8, Hkv=2,
                        D=128, B=16, partition_size=part)
    _check(w, part, 4, expect_groups=False, chunk=chunk)


ROUND_CASES = [
    # B, G, group, prompts, samples, appends: prefixes and own tokens longer
    # than one round of the single-pass kernel (2048 tokens), pieces cut
    # inside a member's tokens
    (16, 1, 16, [4500, 2100], 16, [300, 1, 257, 64, 129, 2, 33, 200]),
    (4, 2, 8, [2049, 40], 8, [1, 700, 3, 2047]),
    (128, 4, 4, [6000], 4, [1, 128, 129, 5]),
    (1, 1, 8, [2100], 5, [3, 1, 2, 40, 9]),
]


@pytest.mark.parametrize("chunk", [0, 512])
@pytest.mark.parametrize("B,G,group,prompts,samples,appends", ROUND_CASES,
                         ids=[f"B{c[0]}-G{c[1]}-g{c[2]}-{c[3][0]}" for c in ROUND_CASES])
def test_single_pass_rounds(B, G, group, prompts, samples, appends, chunk):
    """Also chunked: the group's last item then reads several rounds of the
    members' own tokens, reaching many slots past its own."""
    _require_gpu()
    print(f"[cascade] rounds B={B} G={G} group={group} prompts={prompts} chunk={chunk}",
          flush=True)
    rows = [[appends[(g + j) % len(appends)] for j in range(samples)]
            for g in range(len(prompts))]
    w = W.custom_forks("cascade_rounds", 47, prompts, samples, rows, dtype="bf16", H=2 * G,
                       Hkv=2, D=128, B=B, partition_size=0)
    _check(w, 0, group, chunk=chunk)


@pytest.mark.parametrize("chunk", [0, 256])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "calls"])
def test_prefix_cache_batch_single_pass(fused, chunk):
    """128 requests over 16 cached system prompts: the prompt blocks the
    prefix cache hands to each prompt's requests form the groups."""
    _require_gpu()
    print(f"[cascade] prefix-cache batch fused={fused} chunk={chunk}", flush=True)
    _check(W.prefix_cache_bf16(), 0, 8, fused=fused, chunk=chunk)


@pytest.mark.parametrize("part,chunk", [(0, 0), (64, 0), (0, 32)])
def test_prefix_cache_hits_and_evictions(part, chunk):
    """A tight pool: finished requests' cached blocks are evicted while other
    requests still hit theirs."""
    _require_gpu()
    B = 16
    systems = [3 * B + 5, 5 * B, 2 * B + 1]
    requests = [(0, 7), (1, 3), (0, 2 * B), (2, 1), (-1, 4 * B), (1, B), (0, 9), (2, 3 * B),
                (1, 2), (0, 1)]
    w = W.custom_prefix("cascade_prefix", 53, systems, requests, dtype="bf16", H=8, Hkv=2,
                        D=128, B=B, finished={0, 3, 4, 6}, partition_size=part, num_blocks=24)
    _check(w, part, 4, expect_groups=False, chunk=chunk)


def test_long_prompts_take_a_chunked_plan_by_themselves():
    """Two prompts of ~9k tokens forked 8 ways on a 32q/8kv layer: the step
    chooses 2048-token pieces (the single-pass plan would have 32
    workgroups); one launch and separate calls against the oracle, and
    bit-identical to each other."""
    _require_gpu()
    from paged_kv_cache_123_amd.step import DecodeStep
    w = W.shared_long_prompt_bf16(num_groups=2, prompt=9000)
    print(f"[cascade] {w.notes}", flush=True)
    vals = W.make_values(w, DEV)
    host = {k: to_host(v) for k, v in vals.items()}
    step = DecodeStep(w.num_blocks, w.block_size, w.free_order, w.prefill, w.step, vals,
                      w.scale, 0)
    assert step.cascade == 4 and step.cascade_chunk == 2048
    out = step.run(fused=True).clone()
    torch.cuda.synchronize()
    ora = OracleStep(w)
    kc, vc = host["key_cache"], host["value_cache"]
    ora.apply_copies(kc, vc)
    ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
    check_attention(to_host(out), ora.attention(host["query"], kc, vc), w.dtype, w.name)
    step.run(fused=False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), step.out.view(torch.int16))
