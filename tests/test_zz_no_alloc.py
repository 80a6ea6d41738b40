"""The split-K decode without allocation
(pa_paged_attention_decode_split_noalloc, its workspace a static device
array) against pa_paged_attention_decode_split with a caller workspace:
bit-identical outputs, two calls in a row with the second one smaller, and
both within the attention tolerances of the float64 oracle."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from oracle.dtypes import decode
from oracle_side import OracleStep, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _split_step(name, seed, lens, dtype, H, Hkv, B, P):
    from paged_kv_cache_123_amd.step import DecodeStep
    w = W.custom_decode(name, seed, lens, dtype=dtype, H=H, Hkv=Hkv, D=128, B=B,
                        partition_size=P)
    vals = W.make_values(w, DEV)
    host = {k: to_host(v) for k, v in vals.items()}
    step = DecodeStep(w.num_blocks, w.block_size, w.free_order, w.prefill, w.step, vals,
                      w.scale, P, planned=False)
    step.run()  # copy-on-write, slot mapping, scatter, split attention with a workspace
    torch.cuda.synchronize()
    return w, host, step


def _check_oracle(w, host, step, got):
    ora = OracleStep(w)
    kc, vc = host["key_cache"], host["value_cache"]
    ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
    want = ora.attention(host["query"], kc, vc)
    g = decode(to_host(got), w.dtype)
    err = float(np.abs(g - want).max())
    rel = float(np.linalg.norm(g - want) / np.linalg.norm(want))
    assert err <= 2e-2 and rel <= 5e-3, f"{w.name}: max-abs {err:.3e}, rel-L2 {rel:.3e}"


def test_noalloc_split_equals_the_workspace_call_twice_in_a_row():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from paged_kv_cache_123_amd import ops
    cases = [
        # (lens, dtype, H, Hkv, B, P): the first fills 32 x 32 x 16 partitions
        # (8.4 MB of the array), the second is smaller and must not see
        # anything of the first
        ([4096 - 7 * i for i in range(32)], "bf16", 32, 32, 64, 256),
        ([1, 17, 300, 513, 1000], "f16", 8, 2, 16, 128),
    ]
    for i, (lens, dtype, H, Hkv, B, P) in enumerate(cases):
        print(f"[noalloc] call {i}: {len(lens)} seqs, max len {max(lens)}, {dtype} H={H} "
              f"Hkv={Hkv} B={B} P={P}", flush=True)
        w, host, step = _split_step(f"noalloc{i}", 70 + i, lens, dtype, H, Hkv, B, P)
        out = torch.full_like(step.out, float("nan"))
        ops.paged_attention_decode_split_noalloc(out, step.query, step.key_cache,
                                                 step.value_cache, step.block_tables,
                                                 step.context_lens, step.scale,
                                                 step.max_context_len, P)
        torch.cuda.synchronize()
        assert torch.equal(out, step.out), f"call {i}: differs from the workspace call"
        _check_oracle(w, host, step, out)


def test_noalloc_refuses_a_launch_beyond_its_array():
    from paged_kv_cache_123_amd._lib import PA_EINVAL, lib
    need = lib().pa_split_workspace_bytes(64, 64, 128, 65536, 512)
    assert need > lib().pa_split_workspace_bytes(32, 32, 128, 32768, 512)
    t = torch.zeros(8, dtype=torch.int32, device=DEV)
    st = lib().pa_paged_attention_decode_split_noalloc(
        t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), 4096,
        t.data_ptr(), 64, 64, 8, 128, 16, 65536, 1.0, 2, 512, None)
    assert st == PA_EINVAL
    assert "PA_NOALLOC_WORKSPACE_BYTES" in lib().pa_last_error().decode()
