"""Cache slots that hold no token of any sequence (free blocks, and the
slots past every holder's length in a sequence's last block) are filled with
NaN before the step.  No kernel may let them reach an output: the tiles that
run past a sequence's end, the clamped rows of a partial tile, the chunk
ends of the prefill kernel and the copied tails of the cascade kernel all
stay inside the written slots or mask what they read.  Outputs are checked
against the oracle (which reads only the written slots), for the separate
calls and for the one-launch step."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import OracleStep, to_host
from test_gpu_parity import DEV, _require_gpu, _step, check_attention

pytestmark = pytest.mark.gpu


def _written_slots(ora, num_blocks):
    """[kernel blocks, kernel block size] True where some sequence keeps a
    token after the step."""
    kb = ora.kb
    ok = np.zeros((num_blocks, kb), dtype=bool)
    for r, L in enumerate(ora.context_lens.tolist()):
        for p in range(int(L)):
            b = int(ora.tables[r, p // kb])
            if b >= 0:
                ok[b, p % kb] = True
    return ok


def _poison(vals, ok):
    bad = torch.from_numpy(~ok).to(DEV)  # [NB, B]
    for name in ("key_cache", "value_cache"):
        c = vals[name]  # [NB, H_kv, B, D]
        c.masked_fill_(bad[:, None, :, None], float("nan"))


CASES = [
    ("tiny_fp32", lambda: W.tiny_fp32(), None, 0),
    ("tiny_fp32_split", lambda: W.tiny_fp32(), 16, 0),
    ("llama16", lambda: W.llama7b_fp16(num_seqs=16), None, 0),
    ("llama8_split", lambda: W.llama7b_fp16(num_seqs=8), 256, 0),
    ("gqa32", lambda: W.qwen72b_gqa_bf16(num_seqs=32), None, 0),
    ("shared2_cascade", lambda: W.shared_prefix_bf16(num_groups=2), None, None),
    ("prefix_cache_cascade", lambda: W.prefix_cache_bf16(num_systems=2, per_system=4), None,
     None),
    ("window4", lambda: W.mistral7b_swa_bf16(num_seqs=4), None, 0),
    ("spec4_llama8", lambda: W.llama7b_spec4_fp16(num_seqs=8), None, 0),
    ("prefill_llama2", lambda: W.llama7b_prefill512_fp16(num_seqs=2), None, 0),
    ("prefill_gqa2", lambda: W.qwen72b_prefill512_bf16(num_seqs=2), None, 0),
]


@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
@pytest.mark.parametrize("name,make,part,cascade", CASES, ids=[c[0] for c in CASES])
def test_unwritten_slots_never_reach_an_output(name, make, part, cascade, fused):
    _require_gpu()
    w = make()
    print(f"[poison] {name} fused={fused}", flush=True)
    vals = W.make_values(w, DEV)
    ora = OracleStep(w)
    ok = _written_slots(ora, vals["key_cache"].shape[0])
    # the poison reaches into blocks the step reads: some sequence ends
    # inside a block whose later slots are unwritten
    tails = [(int(ora.tables[r, (int(L) - 1) // ora.kb]), int(L) % ora.kb)
             for r, L in enumerate(ora.context_lens.tolist()) if int(L) % ora.kb]
    assert any(not ok[b, off:].all() for b, off in tails), "no partial block is poisoned"
    _poison(vals, ok)
    host = {k: to_host(v) for k, v in vals.items()}
    step = _step(w, vals, part, cascade=cascade)
    if fused and not step.fused_ok:
        pytest.skip("this step has no one-launch form")
    out = step.run(fused=fused)
    torch.cuda.synchronize()
    kc, vc = host["key_cache"], host["value_cache"]
    ora.apply_copies(kc, vc)
    ora.apply_scatter(kc, vc, host["new_key"], host["new_value"])
    if w.extra.get("queries") == "all":
        want = ora.attention_multi(host["query"], kc, vc)
    else:
        want = ora.attention(host["query"], kc, vc)
    assert np.isfinite(want).all()
    check_attention(to_host(out), want, w.dtype, f"poisoned {name}")
