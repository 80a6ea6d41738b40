"""Seeded synthetic workloads for the paged-KV decode path.

Shared by the tests, bench.py and the oracle side.  A workload is a recipe:
model shape, storage dtype, the pool size and its initial free order, the
host-allocator operations that build the cache before the decode step (add,
append, fork), the tokens the step appends, and value tensors drawn from a
seeded generator.  It holds no part of the method: block tables, slots and
copy-on-write pairs come from replaying the operations through an allocator
(the library's or the oracle's), and attention is computed by the kernels or
by the oracle.

Shapes follow the model families the pages discuss: Llama-7B (32 heads of
128, fp16), a Qwen2.5-72B-style GQA layer (64 query heads sharing 8 KV heads),
parallel sampling with a shared prompt, and a long context cut into
partitions.  Structure comes from numpy.random.default_rng(seed); values come
from a torch generator seeded with the same seed on the target device.

A decode step's context length counts the token the step writes: a sequence
listed with length L is prefilled with L - 1 tokens and the step appends the
L-th, so attention covers L tokens.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


@dataclass
class Workload:
    name: str
    dtype: str                 # storage dtype: "f32" | "f16" | "bf16"
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    scale: float
    sigma: float               # standard deviation of q, K and V values
    seed: int
    free_order: np.ndarray     # int32 [num_blocks], head of the free queue first
    seqs: list                 # sequence ids, one per batch row of the step
    prefill: list              # ("add", s) | ("append", s, n) | ("fork", parent, child)
    step: list                 # (s, n): tokens appended by the step, in order
    context_lens: list         # tokens each row attends over after the step
    partition_size: int = 0    # split-K partition (0: single pass)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.seqs)

    @property
    def num_step_tokens(self) -> int:
        return sum(n for _, n in self.step)

    @property
    def max_context_len(self) -> int:
        return int(max(self.context_lens))

    @property
    def kv_tokens(self) -> int:
        return int(sum(self.context_lens))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def table_width(self) -> int:
        return -(-self.max_context_len // self.block_size)


def _decode_batch(name, seed, lens, *, dtype, H, Hkv, D, B, num_blocks, sigma,
                  partition_size=0, notes="", rng=None):
    rng = rng if rng is not None else np.random.default_rng(seed)
    order = rng.permutation(num_blocks).astype(np.int32)
    prefill, step = [], []
    for s, L in enumerate(lens):
        prefill.append(("add", s))
        if L > 1:
            prefill.append(("append", s, int(L) - 1))
        step.append((s, 1))
    return Workload(name=name, dtype=dtype, num_heads=H, num_kv_heads=Hkv, head_size=D,
                    block_size=B, num_blocks=num_blocks, scale=1.0 / math.sqrt(D), sigma=sigma,
                    seed=seed, free_order=order, seqs=list(range(len(lens))), prefill=prefill,
                    step=step, context_lens=[int(L) for L in lens],
                    partition_size=partition_size, notes=notes)


def _options(w, sliding_window=0, kernel_block_size=0):
    """Record a sliding window and a kernel block size on a workload."""
    if sliding_window:
        w.extra["sliding_window"] = int(sliding_window)
    if kernel_block_size and kernel_block_size != w.block_size:
        w.extra["kernel_block_size"] = int(kernel_block_size)
    return w


def custom_decode(name, seed, lens, *, dtype, H, Hkv, D, B, num_blocks=None, sigma=1.0,
                  partition_size=0, sliding_window=0, kernel_block_size=0):
    """A decode batch with the given context lengths (edge-case tests)."""
    lens = [int(L) for L in lens]
    nb = num_blocks if num_blocks is not None else _blocks_for(lens, B) + 3
    w = _decode_batch(name, seed, lens, dtype=dtype, H=H, Hkv=Hkv, D=D, B=B,
                      num_blocks=nb, sigma=sigma, partition_size=partition_size)
    return _options(w, sliding_window, kernel_block_size)


def custom_forks(name, seed, prompts, samples, appends, *, dtype, H, Hkv, D, B,
                 partition_size=0, sigma=1.0, sliding_window=0, kernel_block_size=0):
    """Parallel-sampling batch for edge-case tests: prompt g is prefilled once
    and forked into ``samples`` sequences; sample j of group g then appends
    appends[g][j] tokens (several tokens per sample, across block and
    partition boundaries)."""
    rng = np.random.default_rng(seed)
    prefill, step, seqs, lens = [], [], [], []
    for g, P in enumerate(prompts):
        lead = g * samples
        prefill += [("add", lead), ("append", lead, int(P))]
        for j in range(1, samples):
            prefill.append(("fork", lead, lead + j))
        for j in range(samples):
            step.append((lead + j, int(appends[g][j])))
            seqs.append(lead + j)
            lens.append(int(P) + int(appends[g][j]))
    nb = _blocks_for(prompts, B) + sum(-(-int(a) // B) + 1 for row in appends for a in row) + 4
    order = rng.permutation(nb).astype(np.int32)
    w = Workload(name=name, dtype=dtype, num_heads=H, num_kv_heads=Hkv, head_size=D,
                 block_size=B, num_blocks=nb, scale=1.0 / math.sqrt(D), sigma=sigma,
                 seed=seed, free_order=order, seqs=seqs, prefill=prefill, step=step,
                 context_lens=lens, partition_size=partition_size)
    return _options(w, sliding_window, kernel_block_size)


def _blocks_for(lens, B) -> int:
    """Pool sizing only: blocks that sequences of these lengths occupy."""
    return int(sum(-(-int(L) // B) for L in lens))


def tiny_fp32(num_seqs=None):
    lens = [7, 9, 16, 37]
    return _decode_batch("tiny_fp32", 1, lens, dtype="f32", H=2, Hkv=2, D=64, B=4,
                         num_blocks=32, sigma=1.0,
                         notes="4 sequences, B=4, MHA 2x64 fp32, 32-block pool")


def llama7b_fp16(num_seqs=64):
    rng = np.random.default_rng(2)
    lens = rng.integers(128, 2049, size=64)[:num_seqs]
    nb = math.ceil(1.1 * _blocks_for(lens, 16))
    return _decode_batch("llama7b_fp16", 2, lens, dtype="f16", H=32, Hkv=32, D=128, B=16,
                         num_blocks=nb, sigma=1.0, rng=rng,
                         notes="Llama-7B layer: 32x128 MHA fp16, B=16, L~U[128,2048], pool +10%")


def qwen72b_gqa_bf16(num_seqs=256):
    rng = np.random.default_rng(3)
    z = rng.standard_normal(256)[:num_seqs]
    lens = np.clip(np.rint(np.exp(math.log(1024.0) + z)), 16, 8192).astype(np.int64)
    nb = _blocks_for(lens, 16)
    return _decode_batch("qwen72b_gqa_bf16", 3, lens, dtype="bf16", H=64, Hkv=8, D=128, B=16,
                         num_blocks=nb, sigma=0.5, rng=rng,
                         notes="GQA 64q/8kv x128 bf16, B=16, lognormal lengths (median 1024, "
                               "sigma 1, clipped [16, 8192]), pool exactly full")


def shared_prefix_bf16(num_groups=16):
    """Parallel sampling: each prompt group's blocks are shared by 8 samples
    (fork), then every sample appends 1-64 tokens of its own."""
    rng = np.random.default_rng(4)
    samples, B = 8, 16
    r = rng.integers(1, 16, size=16)[:num_groups]
    prompts = 1024 + r
    appends = rng.integers(1, 65, size=(16, samples))[:num_groups]
    prefill, step, seqs, lens = [], [], [], []
    for g in range(num_groups):
        lead = g * samples
        prefill += [("add", lead), ("append", lead, int(prompts[g]))]
        for j in range(1, samples):
            prefill.append(("fork", lead, lead + j))
        for j in range(samples):
            step.append((lead + j, int(appends[g, j])))
            seqs.append(lead + j)
            lens.append(int(prompts[g] + appends[g, j]))
    # pool sizing: shared prompt blocks once, plus each sample's own blocks
    own = sum(-(-int(prompts[g] + appends[g, j]) // B) - int(prompts[g]) // B
              for g in range(num_groups) for j in range(samples))
    unique = sum(int(p) // B for p in prompts) + own
    nb = math.ceil(1.1 * unique)
    order = rng.permutation(nb).astype(np.int32)
    return Workload(name="shared_prefix_bf16", dtype="bf16", num_heads=32, num_kv_heads=32,
                    head_size=128, block_size=B, num_blocks=nb, scale=1.0 / math.sqrt(128),
                    sigma=1.0, seed=4, free_order=order, seqs=seqs, prefill=prefill, step=step,
                    context_lens=lens,
                    notes=f"{num_groups} prompts x 8 samples, prompt 1024+U[1,15] shared "
                          "(refcount 8), each sample appends U[1,64] tokens; 32x128 bf16, B=16",
                    extra={"unique_blocks": unique, "prompts": prompts.tolist()})


def shared_long_prompt_bf16(num_groups=2, prompt=16384, samples=8):
    """Parallel sampling over long prompts on a grouped-query layer: each of a
    few prompts of ``prompt`` + U{1..15} tokens is shared by ``samples``
    samples that each append U{1..64} tokens; 32 query heads over 8 KV heads,
    bf16, B = 16.  Few groups over long prefixes: a cascade plan with one
    workgroup per group and KV head has few workgroups."""
    rng = np.random.default_rng(10)
    B = 16
    prompts = prompt + rng.integers(1, 16, size=num_groups)
    appends = rng.integers(1, 65, size=(num_groups, samples))
    prefill, step, seqs, lens = [], [], [], []
    for g in range(num_groups):
        lead = g * samples
        prefill += [("add", lead), ("append", lead, int(prompts[g]))]
        for j in range(1, samples):
            prefill.append(("fork", lead, lead + j))
        for j in range(samples):
            step.append((lead + j, int(appends[g, j])))
            seqs.append(lead + j)
            lens.append(int(prompts[g] + appends[g, j]))
    own = sum(-(-int(prompts[g] + appends[g, j]) // B) - int(prompts[g]) // B
              for g in range(num_groups) for j in range(samples))
    unique = sum(int(p) // B for p in prompts) + own
    nb = math.ceil(1.1 * unique)
    order = rng.permutation(nb).astype(np.int32)
    return Workload(name="shared_long_prompt_bf16", dtype="bf16", num_heads=32, num_kv_heads=8,
                    head_size=128, block_size=B, num_blocks=nb, scale=1.0 / math.sqrt(128),
                    sigma=1.0, seed=10, free_order=order, seqs=seqs, prefill=prefill, step=step,
                    context_lens=lens,
                    notes=f"{num_groups} prompts of {prompt}+U[1,15] tokens x {samples} samples, "
                          "each appends U[1,64]; 32q/8kv x128 bf16, B=16",
                    extra={"unique_blocks": unique, "prompts": prompts.tolist()})


def shared_prefix_cascade_bf16(num_groups=16, partition_size=0, group=8):
    """The shared-prefix batch run through a cascade plan for groups of up to
    ``group`` samples: single pass (``partition_size`` 0: one workgroup per
    group and KV head reads the shared prompt blocks once, then each sample's
    own tokens), or partitions of ``partition_size`` tokens lying wholly inside
    the shared blocks computed once per group."""
    w = shared_prefix_bf16(num_groups)
    w.name = "shared_prefix_cascade_bf16"
    w.partition_size = int(partition_size)
    w.extra["cascade"] = int(group)
    w.notes += (f"; cascade plan, groups of up to {group}, "
                + (f"partitions of {partition_size}" if partition_size else "single pass"))
    return w


def long_context_bf16(num_seqs=32, context_len=32768):
    lens = [context_len] * num_seqs
    nb = math.ceil(1.05 * _blocks_for(lens, 64))
    return _decode_batch("long_context_bf16", 5, lens, dtype="bf16", H=32, Hkv=32, D=128, B=64,
                         num_blocks=nb, sigma=1.0, partition_size=512,
                         notes=f"{num_seqs} x {context_len} tokens, 32x128 MHA bf16, B=64, "
                               "split-K partitions of 512, pool +5%")


def qwen72b_gqa_tp8_bf16(num_seqs=256, partition_size=1024):
    """One GPU's share of the GQA layer under 8-way tensor parallelism: the
    same 256 sequences and lengths with 8 query heads and 1 KV head.  With one
    KV head a single pass has only 256 workgroups, so the share is split into
    partitions of 1024 tokens."""
    w = qwen72b_gqa_bf16(num_seqs)
    w.name = "qwen72b_gqa_tp8_bf16"
    w.num_heads, w.num_kv_heads = 8, 1
    w.partition_size = partition_size
    w.notes = ("GQA layer's share on one of 8 tensor-parallel GPUs: 256 seqs lognormal lengths, "
               "8 query heads sharing 1 KV head, head 128, bf16, B=16")
    return w


def llama7b_spec4_fp16(num_seqs=64, drafts=4):
    """The Llama-7B batch verifying 4 speculative tokens per sequence: every
    sequence appends 4 tokens and each of them is a query (causal)."""
    rng = np.random.default_rng(2)
    lens = rng.integers(128, 2049, size=64)[:num_seqs]
    w = custom_multi("llama7b_spec4_fp16", 2, lens, [drafts] * len(lens), dtype="f16", H=32,
                     Hkv=32, D=128, B=16)
    w.num_blocks = math.ceil(1.1 * _blocks_for(lens, 16))
    w.free_order = np.random.default_rng(12).permutation(w.num_blocks).astype(np.int32)
    w.notes = "Llama-7B layer, 64 seqs L~U[128,2048], 4 speculative tokens each, all queries"
    return w


def llama7b_prefill512_fp16(num_seqs=16, chunk=512):
    """Chunked prefill on the Llama-7B layer: each sequence has a cached
    prefix of U[0, 1536] tokens and appends a ``chunk``-token prefill chunk
    in the step, every new token a query (causal over the chunk)."""
    rng = np.random.default_rng(8)
    prefix = rng.integers(0, 1537, size=num_seqs)
    lens = [int(p) + chunk for p in prefix]
    w = custom_multi("llama7b_prefill512_fp16", 8, lens, [chunk] * num_seqs, dtype="f16",
                     H=32, Hkv=32, D=128, B=16)
    w.notes = (f"{num_seqs} sequences, cached prefix U[0,1536] + a {chunk}-token prefill chunk "
               "(every new token a query, causal); 32x128 MHA fp16, B=16")
    return w


def qwen72b_prefill512_bf16(num_seqs=16, chunk=512):
    """Chunked prefill on the Qwen2.5-72B-style GQA layer (64 query / 8 KV
    heads, bf16): the Llama-7B prefill batch's prefixes and chunks, where one
    K/V row serves 8 query heads of every chunk token (above the matrix-core
    ridge: bound by the MFMA rate, not HBM)."""
    rng = np.random.default_rng(8)
    prefix = rng.integers(0, 1537, size=num_seqs)
    lens = [int(p) + chunk for p in prefix]
    w = custom_multi("qwen72b_prefill512_bf16", 9, lens, [chunk] * num_seqs, dtype="bf16",
                     H=64, Hkv=8, D=128, B=16, sigma=0.5)
    w.notes = (f"{num_seqs} sequences, cached prefix U[0,1536] + a {chunk}-token prefill chunk "
               "(every new token a query, causal); GQA 64q/8kv x 128 bf16, B=16")
    return w


def llama7b_longprefill_fp16(prefix=32256, chunk=512, partition_size=4096):
    """One sequence of the Llama-7B layer with a long cached prefix taking a
    512-token prefill chunk: four query blocks x 32 KV heads give only 128
    workgroups in one pass, so the keys are cut into partitions (the split
    prefill kernel and its merge)."""
    w = custom_multi("llama7b_longprefill_fp16", 10, [prefix + chunk], [chunk], dtype="f16",
                     H=32, Hkv=32, D=128, B=16, partition_size=partition_size)
    w.notes = (f"1 sequence, cached prefix {prefix} + a {chunk}-token prefill chunk (every new "
               f"token a query, causal); 32x128 MHA fp16, B=16, partitions of {partition_size}")
    return w


def qwen72b_longprefill_bf16(prefix=32256, chunk=512, partition_size=4096):
    """The long-prefix prefill chunk on the Qwen2.5-72B-style GQA layer (64
    query / 8 KV heads, bf16): 32 query blocks x 8 KV heads, 256 workgroups in
    one pass (one per CU), partitions by default."""
    w = custom_multi("qwen72b_longprefill_bf16", 11, [prefix + chunk], [chunk], dtype="bf16",
                     H=64, Hkv=8, D=128, B=16, sigma=0.5, partition_size=partition_size)
    w.notes = (f"1 sequence, cached prefix {prefix} + a {chunk}-token prefill chunk; GQA 64q/8kv "
               f"x 128 bf16, B=16, partitions of {partition_size}")
    return w


def qwen72b_gqa_spec2_bf16(num_seqs=256, drafts=2):
    """The GQA batch verifying 2 speculative tokens per sequence (2 x 8 query
    vectors per KV head fill the 16 matrix-core columns)."""
    rng = np.random.default_rng(3)
    z = rng.standard_normal(256)[:num_seqs]
    lens = np.clip(np.rint(np.exp(math.log(1024.0) + z)), 16, 8192).astype(np.int64)
    w = custom_multi("qwen72b_gqa_spec2_bf16", 3, lens, [drafts] * len(lens), dtype="bf16",
                     H=64, Hkv=8, D=128, B=16, sigma=0.5)
    w.notes = "GQA 64q/8kv layer, 256 seqs lognormal lengths, 2 speculative tokens each"
    return w


def custom_prefix(name, seed, systems, requests, *, dtype, H, Hkv, D, B, num_blocks=None,
                  finished=(), partition_size=0, sigma=1.0, vocab=32000):
    """Requests served through the prefix cache.  ``systems``: lengths of the
    shared system prompts; ``requests``: (system index or -1, suffix length)
    per request, in arrival order; ``finished``: requests that end before the
    decode step (freed right after the next request arrives, so their cached
    blocks wait in the LRU queue).  Every other request then decodes one
    token.  Token ids are drawn from ``vocab``."""
    rng = np.random.default_rng(seed)
    prompts = [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in systems]
    prefill, step, seqs, lens = [], [], [], []
    pending = []
    for r, (g, suffix) in enumerate(requests):
        prompt = np.concatenate([prompts[g] if g >= 0 else np.zeros(0, np.int32),
                                 rng.integers(0, vocab, size=int(suffix)).astype(np.int32)])
        prefill.append(("request", r, prompt, b""))
        for f in pending:
            prefill.append(("free", f))
        pending = [r] if r in finished else []
        if r not in finished:
            step.append((r, 1))
            seqs.append(r)
            lens.append(len(prompt) + 1)
    prefill += [("free", f) for f in pending]
    if num_blocks is None:
        num_blocks = _blocks_for([len(op[2]) + 1 for op in prefill if op[0] == "request"], B) + 4
    order = rng.permutation(num_blocks).astype(np.int32)
    return Workload(name=name, dtype=dtype, num_heads=H, num_kv_heads=Hkv, head_size=D,
                    block_size=B, num_blocks=num_blocks, scale=1.0 / math.sqrt(D), sigma=sigma,
                    seed=seed, free_order=order, seqs=seqs, prefill=prefill, step=step,
                    context_lens=lens, partition_size=partition_size)


def prefix_cache_bf16(num_systems=16, per_system=8):
    """Requests that share 16 system prompts of ~1k tokens, each with a
    private question of 16-256 tokens, arriving round-robin over the system
    prompts: the first request of each prompt computes it, the other seven
    take over its full blocks from the prefix cache; then all 128 decode one
    token (32x128 MHA bf16, B=16)."""
    rng = np.random.default_rng(7)
    systems = (1000 + rng.integers(0, 64, size=num_systems)).tolist()
    requests = [(g, int(rng.integers(16, 257))) for _ in range(per_system)
                for g in range(num_systems)]
    w = custom_prefix("prefix_cache_bf16", 7, systems, requests, dtype="bf16", H=32, Hkv=32,
                      D=128, B=16)
    w.notes = (f"{len(requests)} requests over {num_systems} cached system prompts of ~1k "
               "tokens + 16-256 private tokens, one decode token each; 32x128 MHA bf16, B=16")
    return w


def prefix_cache_cascade_bf16(num_systems=16, per_system=8, group=8):
    """The prefix-cache batch run through a single-pass cascade plan: the
    cached system-prompt blocks that a prompt's requests share are read once
    per group of up to ``group`` requests, then each request's own tokens."""
    w = prefix_cache_bf16(num_systems, per_system)
    w.name = "prefix_cache_cascade_bf16"
    w.extra["cascade"] = int(group)
    w.notes += f"; single-pass cascade plan, groups of up to {group}"
    return w


def mistral7b_swa_bf16(num_seqs=64, window=4096):
    """A Mistral-7B-style layer (32 query heads sharing 8 KV heads, head 128)
    with a 4096-token sliding window over contexts up to 16k: attention reads
    the last 4096 tokens of each sequence, and the blocks before the window
    are released before the step."""
    rng = np.random.default_rng(6)
    lens = rng.integers(2048, 16385, size=64)[:num_seqs]
    w = _decode_batch("mistral7b_swa_bf16", 6, lens, dtype="bf16", H=32, Hkv=8, D=128, B=16,
                      num_blocks=math.ceil(1.05 * _blocks_for(lens, 16)), sigma=1.0,
                      partition_size=0, rng=rng,
                      notes=f"{num_seqs} seqs L~U[2048,16384], 32q/8kv x 128 bf16, B=16, "
                            f"sliding window {window}, single pass")
    return _options(w, sliding_window=window)


def cp_decode(name, seed, lens, *, dtype, H, Hkv, D, B, world, interleave, partition_size,
              sigma=1.0, slack=1.0, notes=""):
    """A decode batch spread over a context-parallel group of ``world`` ranks.
    The allocator works in virtual blocks of B * world positions shared by
    the ranks; ``num_blocks`` is the size of each rank's pool (every rank
    holds B slots of each virtual block) and ``block_size`` the physical B."""
    lens = [int(L) for L in lens]
    nb = math.ceil(slack * _blocks_for(lens, B * world)) + 2
    w = _decode_batch(name, seed, lens, dtype=dtype, H=H, Hkv=Hkv, D=D, B=B, num_blocks=nb,
                      sigma=sigma, partition_size=partition_size, notes=notes)
    w.extra = {"cp_world": int(world), "cp_interleave": int(interleave)}
    return w


def cp_prefill(name, seed, lens, *, dtype, H, Hkv, D, B, world, interleave, partition_size,
               sigma=1.0):
    """Context-parallel parity case: the step writes every token of every
    sequence (a whole prompt, spread over the ranks by their slot mappings)
    and the last token of each sequence is the query."""
    lens = [int(L) for L in lens]
    w = cp_decode(name, seed, lens, dtype=dtype, H=H, Hkv=Hkv, D=D, B=B, world=world,
                  interleave=interleave, partition_size=partition_size, sigma=sigma)
    w.prefill = [("add", s) for s in range(len(lens))]
    w.step = [(s, L) for s, L in enumerate(lens)]
    return w


def long_context_cp8_bf16(num_seqs=32, context_len=32768):
    """The long-context batch spread over 8 context-parallel ranks (one token
    at a time in turn): one GPU's share is 32 x 4096 tokens."""
    return cp_decode("long_context_cp8_bf16", 5, [context_len] * num_seqs, dtype="bf16", H=32,
                     Hkv=32, D=128, B=64, world=8, interleave=1, partition_size=4096,
                     slack=1.05,
                     notes=f"{num_seqs} x {context_len} tokens over 8 context-parallel ranks "
                           "(interleave 1), 32x128 MHA bf16, B=64, partitions of 4096")


CONFIGS = {
    "tiny_fp32": tiny_fp32,
    "llama7b_fp16": llama7b_fp16,
    "qwen72b_gqa_bf16": qwen72b_gqa_bf16,
    "shared_prefix_bf16": shared_prefix_bf16,
    "long_context_bf16": long_context_bf16,
    "shared_prefix_cascade_bf16": shared_prefix_cascade_bf16,
    "shared_long_prompt_bf16": shared_long_prompt_bf16,
    "llama7b_spec4_fp16": llama7b_spec4_fp16,
    "llama7b_prefill512_fp16": llama7b_prefill512_fp16,
    "qwen72b_prefill512_bf16": qwen72b_prefill512_bf16,
    "llama7b_longprefill_fp16": llama7b_longprefill_fp16,
    "qwen72b_longprefill_bf16": qwen72b_longprefill_bf16,
    "qwen72b_gqa_spec2_bf16": qwen72b_gqa_spec2_bf16,
    "long_context_cp8_bf16": long_context_cp8_bf16,
    "qwen72b_gqa_tp8_bf16": qwen72b_gqa_tp8_bf16,
    "mistral7b_swa_bf16": mistral7b_swa_bf16,
    "prefix_cache_bf16": prefix_cache_bf16,
    "prefix_cache_cascade_bf16": prefix_cache_cascade_bf16,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)


def custom_multi(name, seed, lens, new_tokens, *, dtype, H, Hkv, D, B, partition_size=0,
                 sigma=1.0, sliding_window=0):
    """A batch whose step appends new_tokens[s] tokens to sequence s (its
    context_lens[s] = lens[s] counts them): speculative drafts or a short
    prefill chunk, every new token being a query."""
    lens = [int(L) for L in lens]
    rng = np.random.default_rng(seed)
    nb = _blocks_for(lens, B) + 3
    order = rng.permutation(nb).astype(np.int32)
    prefill, step = [], []
    for s, (L, n) in enumerate(zip(lens, new_tokens)):
        prefill.append(("add", s))
        if L > n:
            prefill.append(("append", s, L - int(n)))
        step.append((s, int(n)))
    w = Workload(name=name, dtype=dtype, num_heads=H, num_kv_heads=Hkv, head_size=D,
                 block_size=B, num_blocks=nb, scale=1.0 / math.sqrt(D), sigma=sigma,
                 seed=seed, free_order=order, seqs=list(range(len(lens))), prefill=prefill,
                 step=step, context_lens=lens, partition_size=partition_size,
                 extra={"queries": "all"})
    return _options(w, sliding_window)


def make_values(w: Workload, device, chunk_elems: int = 1 << 26):
    """Seeded value tensors of a workload on ``device``.

    Returns dict(key_cache, value_cache [NB, H_kv, B, D], query [S, H, D]
    (or [T, H, D] when every new token is a query, ``w.extra["queries"] ==
    "all"``), new_key, new_value [T, H_kv, D]); every element ~ N(0, sigma^2),
    drawn in fp32 and rounded to the storage dtype.  Unused cache slots hold values
    too, so nothing depends on memory the step never writes.
    """
    import torch

    tdt = getattr(torch, TORCH_DTYPES[w.dtype])
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)

    def draw(shape):
        out = torch.empty(shape, dtype=tdt, device=device)
        flat = out.view(shape[0], -1)
        per_row = flat.shape[1]
        rows = max(1, chunk_elems // max(per_row, 1))
        for i in range(0, shape[0], rows):
            j = min(shape[0], i + rows)
            x = torch.randn((j - i, per_row), generator=gen, device=device, dtype=torch.float32)
            flat[i:j] = (x * w.sigma).to(tdt)
        return out

    kb = w.extra.get("kernel_block_size", w.block_size)  # kernel blocks of the cache
    cache_shape = (w.num_blocks * (w.block_size // kb), w.num_kv_heads, kb, w.head_size)
    return {
        "key_cache": draw(cache_shape),
        "value_cache": draw(cache_shape),
        "query": draw(((w.num_step_tokens if w.extra.get("queries") == "all" else w.num_seqs),
                       w.num_heads, w.head_size)),
        "new_key": draw((w.num_step_tokens, w.num_kv_heads, w.head_size)),
        "new_value": draw((w.num_step_tokens, w.num_kv_heads, w.head_size)),
    }


def make_cp_values(w: Workload, device, ranks=None):
    """Seeded tensors of a context-parallel workload: the step's query,
    new_key and new_value (as ``make_values``), and each listed rank's own
    key/value cache [NB, H_kv, B, D] (``key_caches[r]``), drawn from a
    generator seeded by (seed, rank) so that ranks can be built one at a time."""
    import torch

    world = int(w.extra["cp_world"])
    ranks = list(range(world)) if ranks is None else list(ranks)
    tdt = getattr(torch, TORCH_DTYPES[w.dtype])

    def draw(gen, shape, chunk_rows=64):
        out = torch.empty(shape, dtype=tdt, device=device)
        for i in range(0, shape[0], chunk_rows):
            j = min(shape[0], i + chunk_rows)
            x = torch.randn((j - i,) + tuple(shape[1:]), generator=gen, device=device,
                            dtype=torch.float32)
            out[i:j] = (x * w.sigma).to(tdt)
        return out

    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    vals = {
        "query": draw(gen, (w.num_seqs, w.num_heads, w.head_size)),
        "new_key": draw(gen, (w.num_step_tokens, w.num_kv_heads, w.head_size)),
        "new_value": draw(gen, (w.num_step_tokens, w.num_kv_heads, w.head_size)),
        "key_caches": {}, "value_caches": {},
    }
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_size)
    for r in ranks:
        g = torch.Generator(device=device)
        g.manual_seed(w.seed * 1000 + 1 + r)
        vals["key_caches"][r] = draw(g, shape)
        vals["value_caches"][r] = draw(g, shape)
    return vals
