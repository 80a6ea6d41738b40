"""Benchmark of the paged-KV decode step on one MI355X.

A step is one pass of the whole hot path over one batch: copy-on-write block
copies, slot mapping, cache scatter of the new tokens, and paged decode
attention (single pass, or split-K when the workload uses partitions).  By
default the step runs as one launch (pa_decode_step); --unfused times the four
separate calls.  The host allocator runs once at set-up; the step's inputs are
resident in HBM when the timed region starts.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--unfused] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "paged decode attention: KV tokens/s + achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
# dense matrix-core peaks of MI355X (TFLOP/s) by storage dtype; fp32 is the
# vector peak (the fp32 path runs on the vector ALUs)
MATRIX_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
DEFAULT_WORKLOAD = "llama7b_fp16"
CSRC = os.path.join(REPO, "paged_kv_cache_123_amd", "csrc")
# the attention kernels' sources and the build script that sets their flags
ATTN_SRCS = [os.path.join(CSRC, f) for f in ("attention_kernels.hip", "attention_mfma.hip",
                                             "attention_prefill.hip", "decode_common.h")] + [
    os.path.join(REPO, "paged_kv_cache_123_amd", "build.py")]


def attention_source_hash() -> str:
    """First 16 hex digits of the SHA-256 of the attention kernel sources."""
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def window_of(w) -> int:
    return int(w.extra.get("sliding_window", 0))


def attended(w, context_lens, query_lens=None):
    """Per sequence, the cached positions [lo, L) its queries read: all of
    them, or with a sliding window W those from the first query's window on."""
    W = window_of(w)
    out = []
    for s, L in enumerate(context_lens):
        n = 1 if query_lens is None else int(query_lens[s])
        lo = max(0, int(L) - n + 1 - W) if W else 0
        out.append((lo, int(L)))
    return out


def attended_rows(spans, tables, B) -> int:
    """Distinct cache rows (slots) the queries attend: a block that several
    sequences share counts once."""
    slots = [tables[s, np.arange(lo, L) // B].astype(np.int64) * B + np.arange(lo, L) % B
             for s, (lo, L) in enumerate(spans) if L > lo]
    return int(np.unique(np.concatenate(slots)).size) if slots else 0


def attention_bytes(w, context_lens, query_rows=None, query_lens=None, tables=None) -> int:
    """Algorithmic bytes of one attention launch: every K and V row a query
    reads, once per KV head (with ``tables``, each distinct cache row once,
    however many sequences share its block; else once per sequence), q in,
    out back (one row per sequence, or ``query_rows`` when every new token is
    a query), the table entries of the blocks read and the context lengths.
    The plan does not change it: a cascade plan only reads closer to it, and
    split-K workspace traffic is overhead."""
    e = w.elem_bytes
    B = w.extra.get("kernel_block_size", w.block_size)
    spans = attended(w, context_lens, query_lens)
    rows_read = (attended_rows(spans, tables, B) if tables is not None
                 else sum(L - lo for lo, L in spans))
    kv = rows_read * 2 * w.num_kv_heads * w.head_size * e
    rows = w.num_seqs if query_rows is None else query_rows
    qo = 2 * rows * w.num_heads * w.head_size * e
    tables = 4 * sum((L - 1) // B - lo // B + 1 for lo, L in spans if L > lo)
    return kv + qo + tables + 4 * w.num_seqs


def attention_flops(w, context_lens, query_lens=None) -> int:
    """Algorithmic flops of one attention launch: for every (query token,
    visible key) pair and query head, 2*D for q.k and 2*D for the weighted
    sum of v (exps and the softmax sums are not counted)."""
    W = window_of(w)
    pairs = 0
    for s, L in enumerate(context_lens):
        n = 1 if query_lens is None else int(query_lens[s])
        for i in range(n):
            hi = int(L) - n + i + 1
            lo = max(0, hi - W) if W else 0
            pairs += hi - lo
    return pairs * w.num_heads * 4 * w.head_size


def step_bytes(w, step) -> int:
    """Algorithmic bytes of the whole step: attention plus the slot mapping
    (positions, one table entry, slot: 20 B per token), the scatter (read and
    write of each new K/V row) and the block copies (read + write of K and V)."""
    e = w.elem_bytes
    T = step.num_tokens
    row = w.num_kv_heads * w.head_size * e
    blk = w.num_kv_heads * step.block_size * w.head_size * e  # kernel blocks
    attn = attention_bytes(w, step.context_lens_host, _query_rows(step), _query_lens(step),
                           step.tables_host)
    return (attn + 20 * T
            + 4 * row * T + 4 * blk * len(step.cow_pairs_host))


def _query_rows(step):
    return step.num_tokens if step.all_queries else None


def _query_lens(step):
    return np.diff(step.query_start_loc_host) if step.all_queries else None


def _cow_old_slots(w, step) -> int:
    """Slots before each fork's first new token in its fresh copy-on-write
    tail block: the rows the one-launch step copies."""
    old = 0
    qsl = step.query_start_loc_host
    for r, src in enumerate(step.cow_src_host):
        if src >= 0:
            first_new = int(step.context_lens_host[r]) - int(qsl[r + 1] - qsl[r])
            old += first_new % w.block_size
    return old


def write_bytes(w, step) -> int:
    """The step's cache writes at their minimum: each new token's K/V rows
    written (its read is the attention's read of that token) and its slot (8
    B), and the copied old slots of each copy-on-write tail written (their
    read is the attention's read of those tokens)."""
    row = w.num_kv_heads * w.head_size * w.elem_bytes
    return (2 * row + 8) * step.num_tokens + 2 * row * _cow_old_slots(w, step)


def fused_bytes(w, step) -> int:
    """Algorithmic bytes of the one-launch step: attention (which reads every
    attended row once, the new ones included) plus the step's writes."""
    return (attention_bytes(w, step.context_lens_host, _query_rows(step), _query_lens(step),
                            step.tables_host)
            + write_bytes(w, step))


def time_prefix_cache(w, min_seconds: float = 0.3) -> dict:
    """Host cost of serving the workload's requests through the prefix cache
    (lookup, appends and caching of full blocks on a fresh C++ pool),
    repeated for at least ``min_seconds``."""
    from paged_kv_cache_123_amd.host import Pool

    reqs = [op for op in w.prefill if op[0] == "request"]
    prompt_tokens = sum(len(op[2]) for op in reqs)
    runs, elapsed, hit_tokens = 0, 0.0, 0
    while elapsed < min_seconds:
        pool = Pool(w.num_blocks, w.block_size, w.free_order)
        pool.enable_prefix_caching()
        hit_tokens = 0
        t0 = time.perf_counter()
        for op in w.prefill:
            if op[0] == "request":
                _, s, prompt, extra = op
                done = pool.add_seq_cached(s, prompt, extra)
                pool.append_tokens(s, prompt[done:])
                pool.cache_full_blocks(s)
                hit_tokens += done
            elif op[0] == "free":
                pool.free_seq(op[1])
        elapsed += time.perf_counter() - t0
        runs += 1
    return {"requests": len(reqs), "prompt_tokens": prompt_tokens, "hit_tokens": hit_tokens,
            "hit_fraction": hit_tokens / max(prompt_tokens, 1),
            "us_per_request": elapsed / (runs * max(len(reqs), 1)) * 1e6,
            "note": "C++ allocator through ctypes, one host thread"}


def default_launch(args) -> bool:
    """Whether the run launches the workload's default kernels and plan (the
    configuration the committed counter summaries were taken on)."""
    return (args.cascade is None and args.cascade_chunk is None and args.partition_size is None
            and args.kernel == "auto" and not args.no_prefill_kernel)


def pmc_traffic(workload: str, per_launch_bytes: int):
    """HBM traffic of the attention kernel from a committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(REPO, "profiles", f"paged_attention_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != attention_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def read_reference(nbytes: int = 2 << 30, reps: int = 10):
    """Achievable read bandwidth on this GPU for the access pattern of a paged
    cache: whole 4 KiB blocks in a random order (and, for context, in
    sequential order), with plain and non-temporal loads, timed with HIP events
    around the library's read probe."""
    import torch

    from paged_kv_cache_123_amd import ops
    nblk = nbytes // 4096
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(0)
    rnd = torch.randperm(nblk, generator=g).to(torch.int32).cuda()
    seq = torch.arange(nblk, dtype=torch.int32, device="cuda")
    orders = {"random_4k": (rnd, False), "random_4k_nt": (rnd, True),
              "sequential_4k": (seq, False), "sequential_4k_nt": (seq, True)}
    out = {}
    for name, (order, nt) in orders.items():
        ops.probe_read_blocks(buf, order, sink, non_temporal=nt)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            ops.probe_read_blocks(buf, order, sink, non_temporal=nt)
        b.record()
        torch.cuda.synchronize()
        out[name] = nblk * 4096 / (a.elapsed_time(b) / reps * 1e-3) / 1e9
    del buf
    return out


def cascade_timeline(step, fused: bool) -> dict:
    """One more step of a cascade plan with the kernel's per-workgroup
    timeline: when the workgroups start, how long each spends before its
    first tiles are described (set-up) and streaming them, and when they end,
    in microseconds from the first start; stream times by the wave slot the
    workgroup's first wave took on its SIMD (0: the first workgroup placed on
    it) and by XCD."""
    import torch

    from paged_kv_cache_123_amd import ops
    ops.timeline_reset()
    if fused:
        step.fused()
    else:
        step.attention()
    torch.cuda.synchronize()
    rec = ops.timeline_read().astype(np.int64)
    if len(rec) == 0:
        return {"workgroups": 0, "note": "no cascade launch in this step"}
    us = 0.01  # 100 MHz counter ticks
    t0 = rec[:, 0].min()
    start, setup = (rec[:, 0] - t0) * us, (rec[:, 1] - rec[:, 0]) * us
    stream, end = (rec[:, 2] - rec[:, 1]) * us, (rec[:, 2] - t0) * us
    hw = rec[:, 3] & 0xFFFFFFFF
    slot, xcc = hw & 0xF, (rec[:, 3] >> 32) & 0xF

    def dist(x):
        return {q: round(float(np.percentile(x, p)), 2)
                for q, p in (("min", 0), ("p10", 10), ("median", 50), ("p90", 90), ("max", 100))}
    return {
        "workgroups": int(len(rec)), "start_us": dist(start), "setup_us": dist(setup),
        "stream_us": dist(stream), "end_us": dist(end),
        "stream_us_by_wave_slot": {int(k): round(float(stream[slot == k].mean()), 2)
                                   for k in np.unique(slot)},
        "stream_us_by_xcd": {int(k): round(float(stream[xcc == k].mean()), 2)
                             for k in np.unique(xcc)},
    }


def calibrate_counters() -> dict:
    """Kernels of known byte count for scaling FETCH_SIZE / WRITE_SIZE: the read
    probe over 1 GiB (reads only) and copy_blocks of 2048 blocks of 128 KiB in
    each cache (256 MiB read + 256 MiB written)."""
    import torch

    from paged_kv_cache_123_amd import ops
    nbytes = 1 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    order = torch.arange(nbytes // 4096, dtype=torch.int32, device="cuda")
    ops.probe_read_blocks(buf, order, sink)
    kc = torch.empty((4096, 32, 16, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    pairs = torch.stack([torch.arange(0, 2048), torch.arange(2048, 4096)], 1).cuda()
    ops.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    blk = 32 * 16 * 128 * 2
    return {"probe_read_bytes": nbytes, "copy_blocks_read_bytes": 2 * 2048 * blk,
            "copy_blocks_write_bytes": 2 * 2048 * blk}


def cpu_baseline(w, vals, step, budget_s: float):
    """Oracle attention (float64 NumPy, one BLAS thread) over the first
    sequences of the batch, until about ``budget_s`` of CPU work."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.attention import paged_attention, paged_attention_multi

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    tables = step.tables_host
    lens = step.context_lens_host
    qsl = step.query_start_loc_host
    q = host(step.query)
    # host copies of each sequence's blocks (table entries renumbered)
    per_seq = []
    for s in range(w.num_seqs):
        used = np.unique(tables[s][tables[s] >= 0])
        idx = torch.from_numpy(used.astype(np.int64)).to(step.key_cache.device)
        remap = np.full(w.num_blocks, -1, dtype=np.int64)
        remap[used] = np.arange(used.size)
        row = np.where(tables[s:s + 1] >= 0, remap[np.maximum(tables[s:s + 1], 0)], -1)
        per_seq.append((host(step.key_cache.index_select(0, idx)),
                        host(step.value_cache.index_select(0, idx)), row))
        if sum(int(x) for x in lens[:s + 1]) * w.num_heads * w.head_size > 4e9:
            break  # keep the host copies bounded
    done_tokens, done_seqs, passes, t_used = 0, 0, 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s:
            for s, (kc, vc, row) in enumerate(per_seq):
                t0 = time.perf_counter()
                if step.all_queries:
                    a, b = int(qsl[s]), int(qsl[s + 1])
                    paged_attention_multi(q[a:b], kc, vc, row, lens[s:s + 1], [0, b - a],
                                          w.scale, w.dtype, window=window_of(w))
                else:
                    paged_attention(q[s:s + 1], kc, vc, row, lens[s:s + 1], w.scale, w.dtype,
                                    window=window_of(w))
                t_used += time.perf_counter() - t0
                lo, hi = attended(w, lens[s:s + 1],
                                  None if not step.all_queries else [int(qsl[s + 1] - qsl[s])])[0]
                done_tokens += hi - lo
                done_seqs += 1
                if t_used >= budget_s:
                    break
            passes += 1
    return {"value": done_tokens / t_used, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_seqs} sequence passes over the first {len(per_seq)} of "
                      f"{w.num_seqs} sequences ({done_tokens} KV tokens, all {w.num_heads} "
                      f"heads), float64 NumPy, 1 BLAS thread, {t_used:.1f} s"}


def _cpu_worker(job):
    """One CPU worker of the multi-core oracle baseline: builds host inputs for
    its sequences from the workload recipe (values drawn on the CPU with the
    workload's distribution; each sequence's blocks numbered 0..n-1) and runs
    the oracle over them, one sequence at a time, until its budget is spent."""
    name, rows, budget, seed = job
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle.attention import paged_attention

    w = W.make(name)
    rng = np.random.default_rng([seed, rows[0]])
    B, hkv, D, H = w.block_size, w.num_kv_heads, w.head_size, w.num_heads
    raw = {"f32": np.float32, "f16": np.float16}.get(w.dtype)

    def draw(shape):
        x = (rng.standard_normal(shape, dtype=np.float32) * w.sigma)
        if raw is not None:
            return x.astype(raw)
        return (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 bits (truncated)

    seqs = []
    for r in rows:
        L = int(w.context_lens[r])
        lo, hi = attended(w, [L])[0]
        nb = -(-L // B)
        seqs.append((draw((1, H, D)), draw((nb, hkv, B, D)), draw((nb, hkv, B, D)),
                     np.arange(nb)[None, :], L, hi - lo))
    done, used = 0, 0.0
    with threadpool_limits(limits=1):
        while used < budget:
            for q, kc, vc, table, L, n in seqs:
                t0 = time.perf_counter()
                paged_attention(q, kc, vc, table, [L], w.scale, w.dtype, window=window_of(w))
                used += time.perf_counter() - t0
                done += n
                if used >= budget:
                    break
    return done, used


def cpu_baseline_pool(w, pool, workers: int, budget_s: float):
    """The oracle on ``workers`` processes in parallel over the sequences
    (each with one BLAS thread): aggregate KV tokens per second."""
    rows = [r for r in range(w.num_seqs)]
    jobs = [(w.name, rows[i::workers], budget_s, 1234) for i in range(workers)
            if rows[i::workers]]
    t0 = time.perf_counter()
    res = pool.map(_cpu_worker, jobs)
    wall = time.perf_counter() - t0
    done = sum(r[0] for r in res)
    return {"value": done / max(r[1] for r in res), "unit": "KV tokens/s", "cores": len(jobs),
            "kind": "oracle",
            "sample": f"{len(jobs)} processes over the {w.num_seqs} sequences, each {budget_s:.0f} s "
                      f"of float64 NumPy with one BLAS thread ({done} KV tokens in {wall:.1f} s "
                      "wall); inputs drawn on the host with the workload's shapes and "
                      "distribution"}


def partials_bytes(w, local_lens) -> int:
    """Algorithmic bytes of one rank's partials call: its K/V rows, q, table
    entries and lengths (attention_bytes without the output row), plus the
    fp32 (m, l, o) it writes for every (sequence, query head)."""
    e = w.elem_bytes
    out_row = w.num_seqs * w.num_heads * w.head_size * e
    return (attention_bytes(w, local_lens) - out_row
            + w.num_seqs * w.num_heads * (w.head_size + 2) * 4)


def merge_bytes(w) -> int:
    """Algorithmic bytes of the merge over the group: every rank's (m, l, o)
    read, the output written."""
    world = int(w.extra["cp_world"])
    rows = w.num_seqs * w.num_heads
    return world * rows * (w.head_size + 2) * 4 + rows * w.head_size * w.elem_bytes


def cpu_baseline_cp(w, step, budget_s: float):
    """Oracle rank partials (float64 NumPy, one BLAS thread) over the first
    sequences of the rank's share, until about ``budget_s`` of CPU work."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.attention import paged_attention_partials

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    tables = step.tables_host
    lens = step.local_lens_host
    q = host(step.query)
    per_seq = []
    for s in range(w.num_seqs):
        used = np.unique(tables[s][tables[s] >= 0])
        idx = torch.from_numpy(used.astype(np.int64)).to(step.key_cache.device)
        remap = np.full(w.num_blocks, -1, dtype=np.int64)
        remap[used] = np.arange(used.size)
        row = np.where(tables[s:s + 1] >= 0, remap[np.maximum(tables[s:s + 1], 0)], -1)
        per_seq.append((host(step.key_cache.index_select(0, idx)),
                        host(step.value_cache.index_select(0, idx)), row))
        if len(per_seq) >= 4:
            break  # a few sequences are plenty for a bounded sample
    done_tokens, done_seqs, t_used = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s:
            for s, (kc, vc, row) in enumerate(per_seq):
                t0 = time.perf_counter()
                paged_attention_partials(q[s:s + 1], kc, vc, row, lens[s:s + 1], w.scale,
                                         w.dtype)
                t_used += time.perf_counter() - t0
                done_tokens += int(lens[s])
                done_seqs += 1
                if t_used >= budget_s:
                    break
    return {"value": done_tokens / t_used, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_seqs} rank-partial passes over the first {len(per_seq)} of "
                      f"{w.num_seqs} sequences of the rank's share ({done_tokens} KV tokens, "
                      f"all {w.num_heads} heads), float64 NumPy, 1 BLAS thread, "
                      f"{t_used:.1f} s"}


def main_cp(args, w):
    """One GPU's share of a context-parallel decode step: this rank's slot
    mapping, scatter and partials, then the merge over the group's gathered
    partials (the other ranks' slices are filled once, before timing, by the
    same GPU playing those ranks; the all-gather itself is not timed)."""
    import torch

    import workloads as W
    from paged_kv_cache_123_amd import ops
    from paged_kv_cache_123_amd.cp_step import CPRankStep, alloc_gathered

    world, I = int(w.extra["cp_world"]), int(w.extra["cp_interleave"])
    part = w.partition_size if args.partition_size is None else args.partition_size
    vals = W.make_cp_values(w, "cuda")
    g = alloc_gathered(world, w.num_seqs, w.num_heads, w.head_size, "cuda")
    steps = []
    for r in range(world):
        v = {"key_cache": vals["key_caches"][r], "value_cache": vals["value_caches"][r],
             "query": vals["query"], "new_key": vals["new_key"], "new_value": vals["new_value"]}
        steps.append(CPRankStep(w.num_blocks, w.block_size, world, r, I, w.free_order,
                                w.prefill, w.step, v, w.scale, part, gathered=g))
    # the timed rank: the largest share, then the most new tokens written
    lens = steps[0].context_lens_host
    before = lens - np.bincount([s for s, _ in w.step], weights=[n for _, n in w.step],
                                minlength=len(lens)).astype(np.int32)
    def load(r):
        got = ops.cp_local_context_lens(before, w.block_size, world, r, I)
        return (int(steps[r].local_lens_host.sum()),
                int((steps[r].local_lens_host - got).sum()))
    rank = max(range(world), key=load)
    for r in range(world):
        if r != rank:
            steps[r].run(merge=False)
    st = steps[rank]
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    a_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    a_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        st.slot_mapping_kernel()
        st.scatter()
        a_start[i].record(stream)
        st.partials()
        a_end[i].record(stream)
        st.merge()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in zip(a_start, a_end)]
    attn_avg_ms = float(np.mean(attn_ms))
    attn_stats = {"mean": attn_avg_ms, "p10": float(np.percentile(attn_ms, 10)),
                  "p90": float(np.percentile(attn_ms, 90))}
    local_tokens = int(st.local_lens_host.sum())
    pbytes = partials_bytes(w, st.local_lens_host)
    achieved = pbytes / (attn_avg_ms * 1e-3) / 1e9
    step_b = pbytes + merge_bytes(w) + 20 * st.num_tokens + 4 * w.num_kv_heads * w.head_size \
        * w.elem_bytes * int(load(rank)[1])
    result = {
        "metric": METRIC,
        "value": local_tokens / (ms_per_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "context_parallel_world": world,
            "interleave": I,
            "rank": rank,
            "num_seqs": w.num_seqs,
            "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_size": w.head_size,
            "block_size": w.block_size,
            "kv_tokens": local_tokens,
            "kv_tokens_whole_group": int(lens.sum()),
            "max_context_len": int(st.max_local_len),
            "num_blocks": w.num_blocks,
            "partition_size": part,
            "attention_kernel": args.kernel,
        },
        "step_hbm_gbps": step_b / (ms_per_step * 1e-3) / 1e9,
        "attention_ms": attn_stats,
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_decode_mfma_kernel" if (args.kernel == "mfma" or (
                args.kernel == "auto" and w.num_heads > w.num_kv_heads)) else "paged_decode_kernel")
                      + " + merge_kernel (rank partials)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": pmc_traffic(w.name, pbytes) if default_launch(args) else None,
            "algorithmic_bytes_per_launch": pbytes,
        },
        "wall_s_timed_region": wall,
    }
    if not args.no_read_reference:
        ref = read_reference()
        result["read_reference_gbps"] = ref
        result["roofline"]["frac_of_random_4k_read"] = achieved / max(ref["random_4k"],
                                                                      ref["random_4k_nt"])
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_cp(w, st, args.cpu_budget)
    print(json.dumps(result), flush=True)


# The default run also times these workloads after the metric's own, each
# with its own timed region and roofline (extra keys of the one JSON line):
# the other decode configuration the roofline target names, the long-context
# split-K batch and the shared-prefix batch (on the plan the step chooses).
EXTRA_WORKLOADS = ("qwen72b_gqa_bf16", "long_context_bf16", "shared_prefix_bf16")
# Residency control: a step whose working set is below this many bytes is
# timed on several device copies of its pool and tables in turn, so that no
# repetition finds the previous one's rows in the 256 MB Infinity Cache.
RESIDENCY_BYTES = 1 << 30
DISTRIBUTION_LAUNCHES = 50


def replicas(step, n: int):
    """``n`` steps over independent device copies of the same pool, tables
    and inputs (the first is ``step`` itself)."""
    import copy

    import torch
    out = [step]
    for _ in range(n - 1):
        c = copy.copy(step)
        memo = {}
        for name, t in vars(step).items():
            if isinstance(t, torch.Tensor):
                # tensors that alias each other in the step alias in the copy
                key = (t.data_ptr(), tuple(t.shape), t.dtype)
                if key not in memo:
                    memo[key] = t.clone()
                setattr(c, name, memo[key])
        c._fused_call = None
        out.append(c)
    return out


MAX_REPLICAS = 16


def num_replicas(working_set: int) -> int:
    """Copies of the step's data cycled through so that together they exceed
    the Infinity Cache (1 GiB of working set, at most 16 copies: a smaller
    batch stays cache-resident whatever the rotation)."""
    if working_set >= 2 * RESIDENCY_BYTES:
        return 1
    return min(MAX_REPLICAS, max(2, -(-RESIDENCY_BYTES // max(working_set, 1))))


def time_step(steps, fused: bool, K: int, warmup: int):
    """Warm-up, then K timed steps (HIP events around the whole region, no
    events between steps), then a distribution pass of at least
    DISTRIBUTION_LAUNCHES launches with HIP events around each (the one-launch
    step, or the attention call of the separate calls, launched back to
    back).  Steps cycle over the replicas.  Returns (ms per step, wall seconds of the timed
    region, per-launch milliseconds of the distribution pass)."""
    import torch

    R = len(steps)
    if fused:  # every copy's arguments marshalled before any launch (host only)
        for st in steps:
            st.prepare_fused()

    def one(i, ev=None):
        st = steps[i % R]
        if fused:
            if ev is not None:
                ev[0].record()
            st.fused()
            if ev is not None:
                ev[1].record()
        elif ev is None:
            st.copy_blocks()
            st.slot_mapping_kernel()
            st.scatter()
            st.attention()
        else:
            # the attention launch alone, back to back (the cache writes of
            # every copy are in place from the timed steps): the events then
            # bracket the kernel, not the host's launch of it after a drained
            # queue
            ev[0].record()
            st.attention()
            ev[1].record()

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(K):
        one(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / K
    n = max(K, DISTRIBUTION_LAUNCHES)
    # the pass runs twice and the second is kept: the runtime's first timed
    # events have been seen to stall the host for tens of milliseconds once,
    # and an event pair around a launch then measures the drained queue too
    for _ in range(2):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i in range(n):
            one(i, evs[i])
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    return ms_per_step, wall, launch_ms


def kernel_label(w, step, args, part, fused) -> str:
    cascade = step.cascade
    return (("prefill_kernel (query blocks)" if step.prefill_rows else
             "cascade_decode_kernel" if cascade and not part else
             "paged_decode_mfma_kernel" if (cascade or args.kernel == "mfma" or (
                 args.kernel == "auto" and w.dtype != "f32" and w.head_size == 128
                 and (w.num_heads > w.num_kv_heads or step.attn_max_query_len > 1)))
             else "paged_decode_kernel")
            + (" + merge_kernel" if part or step.cascade_chunk else "")
            + (" (cascade plan)" if cascade else "")
            + (" (one-launch step: copy-on-write + scatter + attention)" if fused else ""))


def measure(args, w, cascade_arg=None):
    """One workload's step on resident inputs: returns (result dict, step,
    values) where the result holds value, ms_per_step, roofline and the
    per-launch statistics."""
    import torch

    import workloads as W
    from paged_kv_cache_123_amd.step import DecodeStep

    part = w.partition_size if args.partition_size is None else args.partition_size
    vals = W.make_values(w, "cuda")
    step = DecodeStep(w.num_blocks, w.block_size, w.free_order, w.prefill, w.step, vals,
                      w.scale, part, all_queries=w.extra.get("queries") == "all",
                      sliding_window=window_of(w),
                      kernel_block_size=w.extra.get("kernel_block_size", 0),
                      cascade=cascade_arg, prefill_kernel=not args.no_prefill_kernel,
                      **({} if args.cascade_chunk is None
                         else {"cascade_chunk": args.cascade_chunk}))
    torch.cuda.synchronize()
    # steps whose cache writes must precede the attention (query blocks of a
    # prefill chunk on the decode kernels; copy-on-write of blocks of several
    # kernel blocks) run as separate calls
    fused = not args.unfused and step.fused_ok
    attn_bytes = (fused_bytes(w, step) if fused
                  else attention_bytes(w, step.context_lens_host, _query_rows(step),
                                       _query_lens(step), step.tables_host))
    R = 1 if args.no_residency_control else num_replicas(step_bytes(w, step))
    steps = replicas(step, R)
    torch.cuda.synchronize()
    ms_per_step, wall, launch_ms = time_step(steps, fused, args.steps, args.warmup)
    # A one-launch step without partitions is a single kernel: its mean
    # launch duration is the timed region over K, which has no events between
    # launches.  Otherwise the mean of the per-launch events.
    single_kernel = fused and part == 0 and not step.cascade_chunk
    attn_avg_ms = ms_per_step if single_kernel else float(np.mean(launch_ms))
    attn_stats = {
        "mean": attn_avg_ms,
        "median": float(np.median(launch_ms)),
        "p10": float(np.percentile(launch_ms, 10)),
        "p90": float(np.percentile(launch_ms, 90)),
        "launches": len(launch_ms),
        "mean_of_launch_events": float(np.mean(launch_ms)),
        "note": ("mean: the timed region over the steps (one kernel launch per step); median, "
                 "p10, p90: HIP events around each launch of a separate pass"
                 if single_kernel else
                 "HIP events around each attention launch of a separate pass"),
    }
    kv_tokens = sum(L - lo for lo, L in attended(w, step.context_lens_host, _query_lens(step)))
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    flops = attention_flops(w, step.context_lens_host, _query_lens(step))
    mpeak = MATRIX_PEAK_TFLOPS[w.dtype]
    # the bound: HBM, or the matrix cores when the flops per algorithmic byte
    # exceed the ridge (several queries per token row: prefill chunks)
    compute_bound = flops / attn_bytes > mpeak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    cascade = step.cascade
    result = {
        "value": kv_tokens / (ms_per_step * 1e-3),
        "unit": "KV tokens/s",
        "ms_per_step": ms_per_step,
        "dtype": w.dtype,
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_size": w.head_size,
            "block_size": w.block_size,
            "kv_tokens": kv_tokens,
            "max_context_len": int(step.max_context_len),
            "num_blocks": w.num_blocks,
            "partition_size": part,
            "cascade_group": cascade,
            "cascade_chunk": step.cascade_chunk,
            "cascade_group_items": int((step.plan_host[:2 * step.num_items:2] < 0).sum())
            if cascade else 0,
            "attention_kernel": args.kernel,
            "fused_step": fused,
            "cow_copies": int(len(step.cow_pairs_host)),
            "step_tokens": int(step.num_tokens),
            "queries_per_sequence": step.max_query_len or 1,
            "sliding_window": window_of(w),
            "context_tokens": int(step.context_lens_host.sum()),
            "pool_copies_in_rotation": R,
        },
        "step_hbm_gbps": step_bytes(w, step) / (ms_per_step * 1e-3) / 1e9,
        "attention_ms": attn_stats,
        "roofline": {
            "bound": "mfma" if compute_bound else "hbm",
            "kernel": kernel_label(w, step, args, part, fused),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            # the committed counts cover the workload's default launch only
            "traffic": (pmc_traffic(w.name + ("_unfused" if args.unfused else ""), attn_bytes)
                        if default_launch(args) else None),
            "algorithmic_bytes_per_launch": attn_bytes,
            "algorithmic_flops_per_launch": flops,
        },
        "wall_s_timed_region": wall,
    }
    if compute_bound:
        tflops = flops / (attn_avg_ms * 1e-3) / 1e12
        result["roofline"].update({
            "achieved": tflops, "peak": mpeak, "unit": "TFLOP/s", "frac": tflops / mpeak,
            "hbm_gbps": achieved, "hbm_frac": achieved / HBM_PEAK_GBPS})
    del steps
    return result, step, vals


def cache_kernels(step, w, reps: int = 50) -> dict:
    """The integer and copy kernels of a step on their own (slot mapping,
    scatter, copy_blocks), each timed with HIP events over ``reps`` launches:
    GB/s over their algorithmic bytes (slot mapping 20 B per token: position,
    table entry and slot; scatter a read and a write of each new K/V row;
    copy_blocks a read and a write of every K and V block of each pair)."""
    import torch
    T = step.num_tokens
    row = w.num_kv_heads * w.head_size * w.elem_bytes
    blk = w.num_kv_heads * step.block_size * w.head_size * w.elem_bytes
    jobs = {"compute_slot_mapping": (step.slot_mapping_kernel, 20 * T, f"{T} tokens"),
            "reshape_and_cache": (step.scatter, 4 * row * T, f"{T} tokens x {row * 2} B"),
            "copy_blocks": (step.copy_blocks, 4 * blk * len(step.cow_pairs_host),
                            f"{len(step.cow_pairs_host)} pairs of {blk} B blocks")}
    out = {}
    for name, (fn, nbytes, what) in jobs.items():
        if nbytes == 0:
            continue
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        out[name] = {"us": us, "algorithmic_bytes": nbytes, "gbps": nbytes / (us * 1e-6) / 1e9,
                     "frac_of_8tbps": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "what": what}
    return out


def compact(res: dict) -> dict:
    """The keys of an extra workload's entry in the JSON line."""
    keep = ("value", "unit", "ms_per_step", "dtype", "config", "step_hbm_gbps", "attention_ms",
            "roofline", "cache_kernels")
    return {k: res[k] for k in keep if k in res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's split-K partition (0 = single pass)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"],
                    help="attention kernel (auto: matrix cores for grouped-query heads)")
    ap.add_argument("--cascade", type=int, default=None,
                    help="cascade plan with groups of at most N sharers (0: off; default: "
                         "the workload's, else the step's own choice)")
    ap.add_argument("--cascade-chunk", type=int, default=None,
                    help="chunked cascade plan: pieces of N prefix tokens per workgroup (0: "
                         "one workgroup per group; default: the step's own choice)")
    ap.add_argument("--no-prefill-kernel", action="store_true",
                    help="attend prefill chunks as 16-token query blocks on the decode kernels")
    ap.add_argument("--unfused", action="store_true",
                    help="time copy_blocks, slot mapping, scatter and attention as four launches "
                         "instead of the one-launch step")
    ap.add_argument("--no-residency-control", action="store_true",
                    help="time one copy of the pool even when its working set fits the caches")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --workload (the default run also times the extra "
                         "workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="processes of the multi-core oracle baseline (default: the usable "
                         "cores, at most 16; 0 = single core only)")
    ap.add_argument("--no-read-reference", action="store_true")
    ap.add_argument("--calibrate-counters", action="store_true",
                    help="only run kernels of known byte count (for rocprofv3 --pmc scaling)")
    ap.add_argument("--timeline", action="store_true",
                    help="after the timing, one more step with the cascade kernel's "
                         "per-workgroup timeline (needs a library built with PA_TIMELINE=1, "
                         "named by PAGEDKV_LIBRARY)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-KV path here runs on a single GPU "
              "(sharding across GPUs is a design note, not code); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    # The multi-core oracle baseline's processes are forked here, before
    # anything touches the GPU; they wait until the GPU timing is done.
    pool, workers = None, 0
    if not args.no_cpu_baseline and not args.calibrate_counters:
        import multiprocessing
        usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1
        workers = min(16, usable) if args.cpu_workers is None else args.cpu_workers
        if workers > 1:
            pool = multiprocessing.get_context("fork").Pool(workers)

    import torch

    import workloads as W
    from paged_kv_cache_123_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_counters:
        print(json.dumps(calibrate_counters()), flush=True)
        return
    ops.set_decode_kernel(args.kernel)
    w = W.make(args.workload)
    if w.extra.get("cp_world"):
        print(f"[bench] workload {w.name}: {w.notes}", file=sys.stderr, flush=True)
        if pool is not None:  # the context-parallel baseline is single-core
            pool.close()
            pool.join()
        main_cp(args, w)
        return
    cascade_arg = w.extra.get("cascade") if args.cascade is None else args.cascade
    print(f"[bench] workload {w.name}: {w.notes}", file=sys.stderr, flush=True)
    res, step, vals = measure(args, w, cascade_arg)
    result = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": res["dtype"], "data": "synthetic"}
    result.update({k: v for k, v in res.items() if k not in result and k != "unit"})
    if args.timeline:
        result["timeline"] = cascade_timeline(step, not args.unfused and step.fused_ok)
    if any(op[0] == "request" for op in w.prefill):
        result["host_prefix_cache"] = time_prefix_cache(w)
    if step.num_tokens > w.num_seqs or len(step.cow_pairs_host):
        result["cache_kernels"] = cache_kernels(step, w)
    if not args.no_read_reference:
        ref = read_reference()
        result["read_reference_gbps"] = ref
        best = max(ref["random_4k"], ref["random_4k_nt"])
        result["roofline"]["frac_of_random_4k_read"] = result["roofline"]["achieved"] / best \
            if result["roofline"]["unit"] == "GB/s" else None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        single = cpu_baseline(w, vals, step, args.cpu_budget)
        if pool is not None and not step.all_queries:
            result["cpu_baseline"] = cpu_baseline_pool(w, pool, workers, args.cpu_budget)
            result["cpu_baseline"]["single_core"] = single
        else:
            result["cpu_baseline"] = single
    if pool is not None:
        pool.close()
        pool.join()
    del step, vals
    torch.cuda.empty_cache()
    if args.workload == DEFAULT_WORKLOAD and not args.no_extras:
        extras = {}
        for name in EXTRA_WORKLOADS:
            we = W.make(name)
            print(f"[bench] extra workload {we.name}: {we.notes}", file=sys.stderr, flush=True)
            r, st, v = measure(args, we, we.extra.get("cascade"))
            if st.num_tokens > we.num_seqs or len(st.cow_pairs_host):
                r["cache_kernels"] = cache_kernels(st, we)
            extras[name] = compact(r)
            del st, v
            torch.cuda.empty_cache()
        result["extra_workloads"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
