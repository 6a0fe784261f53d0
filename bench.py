#!/usr/bin/env python3
"""Benchmark of the paged KV hot path on one MI355X.

Workload (the paged-decode batch): 64 sequences with lengths uniform in
[512, 4096] (the new token included), 16-position pages scattered over a
300,000-page pool, 32 query heads / 8 KV heads of 128, bf16 K/V with fp32
accumulation.  One step is one decode step of the whole batch:

  host   prepare_step: reserve one position per sequence, compute its slot,
         export block tables and lengths (C++ allocator, one call)
  H2D    slots, block tables and lengths from pinned buffers
  GPU    store_kv of the 64 new tokens, then paged decode (+ split merge)

Four disjoint copies of the batch live in the same pool and steps rotate over
them, so consecutive steps read different pages (2.4 GB cycled, well beyond
the 256 MB Infinity Cache).  Sequences keep growing by one token per use.

Printed: one JSON line.  ``value`` = KV bytes the decode steps must read
(sum of lengths x 2 x 8 heads x 128 x 2 bytes) / wall time of the timed steps
(host work and copies included).  ``roofline`` = the decode call's
algorithmic bytes per launch / its median duration over at least 30 calls
timed one by one with HIP events on the launch stream after the step loop
(the mean is reported beside it, and so is the sampled in-step timing),
against the 8 TB/s HBM peak.  ``cpu_baseline`` = the fp64 CPU oracle on a
bounded sample of the same sequences; the prefill, rewind and rollback legs
carry their own.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
METRIC = "paged-decode KV GB/s (% of HBM peak); prefill-append tokens/s (% MFMA peak)"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "pagedattention_pkv_store_amd", "csrc", "device.hip")


def measured_traffic(name: str):
    """HBM bytes per launch of one library call from the committed counter
    summary (FETCH_SIZE / WRITE_SIZE passes, calibrated against a plain copy),
    or None when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha or name not in rec:
        return None
    t = rec[name]
    return int(t["read_bytes"] + t["write_bytes"])


def kv_bytes_per_position(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one position across all KV heads (one layer)."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--call-reps", type=int, default=60,
                    help="decode calls timed one by one after the step loop (at least 30)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="bound on the CPU oracle's sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--cpu-seconds-other", type=float, default=8.0,
                    help="oracle seconds for each of the prefix, rewind and rollback CPU baselines (0: none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefill-reps", type=int, default=30,
                    help="timed repetitions of the prefix-shared prefill leg (0 disables it)")
    ap.add_argument("--int8", type=int, default=1,
                    help="also time the decode batch on INT8 pages (1) or not (0)")
    ap.add_argument("--copy-pairs", type=int, default=4096,
                    help="page pairs of the copy-on-write page-copy leg (0 disables it)")
    ap.add_argument("--codec", type=int, default=1, help="time the Q8 / Q4 KV codec leg (1) or not (0)")
    ap.add_argument("--read-probe", type=int, default=1,
                    help="measure the streaming HBM read ceiling with pkv_stream_read (1) or not (0)")
    ap.add_argument("--rewind", type=int, default=1, help="time the KV rewind append workload (1) or not (0)")
    ap.add_argument("--spec", type=int, default=1,
                    help="time the long-context speculative-rollback workload (1) or not (0)")
    ap.add_argument("--retention-docs", type=int, default=100_000,
                    help="documents of the host retention-pool leg (0 disables it)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="finally copy a buffer of this many MiB three times (a plain copy of known "
                         "size, the reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def prefill_leg(args, torch, pkv, synth, dev: str, kv_int8: bool = False) -> dict:
    """The prefix-shared prefill workload: 256 agent-trace rows (the first
    three 1,000 / 1,400 / 1,900 tokens of one trace, the rest U{1000..8000}
    tokens of 31 others), 16-position pages over a shuffled 100,000-page pool,
    32 / 8 heads of 128, bf16.  The C++ planner sorts the rows and the
    allocator adopts each row's shared full pages from its parent; one step
    stores every row's unshared suffix (store_kv) and runs one causal
    prefill/append over all suffixes.  Q/K/V values are N(0,1) drawn on the
    device from a seeded torch generator (the structure comes from the same
    seeded host generator the parity tests use)."""
    w = synth.prefix_traces(seed=args.seed, values=False)
    ps, hq, hkv, D = w.page_size, w.num_q_heads, w.num_kv_heads, w.head_dim
    n = len(w.row_len)
    t0 = time.perf_counter()
    order, parent, shared = pkv.plan_prefix([w.row_tokens(r) for r in range(n)], ps)
    plan_ms = (time.perf_counter() - t0) * 1e3
    desc = pkv.PoolDesc(pkv.PKV_I8 if kv_int8 else pkv.PKV_BF16, w.num_pages, ps, hkv, D)
    k_pool, v_pool = desc.new_pools(dev, fill=0xFF if kv_int8 else float("nan"))
    alloc = pkv.Allocator(w.num_pages, ps, w.free_order)
    seqs = [-1] * n
    lens = w.row_len.astype(np.int64)
    sh = shared.astype(np.int64)
    for d in order.tolist():
        seqs[d] = alloc.seq_new()
        if parent[d] >= 0:
            alloc.share_prefix(seqs[d], seqs[parent[d]], int(sh[d]))
        alloc.reserve(seqs[d], int(lens[d] - sh[d]))
    n_new = (lens - sh).astype(np.int64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + args.seed)
    n_tr, t_len = w.trace_tokens.shape
    flat = torch.from_numpy(np.concatenate(
        [w.row_trace[d] * t_len + np.arange(sh[d], lens[d]) for d in range(n)])).to(dev)

    def draw(heads):
        x = torch.empty((n_tr * t_len, heads, D), dtype=torch.bfloat16, device=dev)
        for t in range(n_tr):
            x[t * t_len:(t + 1) * t_len] = torch.randn((t_len, heads, D), generator=gen, device=dev).to(torch.bfloat16)
        return x[flat].contiguous()

    q, k_new, v_new = draw(hq), draw(hkv), draw(hkv)
    slots = torch.from_numpy(np.concatenate(
        [alloc.slots(seqs[d], int(sh[d]), int(n_new[d])) for d in range(n)])).to(dev)
    stride = max(alloc.num_blocks(x) for x in seqs)
    bt = torch.from_numpy(alloc.block_tables(seqs, stride)).to(dev)
    d_lens = torch.from_numpy(lens.astype(np.int32)).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(dev)
    max_q, max_len = int(n_new.max()), int(lens.max())
    ws = torch.empty(max(16, pkv.workspace_bytes(desc, n, hq, max_q, max_len)), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(D))

    def step(ev=None):
        if ev:
            ev[0].record()
        pkv.store_kv(desc, k_pool, v_pool, k_new, v_new, slots)
        if ev:
            ev[1].record()
        pkv.prefill_append(desc, k_pool, v_pool, q, cu, bt, d_lens, max_q, max_len, scale, out, ws)
        if ev:
            ev[2].record()

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.prefill_reps)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.prefill_reps
    gc.enable()
    store_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    attn_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    tokens = int(n_new.sum())
    pairs = int(sum((lens[d] * (lens[d] + 1) - sh[d] * (sh[d] + 1)) // 2 for d in range(n)))
    flops = 4.0 * D * hq * pairs
    attn_s = float(attn_ms.mean()) / 1e3
    achieved = flops / attn_s / 1e12
    return {
        "workload": "prefix-shared prefill: 256 agent-trace rows (1,000/1,400/1,900 tokens of one trace, "
                    "then U{1000..8000} of 31 traces), page_size 16, 100k-page shuffled pool, 32 q / 8 KV "
                    "heads, head_dim 128, bf16; step = store_kv of unshared suffixes + one prefill_append",
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "tokens_per_step": tokens,
        "tokens_unshared": int(lens.sum()),
        "ms_per_step": round(wall * 1e3, 3),
        "reps": args.prefill_reps,
        "planner_ms": round(plan_ms, 2),
        "store_kv_avg_us": round(float(store_ms.mean()) * 1e3, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("prefill_append_int8" if kv_int8 else "prefill_append"),
            "kernel": "pkv_prefill_append (prefill_schedule_kernel + paged_prefill_kernel)",
            "kernel_avg_us": round(attn_s * 1e6, 1),
            "kernel_median_us": round(float(np.median(attn_ms)) * 1e3, 1),
            "algorithmic_flops_per_launch": flops,
            "unmasked_pairs": pairs,
        },
    }


def read_probe_leg(args, torch, pkv, dev: str) -> dict:
    """Practical HBM read ceiling: pkv_stream_read (a grid-stride streaming
    read with non-temporal 16-byte loads, eight in flight per thread) over a
    4 GiB buffer, far beyond the 256 MB Infinity Cache, for a few grid sizes;
    the best is reported beside the 8 TB/s nominal peak."""
    nbytes = 4 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    best = None
    for grid in (2048, 4096, 8192, 16384, 32768, 65535):
        sums = torch.empty(grid, dtype=torch.int32, device=dev)
        call = pkv.bind_stream_read(buf, sums)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a, b in evs:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in evs])) / 1e3
        if best is None or t < best[1]:
            best = (grid, t)
    del buf
    torch.cuda.empty_cache()
    grid, t = best
    return {"kernel": "pkv_stream_read (stream_read_kernel)", "bytes": nbytes, "grid": grid,
            "traffic": measured_traffic("stream_read"),
            "kernel_median_us": round(t * 1e6, 1), "gbs": round(nbytes / t / 1e9, 1),
            "frac_of_nominal": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def _append_roofline(kv_bytes: int, qo_bytes: int, t_s: float, traffic_key, kernel: str, timed_ms) -> dict:
    alg = kv_bytes + qo_bytes
    achieved = alg / t_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(traffic_key) if traffic_key else None,
            "kernel": kernel, "kernel_avg_us": round(t_s * 1e6, 1),
            "kernel_median_us": round(float(np.median(timed_ms)) * 1e3, 1), "algorithmic_bytes_per_launch": alg}


def rewind_leg(args, torch, pkv, dev: str) -> dict:
    """KV rewind: 1,000 documents of 300 cached positions (16-position pages
    over a shuffled 32,768-page pool, 32 / 8 heads of 128, bf16).  One pass
    reserves 50 positions per document, stores the question's K/V (store_kv,
    50,000 tokens) and runs a causal 50-query append per document against its
    300 cached positions (prefill_append); the documents are then truncated
    back to 300 on the host (untimed), which hands the same pages back.
    Values are N(0,1) drawn on the device; lengths and placement come from
    the allocator."""
    n_docs, doc_len, q_len, ps, hq, hkv, D, num_pages = 1000, 300, 50, 16, 32, 8, 128, 32_768
    desc = pkv.PoolDesc(pkv.PKV_BF16, num_pages, ps, hkv, D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4000 + args.seed)
    k_pool = torch.randn(desc.pool_shape, generator=gen, device=dev).to(torch.bfloat16)
    v_pool = torch.randn(desc.pool_shape, generator=gen, device=dev).to(torch.bfloat16)
    order = np.random.default_rng(4100 + args.seed).permutation(num_pages).astype(np.int32)
    alloc = pkv.Allocator(num_pages, ps, order)
    seqs = np.array([alloc.seq_new() for _ in range(n_docs)], np.int32)
    alloc.prepare_step(seqs, np.full(n_docs, doc_len, np.int32), 0)      # the cached documents
    n_new = np.full(n_docs, q_len, np.int32)
    stride = -(-(doc_len + q_len) // ps)
    slots, bt, lens = alloc.prepare_step(seqs, n_new, stride)
    d_slots, d_bt, d_lens = (torch.from_numpy(x.copy()).to(dev) for x in (slots, bt, lens))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(dev)
    q = torch.randn((n_docs * q_len, hq, D), generator=gen, device=dev).to(torch.bfloat16)
    k_new = torch.randn((n_docs * q_len, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((n_docs * q_len, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    max_len = doc_len + q_len
    ws = torch.empty(max(16, pkv.workspace_bytes(desc, n_docs, hq, q_len, max_len)), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(D))
    store = pkv.bind_store_kv(desc, k_pool, v_pool, k_new, v_new, d_slots)
    append = pkv.bind_prefill_append(desc, k_pool, v_pool, q, cu, d_bt, d_lens, q_len, max_len, scale, out, ws)
    reps = 30
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(reps)]
    for i in range(reps + 2):
        ev = evs[i - 2] if i >= 2 else None
        if ev:
            ev[0].record()
        store()
        if ev:
            ev[1].record()
        append()
        if ev:
            ev[2].record()
        torch.cuda.synchronize()
        # rewind to the documents, last first, so the free stack hands document
        # 0's pages back first and the next question reuses the same pages
        for x in seqs[::-1].tolist():
            alloc.truncate(x, doc_len)
        s2, b2, l2 = alloc.prepare_step(seqs, n_new, stride)
        assert np.array_equal(s2, slots) and np.array_equal(b2, bt), "truncate then reserve must reuse the pages"
    store_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    attn_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
    assert torch.isfinite(out.float()).all(), "non-finite append output"
    attn_s = float(attn_ms.mean()) / 1e3
    pass_s = attn_s + float(store_ms.mean()) / 1e3
    kv = n_docs * max_len * kv_bytes_per_position(hkv, D, 2)
    qo = 2 * q.numel() * 2
    return {
        "workload": "KV rewind: 1,000 documents x 300 cached positions, page_size 16, 32,768-page shuffled pool, "
                    "32 q / 8 KV heads, head_dim 128, bf16; pass = store_kv of 50,000 question tokens + one causal "
                    "50-query prefill_append per document over its 350 positions",
        "value": round(n_docs * q_len / pass_s, 1), "unit": "tokens/s", "reps": reps,
        "new_tokens_per_pass": n_docs * q_len, "tokens_if_recomputed": n_docs * max_len,
        "store_kv_avg_us": round(float(store_ms.mean()) * 1e3, 1),
        "roofline": _append_roofline(kv, qo, attn_s, "rewind_append",
                                     "pkv_prefill_append (prefill_schedule_kernel + paged_prefill_kernel)", attn_ms),
    }


def spec_leg(args, torch, pkv, synth, dev: str) -> dict:
    """Long-context decode with speculative rollback: 8 sequences with
    contexts U{32K..128K} (the lengths of the seeded workload), 64-position
    pages over a shuffled pool twice the live size, 64 q / 8 KV heads of 128,
    bf16.  A step reserves 5 drafts per sequence, stores their K/V (40
    tokens) and runs a 5-query causal append (the split decode kernel and its
    merge); then each sequence keeps a random 0..5 drafts (host truncate,
    untimed).  The 16-step pattern of kept drafts runs twice: 32 timed steps."""
    B, drafts, steps, ps, hq, hkv, D = 8, 5, 16, 64, 64, 8, 128
    timed_steps = 2 * steps
    ctx = synth.generator(5, "lengths", args.seed).integers(32_768, 131_072, size=B, endpoint=True).astype(np.int64)
    keep = np.random.default_rng(5100 + args.seed).integers(0, drafts + 1, size=(steps, B))
    num_pages = int(2 * sum(-(-int(x + timed_steps * drafts) // ps) for x in ctx))
    desc = pkv.PoolDesc(pkv.PKV_BF16, num_pages, ps, hkv, D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5000 + args.seed)
    k_pool = torch.randn(desc.pool_shape, generator=gen, device=dev).to(torch.bfloat16)
    v_pool = torch.randn(desc.pool_shape, generator=gen, device=dev).to(torch.bfloat16)
    order = np.random.default_rng(5200 + args.seed).permutation(num_pages).astype(np.int32)
    alloc = pkv.Allocator(num_pages, ps, order)
    seqs = np.array([alloc.seq_new() for _ in range(B)], np.int32)
    alloc.prepare_step(seqs, ctx.astype(np.int32), 0)
    max_len = int(ctx.max()) + timed_steps * drafts
    stride = -(-max_len // ps)
    n_new = np.full(B, drafts, np.int32)
    cu = torch.from_numpy(np.arange(0, (B + 1) * drafts, drafts, dtype=np.int32)).to(dev)
    q = torch.randn((B * drafts, hq, D), generator=gen, device=dev).to(torch.bfloat16)
    k_new = torch.randn((B * drafts, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((B * drafts, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(max(16, pkv.workspace_bytes(desc, B, hq, drafts, max_len)), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(D))
    store_ms, attn_ms, kv = [], [], []
    for st in range(timed_steps + 2):           # two untimed warm-up steps, then 32
        slots, bt, lens = alloc.prepare_step(seqs, n_new, stride)
        d_slots, d_bt, d_lens = (torch.from_numpy(x.copy()).to(dev) for x in (slots, bt, lens))
        ev = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
        ev[0].record()
        pkv.store_kv(desc, k_pool, v_pool, k_new, v_new, d_slots)
        ev[1].record()
        pkv.prefill_append(desc, k_pool, v_pool, q, cu, d_bt, d_lens, drafts, max_len, scale, out, ws)
        ev[2].record()
        torch.cuda.synchronize()
        if st >= 2:
            store_ms.append(ev[0].elapsed_time(ev[1]))
            attn_ms.append(ev[1].elapsed_time(ev[2]))
            kv.append(int(lens.astype(np.int64).sum()) * kv_bytes_per_position(hkv, D, 2))
        k = keep[(st - 2) % steps] if st >= 2 else np.zeros(B, np.int64)
        for b, x in enumerate(seqs.tolist()):
            alloc.truncate(x, int(lens[b]) - drafts + int(k[b]))
    assert torch.isfinite(out.float()).all(), "non-finite append output"
    attn_ms = np.array(attn_ms)
    attn_s = float(attn_ms.mean()) / 1e3
    step_s = attn_s + float(np.mean(store_ms)) / 1e3
    qo = 2 * q.numel() * 2
    return {
        "workload": "long-context decode + speculative rollback: 8 sequences, contexts U{32K..128K}, page_size 64, "
                    f"{num_pages:,}-page shuffled pool, 64 q / 8 KV heads, head_dim 128, bf16; step = store_kv of 5 "
                    "drafts per sequence + one 5-query causal prefill_append (split decode kernel + merge), then "
                    "keep 0..5 drafts",
        "value": round(float(np.mean(kv)) / step_s / 1e9, 1), "unit": "GB/s", "steps": timed_steps,
        "ms_per_step": round(step_s * 1e3, 3), "mean_context": round(float(np.mean(kv)) / 4096 / B, 1),
        "store_kv_avg_us": round(float(np.mean(store_ms)) * 1e3, 1),
        "roofline": _append_roofline(int(np.mean(kv)), qo, attn_s, "spec_rollback",
                                     "pkv_prefill_append, 5 queries per sequence (paged_decode_kernel + "
                                     "merge_segments_kernel)", attn_ms),
    }


def copy_pages_leg(args, torch, pkv, dev: str) -> dict:
    """Copy-on-write page copies: ``args.copy_pairs`` (shared, fresh) page
    pairs drawn without repetition from a shuffled 32,768-page pool of the
    decode shape (16 positions x 8 KV heads x 128, bf16), copied in K and V
    by one pkv_copy_pages launch.  HBM bytes per launch = 2 pools x (read +
    write) x 32 KiB x pairs."""
    ps, hkv, D, num_pages = 16, 8, 128, 32_768
    desc = pkv.PoolDesc(pkv.PKV_BF16, num_pages, ps, hkv, D)
    k_pool, v_pool = desc.new_pools(dev, fill=1.0)
    perm = np.random.default_rng(args.seed + 77).permutation(num_pages)[: 2 * args.copy_pairs]
    copies = torch.from_numpy(perm.reshape(2, -1).T.copy().astype(np.int32)).to(dev)
    for _ in range(3):
        pkv.copy_pages(desc, k_pool, v_pool, copies)
    torch.cuda.synchronize()
    reps = 20
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        pkv.copy_pages(desc, k_pool, v_pool, copies)
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    page_bytes = hkv * ps * D * 2
    alg = 2 * 2 * page_bytes * args.copy_pairs
    avg_s = float(ms.mean()) / 1e3
    achieved = alg / avg_s / 1e9
    del k_pool, v_pool
    torch.cuda.empty_cache()
    # context: torch's contiguous device-to-device copy reading and writing
    # the same bytes (alg / 2 each way)
    src = torch.ones(alg // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ref_s = float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3
    del src, dst
    torch.cuda.empty_cache()
    return {
        "workload": f"copy-on-write page copies: {args.copy_pairs} distinct (shared, fresh) page pairs of a shuffled "
                    "32,768-page bf16 pool (16 positions x 8 KV heads x 128), K and V, one pkv_copy_pages launch",
        "pairs": args.copy_pairs,
        "reps": reps,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("copy_pages"),
            "kernel": "pkv_copy_pages (copy_pages_kernel)",
            "kernel_avg_us": round(avg_s * 1e6, 2),
            "kernel_median_us": round(float(np.median(ms)) * 1e3, 2),
            "algorithmic_bytes_per_launch": alg,
        },
        "contiguous_copy_same_bytes_gbs": round(alg / ref_s / 1e9, 1),
    }


def codec_leg(args, torch, pkv, dev: str) -> dict:
    """Group-wise Q8 / Q4 codec of one long prefix: 131,072 positions of 8 KV
    heads x 128 (bf16, 16-position pages scattered over a shuffled pool),
    encoded into a payload and restored into other scattered pages.  HBM
    bytes: encode reads the K/V (2 x n x 8 x 128 x 2) and writes the payload;
    restore reads the payload and writes the K/V."""
    n, hkv, D, ps = 131_072, 8, 128, 16
    pages = n // ps
    num_pages = 2 * pages + 64
    desc = pkv.PoolDesc(pkv.PKV_BF16, num_pages, ps, hkv, D)
    k_pool, v_pool = desc.new_pools(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 5)
    k_pool.normal_(generator=gen)
    v_pool.normal_(generator=gen)
    order = np.random.default_rng(args.seed + 6).permutation(num_pages).astype(np.int32)
    src_bt = torch.from_numpy(order[:pages].copy()).to(dev)
    dst_bt = torch.from_numpy(order[pages:2 * pages].copy()).to(dev)
    kv_bytes = 2 * n * hkv * D * 2
    out = {"workload": "one 131,072-position prefix, 8 KV heads x 128, bf16, 16-position pages scattered over a "
                       "shuffled pool: encode into a packed payload (groups of 64, fp16 scales) and restore into "
                       "other scattered pages"}
    reps = 20
    for bits in (8, 4):
        pay = torch.empty(pkv.codec_payload_bytes(n, hkv, D, bits), dtype=torch.uint8, device=dev)
        res = {}
        for name, call in (("encode", lambda: pkv.codec_encode(desc, k_pool, v_pool, src_bt, n, bits, pay)),
                           ("restore", lambda: pkv.codec_decode(desc, k_pool, v_pool, dst_bt, n, bits, pay))):
            call()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in evs:
                a.record()
                call()
                b.record()
            torch.cuda.synchronize()
            t = float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3
            alg = kv_bytes + pay.numel()
            res[name] = {"kernel_avg_us": round(t * 1e6, 2), "achieved_gbs": round(alg / t / 1e9, 1),
                         "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": alg,
                         "traffic": measured_traffic(f"codec_q{bits}_{name}")}
        out[f"q{bits}"] = res
        del pay
    del k_pool, v_pool
    torch.cuda.empty_cache()
    return out


def retention_leg(args, pkv) -> dict:
    """Host-side KV retention pool: ``args.retention_docs`` documents of
    U{1..64} pages (page size 16) retained with probability_of_reuse ~
    U[0, 1) and recompute_seconds ~ U[0.01, 1), then one eviction down to
    half of their pages (lowest probability * seconds / pages first)."""
    n = args.retention_docs
    rng = np.random.default_rng(args.seed + 99)
    pages = rng.integers(1, 65, size=n)
    prob = rng.random(n)
    secs = 0.01 + 0.99 * rng.random(n)
    alloc = pkv.Allocator(int(pages.sum()), 16)
    seqs = [alloc.seq_new() for _ in range(n)]
    for s_, p_ in zip(seqs, pages.tolist()):
        alloc.reserve(s_, 16 * p_)
    t0 = time.perf_counter()
    for s_, p_, t_ in zip(seqs, prob.tolist(), secs.tolist()):
        alloc.retention_add(s_, p_, t_)
    add_s = time.perf_counter() - t0
    total = alloc.retention_pages()
    t0 = time.perf_counter()
    evicted = alloc.retention_evict(total // 2)
    evict_s = time.perf_counter() - t0
    return {
        "workload": f"host KV retention pool: {n} documents of U{{1..64}} pages, evicted to half their "
                    "pages in one pkv_retention_evict call",
        "retained_pages": int(total),
        "evicted_docs": int(evicted.size),
        "evict_ms": round(evict_s * 1e3, 3),
        "add_us_per_doc_incl_python": round(add_s / n * 1e6, 3),
    }


def cpu_baseline(w, scale: float, budget_s: float):
    """Time the fp64 oracle on whole sequences of the batch until the budget ends."""
    import synth
    from oracle.attention import attend
    threads = _blas_threads()
    per_pos = kv_bytes_per_position(w.num_kv_heads, w.head_dim, 2)
    done_bytes = 0
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:      # whole passes over the batch
        for b in range(len(w.lengths)):
            lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
            k = synth.to_f64(w.k[lo:hi], w.dtype)
            v = synth.to_f64(w.v[lo:hi], w.dtype)
            q = synth.to_f64(w.q[b:b + 1], w.dtype)
            attend(q, k, v, scale)
            done_bytes += (hi - lo) * per_pos
            done += 1
    elapsed = time.perf_counter() - t0
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle decode of {done} sequences ({done / len(w.lengths):.1f} passes "
                  f"over the 64-sequence batch) "
                  f"({done_bytes / 1e6:.1f} MB of K/V, {elapsed:.1f} s incl. bf16->fp64 widening), "
                  f"host cores available {len(os.sched_getaffinity(0))}",
    }


def host_info() -> dict:
    """The host the CPU baselines ran on: CPU model (as lscpu reports it, from
    /proc/cpuinfo), cores available to this process, BLAS threads."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)), "blas_threads": _blas_threads(),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
            "OPENBLAS_NUM_THREADS": os.environ.get("OPENBLAS_NUM_THREADS")}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:
        return 1


def cpu_baseline_prefix(args, budget_s: float) -> dict:
    """The fp64 oracle on the prefix-shared prefill workload: documents of the
    256-row workload (its lengths and its plan from the oracle planner) in a
    seeded order, each one attend() of its unshared suffix over its whole
    context, until the budget is spent.  Values are N(0,1) fp64 of one trace,
    drawn once outside the timed region (the oracle's time does not depend on
    them).  Reported as processed tokens/s and fp64 flop/s."""
    import synth
    from oracle.attention import attend
    from oracle.planner import plan_prefix
    w = synth.prefix_traces(seed=args.seed, values=False)
    n = len(w.row_len)
    _, _, shared = plan_prefix([w.row_tokens(r).tolist() for r in range(n)], w.page_size)
    hq, hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    rng = np.random.default_rng(7000 + args.seed)
    t_len = int(w.row_len.max())
    q = rng.standard_normal((t_len, hq, D))
    k = rng.standard_normal((t_len, hkv, D))
    v = rng.standard_normal((t_len, hkv, D))
    scale = 1.0 / float(np.sqrt(D))
    tokens = pairs = done = 0
    t0 = time.perf_counter()
    for d in rng.permutation(n).tolist():
        if time.perf_counter() - t0 >= budget_s:
            break
        L, sh = int(w.row_len[d]), int(shared[d])
        attend(q[sh:L], k[:L], v[:L], scale)
        tokens += L - sh
        pairs += (L * (L + 1) - sh * (sh + 1)) // 2
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(tokens / el, 1), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "fp64_gflops": round(4.0 * D * hq * pairs / el / 1e9, 2),
            "sample": f"fp64 NumPy oracle on {done} of the 256 prefix-shared rows ({tokens} suffix tokens over "
                      f"their contexts, {pairs} unmasked pairs per head, {el:.1f} s)"}


def cpu_baseline_rewind(args, budget_s: float) -> dict:
    """The fp64 oracle on the KV rewind workload: one 50-query causal append
    over a document's 350 positions per call (32 / 8 heads of 128), repeated
    on fresh seeded N(0,1) documents until the budget is spent; tokens/s."""
    from oracle.attention import attend
    rng = np.random.default_rng(7100 + args.seed)
    q_len, ctx, hq, hkv, D = 50, 350, 32, 8, 128
    scale = 1.0 / float(np.sqrt(D))
    done, busy = 0, 0.0
    while busy < budget_s:
        q = rng.standard_normal((q_len, hq, D))
        k = rng.standard_normal((ctx, hkv, D))
        v = rng.standard_normal((ctx, hkv, D))
        t0 = time.perf_counter()
        attend(q, k, v, scale)
        busy += time.perf_counter() - t0
        done += 1
    return {"value": round(done * q_len / busy, 1), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {done} documents of the rewind workload (50 new queries over 350 "
                      f"positions each, {busy:.1f} s of oracle time)"}


def cpu_baseline_spec(args, budget_s: float) -> dict:
    """The fp64 oracle on the speculative-rollback workload: one 5-draft
    causal append per call over a context of the workload's lengths
    (U{32K..128K}, 64 / 8 heads of 128), until the budget is spent; GB/s of
    bf16 KV the call covers (the unit the GPU leg reports).  One seeded N(0,1)
    fp64 K/V of the longest context is drawn once and read by prefix."""
    import synth
    from oracle.attention import attend
    ctx = synth.generator(5, "lengths", args.seed).integers(32_768, 131_072, size=8, endpoint=True)
    rng = np.random.default_rng(7200 + args.seed)
    drafts, hq, hkv, D = 5, 64, 8, 128
    Lmax = int(ctx.max()) + drafts
    k = rng.standard_normal((Lmax, hkv, D))
    v = rng.standard_normal((Lmax, hkv, D))
    q = rng.standard_normal((drafts, hq, D))
    scale = 1.0 / float(np.sqrt(D))
    done, kv, busy = 0, 0, 0.0
    while busy < budget_s:
        L = int(ctx[done % len(ctx)]) + drafts
        t0 = time.perf_counter()
        attend(q, k[:L], v[:L], scale)
        busy += time.perf_counter() - t0
        kv += L * kv_bytes_per_position(hkv, D, 2)
        done += 1
    return {"value": round(kv / busy / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {done} sequence-steps of the speculative-rollback workload (5 drafts "
                      f"over {kv / 4096 / done:.0f} positions on average, {busy:.1f} s of oracle time)"}


def decode_leg(args, torch, pkv, synth, w, dev: str, kv_int8: bool) -> dict:
    """The paged-decode batch stepped ``args.steps`` times after
    ``args.warmup`` untimed steps (see the module docstring); bf16 pools, or
    INT8 pages (bf16 queries, one fp32 scale per cached vector)."""
    B, hq, hkv, D, ps = len(w.lengths), w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    desc = pkv.PoolDesc(pkv.PKV_I8 if kv_int8 else pkv.PKV_BF16, w.num_pages, ps, hkv, D)
    scale = 1.0 / float(np.sqrt(D))
    per_pos = 2 * hkv * (D + 4) if kv_int8 else kv_bytes_per_position(hkv, D, 2)
    R = args.instances
    total_steps = args.warmup + args.steps
    uses = -(-total_steps // R)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- setup (untimed): pools, R copies of the batch with L-1 positions stored ----
    k_pool, v_pool = desc.new_pools(dev, fill=0xFF if kv_int8 else float("nan"))
    alloc = pkv.Allocator(w.num_pages, ps, w.free_order)
    k_all, v_all = bf16(w.k), bf16(w.v)
    inst = []
    for r in range(R):
        seqs = np.array([alloc.seq_new() for _ in range(B)], np.int32)
        n_ctx = (w.lengths - 1).astype(np.int32)
        slots, _, _ = alloc.prepare_step(seqs, n_ctx, 0)
        rows = torch.from_numpy(np.concatenate(
            [np.arange(w.offsets[b], w.offsets[b + 1] - 1) for b in range(B)])).to(dev)
        pkv.store_kv(desc, k_pool, v_pool, k_all[rows].contiguous(), v_all[rows].contiguous(),
                     torch.from_numpy(slots).to(dev))
        inst.append(seqs)
    last_rows = torch.from_numpy(w.offsets[1:] - 1).to(dev)
    k_new, v_new = k_all[last_rows].contiguous(), v_all[last_rows].contiguous()
    del k_all, v_all
    q = bf16(w.q)
    out = torch.empty_like(q)
    max_len = int(w.lengths.max()) + uses + 1     # + 1: the upload one step ahead
    stride = -(-max_len // ps)
    ws = torch.empty(max(16, pkv.workspace_bytes(desc, B, hq, 1, max_len)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # Upload: step k's slots (int64 [B]), block tables (int32 [B][stride]) and
    # lengths (int32 [B]) go from pinned set k % NSETS to device set k % NSETS
    # in one copy, issued on a copy stream while the previous step's decode
    # runs; the host waits for its event, which has normally fired long
    # before, before launching step k (a copy in line with the kernels costs
    # the copy engine's two hand-offs, about 30 us per step in a kernel
    # trace).  Before a set is refilled the host waits for a timing event
    # recorded after the decode that last read it (at least 5 steps back, so
    # it has long completed).  The compute stream then carries no marker but
    # the timing pair on every TIME_EVERY-th step: each marker leaves the GPU
    # idle for a few microseconds.
    NSETS, TIME_EVERY = 8, 4
    nbytes = B * 8 + B * stride * 4 + B * 4

    def views(buf):
        return (buf[:B * 8].view(torch.int64), buf[B * 8:B * 8 + B * stride * 4].view(torch.int32).view(B, stride),
                buf[B * 8 + B * stride * 4:nbytes].view(torch.int32))

    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream(device=dev)          # default priority
    ones = np.ones(B, np.int32)
    sets = []
    for _ in range(NSETS):
        hb = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        db = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        hs, hbt, hl = views(hb)
        d_slots, d_bt, d_lens = views(db)
        sets.append({
            "host": hb, "dev": db, "np": (hs.numpy(), hbt.numpy(), hl.numpy()),
            "uploaded": torch.cuda.Event(),
            "store": pkv.bind_store_kv(desc, k_pool, v_pool, k_new, v_new, d_slots, stream),
            "decode": pkv.bind_decode(desc, k_pool, v_pool, q, d_bt, d_lens, max_len, scale, out, ws, stream),
        })
    # prepare_step of instance r into pinned set j, marshalled once
    prep = [[alloc.bind_prepare_step(inst[r], ones, stride, *sets[j]["np"]) for j in range(NSETS)]
            for r in range(R)]
    # A small ring of timing-event pairs, read back before reuse (a slot is
    # reused EV_RING marked steps later, long after it completed): many live
    # timing events slow down every record.
    EV_RING = 32
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(EV_RING)]
    slot_timed = [False] * EV_RING        # the slot's last pair belongs to a timed step, unread
    dec_ms = []
    kv_bytes = []                         # every timed step: KV bytes its decode reads
    kv_bytes_timed_calls = []             # the steps whose decode call was timed

    def read_slot(slot: int):
        if slot_timed[slot]:
            a, b = ev[slot]
            b.synchronize()
            dec_ms.append(a.elapsed_time(b))
            slot_timed[slot] = False

    def upload(k: int):
        j = k % NSETS
        st = sets[j]
        if k >= NSETS:
            st["uploaded"].synchronize()      # the copy of step k - NSETS has read the pinned set
            m = k - NSETS + (-(k - NSETS)) % TIME_EVERY   # the marked step in [k - NSETS, k - NSETS + 3]
            ev[(m // TIME_EVERY) % EV_RING][1].synchronize()   # its decode, and step k - NSETS's, are done
        prep[k % R][j]()
        with torch.cuda.stream(copy_stream):
            st["dev"].copy_(st["host"], non_blocking=True)
            st["uploaded"].record(copy_stream)

    def step(k: int, timed: bool):
        st = sets[k % NSETS]
        l_np = st["np"][2]
        # The host waits for this step's copy, which has normally completed
        # during the previous decode; kernels launched after an event is
        # observed complete see what the copy wrote, so the compute stream
        # needs no cross-stream wait (a marker that idles the GPU ~6 us).
        st["uploaded"].synchronize()
        st["store"]()
        marked = k % TIME_EVERY == 0
        if marked:
            slot = (k // TIME_EVERY) % EV_RING
            read_slot(slot)
            ev[slot][0].record(stream)
        st["decode"]()
        if marked:
            ev[slot][1].record(stream)
            slot_timed[slot] = timed
        if timed:
            b = int(l_np.astype(np.int64).sum()) * per_pos
            kv_bytes.append(b)
            if marked:
                kv_bytes_timed_calls.append(b)
        upload(k + 1)                         # the next step's tables, during this decode

    upload(0)
    for k in range(args.warmup):
        step(k, False)
    torch.cuda.synchronize()
    # Keep the garbage collector out of the timed loop: with the workload's
    # arrays alive a full collection takes tens of milliseconds.
    gc.collect()
    gc.freeze()
    gc.disable()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()

    for slot in range(EV_RING):
        read_slot(slot)


    # The last step's decode once more, its tables copied in stream order into
    # a fresh buffer: the timed steps must have read exactly what they uploaded.
    last = sets[(args.warmup + args.steps - 1) % NSETS]
    fresh = torch.empty_like(last["dev"])
    fresh.copy_(last["host"])
    _, f_bt, f_lens = views(fresh)
    out_check = torch.empty_like(out)
    pkv.decode(desc, k_pool, v_pool, q, f_bt, f_lens, max_len, scale, out_check, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_check), "the timed steps' decode differs from a stream-ordered rerun"

    # The decode call alone, timed call by call: CALL_REPS launches back to
    # back, each between its own event pair, over the upload sets of completed
    # steps.  Consecutive sets hold different instances, so consecutive calls
    # read disjoint pages; the pending set (the next step's tables, whose new
    # position is not stored yet) is skipped.
    total = args.warmup + args.steps
    pending = total % NSETS
    ready = sorted({k % NSETS for k in range(max(0, total - NSETS), total)} - {pending})
    call_reps = max(30, args.call_reps)
    call_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(call_reps)]
    call_bytes = []
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(call_ev):
        st = sets[ready[i % len(ready)]]
        a.record(stream)
        st["decode"]()
        b.record(stream)
        call_bytes.append(int(st["np"][2].astype(np.int64).sum()) * per_pos)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in call_ev])
    dec_ms = np.array(dec_ms)
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    total_kv = float(sum(kv_bytes))
    qo_bytes = 2 * B * hq * D * 2                      # q read + out written per launch
    assert len(dec_ms) == len(kv_bytes_timed_calls) > 0, "no timed decode call"
    res = {
        "per_pos": per_pos, "total_kv": total_kv, "wall": wall,
        "in_step_avg_us": float(dec_ms.mean()) * 1e3, "in_step_calls": len(dec_ms),
        "call_ms": call_ms, "alg_per_launch": float(np.mean(call_bytes)) + qo_bytes,
        "dec_avg_s": float(call_ms.mean()) / 1e3, "dec_median_s": float(np.median(call_ms)) / 1e3,
        "timed_calls": len(call_ms),
        "B": B, "hq": hq, "hkv": hkv, "D": D, "ps": ps, "scale": scale,
    }
    res["achieved"] = res["alg_per_launch"] / res["dec_median_s"] / 1e9
    torch.cuda.synchronize()
    del k_pool, v_pool, ws, sets, prep
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the paged path is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch

    import pagedattention_pkv_store_amd as pkv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = synth.decode_batch(seed=args.seed)
    d = decode_leg(args, torch, pkv, synth, w, dev, kv_int8=False)
    B, hq, hkv, D, ps, per_pos = d["B"], d["hq"], d["hkv"], d["D"], d["ps"], d["per_pos"]
    rec = {
        "metric": METRIC,
        "value": round(d["total_kv"] / d["wall"] / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16; lengths U{512..4096}; shuffled free pages)",
        "config": {
            "workload": "paged decode batch: 64 seqs, L~U{512..4096} incl. new token, page_size 16, "
                        "300k-page pool, 32 q heads / 8 KV heads, head_dim 128, bf16 KV, fp32 accumulate; "
                        "step = prepare_step + H2D + store_kv + decode (+LSE merge)",
            "n_seqs": B, "page_size": ps, "num_pages": w.num_pages, "num_q_heads": hq,
            "num_kv_heads": hkv, "head_dim": D, "instances_rotated": args.instances,
            "mean_seq_len": round(float(d["total_kv"] / per_pos / args.steps / B), 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(d["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(d["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode"),
            "kernel": "pkv_decode (paged_decode_kernel + merge_segments_kernel)",
            "achieved_from": "median call",
            "kernel_avg_us": round(d["dec_avg_s"] * 1e6, 2),
            "kernel_median_us": round(d["dec_median_s"] * 1e6, 2),
            "timed_launches": d["timed_calls"],
            "in_step_avg_us": round(d["in_step_avg_us"], 2),
            "in_step_timed_launches": d["in_step_calls"],
            "algorithmic_bytes_per_launch": int(d["alg_per_launch"]),
        },
    }
    if args.int8:
        d8 = decode_leg(args, torch, pkv, synth, w, dev, kv_int8=True)
        rec["int8_decode"] = {
            "workload": "the same decode batch with INT8 pages (int8 codes + one fp32 scale per cached "
                        "vector: 132 bytes per 128-element vector); bf16 queries and outputs",
            "value": round(d8["total_kv"] / d8["wall"] / 1e9, 2),
            "unit": "GB/s",
            "ms_per_step": round(d8["wall"] / args.steps * 1e3, 4),
            "tokens_per_s": round(B * args.steps / d8["wall"], 1),
            "speedup_vs_bf16_step": round(d["wall"] / d8["wall"], 3),
            "roofline": {
                "bound": "hbm",
                "achieved": round(d8["achieved"], 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(d8["achieved"] / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode_int8"),
                "kernel": "pkv_decode on PKV_I8 pools (paged_decode_kernel + merge_segments_kernel)",
                "achieved_from": "median call",
                "kernel_avg_us": round(d8["dec_avg_s"] * 1e6, 2),
                "kernel_median_us": round(d8["dec_median_s"] * 1e6, 2),
                "timed_launches": d8["timed_calls"],
                "algorithmic_bytes_per_launch": int(d8["alg_per_launch"]),
                "speedup_vs_bf16_kernel": round(d["dec_median_s"] / d8["dec_median_s"], 3),
            },
        }
    if args.copy_pairs > 0:
        rec["copy_pages"] = copy_pages_leg(args, torch, pkv, dev)
    if args.codec:
        rec["kv_codec"] = codec_leg(args, torch, pkv, dev)
    if args.retention_docs > 0:
        rec["retention"] = retention_leg(args, pkv)
    if args.prefill_reps > 0:
        rec["prefill_append"] = prefill_leg(args, torch, pkv, synth, dev)
        if args.int8:
            p8 = prefill_leg(args, torch, pkv, synth, dev, kv_int8=True)
            p8["workload"] = ("the same prefix-shared prefill on INT8 pages (codes staged as exact bf16, key "
                              "scales applied to the scores, value scales to the probabilities); bf16 queries "
                              "and outputs")
            p8["roofline"]["kernel"] = "pkv_prefill_append on PKV_I8 pools (prefill_schedule_kernel + paged_prefill_kernel)"
            rec["int8_prefill_append"] = p8
    if args.rewind:
        rec["rewind_append"] = rewind_leg(args, torch, pkv, dev)
    if args.spec:
        rec["spec_rollback"] = spec_leg(args, torch, pkv, synth, dev)
    if args.read_probe:
        probe = read_probe_leg(args, torch, pkv, dev)
        rec["hbm_read_probe"] = probe
        for obj in [rec] + [rec[k] for k in ("int8_decode", "copy_pages", "rewind_append", "spec_rollback") if k in rec]:
            r = obj.get("roofline")
            if r and r.get("bound") == "hbm":
                r["frac_of_measured_read"] = round(r["achieved"] / probe["gbs"], 4)
    if args.copy_calibration_mib > 0:
        n_f32 = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n_f32, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n_f32 * 4
        del src, dst
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, d["scale"], args.cpu_seconds)
        rec["cpu_baseline"]["host"] = host_info()
    if args.cpu_seconds_other > 0:
        for key, fn in (("prefill_append", cpu_baseline_prefix), ("rewind_append", cpu_baseline_rewind),
                        ("spec_rollback", cpu_baseline_spec)):
            if key in rec:
                rec[key]["cpu_baseline"] = fn(args, args.cpu_seconds_other)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
