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
(host work and copies included).  ``roofline`` = the decode kernels' own
algorithmic bytes per launch / their average duration from HIP events on the
launch stream, against the 8 TB/s HBM peak.  ``cpu_baseline`` = the fp64 CPU
oracle on a bounded sample of the same sequences.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged-decode KV GB/s (% of HBM peak); prefill-append tokens/s (% MFMA peak)"


def kv_bytes_per_position(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one position across all KV heads (one layer)."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="bound on the CPU oracle's sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


def cpu_baseline(w, scale: float, budget_s: float):
    """Time the fp64 oracle on whole sequences of the batch until the budget ends."""
    import synth
    from oracle.attention import attend
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the paged path is not sharded across GPUs in this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    import pagedattention_pkv_store_amd as pkv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = synth.decode_batch(seed=args.seed)
    B, hq, hkv, D, ps = len(w.lengths), w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    desc = pkv.PoolDesc(pkv.PKV_BF16, w.num_pages, ps, hkv, D)
    scale = 1.0 / float(np.sqrt(D))
    per_pos = kv_bytes_per_position(hkv, D, 2)
    R = args.instances
    total_steps = args.warmup + args.steps
    uses = -(-total_steps // R)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- setup (untimed): pools, R copies of the batch with L-1 positions stored ----
    k_pool = torch.full(desc.pool_shape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full_like(k_pool, float("nan"))
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
    q = bf16(w.q)
    out = torch.empty_like(q)
    max_len = int(w.lengths.max()) + uses
    stride = -(-max_len // ps)
    ws = torch.empty(max(16, pkv.workspace_bytes(desc, B, hq, 1, max_len)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # pinned staging, double-buffered: the host fills set k%2 while the copy
    # of the previous step's set may still be in flight
    pinned = []
    for _ in range(2):
        pinned.append({
            "slots": torch.empty(B, dtype=torch.int64, pin_memory=True),
            "bt": torch.empty((B, stride), dtype=torch.int32, pin_memory=True),
            "lens": torch.empty(B, dtype=torch.int32, pin_memory=True),
            "done": None,
        })
    d_slots = torch.empty(B, dtype=torch.int64, device=dev)
    d_bt = torch.empty((B, stride), dtype=torch.int32, device=dev)
    d_lens = torch.empty(B, dtype=torch.int32, device=dev)
    ones = np.ones(B, np.int32)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    kv_bytes = []

    def step(k: int, timed_idx: int):
        r = k % R
        buf = pinned[k % 2]
        if buf["done"] is not None:
            buf["done"].synchronize()
        s_np, bt_np, l_np = buf["slots"].numpy(), buf["bt"].numpy(), buf["lens"].numpy()
        alloc.prepare_step(inst[r], ones, stride, s_np, bt_np, l_np)
        d_slots.copy_(buf["slots"], non_blocking=True)
        d_bt.copy_(buf["bt"], non_blocking=True)
        d_lens.copy_(buf["lens"], non_blocking=True)
        e = torch.cuda.Event()
        e.record(stream)
        buf["done"] = e
        pkv.store_kv(desc, k_pool, v_pool, k_new, v_new, d_slots)
        if timed_idx >= 0:
            ev[timed_idx][0].record(stream)
        pkv.decode(desc, k_pool, v_pool, q, d_bt, d_lens, max_len, scale, out, ws)
        if timed_idx >= 0:
            ev[timed_idx][1].record(stream)
            kv_bytes.append(int(l_np.astype(np.int64).sum()) * per_pos)

    for k in range(args.warmup):
        step(k, -1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    total_kv = float(sum(kv_bytes))
    qo_bytes = 2 * B * hq * D * 2                      # q read + out written per launch
    alg_per_launch = total_kv / args.steps + qo_bytes
    dec_avg_s = float(dec_ms.mean()) / 1e3
    achieved = alg_per_launch / dec_avg_s / 1e9
    value = total_kv / wall / 1e9
    assert torch.isfinite(out.float()).all(), "non-finite decode output"

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
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
            "num_kv_heads": hkv, "head_dim": D, "instances_rotated": R,
            "mean_seq_len": round(float(total_kv / per_pos / args.steps / B), 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "pkv_decode (paged_attention_kernel + merge_splits_kernel)",
            "kernel_avg_us": round(dec_avg_s * 1e6, 2),
            "kernel_median_us": round(float(np.median(dec_ms)) * 1e3, 2),
            "algorithmic_bytes_per_launch": int(alg_per_launch),
        },
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, scale, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
