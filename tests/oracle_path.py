"""Oracle-side references for the five workloads, on the same synth inputs.

Uses only ``oracle`` and ``synth``: logical K/V are taken straight from the
generated arrays (what an unpaged computation would see), block tables and
slots from the oracle allocator running the same operation sequence as the
product path, and plans from the oracle planner.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

import synth
from oracle.attention import attend, attend_row
from oracle.paging import Allocator
from oracle.planner import plan_prefix
from oracle.quant import dequantize, quantize


def f64(values, dtype):
    return synth.to_f64(values, dtype)


def kv_f64(values, dtype, kv_int8: bool = False):
    """Logical K or V as attention sees them: the stored values, or for an
    INT8 cache the dequantized codes of each (position, head) vector."""
    x = synth.to_f64(values, dtype)
    return dequantize(*quantize(x)) if kv_int8 else x


def tiny_reference(w: synth.TinyBatch, scale: float):
    alloc = Allocator(w.num_pages, w.page_size, w.free_order)
    seqs = [alloc.seq_new() for _ in w.lengths]
    for b, s in enumerate(seqs):
        alloc.reserve(s, int(w.lengths[b]))
    tables = [alloc.block_table(s) for s in seqs]
    slots = [alloc.slots(s, 0, int(w.lengths[b])) for b, s in enumerate(seqs)]
    prefill, dec = [], []
    for b in range(len(seqs)):
        lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
        k, v, q = f64(w.k[lo:hi], w.dtype), f64(w.v[lo:hi], w.dtype), f64(w.q[lo:hi], w.dtype)
        prefill.append(attend(q, k, v, scale))
        dec.append(attend(q[-1:], k, v, scale)[0])
    return tables, slots, np.concatenate(prefill), np.stack(dec)


def decode_allocator(w, free_order=None):
    """Oracle allocator after the decode workload's operations."""
    alloc = Allocator(w.num_pages, w.page_size, w.free_order if free_order is None else free_order)
    seqs = [alloc.seq_new() for _ in w.lengths]
    for b, s in enumerate(seqs):
        alloc.reserve(s, int(w.lengths[b]) - 1)
    for s in seqs:
        alloc.reserve(s, 1)
    return alloc, seqs


def decode_reference(w: synth.DecodeBatch, scale: float, rows=None,
                     kv_int8: bool = False) -> Dict[Tuple[int, int], np.ndarray]:
    """rows: iterable of (b, h); default all.  Returns {(b, h): o [D]}."""
    B, hq = len(w.lengths), w.num_q_heads
    grp = hq // w.num_kv_heads
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(hq)]
    out = {}
    for b, h in rows:
        lo, L = int(w.offsets[b]), int(w.lengths[b])
        g = h // grp
        k = kv_f64(w.k[lo:lo + L, g], w.dtype, kv_int8)
        v = kv_f64(w.v[lo:lo + L, g], w.dtype, kv_int8)
        out[(b, h)] = attend_row(f64(w.q[b, h], w.dtype), k, v, L - 1, scale)
    return out


def prefix_plan(w: synth.PrefixTraces):
    return plan_prefix([w.row_tokens(r).tolist() for r in range(len(w.row_len))], w.page_size)


def prefix_reference_rows(w: synth.PrefixTraces, shared: List[int], scale: float, rows,
                          kv_int8: bool = False):
    """rows: iterable of (doc, i, h) with i the index among the doc's new queries."""
    grp = w.num_q_heads // w.num_kv_heads
    out = {}
    for d, i, h in rows:
        t = int(w.row_trace[d])
        pos = int(shared[d]) + i
        g = h // grp
        out[(d, i, h)] = attend_row(f64(w.q[t, pos, h], w.dtype), kv_f64(w.k[t, :pos + 1, g], w.dtype, kv_int8),
                                    kv_f64(w.v[t, :pos + 1, g], w.dtype, kv_int8), pos, scale)
    return out


def prefix_reference_full(w: synth.PrefixTraces, shared: List[int], scale: float,
                          kv_int8: bool = False) -> np.ndarray:
    """All rows' suffix outputs, packed in row-id order."""
    outs = []
    for d in range(len(w.row_len)):
        t, L, sh = int(w.row_trace[d]), int(w.row_len[d]), int(shared[d])
        outs.append(attend(f64(w.q[t, sh:L], w.dtype), kv_f64(w.k[t, :L], w.dtype, kv_int8),
                           kv_f64(w.v[t, :L], w.dtype, kv_int8), scale))
    return np.concatenate(outs)


def rewind_reference(w: synth.RewindDocs, scale: float, docs=None, kv_int8: bool = False):
    """[pass1, pass2] outputs [n_docs][q_len][Hq][D] for the listed docs."""
    n = w.doc_k.shape[0]
    docs = range(n) if docs is None else docs
    res = []
    for qq, qk, qv in ((w.q1_q, w.q1_k, w.q1_v), (w.q2_q, w.q2_k, w.q2_v)):
        per = {}
        for d in docs:
            k = np.concatenate([kv_f64(w.doc_k[d], w.dtype, kv_int8), kv_f64(qk[d], w.dtype, kv_int8)])
            v = np.concatenate([kv_f64(w.doc_v[d], w.dtype, kv_int8), kv_f64(qv[d], w.dtype, kv_int8)])
            per[d] = attend(f64(qq[d], w.dtype), k, v, scale)
        res.append(per)
    return res


def spec_reference(w: synth.SpecDecode, scale: float, steps: int, seqs_checked=None,
                   kv_int8: bool = False):
    """Per step, {b: [drafts][Hq][D]} over each sequence's kept logical K/V."""
    B = len(w.ctx_len)
    seqs_checked = range(B) if seqs_checked is None else seqs_checked
    kept_k = {b: [kv_f64(w.ctx_k[w.ctx_offsets[b]:w.ctx_offsets[b + 1]], w.dtype, kv_int8)]
              for b in seqs_checked}
    kept_v = {b: [kv_f64(w.ctx_v[w.ctx_offsets[b]:w.ctx_offsets[b + 1]], w.dtype, kv_int8)]
              for b in seqs_checked}
    res = []
    for st in range(steps):
        per = {}
        for b in seqs_checked:
            dk = kv_f64(w.draft_k[st, b], w.dtype, kv_int8)
            dv = kv_f64(w.draft_v[st, b], w.dtype, kv_int8)
            k = np.concatenate(kept_k[b] + [dk])
            v = np.concatenate(kept_v[b] + [dv])
            per[b] = attend(f64(w.draft_q[st, b], w.dtype), k, v, scale)
            keep = int(w.keep[st, b])
            kept_k[b].append(dk[:keep])
            kept_v[b].append(dv[:keep])
        res.append(per)
    return res
