"""Drive the product path (libpkv through its Python binding) on synth inputs.

Every step here runs in the library: the C++ allocator and planner produce
block tables, slots and plans; the HIP kernels store K/V and compute
attention.  This module only moves data between NumPy and device tensors and
issues the calls in the order a serving loop would.  It never imports the
oracle.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

import pagedattention_pkv_store_amd as pkv
import synth

DEV = "cuda:0"


def dev_tensor(values: np.ndarray, dtype: str) -> torch.Tensor:
    """synth values (fp32 array or bf16 bit array) -> device tensor of that dtype."""
    a = np.ascontiguousarray(values)
    if dtype == synth.F32:
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def desc_of(w, kv_int8: bool = False) -> pkv.PoolDesc:
    if kv_int8:
        assert w.dtype == synth.BF16, "INT8 pages take bf16 K/V and queries"
        dt = pkv.PKV_I8
    else:
        dt = pkv.PKV_BF16 if w.dtype == synth.BF16 else pkv.PKV_F32
    return pkv.PoolDesc(dt, int(w.num_pages), int(w.page_size), int(w.num_kv_heads), int(w.head_dim))


def nan_pools(desc: pkv.PoolDesc):
    """Pools whose every unwritten slot reads as NaN: NaN elements, or for INT8
    pages 0xFF bytes (codes -1, scales NaN)."""
    return desc.new_pools(DEV, fill=0xFF if desc.dtype == pkv.PKV_I8 else float("nan"))


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def i64(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


@dataclass
class Session:
    """A pool pair plus the host allocator that owns its pages."""
    desc: pkv.PoolDesc
    alloc: pkv.Allocator
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    scale: float
    log: Dict[str, list] = field(default_factory=dict)   # tables / slots for checks

    @classmethod
    def open(cls, w, free_order=None, kv_int8: bool = False):
        desc = desc_of(w, kv_int8)
        order = w.free_order if free_order is None else free_order
        alloc = pkv.Allocator(desc.num_pages, desc.page_size, order)
        k, v = nan_pools(desc)
        return cls(desc, alloc, k, v, 1.0 / float(np.sqrt(desc.head_dim)))

    def store(self, seq: int, start: int, k_rows: np.ndarray, v_rows: np.ndarray, dtype: str):
        n = k_rows.shape[0]
        if n == 0:
            return
        slots = self.alloc.slots(seq, start, n)
        self.log.setdefault("slots", []).append((seq, start, slots.copy()))
        pkv.store_kv(self.desc, self.k_pool, self.v_pool, dev_tensor(k_rows, dtype),
                     dev_tensor(v_rows, dtype), i64(slots))

    def store_many(self, items, dtype: str):
        """Store several (seq, start, k_rows, v_rows) in one kernel launch."""
        slots, ks, vs = [], [], []
        for seq, start, k_rows, v_rows in items:
            if k_rows.shape[0] == 0:
                continue
            s = self.alloc.slots(seq, start, k_rows.shape[0])
            self.log.setdefault("slots", []).append((seq, start, s.copy()))
            slots.append(s)
            ks.append(k_rows)
            vs.append(v_rows)
        if not slots:
            return
        pkv.store_kv(self.desc, self.k_pool, self.v_pool, dev_tensor(np.concatenate(ks), dtype),
                     dev_tensor(np.concatenate(vs), dtype), i64(np.concatenate(slots)))

    def tables(self, seqs: List[int]) -> np.ndarray:
        stride = max(1, max(self.alloc.num_blocks(s) for s in seqs))
        bt = self.alloc.block_tables(seqs, stride)
        self.log.setdefault("tables", []).append(bt.copy())
        return bt

    def decode(self, seqs: List[int], q: torch.Tensor) -> torch.Tensor:
        lens = np.array([self.alloc.seq_len(s) for s in seqs], np.int32)
        bt = self.tables(seqs)
        out = torch.empty_like(q)
        max_len = int(lens.max()) if len(lens) else 0
        need = pkv.workspace_bytes(self.desc, len(seqs), q.shape[1], 1, max_len)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        pkv.decode(self.desc, self.k_pool, self.v_pool, q, i32(bt), i32(lens), max_len,
                   self.scale, out, ws)
        return out

    def append(self, seqs: List[int], n_new: List[int], q: torch.Tensor) -> torch.Tensor:
        """Prefill/append: seq b's last n_new[b] positions get queries (packed in q)."""
        lens = np.array([self.alloc.seq_len(s) for s in seqs], np.int32)
        cu = np.zeros(len(seqs) + 1, np.int32)
        cu[1:] = np.cumsum(n_new)
        bt = self.tables(seqs)
        out = torch.empty_like(q)
        max_q = int(max(n_new)) if len(n_new) else 0
        max_len = int(lens.max()) if len(lens) else 0
        pkv.validate_tables(self.desc, bt, lens, cu, max_q)
        need = pkv.workspace_bytes(self.desc, len(seqs), q.shape[1], max_q, max_len)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        pkv.prefill_append(self.desc, self.k_pool, self.v_pool, q, i32(cu), i32(bt), i32(lens),
                           max_q, max_len, self.scale, out, ws)
        return out


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def run_tiny(w: synth.TinyBatch):
    """Store both sequences; causal prefill of every position; decode of the last."""
    s = Session.open(w)
    seqs = [s.alloc.seq_new() for _ in w.lengths]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, int(w.lengths[b]))
    for b, seq in enumerate(seqs):
        lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
        s.store(seq, 0, w.k[lo:hi], w.v[lo:hi], w.dtype)
    prefill = s.append(seqs, [int(x) for x in w.lengths], dev_tensor(w.q, w.dtype))
    last = np.stack([w.q[int(w.offsets[b + 1]) - 1] for b in range(len(seqs))])
    dec = s.decode(seqs, dev_tensor(last, w.dtype))
    torch.cuda.synchronize()
    return s, seqs, prefill, dec


def run_decode(w: synth.DecodeBatch, free_order=None, kv_int8: bool = False):
    """Setup stores positions 0..L-2; the step stores position L-1 and decodes."""
    s = Session.open(w, free_order, kv_int8)
    seqs = [s.alloc.seq_new() for _ in w.lengths]
    items = []
    for b, seq in enumerate(seqs):
        L, lo = int(w.lengths[b]), int(w.offsets[b])
        s.alloc.reserve(seq, L - 1)
        items.append((seq, 0, w.k[lo:lo + L - 1], w.v[lo:lo + L - 1]))
    s.store_many(items, w.dtype)
    items = []
    for b, seq in enumerate(seqs):
        L, lo = int(w.lengths[b]), int(w.offsets[b])
        s.alloc.reserve(seq, 1)
        items.append((seq, L - 1, w.k[lo + L - 1:lo + L], w.v[lo + L - 1:lo + L]))
    s.store_many(items, w.dtype)
    out = s.decode(seqs, dev_tensor(w.q, w.dtype))
    torch.cuda.synchronize()
    return s, seqs, out


def run_prefix(w: synth.PrefixTraces, kv_int8: bool = False):
    """Plan, adopt shared pages in planned order, store every unshared suffix,
    then one prefill/append over all rows' suffixes (rows in id order)."""
    s = Session.open(w, kv_int8=kv_int8)
    n = len(w.row_len)
    order, parent, shared = pkv.plan_prefix([w.row_tokens(r) for r in range(n)], w.page_size)
    seqs = [-1] * n
    items = []
    for d in order.tolist():
        seqs[d] = s.alloc.seq_new()
        if parent[d] >= 0:
            s.alloc.share_prefix(seqs[d], seqs[parent[d]], int(shared[d]))
        L, sh, t = int(w.row_len[d]), int(shared[d]), int(w.row_trace[d])
        s.alloc.reserve(seqs[d], L - sh)
        items.append((seqs[d], sh, w.k[t, sh:L], w.v[t, sh:L]))
    s.store_many(items, w.dtype)
    q = np.concatenate([w.q[int(w.row_trace[d]), int(shared[d]):int(w.row_len[d])] for d in range(n)])
    n_new = [int(w.row_len[d]) - int(shared[d]) for d in range(n)]
    out = s.append(seqs, n_new, dev_tensor(q, w.dtype))
    torch.cuda.synchronize()
    return s, (order, parent, shared), seqs, n_new, out


def run_rewind(w: synth.RewindDocs, kv_int8: bool = False):
    """Documents cached; question 1 appended and answered; truncated back to the
    document; question 2 appended and answered on the kept pages."""
    s = Session.open(w, kv_int8=kv_int8)
    n = w.doc_k.shape[0]
    seqs = [s.alloc.seq_new() for _ in range(n)]
    items = []
    for d, seq in enumerate(seqs):
        s.alloc.reserve(seq, w.doc_len)
        items.append((seq, 0, w.doc_k[d], w.doc_v[d]))
    s.store_many(items, w.dtype)
    outs = []
    for qq, qk, qv in ((w.q1_q, w.q1_k, w.q1_v), (w.q2_q, w.q2_k, w.q2_v)):
        items = []
        for d, seq in enumerate(seqs):
            s.alloc.reserve(seq, w.q_len)
            items.append((seq, w.doc_len, qk[d], qv[d]))
        s.store_many(items, w.dtype)
        q = qq.reshape(n * w.q_len, w.num_q_heads, w.head_dim)
        outs.append(s.append(seqs, [w.q_len] * n, dev_tensor(q, w.dtype)))
        for seq in seqs:
            s.alloc.truncate(seq, w.doc_len)
    torch.cuda.synchronize()
    return s, seqs, outs


def run_spec(w: synth.SpecDecode, steps: Optional[int] = None, kv_int8: bool = False):
    """Each step: reserve the drafts, store them, 5-query causal append, keep a
    prefix of the drafts via truncate."""
    s = Session.open(w, kv_int8=kv_int8)
    B = len(w.ctx_len)
    seqs = [s.alloc.seq_new() for _ in range(B)]
    items = []
    for b, seq in enumerate(seqs):
        lo, hi = int(w.ctx_offsets[b]), int(w.ctx_offsets[b + 1])
        s.alloc.reserve(seq, hi - lo)
        items.append((seq, 0, w.ctx_k[lo:hi], w.ctx_v[lo:hi]))
    s.store_many(items, w.dtype)
    outs = []
    n_steps = w.draft_q.shape[0] if steps is None else steps
    for st in range(n_steps):
        items = []
        for b, seq in enumerate(seqs):
            L = s.alloc.seq_len(seq)
            s.alloc.reserve(seq, w.drafts)
            items.append((seq, L, w.draft_k[st, b], w.draft_v[st, b]))
        s.store_many(items, w.dtype)
        q = w.draft_q[st].reshape(B * w.drafts, w.num_q_heads, w.head_dim)
        outs.append(s.append(seqs, [w.drafts] * B, dev_tensor(q, w.dtype)))
        for b, seq in enumerate(seqs):
            s.alloc.truncate(seq, s.alloc.seq_len(seq) - w.drafts + int(w.keep[st, b]))
    torch.cuda.synchronize()
    return s, seqs, outs
