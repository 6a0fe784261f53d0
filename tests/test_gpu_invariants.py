"""Invariants of the paged method, checked bit for bit on the HIP path.

Where a sequence's K/V sits changes nothing: attention reads the blocks in
place and means the same as over the request's whole valid context ("KV Cache
Management and PagedAttention", "Compute attention over scattered KV").  A
document adopts its parent's pages for the shared prefix instead of computing
them again (Quail docs, "KV", "Execution"), and truncating touches no data,
stale slots being overwritten later (TileInfer.jl docs, "KV cache", "Growing,
rolling back, releasing").  The kernels split work at fixed logical positions,
so the same logical sequences in the same launch shape must give the same bits
whatever the page placement:

* a prefill under two different physical page orders;
* a prefix-shared prefill against the same prefill where every row holds its
  whole sequence in pages of its own;
* a rewind's second question (appended after truncating the first) against the
  same question appended to fresh copies of the documents;
* speculative steps after rollbacks against fresh sequences holding the kept
  tokens.

Each pair of runs issues identical calls apart from the block tables, so any
difference comes from reading a wrong or stale page.
"""

import numpy as np
import pytest
import torch

import synth
from conftest import ensure_library
from gpu_path import Session, dev_tensor, run_prefix, run_rewind, run_spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy()


class _Pools:
    def __init__(self, D, ps, hkv, num_pages, free_order):
        self.dtype, self.head_dim, self.page_size = synth.BF16, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = free_order


@pytest.mark.parametrize("kv_int8", [False, True])
@pytest.mark.parametrize("ctx,news", [
    ([300, 0, 1000], [200, 64, 150]),        # the persistent kernel
    ([2100, 0, 700], [200, 2300, 1]),        # the tiled kernel, KV splits
])
def test_prefill_page_permutation_bit_exact(kv_int8, ctx, news):
    print(f"invariant: prefill page permutation int8={kv_int8} ctx={ctx} new={news}", flush=True)
    D, ps, hq, hkv = 128, 16, 32, 8
    rng = np.random.default_rng(31)
    lens = [c + n for c, n in zip(ctx, news)]
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    q = synth.normal_values(rng, (sum(news), hq, D), synth.BF16)
    pages = 2 * sum(-(-L // ps) for L in lens)
    outs, tables = [], []
    for seed in (1, 2):
        order = np.random.default_rng(seed).permutation(pages).astype(np.int32)
        s = Session.open(_Pools(D, ps, hkv, pages, order), kv_int8=kv_int8)
        seqs = [s.alloc.seq_new() for _ in lens]
        for b, seq in enumerate(seqs):
            s.alloc.reserve(seq, lens[b])
        s.store_many([(seq, 0, kv[b][0], kv[b][1]) for b, seq in enumerate(seqs)], synth.BF16)
        outs.append(_bits(s.append(seqs, news, dev_tensor(q, synth.BF16))))
        tables.append(s.log["tables"][-1])
    assert not np.array_equal(tables[0], tables[1]), "the two runs place the pages differently"
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("shape", ["short", "long"])
def test_prefix_adoption_equals_recomputation_bit_exact(shape):
    """Rows that adopt their parent's pages give the bits of rows that store
    their whole sequence themselves."""
    print(f"invariant: prefix adoption ({shape} contexts)", flush=True)
    if shape == "short":
        w = synth.prefix_traces(n_rows=20, n_traces=5, first_rows=(100, 140, 190), len_lo=100,
                                len_hi=600, trace_len=600, num_pages=1200)
    else:
        w = synth.prefix_traces(n_rows=10, n_traces=3, first_rows=(1000, 1400, 1900), len_lo=1000,
                                len_hi=3000, trace_len=3000, num_pages=4000)
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w)
    assert (shared > 0).sum() >= 3, "the plan shares pages"
    got = _bits(out)
    # every row stores its whole sequence in pages of its own
    f = Session.open(w)
    n = len(w.row_len)
    fresh = []
    for d in range(n):
        seq = f.alloc.seq_new()
        L, t = int(w.row_len[d]), int(w.row_trace[d])
        f.alloc.reserve(seq, L)
        fresh.append((seq, L, t))
    f.store_many([(seq, 0, w.k[t, :L], w.v[t, :L]) for seq, L, t in fresh], w.dtype)
    q = np.concatenate([w.q[int(w.row_trace[d]), int(shared[d]):int(w.row_len[d])] for d in range(n)])
    out_f = f.append([x[0] for x in fresh], n_new, dev_tensor(q, w.dtype))
    assert np.array_equal(got, _bits(out_f))


def test_rewind_second_question_equals_fresh_append_bit_exact():
    """Question 2, appended after question 1 was truncated away, gives the
    bits of question 2 appended to fresh copies of the documents."""
    print("invariant: rewind", flush=True)
    w = synth.rewind_docs(n_docs=40, num_pages=40 * 22 + 10)
    s, seqs, outs = run_rewind(w)
    n = w.doc_k.shape[0]
    f = Session.open(w, free_order=np.random.default_rng(9).permutation(w.num_pages).astype(np.int32))
    fseqs = [f.alloc.seq_new() for _ in range(n)]
    for seq in fseqs:
        f.alloc.reserve(seq, w.doc_len + w.q_len)
    f.store_many([(seq, 0, np.concatenate([w.doc_k[d], w.q2_k[d]]), np.concatenate([w.doc_v[d], w.q2_v[d]]))
                  for d, seq in enumerate(fseqs)], w.dtype)
    q = w.q2_q.reshape(n * w.q_len, w.num_q_heads, w.head_dim)
    out_f = f.append(fseqs, [w.q_len] * n, dev_tensor(q, w.dtype))
    assert np.array_equal(_bits(outs[1]), _bits(out_f))


def test_rollback_equals_fresh_sequences_bit_exact():
    """Each speculative step after rollbacks gives the bits of fresh sequences
    that hold exactly the kept tokens and the step's drafts."""
    print("invariant: speculative rollback", flush=True)
    steps = 4
    w = synth.spec_decode(n_seqs=3, len_lo=2000, len_hi=6000, steps=steps)
    s, seqs, outs = run_spec(w, steps=steps)
    B = len(w.ctx_len)
    # the kept tokens of each sequence before step st: its context, then for
    # every earlier step the first keep[st'] drafts
    for st in range(steps):
        ks, vs = [], []
        for b in range(B):
            lo, hi = int(w.ctx_offsets[b]), int(w.ctx_offsets[b + 1])
            kk, vv = [w.ctx_k[lo:hi]], [w.ctx_v[lo:hi]]
            for p in range(st):
                kk.append(w.draft_k[p, b, :int(w.keep[p, b])])
                vv.append(w.draft_v[p, b, :int(w.keep[p, b])])
            kk.append(w.draft_k[st, b])
            vv.append(w.draft_v[st, b])
            ks.append(np.concatenate(kk))
            vs.append(np.concatenate(vv))
        f = Session.open(w, free_order=np.random.default_rng(40 + st).permutation(w.num_pages).astype(np.int32))
        fseqs = [f.alloc.seq_new() for _ in range(B)]
        for b, seq in enumerate(fseqs):
            f.alloc.reserve(seq, ks[b].shape[0])
        f.store_many([(seq, 0, ks[b], vs[b]) for b, seq in enumerate(fseqs)], w.dtype)
        q = w.draft_q[st].reshape(B * w.drafts, w.num_q_heads, w.head_dim)
        out_f = f.append(fseqs, [w.drafts] * B, dev_tensor(q, w.dtype))
        assert np.array_equal(_bits(outs[st]), _bits(out_f)), f"step {st}"
