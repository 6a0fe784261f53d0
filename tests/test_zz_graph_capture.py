"""Paged attention captured in a HIP graph.

pkv_decode (with a caller workspace), pkv_decode_noalloc (with the library's
static scratch, for callers that cannot allocate, such as code under graph
capture) and pkv_prefill_append enqueue kernel launches only: no allocation,
no memset, no host synchronisation.  Each is captured into a graph here and
replayed several times, with eager work between the replays (the output is
poisoned, the queries are replaced) and a synchronisation after each; every
replay must equal the eager call on the same inputs bit for bit.
"""

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _loaded():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_replays_in_a_graph(noalloc):
    from gpu_path import DEV, Session, dev_tensor, i32
    print(f"graph-captured decode, noalloc={noalloc}", flush=True)
    w = synth.decode_batch(n_seqs=16, len_lo=1, len_hi=1500, num_pages=2000, seed=11)
    s = Session.open(w)
    seqs = [s.alloc.seq_new() for _ in w.lengths]
    items = []
    for b, seq in enumerate(seqs):
        L, lo = int(w.lengths[b]), int(w.offsets[b])
        s.alloc.reserve(seq, L)
        items.append((seq, 0, w.k[lo:lo + L], w.v[lo:lo + L]))
    s.store_many(items, w.dtype)
    bt = i32(s.alloc.block_tables(seqs, max(s.alloc.num_blocks(x) for x in seqs)))
    lens = i32(np.array([s.alloc.seq_len(x) for x in seqs], np.int32))
    max_len = int(w.lengths.max())
    ws = torch.empty(max(16, pkv.workspace_bytes(s.desc, len(seqs), w.num_q_heads, 1, max_len)),
                     dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(12)
    queries = [dev_tensor(w.q, w.dtype)] + [
        dev_tensor(synth.normal_values(rng, w.q.shape, w.dtype), w.dtype) for _ in range(3)]

    def call(q, out):
        if noalloc:
            pkv.decode_noalloc(s.desc, s.k_pool, s.v_pool, q, bt, lens, max_len, s.scale, out)
        else:
            pkv.decode(s.desc, s.k_pool, s.v_pool, q, bt, lens, max_len, s.scale, out, ws)

    # eager results, one per query set
    expect = []
    for qs in queries:
        o = torch.empty_like(qs)
        call(qs, o)
        expect.append(o)
    torch.cuda.synchronize()

    q = queries[0].clone()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, out)                                 # warm-up on the capture's stream kind
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q, out)
    torch.cuda.synchronize()
    for r in range(8):
        k = r % len(queries)
        q.copy_(queries[k])                          # eager work between replays
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, expect[k]), f"replay {r} (query set {k}) differs from the eager call"


@pytest.mark.parametrize("ctx", [300, 2600])
def test_prefill_append_replays_in_a_graph(ctx):
    """The same for pkv_prefill_append, whose schedule kernel writes the
    work records the attention kernel reads within the one captured call: a
    50-query causal append over contexts within 2,048 positions (the
    persistent kernel) and beyond (the tiled kernel with KV splits)."""
    from gpu_path import DEV, Session, dev_tensor, i32
    print(f"graph-captured prefill_append, context {ctx}", flush=True)
    n_new, hq, hkv, D, ps = 50, 32, 8, 128, 16
    lens = [ctx, ctx // 2 + 60, 61]
    w = synth.decode_batch(n_seqs=len(lens), len_lo=1, len_hi=2, num_pages=sum(-(-L // ps) for L in lens) + 9,
                           num_q_heads=hq, num_kv_heads=hkv, head_dim=D, seed=13)
    s = Session.open(w)
    rng = np.random.default_rng(14)
    seqs = [s.alloc.seq_new() for _ in lens]
    items = []
    for seq, L in zip(seqs, lens):
        s.alloc.reserve(seq, L)
        kv = synth.normal_values(rng, (2, L, hkv, D), synth.BF16)
        items.append((seq, 0, kv[0], kv[1]))
    s.store_many(items, synth.BF16)
    n = [n_new] * len(lens)
    cu = i32(np.concatenate([[0], np.cumsum(n)]))
    bt = i32(s.alloc.block_tables(seqs, max(s.alloc.num_blocks(x) for x in seqs)))
    lens_d = i32(np.array(lens, np.int32))
    max_len = max(lens)
    ws = torch.empty(max(16, pkv.workspace_bytes(s.desc, len(seqs), hq, n_new, max_len)), dtype=torch.uint8,
                     device=DEV)
    queries = [dev_tensor(synth.normal_values(rng, (sum(n), hq, D), synth.BF16), synth.BF16) for _ in range(3)]

    def call(q, out):
        pkv.prefill_append(s.desc, s.k_pool, s.v_pool, q, cu, bt, lens_d, n_new, max_len, s.scale, out, ws)

    expect = []
    for qs in queries:
        o = torch.empty_like(qs)
        call(qs, o)
        expect.append(o)
    torch.cuda.synchronize()
    q = queries[0].clone()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q, out)
    torch.cuda.synchronize()
    for r in range(6):
        k = r % len(queries)
        q.copy_(queries[k])
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, expect[k]), f"replay {r} (query set {k}) differs from the eager call"
