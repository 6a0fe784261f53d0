"""Full-size parity: the four large workloads at their stated sizes, in the
launch configuration the benchmark times, on bf16 and INT8 pages, against
the fp64 oracle.

What is compared (bars as everywhere: 2e-2 max-abs and 1e-2 mean-abs for
bf16 K/V with fp32 accumulation; tables, slots and plans bit-exact):

* workload 2, the 64-sequence decode batch: every (sequence, query head)
  output row, 2,048 of 2,048;
* workload 4, KV rewind: every output row of both passes, 1,000 documents x
  50 queries x 32 heads each;
* workload 5, long-context speculative rollback: every step, sequence, draft
  and head, 16 x 8 x 5 x 64 rows;
* workload 3, the prefix-shared prefill: every output row on bf16 pages
  (about 7.1 M (query, head) rows, in 16 shards of documents); on INT8 pages
  every document and every query head at 20 query positions per document
  (the first four, the last four and three seeded runs of four), since the
  oracle's quantization of every trace doubles the cost of a full pass.

The oracle runs per (document or sequence) on a pool of host threads (NumPy
releases the GIL for its array work; BLAS is held to one thread per call).
Each test prints the number of rows it compared.
"""

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle_path as ref
import synth
from conftest import ensure_library
from gpu_path import DEV, host_f64, run_decode, run_prefix, run_rewind, run_spec
from oracle.attention import attend
from oracle.quant import dequantize, quantize

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def pmap(fn, items):
    """fn over items on WORKERS host threads, BLAS one thread per call."""
    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, items))


def check_close(out: np.ndarray, expect: np.ndarray, what: str):
    assert out.shape == expect.shape, what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - expect)
    assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"
    return err


def kv64(values, kv_int8):
    """K or V [..., D] as the attention sees it: the bf16 values, or on INT8
    pages the dequantized codes of each vector (quantized by the oracle)."""
    x = synth.to_f64(values, synth.BF16)
    return dequantize(*quantize(x)) if kv_int8 else x


def bf16_host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu")


def rows_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().double().numpy()


def report(what, n_rows, err, t0):
    print(f"{what}: {n_rows} rows compared, max abs err {err.max():.4g}, mean {err.mean():.3g}, "
          f"{time.perf_counter() - t0:.1f} s", flush=True)


# ---------------------------------------------------------------------------
# workload 2: the paged decode batch, every row
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def w2():
    return synth.decode_batch()


@pytest.mark.parametrize("kv_int8", [False, True], ids=["bf16", "int8"])
def test_full_decode_workload2_every_row(w2, kv_int8):
    print(f"full workload 2 ({'int8' if kv_int8 else 'bf16'})", flush=True)
    t0 = time.perf_counter()
    s, seqs, out = run_decode(w2, kv_int8=kv_int8)
    # slots and block tables: bit-exact against the oracle allocator run through the same operations
    oalloc, _ = ref.decode_allocator(w2)
    for seq, start, slots in s.log.get("slots", []):
        assert slots.tolist() == oalloc.slots(seq, start, len(slots)), "slots differ"
    for x in seqs:
        assert s.alloc.block_table(x).tolist() == oalloc.block_table(x)
    o = host_f64(out)
    B = len(w2.lengths)

    def one(b):
        lo, L = int(w2.offsets[b]), int(w2.lengths[b])
        q = synth.to_f64(w2.q[b:b + 1], synth.BF16)
        return attend(q, kv64(w2.k[lo:lo + L], kv_int8), kv64(w2.v[lo:lo + L], kv_int8), s.scale)[0]

    expect = np.stack(pmap(one, range(B)))
    err = check_close(o, expect, "full decode")
    report("workload 2", B * w2.num_q_heads, err, t0)


# ---------------------------------------------------------------------------
# workload 4: KV rewind, every row of both passes
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def w4():
    return synth.rewind_docs()


@pytest.mark.parametrize("kv_int8", [False, True], ids=["bf16", "int8"])
def test_full_rewind_workload4_every_row(w4, kv_int8):
    print(f"full workload 4 ({'int8' if kv_int8 else 'bf16'})", flush=True)
    t0 = time.perf_counter()
    s, seqs, outs = run_rewind(w4, kv_int8=kv_int8)
    n = w4.doc_k.shape[0]
    got = [bf16_host(o).view(n, w4.q_len, w4.num_q_heads, w4.head_dim) for o in outs]
    passes = ((w4.q1_q, w4.q1_k, w4.q1_v), (w4.q2_q, w4.q2_k, w4.q2_v))

    def one(args):
        p, d = args
        qq, qk, qv = passes[p]
        k = np.concatenate([kv64(w4.doc_k[d], kv_int8), kv64(qk[d], kv_int8)])
        v = np.concatenate([kv64(w4.doc_v[d], kv_int8), kv64(qv[d], kv_int8)])
        e = attend(synth.to_f64(qq[d], synth.BF16), k, v, s.scale)
        o = rows_f64(got[p][d])
        assert np.isfinite(o).all(), f"rewind pass {p + 1} doc {d}: non-finite output"
        err = np.abs(o - e)
        return err.max(), err.sum(), err.size

    res = pmap(one, [(p, d) for p in range(2) for d in range(n)])
    mx = max(r[0] for r in res)
    mean = sum(r[1] for r in res) / sum(r[2] for r in res)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"full rewind: max {mx:.3g} mean {mean:.3g}"
    report("workload 4", 2 * n * w4.q_len * w4.num_q_heads, np.array([mx, mean]), t0)


# ---------------------------------------------------------------------------
# workload 5: long-context decode with speculative rollback, every row
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def w5():
    return synth.spec_decode()


@pytest.fixture(scope="module")
def spec_outputs(w5):
    s, seqs, outs = run_spec(w5)
    return s.scale, [host_f64(o).reshape(len(w5.ctx_len), w5.drafts, w5.num_q_heads, w5.head_dim)
                     for o in outs]


def _spec_check(w5, scale, outs, b, kv_int8):
    """Every step of sequence b: its logical K/V are the context, the drafts
    kept by earlier steps, then this step's drafts (one fp64 buffer, written
    in place as the sequence grows and rolls back)."""
    lo, L0 = int(w5.ctx_offsets[b]), int(w5.ctx_len[b])
    steps = w5.draft_q.shape[0]
    cap = L0 + steps * w5.drafts
    K = np.empty((cap, w5.num_kv_heads, w5.head_dim))
    V = np.empty_like(K)
    K[:L0] = kv64(w5.ctx_k[lo:lo + L0], kv_int8)
    V[:L0] = kv64(w5.ctx_v[lo:lo + L0], kv_int8)
    kept = L0
    worst, total, count = 0.0, 0.0, 0
    for st in range(steps):
        K[kept:kept + w5.drafts] = kv64(w5.draft_k[st, b], kv_int8)
        V[kept:kept + w5.drafts] = kv64(w5.draft_v[st, b], kv_int8)
        e = attend(synth.to_f64(w5.draft_q[st, b], synth.BF16), K[:kept + w5.drafts], V[:kept + w5.drafts], scale)
        o = outs[st][b]
        assert np.isfinite(o).all(), f"spec step {st} seq {b}: non-finite output"
        err = np.abs(o - e)
        assert err.max() <= BF16_MAX, f"spec step {st} seq {b}: max abs err {err.max():.3g}"
        worst, total, count = max(worst, err.max()), total + err.sum(), count + err.size
        kept += int(w5.keep[st, b])
    return worst, total, count


@pytest.mark.parametrize("b", range(8))
def test_full_spec_workload5_every_row(w5, spec_outputs, b):
    print(f"full workload 5, sequence {b}", flush=True)
    t0 = time.perf_counter()
    scale, outs = spec_outputs
    worst, total, count = _spec_check(w5, scale, outs, b, kv_int8=False)
    assert total / count <= BF16_MEAN, f"spec seq {b}: mean abs err {total / count:.3g}"
    report(f"workload 5 sequence {b} (16 steps)", count // w5.head_dim, np.array([worst, total / count]), t0)


# ---------------------------------------------------------------------------
# workload 3: prefix-shared prefill
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def w3():
    return synth.prefix_traces()


def _check_plan(w3, s, order, parent, shared, seqs):
    o_order, o_parent, o_shared = ref.prefix_plan(w3)
    assert order.tolist() == o_order and shared.tolist() == o_shared
    assert [None if p < 0 else int(p) for p in parent] == o_parent
    assert shared[:3].tolist() == [0, 992, 1392]
    # adopted pages are the parent's own: the child's first shared/ps table entries
    ps = w3.page_size
    for d in range(len(seqs)):
        if parent[d] >= 0:
            nb = int(shared[d]) // ps
            assert (s.alloc.block_table(seqs[d])[:nb].tolist()
                    == s.alloc.block_table(seqs[int(parent[d])])[:nb].tolist())


@pytest.fixture(scope="module")
def prefix_bf16(w3):
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w3)
    _check_plan(w3, s, order, parent, shared, seqs)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    return s.scale, shared, cu, bf16_host(out)


SHARDS = 16


@pytest.mark.parametrize("shard", range(SHARDS))
def test_full_prefix_workload3_every_row(w3, prefix_bf16, shard):
    """Every output row of the documents d with d % 16 == shard, bf16 pages.
    The oracle runs per (document, KV head): attend() over that head's K/V
    with the query heads that map to it (h // (Hq / Hkv) == g), so the
    score blocks stay one head group wide."""
    print(f"full workload 3, shard {shard}", flush=True)
    t0 = time.perf_counter()
    scale, shared, cu, got = prefix_bf16
    grp = w3.num_q_heads // w3.num_kv_heads
    docs = [d for d in range(len(w3.row_len)) if d % SHARDS == shard]

    def one(job):
        d, g = job
        t, L, sh = int(w3.row_trace[d]), int(w3.row_len[d]), int(shared[d])
        heads = slice(g * grp, (g + 1) * grp)
        ex = attend(synth.to_f64(w3.q[t, sh:L, heads], synth.BF16), synth.to_f64(w3.k[t, :L, g:g + 1], synth.BF16),
                    synth.to_f64(w3.v[t, :L, g:g + 1], synth.BF16), scale)
        o = rows_f64(got[cu[d]:cu[d + 1], heads])
        assert np.isfinite(o).all(), f"prefix doc {d} head group {g}: non-finite output"
        err = np.abs(o - ex)
        return err.max(), err.sum(), err.size

    res = pmap(one, [(d, g) for d in docs for g in range(w3.num_kv_heads)])
    mx = max(r[0] for r in res)
    mean = sum(r[1] for r in res) / sum(r[2] for r in res)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"full prefix shard {shard}: max {mx:.3g} mean {mean:.3g}"
    n_rows = sum(r[2] for r in res) // w3.head_dim
    assert n_rows == sum(int(cu[d + 1] - cu[d]) for d in docs) * w3.num_q_heads
    report(f"workload 3 shard {shard} ({len(docs)} documents, every row)", n_rows, np.array([mx, mean]), t0)


RUN = 4   # query positions per run


def _prefix_runs(n_new: int, rng) -> list:
    """(first, end) index ranges among a document's new queries: the first
    RUN, the last RUN and three seeded runs (each clipped to the suffix)."""
    runs = {(0, min(RUN, n_new)), (max(0, n_new - RUN), n_new)}
    for _ in range(3):
        a = int(rng.integers(0, max(1, n_new - RUN + 1)))
        runs.add((a, min(n_new, a + RUN)))
    return sorted(runs)


def test_full_prefix_workload3_int8_every_document(w3):
    """INT8 pages: every document and every query head, at 20 query positions
    per document (the first four, the last four and three seeded runs of
    four), against the oracle over the dequantized values."""
    print("full workload 3 (int8)", flush=True)
    t0 = time.perf_counter()
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w3, kv_int8=True)
    _check_plan(w3, s, order, parent, shared, seqs)
    got = bf16_host(out)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    rng = np.random.default_rng(11)
    jobs = [(d, a, e) for d in range(len(seqs)) for a, e in _prefix_runs(int(n_new[d]), rng)]

    def one(job):
        d, a, e = job
        t, sh = int(w3.row_trace[d]), int(shared[d])
        end = sh + e                            # the run's queries are the last e - a of positions < end
        ex = attend(synth.to_f64(w3.q[t, sh + a:end], synth.BF16), kv64(w3.k[t, :end], True),
                    kv64(w3.v[t, :end], True), s.scale)
        o = rows_f64(got[cu[d] + a:cu[d] + e])
        assert np.isfinite(o).all(), f"prefix doc {d} rows {a}..{e}: non-finite output"
        err = np.abs(o - ex)
        return err.max(), err.sum(), err.size

    res = pmap(one, jobs)
    mx = max(r[0] for r in res)
    mean = sum(r[1] for r in res) / sum(r[2] for r in res)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"full prefix int8: max {mx:.3g} mean {mean:.3g}"
    n_rows = sum(r[2] for r in res) // w3.head_dim
    assert len({d for d, _, _ in jobs}) == len(seqs)
    report(f"workload 3 int8 ({len(jobs)} runs over all {len(seqs)} documents)", n_rows, np.array([mx, mean]), t0)
