"""GPU parity: libpkv's HIP path against the fp64 oracle on the same inputs.

Bars: block tables, slots, plans and the stored pool contents are bit-exact;
attention is within 1e-5 max-abs of the oracle for fp32 and within 2e-2
max-abs and 1e-2 mean-abs for bf16 K/V with fp32 accumulation.  Pools start
NaN-filled, so any read of a slot that was never written (or of another
sequence's page) would turn an output into NaN.

Small cases run the oracle on every output.  The full-size workloads (at
their stated sizes, in the launch configuration the benchmark times) are in
test_gpu_full.py.
"""

import math

import numpy as np
import pytest
import torch

import oracle_path as ref
import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library
from gpu_path import (DEV, Session, dev_tensor, host_f64, i32, i64, run_decode, run_prefix,
                      run_rewind, run_spec, run_tiny)
from oracle.attention import attend, attend_row, paged_attention
from oracle.paging import Allocator as OracleAllocator
from oracle.paging import store_rows
from oracle.quant import dequantize, quantize

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def check_close(out: np.ndarray, expect: np.ndarray, dtype: str, what: str):
    assert out.shape == expect.shape, what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - expect)
    if dtype == synth.F32:
        assert err.max() <= F32_TOL, f"{what}: max abs err {err.max():.3g}"
    else:
        assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"


def check_slots_and_tables(session: Session, oalloc: OracleAllocator, seqs):
    for seq, start, slots in session.log.get("slots", []):
        assert slots.tolist() == oalloc.slots(seq, start, len(slots)), "slots differ"
    for s in seqs:
        assert session.alloc.block_table(s).tolist() == oalloc.block_table(s)


# ---------------------------------------------------------------------------
# store_kv
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,ps,hkv", [(synth.BF16, 128, 16, 8), (synth.F32, 64, 3, 2),
                                            (synth.BF16, 64, 1, 1), (synth.F32, 128, 64, 4)])
def test_store_kv_bit_exact(dtype, D, ps, hkv):
    print(f"store_kv dtype={dtype} D={D} ps={ps} hkv={hkv}", flush=True)
    rng = np.random.default_rng(7)
    num_pages = 37
    T = 50
    slots = rng.permutation(num_pages * ps)[:T].astype(np.int64)
    slots[3] = -1                              # padding token: skipped
    slots[7] = num_pages * ps                  # out of range: skipped
    kv = synth.normal_values(rng, (2, T, hkv, D), dtype)
    desc = pkv.PoolDesc(pkv.PKV_BF16 if dtype == synth.BF16 else pkv.PKV_F32, num_pages, ps, hkv, D)
    kp = torch.zeros(desc.pool_shape, dtype=desc.torch_dtype(), device=DEV)
    vp = torch.zeros_like(kp)
    pkv.store_kv(desc, kp, vp, dev_tensor(kv[0], dtype), dev_tensor(kv[1], dtype), i64(slots))
    torch.cuda.synchronize()
    for pool, vals in ((kp, kv[0]), (vp, kv[1])):
        expect = np.zeros(desc.pool_shape)
        store_rows(expect, slots, synth.to_f64(vals, dtype))
        assert np.array_equal(host_f64(pool), expect)


# ---------------------------------------------------------------------------
# workload 1: tiny fp32 (page_size 4, 6 pages, lengths 7 and 6)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("free_order", [None, [3, 0, 1, 4, 5, 2]])
def test_tiny_fp32(free_order):
    print(f"tiny fp32 free_order={free_order}", flush=True)
    w = synth.tiny_batch(free_order=free_order)
    s, seqs, prefill, dec = run_tiny(w)
    tables, slots, ref_prefill, ref_dec = ref.tiny_reference(w, s.scale)
    assert [s.alloc.block_table(q).tolist() for q in seqs] == tables
    assert [x[2].tolist() for x in s.log["slots"]] == slots
    if free_order is not None:
        assert tables == [[3, 0], [1, 4]]      # the blog's Figure 2 mapping
    check_close(host_f64(prefill), ref_prefill, w.dtype, "tiny prefill")
    check_close(host_f64(dec), ref_dec, w.dtype, "tiny decode")
    # first query of each sequence sees only position 0: output = v_0 exactly
    p = host_f64(prefill)
    for b in range(2):
        lo = int(w.offsets[b])
        for h in range(w.num_q_heads):
            assert np.array_equal(p[lo, h], synth.to_f64(w.v[lo, 0], w.dtype))
    # 13 of 16 slots filled; the 3 empty slots are untouched NaN
    kp = host_f64(s.k_pool)
    assert np.isnan(kp).sum() == (6 * 4 - 13) * 64


# ---------------------------------------------------------------------------
# workload 2 shape: paged decode
# ---------------------------------------------------------------------------
def _decode_full_check(w, s, seqs, out):
    oalloc, oseqs = ref.decode_allocator(w)
    assert oseqs == seqs
    check_slots_and_tables(s, oalloc, seqs)
    expect = ref.decode_reference(w, s.scale)
    o = host_f64(out)
    e = np.stack([np.stack([expect[(b, h)] for h in range(w.num_q_heads)])
                  for b in range(len(seqs))])
    check_close(o, e, w.dtype, "decode")


@pytest.mark.parametrize("n_seqs,len_lo,len_hi", [(24, 1, 1500), (64, 1, 200), (3, 4000, 9000)])
def test_decode_bf16(n_seqs, len_lo, len_hi):
    print(f"decode bf16 B={n_seqs} L=[{len_lo},{len_hi}]", flush=True)
    total_pages = n_seqs * (-(-len_hi // 16)) + 64
    w = synth.decode_batch(n_seqs=n_seqs, len_lo=len_lo, len_hi=len_hi, num_pages=total_pages,
                           seed=n_seqs)
    s, seqs, out = run_decode(w)
    _decode_full_check(w, s, seqs, out)


@pytest.mark.parametrize("kv_int8", [False, True])
def test_decode_many_sequences(kv_int8):
    """300 sequences: each wave scans the block counts in five 64-sequence
    chunks, and ranges start in every chunk."""
    print(f"decode 300 sequences int8={kv_int8}", flush=True)
    w = synth.decode_batch(n_seqs=300, len_lo=1, len_hi=400, num_pages=300 * 25 + 64, seed=300)
    s, seqs, out = run_decode(w, kv_int8=kv_int8)
    if kv_int8:
        expect = ref.decode_reference(w, s.scale, kv_int8=True)
        o = host_f64(out)
        e = np.stack([np.stack([expect[(b, h)] for h in range(w.num_q_heads)]) for b in range(len(seqs))])
        check_close(o, e, w.dtype, "int8 decode, 300 sequences")
    else:
        _decode_full_check(w, s, seqs, out)


def test_short_append_many_sequences():
    """Prefill/append with at most 3 new queries per sequence (the decode
    kernel family) over 200 sequences, some with none, including those on
    64-sequence chunk boundaries."""
    rng = np.random.default_rng(200)
    n = 200
    hq, hkv, D = 32, 8, 128
    n_new = rng.integers(0, 4, size=n)
    for b in (0, 63, 64, 127, 128, 199):
        n_new[b] = 0
    n_new[1] = 3
    lens = [int(x) for x in rng.integers(1, 300, size=n) + n_new]
    pages = sum(-(-L // 16) for L in lens) + 8
    s = Session.open(_Pools(synth.BF16, D, 16, hkv, pages, seed=7))
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
        s.store(seq, 0, kv[b][0], kv[b][1], synth.BF16)
    qs = [synth.normal_values(rng, (int(k), hq, D), synth.BF16) for k in n_new]
    out = host_f64(s.append(seqs, [int(k) for k in n_new], dev_tensor(np.concatenate(qs), synth.BF16)))
    row = 0
    for b in range(n):
        if n_new[b]:
            e = attend(synth.to_f64(qs[b], synth.BF16), synth.to_f64(kv[b][0], synth.BF16),
                       synth.to_f64(kv[b][1], synth.BF16), s.scale)
            check_close(out[row:row + n_new[b]], e, synth.BF16, f"short append seq {b}")
        row += int(n_new[b])


def test_decode_gather_form_equals_logical():
    """A host copy of the device pools, read through the oracle's block tables,
    reproduces the logical K/V bit for bit (store_kv + slots placed every row)."""
    w = synth.decode_batch(n_seqs=6, len_lo=1, len_hi=90, num_pages=160, page_size=4,
                           num_q_heads=4, num_kv_heads=2, head_dim=64, dtype=synth.F32)
    s, seqs, out = run_decode(w)
    oalloc, _ = ref.decode_allocator(w)
    kp, vp = host_f64(s.k_pool), host_f64(s.v_pool)
    tables = [oalloc.block_table(q) for q in seqs]
    cu = np.arange(len(seqs) + 1)
    gathered = paged_attention(synth.to_f64(w.q, w.dtype), cu, w.lengths, tables, kp, vp, s.scale)
    logical = np.stack([attend(synth.to_f64(w.q[b:b + 1], w.dtype),
                               synth.to_f64(w.k[w.offsets[b]:w.offsets[b + 1]], w.dtype),
                               synth.to_f64(w.v[w.offsets[b]:w.offsets[b + 1]], w.dtype), s.scale)[0]
                        for b in range(len(seqs))])
    assert np.array_equal(gathered, logical)
    check_close(host_f64(out), logical, w.dtype, "decode fp32")


@pytest.mark.parametrize("dtype,D,ps,hq,hkv,len_hi", [
    (synth.F32, 128, 16, 8, 2, 700),
    (synth.F32, 64, 1, 4, 4, 300),
    (synth.BF16, 64, 4, 16, 1, 900),
    (synth.BF16, 128, 3, 8, 8, 500),
    (synth.BF16, 128, 256, 16, 1, 2000),
    (synth.BF16, 128, 64, 64, 8, 5000),
])
def test_decode_variants(dtype, D, ps, hq, hkv, len_hi):
    print(f"decode variant {dtype} D={D} ps={ps} hq={hq} hkv={hkv}", flush=True)
    n = 9
    w = synth.decode_batch(n_seqs=n, len_lo=1, len_hi=len_hi, page_size=ps,
                           num_pages=n * (-(-len_hi // ps)) + 5, num_q_heads=hq,
                           num_kv_heads=hkv, head_dim=D, dtype=dtype, seed=D + ps)
    s, seqs, out = run_decode(w)
    _decode_full_check(w, s, seqs, out)


def test_decode_page_permutation_bit_exact():
    w = synth.decode_batch(n_seqs=16, len_lo=1, len_hi=1200, num_pages=2000, seed=3)
    outs = []
    for k in range(3):
        order = np.random.default_rng(100 + k).permutation(w.num_pages).astype(np.int32)
        _, _, out = run_decode(w, free_order=order)
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_decode_edge_cases():
    # empty batch is a no-op; a one-position sequence returns its value exactly
    w = synth.decode_batch(n_seqs=2, len_lo=1, len_hi=1, num_pages=4, seed=1)
    s, seqs, out = run_decode(w)
    o = host_f64(out)
    for b in range(2):
        for h in range(w.num_q_heads):
            assert np.array_equal(o[b, h], synth.to_f64(w.v[b, h // 4], w.dtype))
    q = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device=DEV)
    empty = torch.zeros((0, 1), dtype=torch.int32, device=DEV)
    pkv.decode(s.desc, s.k_pool, s.v_pool, q, empty, torch.zeros(0, dtype=torch.int32, device=DEV),
               0, 0.1, torch.empty_like(q))
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# workload 3 shape: prefix-shared prefill
# ---------------------------------------------------------------------------
def test_prefix_shared_prefill_reduced():
    print("prefix reduced", flush=True)
    w = synth.prefix_traces(n_rows=20, n_traces=5, first_rows=(100, 140, 190), len_lo=100,
                            len_hi=600, trace_len=600, num_pages=1200)
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w)
    o_order, o_parent, o_shared = ref.prefix_plan(w)
    assert order.tolist() == o_order
    assert [None if p < 0 else int(p) for p in parent] == o_parent
    assert shared.tolist() == o_shared
    assert shared[:3].tolist() == [0, 96, 128]
    check_close(host_f64(out), ref.prefix_reference_full(w, o_shared, s.scale), w.dtype, "prefix")
    # pages were adopted, not copied: child's first pages are its parent's
    for d in range(len(seqs)):
        if parent[d] >= 0:
            npg = shared[d] // w.page_size
            assert (s.alloc.block_table(seqs[d])[:npg] ==
                    s.alloc.block_table(seqs[parent[d]])[:npg]).all()


def test_prefix_paper_rows():
    """The three rows of the sharing-plan example (1,000 / 1,400 / 1,900 tokens)."""
    w = synth.prefix_traces(n_rows=3, n_traces=2, trace_len=1900, len_hi=1900, num_pages=400,
                            num_q_heads=8, num_kv_heads=2)
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w)
    assert shared.tolist() == [0, 992, 1392] and parent.tolist() == [-1, 0, 1]
    assert sum(n_new) == 1916
    check_close(host_f64(out), ref.prefix_reference_full(w, shared.tolist(), s.scale), w.dtype,
                "prefix paper rows")


# ---------------------------------------------------------------------------
# workload 4 shape: KV rewind
# ---------------------------------------------------------------------------
def test_rewind_reduced():
    print("rewind reduced", flush=True)
    w = synth.rewind_docs(n_docs=24, num_pages=24 * 22 + 10)
    s, seqs, outs = run_rewind(w)
    expect = ref.rewind_reference(w, s.scale)
    for p in range(2):
        o = host_f64(outs[p]).reshape(24, w.q_len, w.num_q_heads, w.head_dim)
        e = np.stack([expect[p][d] for d in range(24)])
        check_close(o, e, w.dtype, f"rewind pass {p + 1}")


def test_truncated_slots_are_never_read():
    """After truncate, the dropped positions' slots hold stale data; poison them
    with NaN and decode the kept sequence: the output stays finite and exact."""
    w = synth.decode_batch(n_seqs=4, len_lo=40, len_hi=60, num_pages=40, page_size=16, seed=5)
    s, seqs, _ = run_decode(w)
    stale = []
    for b, seq in enumerate(seqs):
        L = s.alloc.seq_len(seq)
        stale.append(s.alloc.slots(seq, L - 7, 7))
        s.alloc.truncate(seq, L - 7)
    st = np.concatenate(stale)
    nan_rows = torch.full((len(st), w.num_kv_heads, w.head_dim), float("nan"),
                          dtype=torch.bfloat16, device=DEV)
    pkv.store_kv(s.desc, s.k_pool, s.v_pool, nan_rows, nan_rows, i64(st))
    q = dev_tensor(w.q, w.dtype)
    out = host_f64(s.decode(seqs, q))
    for b in range(4):
        L = int(w.lengths[b]) - 7
        lo = int(w.offsets[b])
        for h in range(w.num_q_heads):
            e = attend_row(synth.to_f64(w.q[b, h], w.dtype), synth.to_f64(w.k[lo:lo + L, h // 4], w.dtype),
                           synth.to_f64(w.v[lo:lo + L, h // 4], w.dtype), L - 1, s.scale)
            assert np.isfinite(out[b, h]).all()
            assert np.abs(out[b, h] - e).max() <= BF16_MAX


@pytest.mark.parametrize("dtype,kv_int8,D", [(synth.F32, False, 64), (synth.BF16, False, 128),
                                         (synth.BF16, True, 128)])
def test_positions_past_the_table_row_are_not_read(dtype, kv_int8, D):
    """seq_lens entries past bt_stride * page_size, or past max_seq_len, read
    only the positions the row and the bound cover.  The table buffer runs on
    past the last row into entries naming never-written (NaN) pages, and rows
    sit back to back, so a read past a row would show as a NaN or as another
    sequence's keys."""
    print(f"positions past the row {dtype} int8={kv_int8} D={D}", flush=True)
    rng = np.random.default_rng(D + 5 * kv_int8)
    ps, stride, n, hq, hkv = 4, 5, 3, 16, 2
    cap = ps * stride
    pools = _Pools(dtype, D, ps, hkv, n * stride + 4, seed=9)
    s = Session.open(pools, kv_int8=kv_int8)
    seqs = [s.alloc.seq_new() for _ in range(n)]
    kv = synth.normal_values(rng, (n, 2, cap, hkv, D), dtype)
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, cap)
        s.store(seq, 0, kv[b, 0], kv[b, 1], dtype)
    bt = s.alloc.block_tables(seqs, stride)
    unused = sorted(set(range(pools.num_pages)) - set(bt.ravel().tolist()))
    buf = i32(np.concatenate([bt.ravel(), np.resize(np.array(unused, np.int32), 64)]))
    d_bt = buf[: n * stride].view(n, stride)

    def logical(b, n_pos):
        k = synth.to_f64(kv[b, 0, :n_pos], dtype)
        v = synth.to_f64(kv[b, 1, :n_pos], dtype)
        if kv_int8:
            k, v = dequantize(*quantize(k)), dequantize(*quantize(v))
        return k, v

    def run_decode_call(lens, max_len):
        q = synth.normal_values(rng, (n, hq, D), dtype)
        out = torch.empty((n, hq, D), dtype=s.desc.torch_dtype(), device=DEV)
        ws = torch.empty(max(16, pkv.workspace_bytes(s.desc, n, hq, 1, max_len)), dtype=torch.uint8, device=DEV)
        pkv.decode(s.desc, s.k_pool, s.v_pool, dev_tensor(q, dtype), d_bt, i32(lens), max_len, s.scale, out, ws)
        return q, host_f64(out)

    # past the row: every query sees the row's cap positions
    lens = np.array([cap + 7, cap + 100, cap], np.int32)
    q, o = run_decode_call(lens, int(lens.max()))
    for b in range(n):
        k, v = logical(b, cap)
        check_close(o[b:b + 1], attend(synth.to_f64(q[b:b + 1], dtype), k, v, s.scale), dtype, f"decode row {b}")
    # past max_seq_len: the first 13 positions only
    q, o = run_decode_call(np.full(n, cap, np.int32), 13)
    for b in range(n):
        k, v = logical(b, 13)
        check_close(o[b:b + 1], attend(synth.to_f64(q[b:b + 1], dtype), k, v, s.scale), dtype, f"bounded row {b}")
    # append: 8, 7 and 2 queries (64 rows per KV head: the multi-query tiles)
    n_new = np.array([8, 7, 2], np.int32)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    q = synth.normal_values(rng, (int(cu[-1]), hq, D), dtype)
    out = torch.empty((int(cu[-1]), hq, D), dtype=s.desc.torch_dtype(), device=DEV)
    max_len = int(lens.max())
    ws = torch.empty(max(16, pkv.workspace_bytes(s.desc, n, hq, 8, max_len)), dtype=torch.uint8, device=DEV)
    pkv.prefill_append(s.desc, s.k_pool, s.v_pool, dev_tensor(q, dtype), i32(cu), d_bt, i32(lens), 8, max_len,
                       s.scale, out, ws)
    o = host_f64(out)
    for b in range(n):
        qb = synth.to_f64(q[cu[b]:cu[b + 1]], dtype)
        e = []
        for i in range(n_new[b]):        # query i at position lens - n_new + i sees at most cap positions
            k, v = logical(b, min(int(lens[b] - n_new[b]) + i + 1, cap))
            e.append(attend(qb[i:i + 1], k, v, s.scale))
        check_close(o[cu[b]:cu[b + 1]], np.concatenate(e), dtype, f"append row {b}")


# ---------------------------------------------------------------------------
# workload 5 shape: long decode + speculative rollback
# ---------------------------------------------------------------------------
def test_spec_rollback_reduced():
    print("spec reduced", flush=True)
    w = synth.spec_decode(n_seqs=3, len_lo=2000, len_hi=6000, steps=4)
    s, seqs, outs = run_spec(w)
    expect = ref.spec_reference(w, s.scale, 4)
    for st in range(4):
        o = host_f64(outs[st]).reshape(3, w.drafts, w.num_q_heads, w.head_dim)
        check_close(o, np.stack([expect[st][b] for b in range(3)]), w.dtype, f"spec step {st}")


def test_prefill_mixed_query_counts():
    """Sequences with 0, 1, 17 and 300 new queries in one launch."""
    rng = np.random.default_rng(3)
    lens = [50, 1, 40, 700]
    n_new = [0, 1, 17, 300]
    hq, hkv, D = 32, 8, 128
    w = synth.decode_batch(n_seqs=4, num_pages=200, num_q_heads=hq, seed=11)
    s = Session.open(w)
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
        s.store(seq, 0, kv[b][0], kv[b][1], synth.BF16)
    qs = [synth.normal_values(rng, (n, hq, D), synth.BF16) for n in n_new]
    out = host_f64(s.append(seqs, n_new, dev_tensor(np.concatenate(qs), synth.BF16)))
    row = 0
    for b in range(4):
        if n_new[b]:
            e = attend(synth.to_f64(qs[b], synth.BF16), synth.to_f64(kv[b][0], synth.BF16),
                       synth.to_f64(kv[b][1], synth.BF16), s.scale)
            check_close(out[row:row + n_new[b]], e, synth.BF16, f"mixed seq {b}")
        row += n_new[b]


class _Pools:
    """Minimal pool description for hand-built prefill cases."""

    def __init__(self, dtype, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = dtype, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


@pytest.mark.parametrize("ps,n_seqs", [(16, 120), (4, 40), (2, 40), (3, 40)])
def test_persistent_prefill_item_mix(ps, n_seqs):
    """Short appends over short contexts in one launch: sequences with 0..200
    cached positions and 13..140 new queries (bf16, D 128, 32 q / 8 KV
    heads), so the persistent kernel walks many work items per workgroup of
    1..6 tiles and 1..3 row tiles each.  With page sizes 16 and 4 its K/V
    tiles go through a ring of three LDS buffers that runs on across item
    boundaries, and an item of one tile takes the next item's queries in the
    same iteration; page sizes 2 and 3 take the register-staged tiles with
    per-lane page lookups.  Every output row is checked against the oracle."""
    print(f"persistent item mix: page size {ps}, {n_seqs} sequences", flush=True)
    rng = np.random.default_rng(2024 + ps)
    hq, hkv, D = 32, 8, 128
    ctx = rng.integers(0, 201, n_seqs)
    ctx[:4] = [0, 1, 63, 64]
    news = rng.integers(13, 141, n_seqs)
    news[:4] = [13, 50, 64, 140]
    lens = [int(c + n) for c, n in zip(ctx, news)]
    pages = sum(-(-L // ps) for L in lens) + 5
    s = Session.open(_Pools(synth.BF16, D, ps, hkv, pages, seed=77 + ps))
    seqs = [s.alloc.seq_new() for _ in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    s.store_many([(seq, 0, kv[b][0], kv[b][1]) for b, seq in enumerate(seqs)], synth.BF16)
    qs = [synth.normal_values(rng, (int(n), hq, D), synth.BF16) for n in news]
    out = host_f64(s.append(seqs, [int(n) for n in news], dev_tensor(np.concatenate(qs), synth.BF16)))
    row = 0
    for b in range(n_seqs):
        e = attend(synth.to_f64(qs[b], synth.BF16), synth.to_f64(kv[b][0], synth.BF16),
                   synth.to_f64(kv[b][1], synth.BF16), s.scale)
        check_close(out[row:row + int(news[b])], e, synth.BF16, f"item mix seq {b} (ctx {ctx[b]}, new {news[b]})")
        row += int(news[b])


def test_persistent_prefill_schedule_passes():
    """1,100 sequences of 8 KV heads: 1,100 blocks of 8 units, so the
    schedule kernel takes two passes of 1,024 blocks (the row offsets carry
    from one pass to the next in each of its workgroups, which store the
    records of every 16th block), and the persistent kernel runs over the
    records of both passes; every output row is checked against the
    oracle."""
    rng = np.random.default_rng(1100)
    n_seqs, hq, hkv, D, ps = 1100, 32, 8, 128, 16
    ctx = rng.integers(0, 61, n_seqs)
    news = rng.integers(13, 21, n_seqs)
    lens = [int(c + n) for c, n in zip(ctx, news)]
    pages = sum(-(-L // ps) for L in lens) + 5
    s = Session.open(_Pools(synth.BF16, D, ps, hkv, pages, seed=1100))
    seqs = [s.alloc.seq_new() for _ in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    s.store_many([(seq, 0, kv[b][0], kv[b][1]) for b, seq in enumerate(seqs)], synth.BF16)
    qs = [synth.normal_values(rng, (int(n), hq, D), synth.BF16) for n in news]
    print(f"schedule passes: {n_seqs} sequences, {int(news.sum())} queries", flush=True)
    out = host_f64(s.append(seqs, [int(n) for n in news], dev_tensor(np.concatenate(qs), synth.BF16)))
    row = 0
    for b in range(n_seqs):
        e = attend(synth.to_f64(qs[b], synth.BF16), synth.to_f64(kv[b][0], synth.BF16),
                   synth.to_f64(kv[b][1], synth.BF16), s.scale)
        check_close(out[row:row + int(news[b])], e, synth.BF16, f"schedule passes seq {b}")
        row += int(news[b])


@pytest.mark.parametrize("D,ps,hq,hkv,ctx,news", [
    (128, 16, 32, 8, [2100, 0, 3000], [200, 2300, 1]),     # every wave row count, one sequence all-new
    (128, 64, 8, 8, [5000, 2040], [17, 63]),               # group 1: rows 17 and 63 of one tile
    (128, 256, 16, 2, [9000], [65]),                       # a long split context, group 8
    (128, 32, 32, 4, [2500, 2600, 0], [64, 129, 2100]),
])
def test_prefill_long_context_variants(D, ps, hq, hkv, ctx, news):
    """Appends over contexts above 2048 positions (the tiled prefill kernels,
    not the persistent one): ragged row counts per wave and tile, one or
    several KV splits, GQA groups 1..8, page sizes 16..256."""
    test_prefill_variants(synth.BF16, D, ps, hq, hkv, ctx, news)


@pytest.mark.parametrize("dtype,D,ps,hq,hkv,ctx,news", [
    (synth.BF16, 128, 16, 32, 8, [300, 0, 1000], [200, 64, 150]),
    (synth.BF16, 64, 3, 8, 8, [100, 37], [49, 130]),
    (synth.BF16, 128, 64, 16, 2, [500, 20, 90, 0], [80, 300, 13, 64]),
    (synth.BF16, 128, 1, 1, 1, [3000], [60]),
    (synth.BF16, 64, 16, 6, 3, [2500, 700], [100, 20]),
    (synth.F32, 64, 4, 4, 2, [100, 30], [70, 40]),
    (synth.BF16, 128, 256, 16, 1, [600, 0], [100, 40]),
    (synth.BF16, 64, 256, 32, 2, [2500], [33]),
])
def test_prefill_variants(dtype, D, ps, hq, hkv, ctx, news):
    """Append of several queries per sequence over cached positions: GQA groups
    1..16, page sizes 1..256 (power of two or not), one or several KV splits,
    KV-head counts that do or do not fill blocks of 8 units."""
    print(f"prefill variant {dtype} D={D} ps={ps} hq={hq} hkv={hkv} ctx={ctx} new={news}", flush=True)
    rng = np.random.default_rng(D * 7 + ps)
    lens = [c + n for c, n in zip(ctx, news)]
    pages = sum(-(-L // ps) for L in lens) + 3
    s = Session.open(_Pools(dtype, D, ps, hkv, pages, seed=ps + hq))
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), dtype) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
        s.store(seq, 0, kv[b][0], kv[b][1], dtype)
    qs = [synth.normal_values(rng, (n, hq, D), dtype) for n in news]
    out = host_f64(s.append(seqs, news, dev_tensor(np.concatenate(qs), dtype)))
    row = 0
    for b in range(len(lens)):
        if news[b]:
            e = attend(synth.to_f64(qs[b], dtype), synth.to_f64(kv[b][0], dtype),
                       synth.to_f64(kv[b][1], dtype), s.scale)
            check_close(out[row:row + news[b]], e, dtype, f"prefill variant seq {b}")
        row += news[b]
