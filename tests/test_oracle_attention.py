"""Pins for the oracle's paged attention.

Nothing here re-types the oracle's formula.  The checks are:
* closed forms: one visible key gives its value exactly; a zero query (or equal
  keys) gives the plain mean of the visible values;
* a library special case: torch's scaled_dot_product_attention in float64 on
  the CPU, with an explicit boolean mask and the KV heads repeated per group;
* brute force: scalar math.exp loops on tiny inputs;
* invariants from "KV Cache Management and PagedAttention", "Compute attention
  over scattered KV": the result does not depend on where pages sit; decode of
  the last position equals the last row of a causal prefill; a prefix-shared
  append equals the unshared computation.
"""

import math
import random

import numpy as np
import pytest
import torch

from oracle.attention import attend, attend_row, gather_kv, paged_attention
from oracle.paging import Allocator, store_rows


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = _rand(rng, 3, 4, 8)
    k = _rand(rng, 3, 2, 8)
    v = _rand(rng, 3, 2, 8)
    out = attend(q, k, v, 0.3)  # n == L: query 0 sees only position 0
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(2)
    L, n = 9, 4
    k = _rand(rng, L, 1, 16)
    v = _rand(rng, L, 1, 16)
    q = np.zeros((n, 2, 16))
    out = attend(q, k, v, 1.0)
    for i in range(n):
        p = L - n + i
        np.testing.assert_allclose(out[i, 0], v[: p + 1, 0].mean(axis=0), rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[i, 1], v[: p + 1, 0].mean(axis=0), rtol=0, atol=1e-15)


def test_equal_keys_give_mean():
    rng = np.random.default_rng(3)
    L = 7
    k = np.repeat(_rand(rng, 1, 1, 8), L, axis=0)
    v = _rand(rng, L, 1, 8)
    q = _rand(rng, 1, 1, 8)
    out = attend(q, k, v, 0.5)
    np.testing.assert_allclose(out[0, 0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)


def _sdpa_reference(q, k, v, scale):
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][n][D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    start = L - n
    mask = torch.arange(L)[None, :] <= (start + torch.arange(n))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,L,hq,hkv,d", [(1, 1, 1, 1, 4), (1, 37, 8, 2, 16), (5, 5, 4, 4, 8),
                                          (6, 40, 8, 1, 32), (50, 350, 4, 1, 64),
                                          (3, 130, 6, 3, 128)])
def test_matches_fp64_sdpa(n, L, hq, hkv, d):
    rng = np.random.default_rng(n * 1000 + L)
    q, k, v = _rand(rng, n, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    scale = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(attend(q, k, v, scale), _sdpa_reference(q, k, v, scale),
                               rtol=0, atol=1e-12)


def _scalar_attention(q, k, v, scale):
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    grp = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(n)]
    for i in range(n):
        pos = L - n + i
        for h in range(hq):
            g = h // grp
            scores = []
            for j in range(pos + 1):
                s = 0.0
                for x in range(d):
                    s += float(q[i][h][x]) * float(k[j][g][x])
                scores.append(scale * s)
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            tot = sum(ws)
            for x in range(d):
                out[i][h][x] = sum(ws[j] * float(v[j][g][x]) for j in range(pos + 1)) / tot
    return np.array(out)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rnd = random.Random(seed)
    d = rnd.choice([1, 2, 8])
    hkv = rnd.choice([1, 2])
    grp = rnd.choice([1, 2, 4])
    L = rnd.randrange(1, 10)
    n = rnd.randrange(1, L + 1)
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, n, hkv * grp, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    scale = rnd.choice([1.0, 0.125, 1 / math.sqrt(d)])
    np.testing.assert_allclose(attend(q, k, v, scale), _scalar_attention(q, k, v, scale),
                               rtol=0, atol=1e-12)


def test_attend_row_matches_attend():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 4, 4, 16), _rand(rng, 20, 2, 16), _rand(rng, 20, 2, 16)
    full = attend(q, k, v, 0.25)
    for i in range(4):
        for h in range(4):
            row = attend_row(q[i, h], k[:, h // 2], v[:, h // 2], 16 + i, 0.25)
            np.testing.assert_allclose(row, full[i, h], rtol=0, atol=1e-14)


def _store(pool, alloc, seq, values, start):
    store_rows(pool, alloc.slots(seq, start, values.shape[0]), values)


def test_store_rows_places_each_row_at_its_slot():
    pool = np.zeros((3, 2, 4, 5))
    rows = np.arange(3 * 2 * 5, dtype=float).reshape(3, 2, 5) + 1
    store_rows(pool, [9, 2, -1], rows)
    assert np.array_equal(pool[2, :, 1, :], rows[0])   # slot 9 = page 2, offset 1
    assert np.array_equal(pool[0, :, 2, :], rows[1])   # slot 2 = page 0, offset 2
    assert np.count_nonzero(pool) == 2 * 2 * 5          # slot -1 skipped


@pytest.mark.parametrize("ps", [1, 3, 4, 16])
def test_page_permutation_changes_nothing(ps):
    rng = np.random.default_rng(ps)
    lens = [7, 6, 19, 1]
    hq, hkv, d = 4, 2, 8
    k = [_rand(rng, L, hkv, d) for L in lens]
    v = [_rand(rng, L, hkv, d) for L in lens]
    q = [_rand(rng, 1, hq, d) for _ in lens]
    outs = []
    for perm_seed in range(3):
        npages = 40
        order = list(range(npages))
        random.Random(perm_seed).shuffle(order)
        alloc = Allocator(npages, ps, order)
        kp = np.full((npages, hkv, ps, d), np.nan)
        vp = np.full((npages, hkv, ps, d), np.nan)
        tables = []
        for b, L in enumerate(lens):
            s = alloc.seq_new()
            alloc.reserve(s, L)
            _store(kp, alloc, s, k[b], 0)
            _store(vp, alloc, s, v[b], 0)
            tables.append(alloc.block_table(s))
        cu = np.arange(len(lens) + 1)
        outs.append(paged_attention(np.concatenate(q), cu, lens, tables, kp, vp, 0.35))
        # the gather form equals the logical form bit for bit
        for b, L in enumerate(lens):
            assert np.array_equal(gather_kv(kp, tables[b], L), k[b])
            assert np.array_equal(outs[-1][b:b + 1], attend(q[b], k[b], v[b], 0.35))
    assert not np.isnan(outs[0]).any()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_decode_equals_last_row_of_causal_prefill():
    rng = np.random.default_rng(9)
    L = 23
    q, k, v = _rand(rng, L, 4, 8), _rand(rng, L, 1, 8), _rand(rng, L, 1, 8)
    full = attend(q, k, v, 0.3)
    last = attend(q[-1:], k, v, 0.3)
    np.testing.assert_allclose(last[0], full[-1], rtol=0, atol=1e-15)


def test_prefix_shared_append_equals_unshared():
    # A child that adopts its parent's first 8 positions and appends 5 gets the
    # same result as a fresh causal prefill over its own 13 positions.
    rng = np.random.default_rng(11)
    ps, hq, hkv, d = 4, 2, 1, 8
    k = _rand(rng, 13, hkv, d)
    v = _rand(rng, 13, hkv, d)
    q = _rand(rng, 13, hq, d)
    alloc = Allocator(10, ps, list(range(9, -1, -1)))
    kp = np.full((10, hkv, ps, d), np.nan)
    vp = np.full((10, hkv, ps, d), np.nan)
    parent = alloc.seq_new()
    alloc.reserve(parent, 10)
    _store(kp, alloc, parent, k[:10], 0)
    _store(vp, alloc, parent, v[:10], 0)
    child = alloc.seq_new()
    alloc.share_prefix(child, parent, 8)
    alloc.reserve(child, 5)
    _store(kp, alloc, child, k[8:], 8)
    _store(vp, alloc, child, v[8:], 8)
    out = paged_attention(q[8:], [0, 5], [13], [alloc.block_table(child)], kp, vp, 0.4)
    np.testing.assert_allclose(out, attend(q, k, v, 0.4)[8:], rtol=0, atol=1e-15)


def test_rewind_second_pass_equals_fresh_prefill():
    rng = np.random.default_rng(12)
    ps, hq, hkv, d, doc, ql = 16, 4, 2, 8, 30, 5
    dk, dv = _rand(rng, doc, hkv, d), _rand(rng, doc, hkv, d)
    q1 = [_rand(rng, ql, hq, d), _rand(rng, ql, hkv, d), _rand(rng, ql, hkv, d)]
    q2 = [_rand(rng, ql, hq, d), _rand(rng, ql, hkv, d), _rand(rng, ql, hkv, d)]
    alloc = Allocator(8, ps)
    kp = np.full((8, hkv, ps, d), np.nan)
    vp = np.full((8, hkv, ps, d), np.nan)
    s = alloc.seq_new()
    alloc.reserve(s, doc)
    _store(kp, alloc, s, dk, 0)
    _store(vp, alloc, s, dv, 0)
    alloc.reserve(s, ql)
    _store(kp, alloc, s, q1[1], doc)
    _store(vp, alloc, s, q1[2], doc)
    alloc.truncate(s, doc)   # the stale q1 KV stays in the page; never read
    alloc.reserve(s, ql)
    _store(kp, alloc, s, q2[1], doc)
    _store(vp, alloc, s, q2[2], doc)
    out = paged_attention(q2[0], [0, ql], [doc + ql], [alloc.block_table(s)], kp, vp, 0.3)
    fresh = attend(q2[0], np.concatenate([dk, q2[1]]), np.concatenate([dv, q2[2]]), 0.3)
    np.testing.assert_allclose(out, fresh, rtol=0, atol=1e-15)
