"""Pins for the oracle's block-table / slot model and page allocator.

The worked example is the blog "KV Cache Management and PagedAttention"
(Figures 1-4), stored in tests/golden/blog_block_example.json.  The remaining
checks are invariants that any correct allocator must keep.
"""

import random

import pytest

from oracle.paging import (Allocator, InvalidArgument, OutOfPages, SharedPageWrite,
                           pool_element_index, slot_of)


def test_blog_block_counts(golden):
    ex = golden("blog_block_example.json")
    bs = ex["block_size"]
    assert ex["capacity_slots"] // bs == ex["capacity_blocks"]
    a = Allocator(ex["capacity_blocks"], bs, ex["free_order_reading"])
    b = a.seq_new()
    c = a.seq_new()
    a.reserve(b, ex["B_positions_before"])
    a.reserve(c, ex["C_positions"])
    assert len(a.block_table(b)) == ex["blocks_B"]
    assert len(a.block_table(c)) == ex["blocks_C"]
    allocated = (len(a.block_table(b)) + len(a.block_table(c))) * bs
    assert allocated == ex["allocated_slots"]
    assert a.num_free() * bs == ex["free_slots_after_allocation"]
    # B's next input (position 6) fits its last block: no new block.
    a.reserve(b, ex["B_positions_after"] - ex["B_positions_before"])
    assert len(a.block_table(b)) == ex["blocks_B"]
    filled = a.seq_len(b) + a.seq_len(c)
    assert filled == ex["filled_after_step"]
    assert allocated - filled == ex["empty_after_step"]


def test_blog_lookup_and_growth(golden):
    ex = golden("blog_block_example.json")
    bs = ex["block_size"]
    a = Allocator(ex["capacity_blocks"], bs, ex["free_order_reading"])
    b = a.seq_new()
    c = a.seq_new()
    a.reserve(b, ex["B_positions_after"])
    a.reserve(c, ex["C_positions"])
    assert a.block_table(b) == ex["table_B"]
    assert a.block_table(c) == ex["table_C"]
    a.reserve(b, 1)  # position 7: the last empty slot of P0
    assert a.block_table(b) == ex["table_B"]
    a.reserve(b, 1)  # position 8: both blocks full -> new block
    assert a.block_table(b) == ex["table_B_after_position_8"]
    for row in ex["lookup"]:
        p = row["position"]
        assert p // bs == row["logical_block"]
        assert p % bs == row["offset"]
        assert a.block_table(b)[row["logical_block"]] == row["physical_block"]
        assert a.slots(b, p, 1) == [row["physical_block"] * bs + row["offset"]]
    # Attention at position 8 reads 9 positions: 4 in P3, 4 in P0, 1 in P5.
    att = ex["attention_at_position_8"]
    used = a.slots(b, 0, 9)
    assert len(used) == att["positions"]
    per_block = {}
    for s in used:
        per_block[str(s // bs)] = per_block.get(str(s // bs), 0) + 1
    assert per_block == att["per_block"]
    assert not ({s // bs for s in used} & set(att["excluded_blocks"]))
    assert len(a.block_table(b)) * bs - a.seq_len(b) == att["unused_slots_in_last_block"]


def test_slot_formula_zero_based():
    table = [7, 2, 9]
    assert [slot_of(table, p, 4) for p in range(12)] == \
        [28, 29, 30, 31, 8, 9, 10, 11, 36, 37, 38, 39]


def test_pool_element_index_is_row_major_of_reversed_shape():
    import numpy as np
    npages, hkv, ps, d = 3, 2, 4, 5
    pool = np.arange(npages * hkv * ps * d).reshape(npages, hkv, ps, d)
    # TileInfer's (head_dim, page_size, kv_heads, num_pages) column-major array
    # is this array's transpose with Fortran order: same bytes.
    col_major = np.asfortranarray(pool.transpose(3, 2, 1, 0))
    flat = col_major.ravel(order="F")
    for page in range(npages):
        for g in range(hkv):
            for off in range(ps):
                for x in range(d):
                    i = pool_element_index(page, g, off, x, hkv, ps, d)
                    assert flat[i] == pool[page, g, off, x]
                    assert col_major[x, off, g, page] == flat[i]


def test_out_of_pages_leaves_state_unchanged():
    a = Allocator(4, 4)
    s = a.seq_new()
    a.reserve(s, 10)
    before = (a.block_table(s), a.seq_len(s), a.num_free(), list(a.refcount))
    with pytest.raises(OutOfPages):
        a.reserve(s, 7)  # needs 2 more pages, 1 free
    assert (a.block_table(s), a.seq_len(s), a.num_free(), list(a.refcount)) == before
    a.reserve(s, 6)  # exactly fills the pool
    assert a.num_free() == 0


def test_truncate_then_reserve_returns_same_pages():
    a = Allocator(16, 4, list(range(15, -1, -1)))
    s = a.seq_new()
    a.reserve(s, 23)
    table = a.block_table(s)
    a.truncate(s, 9)  # keep 3 blocks
    assert a.block_table(s) == table[:3]
    a.reserve(s, 14)
    assert a.block_table(s) == table


def test_rewind_frees_three_pages_per_document():
    a = Allocator(64, 16)
    s = a.seq_new()
    a.reserve(s, 300)
    assert len(a.block_table(s)) == 19
    a.reserve(s, 50)
    assert len(a.block_table(s)) == 22
    free_before = a.num_free()
    a.truncate(s, 300)
    assert a.num_free() - free_before == 3
    assert a.seq_len(s) == 300


def test_share_prefix_refcounts_and_release():
    a = Allocator(10, 4)
    p = a.seq_new()
    a.reserve(p, 10)
    c = a.seq_new()
    a.share_prefix(c, p, 8)
    assert a.block_table(c) == a.block_table(p)[:2]
    assert [a.refcount[x] for x in a.block_table(p)] == [2, 2, 1]
    a.reserve(c, 3)
    assert a.block_table(c)[:2] == a.block_table(p)[:2]
    a.release(p)
    # shared pages stay with the child; the parent's own page returns
    assert all(a.refcount[x] == 1 for x in a.block_table(c))
    assert a.num_free() == 10 - 3
    with pytest.raises(InvalidArgument):
        a.share_prefix(a.seq_new(), c, 6)  # not whole pages


def test_write_into_shared_partial_page_is_refused():
    a = Allocator(10, 4)
    p = a.seq_new()
    a.reserve(p, 8)
    c = a.seq_new()
    a.share_prefix(c, p, 8)
    a.truncate(p, 6)  # parent now ends inside a page the child also holds
    with pytest.raises(SharedPageWrite):
        a.reserve(p, 1)


def _check_invariants(a, live):
    counts = [0] * a.num_pages
    for s in live:
        t = a.block_table(s)
        assert len(t) == -(-a.seq_len(s) // a.page_size)
        for x in t:
            counts[x] += 1
    assert counts == a.refcount
    free = a.free_pages()
    assert len(set(free)) == len(free)
    assert set(free) == {x for x in range(a.num_pages) if counts[x] == 0}


@pytest.mark.parametrize("seed", range(20))
def test_random_operation_sequences_keep_invariants(seed):
    rnd = random.Random(seed)
    ps = rnd.choice([1, 2, 3, 4, 16])
    a = Allocator(40, ps, rnd.sample(range(40), 40))
    live = []
    for _ in range(300):
        op = rnd.random()
        try:
            if op < 0.15 or not live:
                live.append(a.seq_new())
            elif op < 0.55:
                a.reserve(rnd.choice(live), rnd.randrange(0, 3 * ps + 2))
            elif op < 0.75:
                s = rnd.choice(live)
                a.truncate(s, rnd.randrange(0, a.seq_len(s) + 1))
            elif op < 0.85:
                s = rnd.choice(live)
                a.release(s)
                live.remove(s)
            else:
                p = rnd.choice(live)
                c = a.seq_new()
                live.append(c)
                a.share_prefix(c, p, ps * rnd.randrange(0, a.seq_len(p) // ps + 1))
        except (OutOfPages, SharedPageWrite):
            pass
        _check_invariants(a, live)
