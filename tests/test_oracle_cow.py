"""Pins for the oracle's copy-on-write allocator rule and page copy
("KV Cache Management and PagedAttention": "Share common KV across responses"
(Figure 5), "Split shared blocks when a write is needed" (Figure 6), "Return
blocks after a request ends").

The checks are the blog's worked example (tests/golden/blog_cow_example.json),
the rule it states for a shared block that is already full, all-or-nothing
behaviour, and an end-to-end invariant: after any sequence of forks, copy-on-
write reserves, page copies and stores, every response's K/V read through its
own block table is exactly its prompt followed by its own tokens.
"""

import numpy as np
import pytest

from oracle.attention import gather_kv
from oracle.paging import Allocator, OutOfPages, copy_pages, store_rows


def _page(name):
    return int(name[1:])


def test_blog_figure6_walkthrough(golden):
    g = golden("blog_cow_example.json")
    ps = g["block_size"]
    a = Allocator(8, ps)
    r1 = a.seq_new()
    a.reserve(r1, g["input_tokens"])
    r2 = a.seq_new()
    a.fork(r2, r1)
    # both responses map L0 -> P0, L1 -> P1; 2 physical blocks instead of 4
    assert a.block_table(r1) == [_page(x) for x in g["after_input"]["response_1"]]
    assert a.block_table(r2) == [_page(x) for x in g["after_input"]["response_2"]]
    assert 8 - a.num_free() == g["after_input"]["physical_blocks"] == g["blocks_shared"]
    assert 2 * -(-g["input_tokens"] // ps) == g["blocks_if_each_response_copies"]
    # response 1 processes a0: P1 is copied to P2, response 1 now maps L1 -> P2
    s = g["after_a0"]
    assert a.reserve_cow(r1, 1) == (_page(s["copy"][0]), _page(s["copy"][1]))
    assert a.block_table(r1) == [_page(x) for x in s["response_1"]]
    assert a.block_table(r2) == [_page(x) for x in s["response_2"]]
    assert a.slots(r1, 6, 1) == [_page(s["a0_block"]) * ps + s["a0_offset"]]
    assert a.refcount[_page("P1")] == s["refcount_P1"]
    assert 8 - a.num_free() == s["physical_blocks"]
    # response 2 processes b0: no copy, it writes into P1's next slot
    s = g["after_b0"]
    assert a.reserve_cow(r2, 1) is s["copy"]
    assert a.block_table(r2) == [_page(x) for x in s["response_2"]]
    assert a.slots(r2, 6, 1) == [_page(s["b0_block"]) * ps + s["b0_offset"]]
    assert a.refcount[_page("P0")] == s["refcount_P0"]
    assert 8 - a.num_free() == s["physical_blocks"]


def test_plain_reserve_still_refuses_shared_partial_page():
    a = Allocator(8, 4)
    r1 = a.seq_new()
    a.reserve(r1, 6)
    r2 = a.seq_new()
    a.fork(r2, r1)
    from oracle.paging import SharedPageWrite
    with pytest.raises(SharedPageWrite):
        a.reserve(r1, 1)


def test_full_shared_block_stays_shared():
    """A shared block that is already full stays shared; each response gets a
    new block for its next positions and nothing is copied."""
    a = Allocator(8, 4)
    r1 = a.seq_new()
    a.reserve(r1, 8)
    r2 = a.seq_new()
    a.fork(r2, r1)
    assert a.reserve_cow(r1, 1) is None and a.reserve_cow(r2, 3) is None
    assert a.block_table(r1)[:2] == a.block_table(r2)[:2] == [0, 1]
    assert a.block_table(r1)[2] != a.block_table(r2)[2]
    assert a.refcount[0] == a.refcount[1] == 2


def test_copy_page_is_taken_before_growth_pages_and_all_or_nothing():
    a = Allocator(5, 4, [4, 3, 2, 1, 0])
    r1 = a.seq_new()
    a.reserve(r1, 6)                       # pages 4, 3
    r2 = a.seq_new()
    a.fork(r2, r1)
    # 6 + 7 = 13 positions: the copy page (2), then pages 1 and 0
    assert a.reserve_cow(r2, 7) == (3, 2)
    assert a.block_table(r2) == [4, 2, 1, 0]
    r3 = a.seq_new()
    a.fork(r3, r1)
    before = (a.block_table(r1), a.block_table(r3), list(a.refcount), a.free_pages(), a.seq_len(r3))
    with pytest.raises(OutOfPages):         # a copy is needed and no page is free
        a.reserve_cow(r3, 1)
    assert (a.block_table(r1), a.block_table(r3), list(a.refcount), a.free_pages(), a.seq_len(r3)) == before


def test_release_after_split_returns_only_unshared_blocks():
    a = Allocator(8, 4)
    r1 = a.seq_new()
    a.reserve(r1, 6)
    r2 = a.seq_new()
    a.fork(r2, r1)
    a.reserve_cow(r1, 1)                   # r1: [0, 2], r2: [0, 1]
    a.release(r1)
    assert a.refcount[:3] == [1, 1, 0] and 2 in a.free_pages()
    assert a.block_table(r2) == [0, 1]


def test_rewind_into_shared_block_copies_on_next_write():
    """Truncating back into a block another sequence references and writing
    again copies the block first (the same rule after a rewind)."""
    a = Allocator(8, 4)
    r1 = a.seq_new()
    a.reserve(r1, 10)                      # [0, 1, 2]
    r2 = a.seq_new()
    a.fork(r2, r1)
    a.truncate(r2, 5)                      # r2: [0, 1], block 1 shared and partial
    assert a.reserve_cow(r2, 1) == (1, a.block_table(r2)[1])
    assert a.block_table(r1) == [0, 1, 2] and a.refcount[1] == 1


@pytest.mark.parametrize("seed", range(6))
def test_every_response_reads_prompt_then_its_own_tokens(seed):
    """Fork a prompt into several responses, grow each by copy-on-write
    reserves, device-side page copies and stores, in random interleaving; then
    each response's K/V read through its block table is exactly its prompt
    followed by its own tokens (and the prompt's own table is untouched)."""
    rng = np.random.default_rng(seed)
    ps = int(rng.choice([1, 3, 4, 16]))
    hkv, d = 2, 4
    num_pages = 200
    a = Allocator(num_pages, ps, rng.permutation(num_pages))
    pool = np.full((num_pages, hkv, ps, d), np.nan)
    L0 = int(rng.integers(1, 40))
    prompt_rows = rng.standard_normal((L0, hkv, d))
    root = a.seq_new()
    a.reserve(root, L0)
    store_rows(pool, a.slots(root, 0, L0), prompt_rows)
    responses = []
    for _ in range(int(rng.integers(2, 5))):
        r = a.seq_new()
        a.fork(r, root)
        responses.append((r, [prompt_rows]))
    for _ in range(30):
        r, rows = responses[int(rng.integers(len(responses)))]
        n = int(rng.integers(1, 6))
        start = a.seq_len(r)
        copy = a.reserve_cow(r, n)
        if copy is not None:
            copy_pages(pool, [copy])
        new_rows = rng.standard_normal((n, hkv, d))
        store_rows(pool, a.slots(r, start, n), new_rows)
        rows.append(new_rows)
    for r, rows in responses:
        expect = np.concatenate(rows)
        assert np.array_equal(gather_kv(pool, a.block_table(r), a.seq_len(r)), expect)
    assert np.array_equal(gather_kv(pool, a.block_table(root), L0), prompt_rows)
