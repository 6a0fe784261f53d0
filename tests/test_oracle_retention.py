"""Pins for the oracle's KV retention pool (Quail docs, "KV", "KV retention").

Priorities and eviction orders below are worked out by hand from the page's
rule, priority = probability_of_reuse * recompute_seconds / pages, and the
readings listed in oracle/retention.py (pages counted at entry, ties evicted
in entry order, eviction releases the sequence).
"""

import pytest

from oracle.paging import Allocator, InvalidArgument
from oracle.retention import RetentionPool, priority


def test_priority_hand_values():
    assert priority(0.5, 2.0, 4) == 0.25
    assert priority(1.0, 3.0, 1) == 3.0
    assert priority(0.9, 10.0, 30) == pytest.approx(0.3)
    assert priority(0.0, 5.0, 2) == 0.0


def _docs(alloc, page_counts, ps):
    seqs = []
    for n in page_counts:
        s = alloc.seq_new()
        alloc.reserve(s, n * ps - 1)          # n pages, the last one partial
        seqs.append(s)
    return seqs


def test_hand_built_eviction_order():
    # pages 2, 4, 1, 3; priorities 0.5*2/2 = 0.5, 0.9*10/4 = 2.25, 0.2*1/1 = 0.2,
    # 0.5*6/3 = 1.0 -> lowest first: doc 2, doc 0, doc 3, doc 1
    a = Allocator(20, 4)
    d = _docs(a, [2, 4, 1, 3], 4)
    pool = RetentionPool(a)
    for s, p, t in zip(d, [0.5, 0.9, 0.2, 0.5], [2.0, 10.0, 1.0, 6.0]):
        pool.add(s, p, t)
    assert pool.pages() == 10
    assert pool.evict(10) == []                          # at the limit: nothing to do
    assert pool.evict(6) == [d[2], d[0], d[3]]           # 10 -> 9 -> 7 -> 4 pages
    assert pool.retained() == [d[1]]
    assert a.num_free() == 20 - 4                        # evicted pages went back
    assert pool.evict(0) == [d[1]] and a.num_free() == 20


def test_ties_go_in_entry_order():
    a = Allocator(20, 2)
    d = _docs(a, [2, 1, 4], 2)
    pool = RetentionPool(a)
    pool.add(d[0], 0.5, 2.0)      # 0.5
    pool.add(d[1], 0.25, 2.0)     # 0.5
    pool.add(d[2], 1.0, 2.0)      # 0.5
    assert pool.evict(1) == [d[0], d[1], d[2]]


def test_per_page_value_decides_not_the_total():
    """The same total saving spread over more pages is worth less per page."""
    a = Allocator(20, 4)
    small, large = _docs(a, [1, 5], 4)
    pool = RetentionPool(a)
    pool.add(large, 1.0, 5.0)     # 1.0 per page
    pool.add(small, 0.5, 4.0)     # 2.0 per page
    assert pool.evict(1) == [large]


def test_take_and_recompute():
    a = Allocator(20, 4)
    d = _docs(a, [2, 2, 2], 4)
    pool = RetentionPool(a)
    for s, p in zip(d, [0.1, 0.5, 0.9]):
        pool.add(s, p, 1.0)
    assert pool.take(d[1]) is True                       # reused: leaves the pool, stays alive
    assert a.seq_len(d[1]) == 7
    assert pool.evict(2) == [d[0]]                       # d[1] is no longer a candidate
    assert pool.take(d[0]) is False                      # evicted: the operator recomputes
    with pytest.raises(InvalidArgument):
        a.seq_len(d[0])                                  # released


def test_shared_pages_survive_eviction():
    """Evicting a retained document whose pages another sequence also
    references releases its references only."""
    a = Allocator(10, 4)
    doc = a.seq_new()
    a.reserve(doc, 12)
    child = a.seq_new()
    a.share_prefix(child, doc, 8)
    pool = RetentionPool(a)
    pool.add(doc, 0.5, 1.0)
    assert pool.evict(0) == [doc]
    assert a.num_free() == 10 - 2 and a.block_table(child) == [0, 1]


def test_limit_leaves_room_for_two_forward_passes():
    """The caller's limit: pool pages minus the pages two forward passes need."""
    a = Allocator(100, 4)
    pages_per_pass = 10
    limit = a.num_pages - 2 * pages_per_pass
    d = _docs(a, [30, 30, 30], 4)
    pool = RetentionPool(a)
    for s, p in zip(d, [0.3, 0.2, 0.1]):
        pool.add(s, p, 1.0)
    assert pool.evict(limit) == [d[2]]
    assert a.num_free() >= 2 * pages_per_pass


def test_rejects_bad_input():
    a = Allocator(10, 4)
    s = a.seq_new()
    pool = RetentionPool(a)
    with pytest.raises(InvalidArgument):
        pool.add(s, 0.5, 1.0)                            # no pages
    a.reserve(s, 3)
    pool.add(s, 0.5, 1.0)
    with pytest.raises(InvalidArgument):
        pool.add(s, 0.5, 1.0)                            # twice
    with pytest.raises(InvalidArgument):
        pool.evict(-1)
