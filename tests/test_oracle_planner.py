"""Pins for the oracle's prefix-sharing planner and the rewind accounting.

Printed examples: Quail docs "KV", sections "The sharing plan" and "KV rewind"
(tests/golden/quail_sharing_plan.json, tests/golden/quail_rewind.json).
Brute force on tiny alphabets checks that the sorted-adjacent plan shares the
longest whole-page prefix any earlier document offers and that the parent
reached by following links holds the very pages the preceding document holds.
"""

import itertools
import random

import pytest

from oracle.paging import Allocator
from oracle.planner import common_prefix_length, plan_prefix, processed_tokens


def test_quail_sharing_plan_example(golden):
    ex = golden("quail_sharing_plan.json")
    trace = list(range(10_000, 10_000 + max(ex["row_lengths"])))
    rows = [trace[:n] for n in ex["row_lengths"]]
    order, parent, shared = plan_prefix(rows, ex["page_size"])
    assert order == ex["order"]
    assert parent == ex["parent"]
    assert shared == ex["shared"]
    assert [len(r) - s for r, s in zip(rows, shared)] == ex["processed_per_row"]
    assert processed_tokens(rows, shared) == ex["processed_with_sharing"]
    assert sum(map(len, rows)) == ex["processed_without_sharing"]


def test_quail_sharing_plan_example_shuffled_input(golden):
    ex = golden("quail_sharing_plan.json")
    trace = list(range(5, 5 + max(ex["row_lengths"])))
    perm = [2, 0, 1]
    rows = [trace[:ex["row_lengths"][i]] for i in perm]
    order, parent, shared = plan_prefix(rows, ex["page_size"])
    # same plan, relabelled: document ids follow the input order
    inv = {old: new for new, old in enumerate(perm)}
    assert order == [inv[i] for i in ex["order"]]
    assert [shared[inv[i]] for i in range(3)] == ex["shared"]
    assert [None if parent[inv[i]] is None else perm[parent[inv[i]]]
            for i in range(3)] == ex["parent"]


def test_quail_rewind_accounting(golden):
    ex = golden("quail_rewind.json")
    ps = 16
    per_doc_pages = -(-(ex["document_tokens"] + ex["question_tokens"]) // ps)
    a = Allocator(ex["documents"] * per_doc_pages, ps)
    docs = [a.seq_new() for _ in range(ex["documents"])]
    new_with, new_without = 0, 0
    for s in docs:
        a.reserve(s, ex["document_tokens"])
        a.reserve(s, ex["question_tokens"])            # first question
        a.truncate(s, ex["document_tokens"])           # rewind: drop its KV
        before = a.seq_len(s)
        a.reserve(s, ex["question_tokens"])            # second question
        new_with += a.seq_len(s) - before
        new_without += ex["document_tokens"] + ex["question_tokens"]
    assert new_with == ex["new_tokens_with_rewind"]
    assert new_without == ex["new_tokens_without_rewind"]


def _brute_force_checks(docs, ps):
    order, parent, shared = plan_prefix(docs, ps)
    n = len(docs)
    assert sorted(order) == list(range(n))
    # order is sorted lexicographically and stable on ties
    for k in range(1, n):
        a, b = docs[order[k - 1]], docs[order[k]]
        assert list(a) <= list(b)
        if list(a) == list(b):
            assert order[k - 1] < order[k]
    pos = {d: k for k, d in enumerate(order)}
    for d in range(n):
        s = shared[d]
        assert s % ps == 0
        assert 0 <= s <= max(0, len(docs[d]) - 1)
        # maximal: no earlier document offers more whole pages
        best = 0
        for e in order[: pos[d]]:
            lcp = common_prefix_length(docs[d], docs[e])
            best = max(best, ps * (max(0, min(lcp, len(docs[d]) - 1)) // ps))
        assert s == best
        if s == 0:
            assert parent[d] is None
        else:
            p = parent[d]
            assert pos[p] < pos[d]
            assert list(docs[p][:s]) == list(docs[d][:s])
    # Allocate in planned order: the child's shared pages are exactly the
    # pages its sorted predecessor holds for that prefix.
    alloc = Allocator(sum(-(-len(x) // ps) for x in docs) + 1, ps)
    seqs = {}
    for k, d in enumerate(order):
        seqs[d] = alloc.seq_new()
        if parent[d] is not None:
            alloc.share_prefix(seqs[d], seqs[parent[d]], shared[d])
        alloc.reserve(seqs[d], len(docs[d]) - shared[d])
        if k > 0 and shared[d] > 0:
            q = order[k - 1]
            npg = shared[d] // ps
            assert alloc.block_table(seqs[d])[:npg] == alloc.block_table(seqs[q])[:npg]
    return order, parent, shared


@pytest.mark.parametrize("seed", range(40))
def test_planner_brute_force_tiny_alphabets(seed):
    rnd = random.Random(seed)
    ps = rnd.choice([1, 2, 3, 4])
    n = rnd.randrange(1, 9)
    alpha = rnd.choice([1, 2, 3])
    base = [rnd.randrange(alpha) for _ in range(14)]
    docs = []
    for _ in range(n):
        if rnd.random() < 0.6:
            cut = rnd.randrange(0, 15)
            tail = [rnd.randrange(alpha) for _ in range(rnd.randrange(0, 4))]
            docs.append(base[:cut] + tail)
        else:
            docs.append([rnd.randrange(alpha) for _ in range(rnd.randrange(0, 12))])
    _brute_force_checks(docs, ps)


def test_planner_exhaustive_small():
    # every multiset of 3 documents over {0,1} with lengths <= 4
    words = [list(w) for L in range(5) for w in itertools.product([0, 1], repeat=L)]
    rnd = random.Random(0)
    for _ in range(400):
        docs = [rnd.choice(words) for _ in range(3)]
        for ps in (1, 2):
            _brute_force_checks(docs, ps)


def test_parent_chain_follows_links():
    # three nested prefixes and a fourth row equal to the second: the fourth
    # row's predecessor (row 1) reuses the whole shared prefix from row 0,
    # so the plan follows row 1's parent link.
    ps = 4
    t = list(range(100))
    docs = [t[:9], t[:13], t[:20], t[:13]]
    order, parent, shared = plan_prefix(docs, ps)
    assert order == [0, 1, 3, 2]
    assert shared == [0, 8, 12, 12]
    assert parent[1] == 0
    # row 3 follows row 1 (shared 8 < 12 -> row 1 supplies), row 2 follows row 3
    # (shared 12 >= 12 -> walk to row 1)
    assert parent[3] == 1
    assert parent[2] == 1
    _brute_force_checks(docs, ps)
