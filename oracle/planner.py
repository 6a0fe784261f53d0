"""The prefix-sharing plan (order, parent, shared), written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Quail docs "KV", section "The sharing plan".  The planner has every
document before execution; it sorts documents by their token sequence,
compares each document with its neighbour in that order to find the common
prefix, shares only whole pages, always leaves a document's final token to be
computed, and, when the preceding document itself reuses the entire shared
prefix, follows parent links to the document that supplies those pages.  The
plan is a triple (order, parent, shared).

Readings (also listed in the design notes):
* "sorts documents by token sequence": lexicographic order of the token-id
  lists, a proper prefix before its extensions, equal lists kept in input
  order (a stable sort).
* ``parent`` and ``shared`` are indexed by original document id; ``order[k]``
  is the document at sorted position k; ``parent`` holds document ids, None
  for a document that shares nothing.
* "leaves the final token": the shareable length is capped at len - 1 before
  it is rounded down to whole pages.
* "follows parent links": starting at the preceding document q, while the
  current candidate has a parent and shares at least the new prefix length s,
  move to its parent.  The pages' example never walks a link, so this loop is
  pinned only by the invariant that the chosen parent's first s/page_size
  pages are the very pages the preceding document holds: which of several
  equivalent parents is chosen is parity unpinned (no attention output can
  depend on it).
* The cost rule ("savings exceed additional KV write costs") gives no
  constants; the plainest reading shares whenever at least one page is whole.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple


def common_prefix_length(a: Sequence[int], b: Sequence[int]) -> int:
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


def plan_prefix(docs: Sequence[Sequence[int]], page_size: int
                ) -> Tuple[List[int], List[Optional[int]], List[int]]:
    """Return (order, parent, shared) for the documents ``docs``."""
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    docs = [list(map(int, d)) for d in docs]
    n = len(docs)
    order = sorted(range(n), key=lambda d: docs[d])  # Python's sort is stable
    parent: List[Optional[int]] = [None] * n
    shared = [0] * n
    for k in range(1, n):
        d = order[k]
        q = order[k - 1]
        lcp = common_prefix_length(docs[d], docs[q])
        computable = max(0, min(lcp, len(docs[d]) - 1))
        s = page_size * (computable // page_size)
        if s == 0:
            continue
        p = q
        while parent[p] is not None and shared[p] >= s:
            p = parent[p]
        parent[d] = p
        shared[d] = s
    return order, parent, shared


def processed_tokens(docs: Sequence[Sequence[int]], shared: Sequence[int]) -> int:
    """Document tokens computed under the plan: each length minus its shared part."""
    return sum(len(d) - s for d, s in zip(docs, shared))
