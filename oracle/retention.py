"""KV retention pool with priority eviction, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Quail docs, "KV", section "KV retention".  Retained KV lets a later
operator reuse a document's keys and values instead of running the document
through the model a second time.  What is retained is bounded: the budget is
the memory left after setting aside enough for two forward passes.  Over
budget, entries go in increasing order of

    priority = probability_of_reuse * recompute_seconds / pages

which is the expected compute saved per page held: ``probability_of_reuse``
is the chance that a later operator reads the document, ``recompute_seconds``
the cost of processing it anew, and ``pages`` its page count.  An operator
that finds its document's KV gone simply recomputes it.

Readings (also listed in the design notes):
* The unit of retention is a sequence of the page allocator; removing it is
  releasing it (its pages return to the free stack unless another sequence
  still references them).
* ``pages`` is the sequence's page count when it enters the pool (retained
  KV does not grow).
* The pool is full when the sum of its sequences' page counts exceeds the
  limit; eviction removes lowest-priority sequences until it does not.  The
  limit itself (the pool's pages minus the pages of two forward passes) is the
  caller's number.
* Equal priorities: the sequence that entered the pool first goes first.
* Taking a sequence back (a later operator reuses it) removes it from the
  pool without releasing it; taking one that was evicted reports it gone.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

from .paging import Allocator, InvalidArgument


def priority(probability_of_reuse: float, recompute_seconds: float, pages: int) -> float:
    """Estimated compute saved per page of retained KV."""
    return probability_of_reuse * recompute_seconds / pages


class RetentionPool:
    def __init__(self, alloc: Allocator):
        self.alloc = alloc
        self._entries: Dict[int, Tuple[float, int, int]] = {}   # seq -> (priority, order, pages)
        self._order = 0

    def add(self, seq: int, probability_of_reuse: float, recompute_seconds: float) -> None:
        pages = len(self.alloc.block_table(seq))
        if seq in self._entries:
            raise InvalidArgument("sequence already retained")
        if pages == 0:
            raise InvalidArgument("an empty sequence holds no KV")
        if not (probability_of_reuse >= 0 and recompute_seconds >= 0):
            raise InvalidArgument("probability and seconds must be >= 0")
        self._entries[seq] = (priority(probability_of_reuse, recompute_seconds, pages), self._order, pages)
        self._order += 1

    def pages(self) -> int:
        return sum(p for _, _, p in self._entries.values())

    def evict(self, limit_pages: int) -> List[int]:
        """Remove lowest-priority sequences until the pool's pages fit the limit;
        returns them in eviction order."""
        if limit_pages < 0:
            raise InvalidArgument("limit must be >= 0")
        evicted = []
        while self.pages() > limit_pages:
            seq = min(self._entries, key=lambda s: self._entries[s][:2])
            del self._entries[seq]
            self.alloc.release(seq)
            evicted.append(seq)
        return evicted

    def take(self, seq: int) -> bool:
        """A later operator reuses ``seq``: True (and the pool lets it go) when
        its KV is still retained, False when it was evicted or never added."""
        if seq in self._entries:
            del self._entries[seq]
            return True
        return False

    def retained(self) -> List[int]:
        return sorted(self._entries, key=lambda s: self._entries[s][1])
