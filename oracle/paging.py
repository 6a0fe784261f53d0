"""Block tables, slots and the page allocator, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources
-------
* TileInfer.jl docs, "KV cache" -- "Pages and block tables": a sequence owns a
  block table (its pages in order); position p lives in page
  ``block_table[p / page_size]`` at offset ``p % page_size``; a BlockManager
  hands out pages from a stack of free page ids; a slot is a flat pool index
  made of page and offset.  "Growing, rolling back, releasing": ``reserve!``
  (pages for the next n positions, OutOfPagesError when exhausted),
  ``truncate!`` (keep the first n positions, return pages no longer needed,
  nothing copied or cleared), ``release!`` (return all pages).
* "KV Cache Management and PagedAttention" -- "Allocate blocks as needed"
  (Figure 1), "Connect token order to storage locations" (Figure 2: 0-based
  logical blocks and in-block positions), "Grow the allocation as generation
  proceeds" (Figure 3: a new block only when the last one is full), "Return
  blocks after a request ends" (reference counts; a page with no references
  returns to the pool).
* Quail docs "KV" -- "Paged KV": several documents may reference one page; a
  page is free when nothing references it.  "Execution": a document
  references its parent's shared pages without copying them.

Readings where the pages leave a choice open (each one is listed in the design
notes):
* 0-based indices (the blog's Figure 2 text; the Julia page is 1-based).
* slot = page * page_size + offset, one slot per position covering every KV
  head of that position.
* The free stack pops ``free_order[0]`` first; pages dropped by a truncate are
  pushed last-logical-block first, so truncate followed by reserve hands back
  the same pages in the same order.
* Every allocator call is all-or-nothing: on error the state is unchanged.
* ``reserve`` refuses to write a new position into a page that another
  sequence also references (``SharedPageWrite``).  ``reserve_cow`` is the
  copy-on-write form ("KV Cache Management and PagedAttention", "Split shared
  blocks when a write is needed", Figure 6): the writing sequence first gets
  a fresh page holding a copy of the shared one (popped before any page the
  growth needs), the shared page loses that reference, and the copy is
  returned for the device to perform.  The whole page is copied.
* ``fork`` makes an empty sequence reference every page of another one, the
  partial last page included ("Share common KV across responses", Figure 5).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class AllocatorError(Exception):
    """Base class of the allocator's errors."""


class OutOfPages(AllocatorError):
    """The free stack holds fewer pages than a reserve needs."""


class InvalidArgument(AllocatorError):
    """A call's arguments contradict the allocator state."""


class SharedPageWrite(AllocatorError):
    """A reserve would write into a page referenced by another sequence."""


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def slot_of(block_table: Sequence[int], p: int, page_size: int) -> int:
    """Slot of logical position p: its page times page_size plus its offset."""
    return int(block_table[p // page_size]) * page_size + p % page_size


def pool_element_index(page: int, kv_head: int, offset: int, d: int,
                       num_kv_heads: int, page_size: int, head_dim: int) -> int:
    """Flat index of one element of a pool laid out [page][kv_head][offset][d].

    This is the TileInfer.jl pool shape (head_dim, page_size, kv_heads,
    num_pages) in column-major order, i.e. the same bytes read row-major with
    the axes reversed.
    """
    return ((page * num_kv_heads + kv_head) * page_size + offset) * head_dim + d


class Allocator:
    """Reference page allocator: a free stack, block tables and refcounts."""

    def __init__(self, num_pages: int, page_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_pages < 0 or page_size < 1:
            raise InvalidArgument("num_pages must be >= 0 and page_size >= 1")
        order = list(range(num_pages)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_pages)):
            raise InvalidArgument("free_order must be a permutation of the page ids")
        self.num_pages = num_pages
        self.page_size = page_size
        # The top of the stack is the end of the list: the first pop returns
        # free_order[0].
        self._free: List[int] = list(reversed(order))
        self.refcount: List[int] = [0] * num_pages
        self._tables: Dict[int, List[int]] = {}
        self._lens: Dict[int, int] = {}
        self._next_id = 0

    # -- queries -----------------------------------------------------------
    def num_free(self) -> int:
        return len(self._free)

    def seq_len(self, seq: int) -> int:
        self._check(seq)
        return self._lens[seq]

    def block_table(self, seq: int) -> List[int]:
        self._check(seq)
        return list(self._tables[seq])

    def slots(self, seq: int, start: int, n: int) -> List[int]:
        """Slots of positions start .. start+n-1 of ``seq``."""
        self._check(seq)
        if start < 0 or n < 0 or start + n > self._lens[seq]:
            raise InvalidArgument("slot range outside the sequence")
        table = self._tables[seq]
        return [slot_of(table, p, self.page_size) for p in range(start, start + n)]

    def free_pages(self) -> List[int]:
        """Free page ids, next pop first."""
        return list(reversed(self._free))

    # -- mutations -----------------------------------------------------------
    def seq_new(self) -> int:
        seq = self._next_id
        self._next_id += 1
        self._tables[seq] = []
        self._lens[seq] = 0
        return seq

    def reserve(self, seq: int, n: int) -> None:
        """Extend ``seq`` by n positions, popping pages only when needed."""
        self._check(seq)
        if n < 0:
            raise InvalidArgument("n must be >= 0")
        length = self._lens[seq]
        table = self._tables[seq]
        ps = self.page_size
        if n > 0 and length % ps != 0 and self.refcount[table[length // ps]] > 1:
            raise SharedPageWrite("next position falls in a page other sequences reference")
        need = ceil_div(length + n, ps) - len(table)
        if need > len(self._free):
            raise OutOfPages(f"need {need} pages, {len(self._free)} free")
        for _ in range(need):
            page = self._free.pop()
            self.refcount[page] = 1
            table.append(page)
        self._lens[seq] = length + n

    def truncate(self, seq: int, n_keep: int) -> None:
        """Keep the first n_keep positions; drop references to later pages."""
        self._check(seq)
        if n_keep < 0 or n_keep > self._lens[seq]:
            raise InvalidArgument("n_keep outside 0..len")
        table = self._tables[seq]
        keep_blocks = ceil_div(n_keep, self.page_size)
        for i in range(len(table) - 1, keep_blocks - 1, -1):
            page = table[i]
            self.refcount[page] -= 1
            if self.refcount[page] == 0:
                self._free.append(page)
        del table[keep_blocks:]
        self._lens[seq] = n_keep

    def release(self, seq: int) -> None:
        """Drop every reference of ``seq`` and retire its id."""
        self.truncate(seq, 0)
        del self._tables[seq]
        del self._lens[seq]

    def share_prefix(self, child: int, parent: int, n_tokens: int) -> None:
        """Make an empty ``child`` reference the parent's first n_tokens."""
        self._check(child)
        self._check(parent)
        if child == parent:
            raise InvalidArgument("child and parent must differ")
        if self._lens[child] != 0:
            raise InvalidArgument("child must be empty")
        if n_tokens < 0 or n_tokens % self.page_size != 0 or n_tokens > self._lens[parent]:
            raise InvalidArgument("n_tokens must be whole pages within the parent")
        pages = self._tables[parent][: n_tokens // self.page_size]
        for page in pages:
            self.refcount[page] += 1
        self._tables[child] = list(pages)
        self._lens[child] = n_tokens

    def fork(self, child: int, parent: int) -> None:
        """Make an empty ``child`` reference all of the parent's pages (two
        responses to one input share its blocks, the last partial one too)."""
        self._check(child)
        self._check(parent)
        if child == parent:
            raise InvalidArgument("child and parent must differ")
        if self._lens[child] != 0:
            raise InvalidArgument("child must be empty")
        for page in self._tables[parent]:
            self.refcount[page] += 1
        self._tables[child] = list(self._tables[parent])
        self._lens[child] = self._lens[parent]

    def reserve_cow(self, seq: int, n: int) -> Optional[Tuple[int, int]]:
        """reserve() with copy-on-write: when the first new position falls in
        a partially filled page that other sequences also reference, ``seq``
        first takes a fresh page, its table points there, and (shared page,
        fresh page) is returned: the device must copy the shared page into the
        fresh one before anything is written to it.  All-or-nothing."""
        self._check(seq)
        if n < 0:
            raise InvalidArgument("n must be >= 0")
        length = self._lens[seq]
        table = self._tables[seq]
        ps = self.page_size
        copy_needed = n > 0 and length % ps != 0 and self.refcount[table[length // ps]] > 1
        need = ceil_div(length + n, ps) - len(table) + (1 if copy_needed else 0)
        if need > len(self._free):
            raise OutOfPages(f"need {need} pages, {len(self._free)} free")
        copy = None
        if copy_needed:
            shared = table[length // ps]
            fresh = self._free.pop()
            self.refcount[shared] -= 1
            self.refcount[fresh] = 1
            table[length // ps] = fresh
            copy = (shared, fresh)
        self.reserve(seq, n)
        return copy

    def _check(self, seq: int) -> None:
        if seq not in self._tables:
            raise InvalidArgument(f"unknown sequence {seq}")


def store_rows(pool, slots: Sequence[int], rows) -> None:
    """Write rows[t] ([Hkv][D]) into ``pool`` ([num_pages][Hkv][ps][D]) at slots[t].

    The plain statement of TileInfer.jl's store_kv! ("Pages and block
    tables"): each new token's vectors go to its slot's page and offset, for
    every KV head.  Slots outside the pool are skipped.
    """
    page_size = pool.shape[2]
    limit = pool.shape[0] * page_size
    for t, slot in enumerate(slots):
        slot = int(slot)
        if 0 <= slot < limit:
            pool[slot // page_size, :, slot % page_size, :] = rows[t]


def copy_pages(pool, copies: Sequence[Tuple[int, int]]) -> None:
    """The device half of copy-on-write: page dst of ``pool`` (every KV head,
    every offset) becomes a copy of page src, for each (src, dst)."""
    for src, dst in copies:
        pool[int(dst)] = pool[int(src)]

