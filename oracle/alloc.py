"""Slot allocation and row writing -- TEST INFRASTRUCTURE ONLY (part of the
oracle; see the package docstring).

What the pages describe ([XPU] "How SGLang stores the KV cache: two pools and
a page size", its token and paged allocators and write_cache_indices; [BACKEND]
the opening table, page-aligned allocation row):

* The free list holds page ids (slots when page_size is 1).  Allocation takes
  entries from its front, in order; freeing puts page ids back at its end.
  Here it is a ring of fixed capacity: ``pages[(head + k) % capacity]`` for
  ``k < size`` are the free entries, front first.
* ``alloc`` (page aligned) takes ``need / page_size`` pages from the front
  and expands each page p to the slots ``p * page_size + offset``.
* ``alloc_extend`` / ``alloc_decode`` grow each request from ``prefix_len``
  to ``seq_len`` tokens: the free part of the request's last, partially used
  page is filled first (the slots right after ``last_loc``), then whole new
  pages are taken for the rest, request after request.  A new page p gives
  slots ``p * page_size + offset``, so every page of a request holds
  consecutive logical positions.  When the free list is too short nothing is
  taken and the call reports it (the pages' ``None`` back-pressure).
* ``write_req_to_token`` fills each request's table row: its reused prefix
  slots in columns ``[0, prefix_len)`` and its freshly allocated slots in
  ``[prefix_len, seq_len)``, taken from the batch's ``out_cache_loc`` in
  request order.

Plain Python loops, sized for small inputs.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .indices import ceil_div


class FreeRing:
    """Free page ids, front at ``head``: entries ``(head + k) % capacity``
    for ``k < size``."""

    def __init__(self, pages: Sequence[int], capacity: int, head: int = 0):
        assert len(pages) <= capacity
        self.capacity = capacity
        self.buf = np.full(capacity, -1, np.int64)
        self.head = head % capacity
        self.size = len(pages)
        for k, p in enumerate(pages):
            self.buf[(self.head + k) % capacity] = p

    def front(self, k: int) -> int:
        """k-th free entry from the front."""
        assert 0 <= k < self.size
        return int(self.buf[(self.head + k) % self.capacity])

    def contents(self) -> List[int]:
        return [self.front(k) for k in range(self.size)]


def new_pages_needed(prefix_len: int, seq_len: int, page_size: int) -> int:
    """Whole pages a request takes when it grows from prefix_len to seq_len:
    the pages its longer length spans minus those it already holds."""
    return ceil_div(seq_len, page_size) - ceil_div(prefix_len, page_size)


def alloc(ring: FreeRing, page_size: int, need: int) -> Optional[np.ndarray]:
    """Page-aligned allocation of ``need`` slots (a multiple of page_size):
    the first need / page_size free pages, each expanded to its slots; None
    (ring untouched) when too few are free."""
    assert need % page_size == 0
    n = need // page_size
    if n > ring.size:
        return None
    pages = [ring.front(k) for k in range(n)]
    ring.head = (ring.head + n) % ring.capacity
    ring.size -= n
    return np.asarray([p * page_size + o for p in pages for o in range(page_size)], np.int64)


def alloc_extend(ring: FreeRing, page_size: int, prefix_lens: Sequence[int], seq_lens: Sequence[int],
                 last_loc: Sequence[int]) -> Optional[np.ndarray]:
    """Slots for every new token of the batch (request after request), or
    None -- with the ring untouched -- when the ring holds too few pages.
    ``last_loc[i]`` is the slot of request i's last cached token (ignored
    when its prefix is empty)."""
    need = [new_pages_needed(int(p), int(s), page_size) for p, s in zip(prefix_lens, seq_lens)]
    if sum(need) > ring.size:
        return None
    out = []
    taken = 0  # pages taken by earlier requests
    for i, (p, s) in enumerate(zip(prefix_lens, seq_lens)):
        p, s = int(p), int(s)
        held = ceil_div(p, page_size)  # pages the request already holds
        for t in range(p, s):
            page_idx = t // page_size
            if page_idx < held:  # the free part of the last page
                page = int(last_loc[i]) // page_size
            else:
                page = ring.front(taken + page_idx - held)
            out.append(page * page_size + t % page_size)
        taken += need[i]
    ring.head = (ring.head + taken) % ring.capacity
    ring.size -= taken
    return np.asarray(out, np.int64)


def alloc_decode(ring: FreeRing, page_size: int, seq_lens: Sequence[int], last_loc: Sequence[int]):
    """One new token per request: alloc_extend from seq_len - 1 to seq_len."""
    return alloc_extend(ring, page_size, [int(s) - 1 for s in seq_lens], seq_lens, last_loc)


def free_pages(ring: FreeRing, page_ids: Sequence[int]) -> bool:
    """Put page ids back at the end of the ring (False, untouched, if they
    do not fit)."""
    if ring.size + len(page_ids) > ring.capacity:
        return False
    for k, p in enumerate(page_ids):
        ring.buf[(ring.head + ring.size + k) % ring.capacity] = int(p)
    ring.size += len(page_ids)
    return True


def pages_of_slots(slots: Sequence[int], page_size: int) -> np.ndarray:
    """The distinct pages a set of freed slots occupies (what goes back to
    the free list), in increasing order."""
    return np.unique(np.asarray(slots, np.int64) // page_size)


def write_req_to_token(req_to_token: np.ndarray, req_pool_indices: Sequence[int], prefix_lens: Sequence[int],
                       seq_lens: Sequence[int], out_cache_loc: Sequence[int],
                       prefix_slots: Optional[Sequence[Sequence[int]]] = None) -> np.ndarray:
    """A copy of the table with every request's row written: prefix slots
    (when given) in [0, prefix_len), then its new slots in [prefix_len,
    seq_len) from out_cache_loc, request after request."""
    table = np.array(req_to_token, copy=True)
    pt = 0
    for i, (p, s) in enumerate(zip(prefix_lens, seq_lens)):
        r, p, s = int(req_pool_indices[i]), int(p), int(s)
        if prefix_slots is not None:
            table[r, :p] = np.asarray(prefix_slots[i])[:p]
        table[r, p:s] = np.asarray(out_cache_loc)[pt:pt + s - p]
        pt += s - p
    return table
