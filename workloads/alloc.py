"""Seeded inputs for slot allocation: a shuffled free list of page ids
(taken as a ring that wraps past its end) and a batch of requests that
already hold some tokens and grow.  Inputs only: no allocation arithmetic.

A request holding p > 0 tokens gets its own held page, outside the free
list, and last_loc is the slot of its token p - 1 on that page (page *
page_size + (p - 1) % page_size), as a page-contiguous row would have it."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class GrowthBatch:
    page_size: int
    num_pages: int        # page ids are 0 .. num_pages - 1
    capacity: int         # ring slots
    head: int             # ring index of the first free entry
    free: np.ndarray      # free page ids, front first
    prefix_lens: np.ndarray
    seq_lens: np.ndarray
    last_loc: np.ndarray

    def ring_buffer(self) -> np.ndarray:
        buf = np.full(self.capacity, -1, np.int32)
        idx = (self.head + np.arange(len(self.free))) % self.capacity
        buf[idx] = self.free
        return buf


def growth_batch(seed: int, bs: int, page_size: int, max_prefix: int, max_new: int, num_free: int,
                 spare: int = 7, decode: bool = False) -> GrowthBatch:
    """bs requests with prefix lengths in [0, max_prefix) (the first empty,
    the second page aligned, the third mid-page, one growing by nothing when
    bs > 3) that grow by [1, max_new) tokens (exactly one when decode);
    num_free shuffled free pages in a ring of num_free + spare entries whose
    head sits near its end, so the batch's pages wrap around."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, max_prefix, bs).astype(np.int64)
    new = np.ones(bs, np.int64) if decode else rng.integers(1, max(max_new, 2), bs).astype(np.int64)
    if bs > 0 and not decode:
        prefix[0] = 0
    if bs > 1:
        prefix[1] = 2 * page_size
    if bs > 2:
        prefix[2] = page_size + page_size // 2 + 1 if page_size > 1 else 5
    if bs > 3 and not decode:
        new[3] = 0
    if decode:
        prefix = np.maximum(prefix, 0)
    seq = prefix + new
    num_pages = num_free + bs + 1
    ids = rng.permutation(num_pages)
    free, held = ids[:num_free], ids[num_free:num_free + bs]
    last = np.where(prefix > 0, held * page_size + (prefix - 1) % page_size, -1)
    cap = num_free + spare
    head = cap - min(3, cap)
    return GrowthBatch(page_size, num_pages, cap, head, free.astype(np.int32), prefix.astype(np.int32),
                       seq.astype(np.int32), last.astype(np.int32))


@dataclass
class ServingAlloc:
    """One serving step's allocation work: bs requests holding page-aligned
    prefixes grow by new_lens tokens (one each for decode)."""
    page_size: int
    num_pages: int
    prefix_lens: np.ndarray
    seq_lens: np.ndarray
    req_pool_indices: np.ndarray
    table_width: int


def serving_alloc(decode: bool, seed: int = 0) -> ServingAlloc:
    """Decode: 4096 requests, page_size 16, prefixes page aligned in
    [512, 4096), so every request opens a new page (the allocator's busiest
    decode step).  Extend: 64 requests, page_size 16, page-aligned prefixes
    in [0, 4096) growing by U[1, 2048] tokens.  A 65536-page (1M-slot) pool;
    rows are a seeded shuffle of a 4097- or 65-row table of width 8192."""
    rng = np.random.default_rng(seed)
    ps = 16
    bs = 4096 if decode else 64
    lo = 512 if decode else 0
    prefix = rng.integers(lo // ps, 4096 // ps, bs) * ps
    new = np.ones(bs, np.int64) if decode else rng.integers(1, 2049, bs)
    rpi = rng.permutation(bs + 1)[:bs]
    return ServingAlloc(ps, 65536, prefix.astype(np.int32), (prefix + new).astype(np.int32), rpi.astype(np.int32),
                        8192)
