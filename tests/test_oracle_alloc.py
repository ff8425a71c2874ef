"""Pins of the oracle's slot allocation and row writing ([XPU] "How SGLang
stores the KV cache: two pools and a page size": the token and paged
allocators and write_cache_indices).  CPU only.

The batched allocation formula is checked against a token-by-token growth
simulation built on a plain deque (a new page is popped whenever a token
starts one, otherwise the token takes the slot after its predecessor), the
page-aligned expansion against numpy's repeat/tile, freeing against
numpy's unique, and a long random schedule against ownership invariants."""
from collections import deque

import numpy as np
import pytest

import oracle


def grow_token_by_token(free, page_size, prefix_lens, seq_lens, last_loc):
    """Independent restatement: each new token either opens a page (pop the
    front of the free deque) or continues the slot of the token before it."""
    out = []
    for p, s, last in zip(prefix_lens, seq_lens, last_loc):
        prev = last
        for t in range(p, s):
            if t % page_size == 0:
                prev = free.popleft() * page_size
            else:
                prev = prev + 1
            out.append(prev)
    return out


def random_batch(rng, bs, page_size, max_len, free):
    """Requests that already hold prefix_len tokens (allocated from `free`
    token by token, so last_loc is consistent) and grow to seq_len."""
    prefix = rng.integers(0, max_len, bs)
    seq = prefix + rng.integers(0, max_len, bs)
    prefix[0] = 0  # an empty prefix
    if bs > 1:
        prefix[1] = page_size * 2  # page aligned
        seq[1] = prefix[1] + 1
    if bs > 2:
        seq[2] = prefix[2]  # nothing new
    last = []
    for p in prefix:
        slots = grow_token_by_token(free, page_size, [0], [int(p)], [-1])
        last.append(slots[-1] if slots else -1)
    return prefix.tolist(), seq.tolist(), last


@pytest.mark.parametrize("page_size", [1, 2, 16, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_alloc_extend_matches_token_by_token_growth(page_size, seed):
    rng = np.random.default_rng(seed)
    num_pages = 4000 // page_size + 64
    pages = rng.permutation(num_pages).tolist()
    free = deque(pages)
    prefix, seq, last = random_batch(rng, 7, page_size, 150, free)
    remaining = list(free)
    cap = num_pages + 5
    ring = oracle.FreeRing(remaining, cap, head=int(rng.integers(0, cap)))  # wraps around the end
    got = oracle.alloc_extend(ring, page_size, prefix, seq, last)
    want = grow_token_by_token(free, page_size, prefix, seq, last)
    assert got.tolist() == want
    assert ring.contents() == list(free)


@pytest.mark.parametrize("page_size", [1, 16])
def test_alloc_decode_is_one_token_of_growth(page_size):
    rng = np.random.default_rng(3)
    free = deque(rng.permutation(600).tolist())
    prefix, _, last = random_batch(rng, 9, page_size, 100, free)
    seq = [p + 1 for p in prefix]
    ring = oracle.FreeRing(list(free), 700)
    got = oracle.alloc_decode(ring, page_size, seq, last)
    assert got.tolist() == grow_token_by_token(free, page_size, prefix, seq, last)
    assert ring.contents() == list(free)


def test_token_allocator_starts_at_one_and_pops_in_order():
    # page_size 1: the free list starts as 1 .. size (slot 0 reserved) and an
    # allocation of n returns its first n entries.
    ring = oracle.FreeRing(np.arange(1, 101).tolist(), 100)
    assert oracle.alloc(ring, 1, 5).tolist() == [1, 2, 3, 4, 5]
    assert oracle.alloc_extend(ring, 1, [0, 3], [2, 6], [-1, 9]).tolist() == [6, 7, 8, 9, 10]
    assert ring.size == 90 and ring.front(0) == 11


@pytest.mark.parametrize("page_size", [4, 64])
def test_page_aligned_alloc_expands_whole_pages(page_size):
    ring = oracle.FreeRing([9, 2, 30, 7], 8)
    got = oracle.alloc(ring, page_size, 3 * page_size)
    want = np.repeat([9, 2, 30], page_size) * page_size + np.tile(np.arange(page_size), 3)
    assert np.array_equal(got, want)
    assert ring.contents() == [7]
    # the growth path from an empty prefix takes the same slots
    ring2 = oracle.FreeRing([9, 2, 30, 7], 8)
    assert np.array_equal(oracle.alloc_extend(ring2, page_size, [0], [3 * page_size], [-1]), want)


def test_page_counts_closed_form():
    for ps in (1, 2, 16, 64):
        for p in range(0, 140, 7):
            for s in range(p, p + 140, 11):
                pages_before = -(-p // ps)
                pages_after = -(-s // ps)
                assert oracle.new_pages_needed(p, s, ps) == pages_after - pages_before
    assert oracle.new_pages_needed(16, 17, 16) == 1
    assert oracle.new_pages_needed(15, 16, 16) == 0
    assert oracle.new_pages_needed(0, 0, 16) == 0


def test_allocation_failure_takes_nothing():
    ring = oracle.FreeRing([5, 6, 7], 4, head=3)
    before = (ring.head, ring.size, ring.buf.copy())
    # needs ceil(40/16) + ceil(10/16) = 4 pages, 3 are free
    assert oracle.alloc_extend(ring, 16, [0, 0], [40, 10], [-1, -1]) is None
    assert oracle.alloc(ring, 16, 64) is None
    assert (ring.head, ring.size) == before[:2] and np.array_equal(ring.buf, before[2])
    # exactly the free count succeeds and empties the ring
    got = oracle.alloc_extend(ring, 16, [0, 0], [32, 8], [-1, -1])
    assert ring.size == 0 and len(got) == 40


def test_free_returns_sorted_distinct_pages_to_the_back():
    ps = 16
    ring = oracle.FreeRing([100, 101], 16)
    slots = np.array([3 * ps + 1, 7 * ps, 3 * ps + 5, 7 * ps + 15, 1 * ps + 2, 3 * ps + 1])
    pages = oracle.pages_of_slots(slots, ps)
    assert pages.tolist() == np.unique(slots // ps).tolist() == [1, 3, 7]
    assert oracle.free_pages(ring, pages)
    assert ring.contents() == [100, 101, 1, 3, 7]
    # the older free pages are handed out first
    assert oracle.alloc(ring, ps, 2 * ps)[::ps].tolist() == [100 * ps, 101 * ps]
    # a free that does not fit changes nothing
    full = oracle.FreeRing(list(range(4)), 5)
    assert not oracle.free_pages(full, [9, 10])
    assert full.contents() == [0, 1, 2, 3]


def test_write_req_to_token_rows():
    rng = np.random.default_rng(4)
    table = np.full((6, 40), -3, np.int64)
    rows = [4, 1, 5]
    prefix = [0, 7, 12]
    seq = [9, 7, 30]
    new = [s - p for p, s in zip(prefix, seq)]
    out_cache_loc = rng.integers(0, 1000, sum(new))
    pre = [rng.integers(1000, 2000, p) for p in prefix]
    got = oracle.write_req_to_token(table, rows, prefix, seq, out_cache_loc, pre)
    pieces = np.split(out_cache_loc, np.cumsum(new)[:-1])
    for r, p, s, piece, pr in zip(rows, prefix, seq, pieces, pre):
        assert np.array_equal(got[r, :s], np.concatenate([pr, piece]))
        assert (got[r, s:] == -3).all()
    untouched = [r for r in range(6) if r not in rows]
    assert (got[untouched] == -3).all()
    # without prefix slots the prefix columns keep what the row held
    got2 = oracle.write_req_to_token(got, rows, prefix, seq, out_cache_loc[::-1].copy())
    for r, p in zip(rows, prefix):
        assert np.array_equal(got2[r, :p], got[r, :p])


@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_random_schedule_keeps_ownership_invariants(page_size):
    """Requests arrive, prefill in chunks, decode and finish; every page is
    either free or owned by exactly one request, every row is contiguous
    inside its pages, and freeing everything restores the full free list."""
    rng = np.random.default_rng(page_size)
    num_pages = 3000 // page_size + 40
    ring = oracle.FreeRing(list(range(num_pages)), num_pages)
    width = 600
    table = np.full((12, width), -1, np.int64)
    live = {}  # row -> length
    for step in range(120):
        rows = [r for r in range(12) if r not in live]
        if rows and rng.random() < 0.4:
            live[rows[0]] = 0
        if not live:
            continue
        batch = sorted(live)
        prefix = [live[r] for r in batch]
        grow = rng.integers(1, 40, len(batch)) if rng.random() < 0.3 else np.ones(len(batch), np.int64)
        seq = [min(p + int(g), width) for p, g in zip(prefix, grow)]
        last = [int(table[r, p - 1]) if p else -1 for r, p in zip(batch, prefix)]
        slots = oracle.alloc_extend(ring, page_size, prefix, seq, last)
        if slots is not None:
            table = oracle.write_req_to_token(table, batch, prefix, seq, slots)
            for r, s in zip(batch, seq):
                live[r] = s
        done = [r for r in batch if live[r] >= width or rng.random() < 0.05]
        for r in done:
            assert oracle.free_pages(ring, oracle.pages_of_slots(table[r, :live[r]], page_size))
            table[r] = -1
            del live[r]
        owned = []
        for r, L in live.items():
            assert oracle.in_page_contiguous(table, [r], [0], [L], page_size) == [True]
            owned += oracle.pages_of_slots(table[r, :L], page_size).tolist()
        assert len(owned) == len(set(owned))
        assert sorted(owned + ring.contents()) == list(range(num_pages))
    for r, L in list(live.items()):
        oracle.free_pages(ring, oracle.pages_of_slots(table[r, :L], page_size))
    assert sorted(ring.contents()) == list(range(num_pages))
