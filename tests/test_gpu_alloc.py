"""GPU parity of the device slot allocator and row writing against the
oracle ([XPU] "How SGLang stores the KV cache: two pools and a page size").
Everything here is integer work: slots, ring contents, ring state and table
rows must match bit for bit.  Batches span several 256-request scan chunks
and several token blocks; rings wrap past their end."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_38_amd as P
from workloads.alloc import growth_batch, serving_alloc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def device_ring(b):
    """A FreeList holding batch b's ring, plus the oracle's copy."""
    fl = P.kv_free_list_create(b.page_size, b.num_pages, capacity=b.capacity, count=0, device=DEV)
    fl.pages.copy_(torch.from_numpy(b.ring_buffer()))
    fl.state.copy_(torch.tensor([b.head, len(b.free)], dtype=torch.int32))
    ring = oracle.FreeRing(b.free.tolist(), b.capacity, head=b.head)
    return fl, ring


def t32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def assert_ring_equal(fl, ring, what):
    torch.cuda.synchronize()
    head, size = fl.state.cpu().tolist()
    assert (head, size) == (ring.head, ring.size), f"{what}: state {(head, size)} vs {(ring.head, ring.size)}"
    assert np.array_equal(fl.pages.cpu().numpy(), ring.buf.astype(np.int32)), f"{what}: ring contents differ"


def status(fl):
    torch.cuda.synchronize()
    return int(fl.status.item())


@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("bs", [5, 300])
def test_alloc_extend_matches_oracle(page_size, bs):
    b = growth_batch(seed=bs + page_size, bs=bs, page_size=page_size, max_prefix=300, max_new=160,
                     num_free=bs * 200 // page_size + 50)
    print(f"alloc_extend ps {page_size} bs {bs} new {int((b.seq_lens - b.prefix_lens).sum())}", flush=True)
    fl, ring = device_ring(b)
    want = oracle.alloc_extend(ring, page_size, b.prefix_lens, b.seq_lens, b.last_loc)
    assert want is not None
    out = torch.full((len(want) + 9,), -5, dtype=torch.int32, device=DEV)
    P.kv_alloc_extend(fl, t32(b.prefix_lens), t32(b.seq_lens), t32(b.last_loc), out)
    assert status(fl) == P.PKV_ALLOC_OK
    got = out.cpu().numpy()
    assert np.array_equal(got[:len(want)], want.astype(np.int32))
    assert (got[len(want):] == -5).all()
    assert_ring_equal(fl, ring, "alloc_extend")


@pytest.mark.parametrize("page_size", [1, 16])
@pytest.mark.parametrize("bs", [1, 700, 8000])
def test_alloc_decode_matches_oracle(page_size, bs):
    b = growth_batch(seed=bs, bs=bs, page_size=page_size, max_prefix=500, max_new=1,
                     num_free=bs // 2 + bs // page_size + 20, decode=True)
    print(f"alloc_decode ps {page_size} bs {bs}", flush=True)
    fl, ring = device_ring(b)
    want = oracle.alloc_decode(ring, page_size, b.seq_lens, b.last_loc)
    assert want is not None
    out = torch.full((bs,), -5, dtype=torch.int32, device=DEV)
    P.kv_alloc_decode(fl, t32(b.seq_lens), t32(b.last_loc), out)
    assert status(fl) == P.PKV_ALLOC_OK
    assert np.array_equal(out.cpu().numpy(), want.astype(np.int32))
    assert_ring_equal(fl, ring, "alloc_decode")


def test_denied_allocations_change_nothing():
    b = growth_batch(seed=9, bs=40, page_size=16, max_prefix=100, max_new=90, num_free=60)
    fl, ring = device_ring(b)
    need = sum(oracle.new_pages_needed(int(p), int(s), 16) for p, s in zip(b.prefix_lens, b.seq_lens))
    assert need > len(b.free)  # too few pages
    new = int((b.seq_lens - b.prefix_lens).sum())
    out = torch.full((max(new, 16 * (len(b.free) + 1)),), -5, dtype=torch.int32, device=DEV)
    pre, seq, last = t32(b.prefix_lens), t32(b.seq_lens), t32(b.last_loc)
    cases = [
        ("no space", lambda: P.kv_alloc_extend(fl, pre, seq, last, out), P.PKV_ALLOC_NO_SPACE),
        ("out capacity", lambda: P.kv_alloc_extend(fl, pre, seq, last, out[:new - 1]), P.PKV_ALLOC_OUT_CAPACITY),
        ("bad lengths", lambda: P.kv_alloc_extend(fl, seq, pre, last, out), P.PKV_ALLOC_BAD_LENGTHS),
        ("decode from 0", lambda: P.kv_alloc_decode(fl, t32(np.zeros(40)), last, out), P.PKV_ALLOC_BAD_LENGTHS),
        ("aligned alloc", lambda: P.kv_alloc(fl, 16 * (len(b.free) + 1), out), P.PKV_ALLOC_NO_SPACE),
    ]
    for what, call, code in cases:
        call()
        assert status(fl) == code, what
        assert (out.cpu().numpy() == -5).all(), what
        assert_ring_equal(fl, ring, what)
    # an empty batch is granted and takes nothing
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    P.kv_alloc_extend(fl, e, e, e, out)
    assert status(fl) == P.PKV_ALLOC_OK
    assert_ring_equal(fl, ring, "empty batch")


@pytest.mark.parametrize("page_size", [1, 64])
def test_page_aligned_alloc_matches_oracle(page_size):
    b = growth_batch(seed=2, bs=0, page_size=page_size, max_prefix=1, max_new=1, num_free=3000)
    fl, ring = device_ring(b)
    for n in (0, 1, 777, 1500):
        want = oracle.alloc(ring, page_size, n * page_size)
        out = torch.full((n * page_size + 3,), -5, dtype=torch.int32, device=DEV)
        P.kv_alloc(fl, n * page_size, out)
        assert status(fl) == P.PKV_ALLOC_OK
        got = out.cpu().numpy()
        assert np.array_equal(got[:n * page_size], want.astype(np.int32)) and (got[n * page_size:] == -5).all()
        assert_ring_equal(fl, ring, f"alloc {n} pages")


@pytest.mark.parametrize("page_size", [1, 16])
def test_free_matches_oracle(page_size):
    rng = np.random.default_rng(page_size)
    num_pages = 40000  # bitmap of 1250 words: more than one pass of the compacting block
    free = rng.permutation(num_pages)[:5000].astype(np.int32)
    cap = 12000
    fl = P.kv_free_list_create(page_size, num_pages, capacity=cap, count=0, device=DEV)
    ring = oracle.FreeRing(free.tolist(), cap, head=cap - 100)
    fl.pages.copy_(torch.from_numpy(ring.buf.astype(np.int32)))
    fl.state.copy_(torch.tensor([ring.head, ring.size], dtype=torch.int32))
    owned = np.setdiff1d(np.arange(num_pages), free)
    pick = rng.choice(owned, 3000, replace=False)
    slots = (pick[:, None] * page_size + rng.integers(0, page_size, (3000, 2))).reshape(-1)
    slots = np.concatenate([slots, slots[:50], [-1, -7, num_pages * page_size, num_pages * page_size + page_size - 1]])
    rng.shuffle(slots)
    kept = slots[(slots >= 0) & (slots // page_size < num_pages)]
    assert oracle.free_pages(ring, oracle.pages_of_slots(kept, page_size))
    P.kv_free(fl, t32(slots))
    assert status(fl) == P.PKV_ALLOC_OK
    assert_ring_equal(fl, ring, "free")
    # a free that would overflow the ring is refused whole
    more = np.setdiff1d(owned, pick)[: cap - ring.size + 1] * page_size
    P.kv_free(fl, t32(more))
    assert status(fl) == P.PKV_ALLOC_RING_FULL
    assert_ring_equal(fl, ring, "ring full")
    # and an empty free is a no-op
    P.kv_free(fl, torch.empty(0, dtype=torch.int32, device=DEV))
    assert status(fl) == P.PKV_ALLOC_OK
    assert_ring_equal(fl, ring, "empty free")


def test_free_list_init_matches_clear():
    fl = P.kv_free_list_create(1, 5000, capacity=6000, first=1, count=5000, device=DEV)
    ring = oracle.FreeRing(list(range(1, 5001)), 6000)
    torch.cuda.synchronize()
    assert fl.state.cpu().tolist() == [ring.head, ring.size]
    assert np.array_equal(fl.pages.cpu().numpy()[:5000], ring.buf[:5000].astype(np.int32))


@pytest.mark.parametrize("with_prefix", [False, True])
def test_write_req_to_token_matches_oracle(with_prefix):
    rng = np.random.default_rng(11)
    rows, width, bs = 50, 3100, 37
    table = rng.integers(-9, 10**6, (rows, width)).astype(np.int32)
    rpi = rng.permutation(rows)[:bs]
    prefix = rng.integers(0, 2000, bs)
    seq = prefix + rng.integers(0, 1100, bs)
    prefix[0], seq[0] = 0, 1024  # exactly one chunk
    seq[1] = prefix[1]           # nothing new
    seq[2] = width               # the full row
    new = (seq - prefix).astype(np.int64)
    out_cache_loc = rng.integers(0, 10**6, int(new.sum())).astype(np.int32)
    pre = [rng.integers(0, 10**6, p).astype(np.int32) if (with_prefix and i % 5) else None
           for i, p in enumerate(prefix)]
    pre_or = [np.asarray(x) if x is not None else table[rpi[i], :prefix[i]] for i, x in enumerate(pre)]
    want = oracle.write_req_to_token(table, rpi, prefix, seq, out_cache_loc, pre_or if with_prefix else None)
    dt = t32(table)
    pre_dev = [t32(x) if x is not None else None for x in pre]
    P.write_req_to_token(dt, t32(rpi), t32(prefix), t32(seq), t32(out_cache_loc), int(seq.max()),
                         prefix_ptrs=pre_dev if with_prefix else None)
    torch.cuda.synchronize()
    assert np.array_equal(dt.cpu().numpy(), want.astype(np.int32))


@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_serving_schedule_matches_oracle(page_size):
    """Requests arrive, prefill in chunks, decode and finish, through the
    device allocator and row writing, side by side with the oracle; table,
    ring and status agree after every step."""
    rng = np.random.default_rng(100 + page_size)
    num_pages = 2000 // page_size + 40
    width, nrows = 400, 12
    fl = P.kv_free_list_create(page_size, num_pages, device=DEV)
    ring = oracle.FreeRing(list(range(num_pages)), num_pages)
    table = np.full((nrows, width), -1, np.int64)
    dt = torch.full((nrows, width), -1, dtype=torch.int32, device=DEV)
    live = {}
    for step in range(40):
        free_rows = [r for r in range(nrows) if r not in live]
        if free_rows and rng.random() < 0.5:
            live[free_rows[0]] = 0
        if not live:
            continue
        batch = sorted(live)
        prefix = np.array([live[r] for r in batch])
        grow = rng.integers(1, 60, len(batch)) if rng.random() < 0.4 else np.ones(len(batch), np.int64)
        seq = np.minimum(prefix + grow, width)
        last = np.array([table[r, p - 1] if p else -1 for r, p in zip(batch, prefix)])
        want = oracle.alloc_extend(ring, page_size, prefix, seq, last)
        out = torch.empty(int((seq - prefix).sum()), dtype=torch.int32, device=DEV)
        P.kv_alloc_extend(fl, t32(prefix), t32(seq), t32(last), out)
        st = status(fl)
        if want is None:
            assert st == P.PKV_ALLOC_NO_SPACE, f"step {step}"
        else:
            assert st == P.PKV_ALLOC_OK, f"step {step}"
            assert np.array_equal(out.cpu().numpy(), want.astype(np.int32)), f"step {step}"
            table = oracle.write_req_to_token(table, batch, prefix, seq, want)
            P.write_req_to_token(dt, t32(batch), t32(prefix), t32(seq), out, width)
            for r, s in zip(batch, seq):
                live[r] = int(s)
        for r in [r for r in batch if live[r] >= width or rng.random() < 0.08]:
            slots = table[r, :live[r]]
            assert oracle.free_pages(ring, oracle.pages_of_slots(slots, page_size))
            P.kv_free(fl, dt[r, :live[r]].contiguous())
            assert status(fl) == P.PKV_ALLOC_OK, f"step {step}"
            table[r] = -1
            dt[r] = -1
            del live[r]
        torch.cuda.synchronize()
        assert np.array_equal(dt.cpu().numpy(), table.astype(np.int32)), f"step {step}"
        assert_ring_equal(fl, ring, f"step {step}")


@pytest.mark.parametrize("decode", [True, False])
def test_serving_alloc_full_size(decode):
    """The allocator's benchmark steps at full size (decode: 4096 requests
    each opening a page; extend: 64 requests growing by up to 2048 tokens;
    a 65536-page pool), in bench.py's call sequence -- alloc, row write,
    free of the same slots -- twice, so the second step starts from a ring
    the first one advanced.  Slots, table, ring and status bit for bit."""
    w = serving_alloc(decode)
    bs = len(w.seq_lens)
    print(f"full-size allocation step (decode={decode}): {bs} requests", flush=True)
    fl = P.kv_free_list_create(w.page_size, w.num_pages, device=DEV)
    ring = oracle.FreeRing(list(range(w.num_pages)), w.num_pages)
    new = int((w.seq_lens - w.prefix_lens).sum())
    out = torch.empty(new, dtype=torch.int32, device=DEV)
    dt = torch.zeros((bs + 1, w.table_width), dtype=torch.int32, device=DEV)
    table = np.zeros((bs + 1, w.table_width), np.int64)
    last = np.full(bs, -1)
    for step in range(2):
        if decode:
            P.kv_alloc_decode(fl, t32(w.seq_lens), t32(last), out)
        else:
            P.kv_alloc_extend(fl, t32(w.prefix_lens), t32(w.seq_lens), t32(last), out)
        P.write_req_to_token(dt, t32(w.req_pool_indices), t32(w.prefix_lens), t32(w.seq_lens), out,
                             int(w.seq_lens.max()))
        P.kv_free(fl, out)
        want = oracle.alloc_extend(ring, w.page_size, w.prefix_lens, w.seq_lens, last)
        table = oracle.write_req_to_token(table, w.req_pool_indices, w.prefix_lens, w.seq_lens, want)
        assert oracle.free_pages(ring, oracle.pages_of_slots(want, w.page_size))
        assert status(fl) == P.PKV_ALLOC_OK, f"step {step}"
        assert np.array_equal(out.cpu().numpy(), want.astype(np.int32)), f"step {step}: slots"
        assert np.array_equal(dt.cpu().numpy(), table.astype(np.int32)), f"step {step}: table"
        assert_ring_equal(fl, ring, f"step {step}")
