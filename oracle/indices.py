"""Index math of the paged KV cache (oracle; test infrastructure only).

Closed-form integer code for what each table holds:

* [XPU] "From slots to a page table: how attention reads the cache": a key at
  logical position ``t`` lives at slot ``page_table[req, t // ps] * ps +
  t % ps``; the page table is recovered from the token-granular
  ``req_to_token`` by taking every ``ps``-th column and dividing by ``ps``
  (the identity at ``ps == 1``).  This needs a request's tokens to be
  contiguous inside each page ([XPU] "How SGLang stores the KV cache").
* [BACKEND] "kv_indptr 和 kv_indices": ``kv_indptr`` (``[bs+1]``) is the
  prefix sum of per-request page counts and ``kv_indices`` lists each
  request's page ids in order; "init_forward_metadata()": the padded block
  table is ``[bs, ceil(max_len / ps)]`` filled with ``-1`` and then with each
  request's page ids.
* [BACKEND] "例子": ``qo_indptr`` is the prefix sum of ``seq_lens -
  prefix_lens``.
* [XPU] "Approach 1: page-align the encoder": ``ceil_align(x, ps)``.
"""
from typing import List, Sequence

import numpy as np


def ceil_div(a, b):
    return -(-np.asarray(a, dtype=np.int64) // int(b))


def ceil_align(x, a: int):
    """Smallest multiple of ``a`` that is >= ``x`` ([XPU] Approach 1)."""
    return ceil_div(x, a) * int(a)


def page_ids_from_token_table(req_to_token: np.ndarray, row: int, kv_start: int, kv_len: int,
                              page_size: int) -> np.ndarray:
    """Page ids covering columns ``[kv_start, kv_start + kv_len)`` of one row:
    every ``page_size``-th column, divided by ``page_size``."""
    cols = int(kv_start) + np.arange(0, int(kv_len), int(page_size), dtype=np.int64)
    return (np.asarray(req_to_token)[int(row), cols].astype(np.int64) // int(page_size)).astype(np.int32)


def build_csr(req_to_token, req_pool_indices, kv_start, kv_lens, page_size):
    """(kv_indptr [bs+1], kv_indices [sum pages]) for page-granular access."""
    bs = len(kv_lens)
    starts = np.zeros(bs, np.int64) if kv_start is None else np.asarray(kv_start, np.int64)
    lists = [page_ids_from_token_table(req_to_token, req_pool_indices[i], starts[i], kv_lens[i], page_size)
             for i in range(bs)]
    counts = np.array([len(x) for x in lists], dtype=np.int64)
    kv_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    kv_indices = (np.concatenate(lists) if bs else np.zeros(0)).astype(np.int32)
    return kv_indptr, kv_indices


def build_block_table(req_to_token, req_pool_indices, kv_start, kv_lens, page_size, max_blocks):
    """``[bs, max_blocks]`` int32: each request's page ids, then ``-1``."""
    bs = len(kv_lens)
    starts = np.zeros(bs, np.int64) if kv_start is None else np.asarray(kv_start, np.int64)
    out = np.full((bs, int(max_blocks)), -1, dtype=np.int32)
    for i in range(bs):
        ids = page_ids_from_token_table(req_to_token, req_pool_indices[i], starts[i], kv_lens[i], page_size)
        assert len(ids) <= max_blocks, "block table too narrow"
        out[i, :len(ids)] = ids
    return out


def last_page_len(kv_lens, page_size):
    """Valid tokens on each request's last page; 0 for an empty request."""
    L = np.asarray(kv_lens, dtype=np.int64)
    n = ceil_div(L, page_size)
    return np.where(L > 0, L - (n - 1) * int(page_size), 0).astype(np.int32)


def slots_from_token_table(req_to_token, row, kv_start, kv_len) -> np.ndarray:
    """Slots of logical tokens 0..kv_len-1 read straight from the token table."""
    return np.asarray(req_to_token)[int(row), int(kv_start):int(kv_start) + int(kv_len)].astype(np.int64)


def slots_from_pages(page_ids, page_size, kv_len) -> np.ndarray:
    """slot(t) = page_ids[t // ps] * ps + t % ps for t < kv_len ([XPU])."""
    t = np.arange(int(kv_len), dtype=np.int64)
    pid = np.asarray(page_ids, dtype=np.int64)[t // int(page_size)]
    assert (pid >= 0).all(), "a -1 (unused) block-table entry inside a request's length"
    return pid * int(page_size) + t % int(page_size)


def slots_from_csr(kv_indptr, kv_indices, i, page_size, kv_len) -> np.ndarray:
    a, b = int(kv_indptr[i]), int(kv_indptr[i + 1])
    return slots_from_pages(np.asarray(kv_indices)[a:b], page_size, kv_len)


def slots_from_block_table(block_table, i, page_size, kv_len) -> np.ndarray:
    return slots_from_pages(np.asarray(block_table)[i], page_size, kv_len)


def qo_indptr(seq_lens, prefix_lens) -> np.ndarray:
    """Prefix sum of new-token counts ([BACKEND] "计算 Query/Output 指针")."""
    n = np.asarray(seq_lens, np.int64) - np.asarray(prefix_lens, np.int64)
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)


def token_indptr(lens) -> np.ndarray:
    """Prefix sum of per-request token counts (``cu_seqlens`` /
    the page_size-1 ``kv_indptr`` of [BACKEND] "计算 KV 指针")."""
    return np.concatenate([[0], np.cumsum(np.asarray(lens, np.int64))]).astype(np.int32)


def in_page_contiguous(req_to_token, rows: Sequence[int], kv_start, kv_lens, page_size) -> List[bool]:
    """Per request: do its tokens sit in consecutive slots inside every page
    and start each page at offset 0 -- the invariant page-granular access
    relies on ([XPU] "How SGLang stores the KV cache")."""
    res = []
    for i, r in enumerate(rows):
        s = slots_from_token_table(req_to_token, r, kv_start[i], kv_lens[i])
        t = np.arange(len(s), dtype=np.int64)
        pages = page_ids_from_token_table(req_to_token, r, kv_start[i], kv_lens[i], page_size).astype(np.int64)
        res.append(bool(np.array_equal(s, pages[t // page_size] * page_size + t % page_size)))
    return res
