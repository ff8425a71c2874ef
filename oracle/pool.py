"""KV pool geometry and the KV append (oracle; test infrastructure only).

[MINI] "The KV pool: one preallocated block of memory": one tensor
``[2, layers, pages, page_size, kv_heads, head_dim]`` allocated once; row ``j``
of the per-token flattening ``[pages*page_size, kv_heads, head_dim]`` is where
the pool's ``j``-th token lives; ``store_kv`` writes each new token's K and V
at its location by indexed assignment.
"""
import numpy as np


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes one token's K and V take over all layers: 2 (K and V) x layers x
    KV heads x head_dim x element size ([MINI] self-test answer 1 and the
    Llama-3.1-8B exercise)."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def tokens_that_fit(budget_bytes: int, per_token_bytes: int) -> int:
    """Whole tokens a byte budget holds ([MINI] "What it prints")."""
    return budget_bytes // per_token_bytes


def pool_shape(num_layers: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int):
    """[K/V, layer, page, offset in page, KV head, dim] ([MINI] MHAKVCache)."""
    return (2, num_layers, num_pages, page_size, num_kv_heads, head_dim)


def per_token_shape(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int):
    """One layer's buffer flattened per token ([MINI] ``_storage_shape``)."""
    return (num_pages * page_size, num_kv_heads, head_dim)


def page_of(slot, page_size: int):
    """Page holding a slot: slot // page_size ([BACKEND] "页表构建" table)."""
    return np.asarray(slot) // page_size


def offset_of(slot, page_size: int):
    """Offset of a slot inside its page: slot % page_size."""
    return np.asarray(slot) % page_size


def store(pool_flat: np.ndarray, rows: np.ndarray, out_loc: np.ndarray) -> np.ndarray:
    """Return a copy of one layer's per-token pool view with ``rows[i]``
    written at slot ``out_loc[i]`` ([MINI] ``store_cache``: ``k_cache[idx] =
    k.view(n, H, D)``).  Raw element values are copied bit for bit.

    Duplicate slots are only meaningful for writes to the padding page
    (dummy requests); numpy keeps the last writer, which is one valid
    outcome of such a race."""
    out = np.array(pool_flat, copy=True)
    idx = np.asarray(out_loc, dtype=np.int64)
    rows = np.asarray(rows).reshape((idx.shape[0],) + out.shape[1:])
    if idx.size:
        assert idx.min() >= 0 and idx.max() < out.shape[0], "slot out of range"
    out[idx] = rows
    return out
