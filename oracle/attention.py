"""Softmax attention over gathered K/V, in fp64 (oracle; test infrastructure
only).

What the paged kernels must reproduce, for each request ``i`` with ``n_i``
query tokens and ``L_i`` keys, each query head ``h`` reading KV head
``h // (Hq / Hkv)`` (contiguous grouping):

    s[j, t] = scale * <q[j, h], K[t, g]>          t < L_i, visible(j, t)
    o[j, h] = sum_t exp(s[j, t] - m) V[t, g] / sum_t exp(s[j, t] - m)
    lse[j, h] = m + log(sum_t exp(s[j, t] - m)),   m = max_t s[j, t]

Visibility: non-causal -> every key; causal -> bottom-right alignment, the
``j``-th of ``n`` new queries sits at position ``L - n + j`` and sees keys
``0 .. L - n + j`` (the vLLM-Omni notes, "Attention execution": a causal
segment ``Q[s:e]`` sees ``K[:e]``; decode is the case ``n = 1``).  A query
with no visible key (``L = 0``) gets ``o = 0`` and ``lse = -inf`` (the SGLang
encoder-decoder post, "Approach 2": an empty KV returns a zero context).

Keys and values are the exact stored values, gathered by slot: paged and
dense attention describe the same result ([OMNI] "Dense and paged
representation").

Softcap (the SGLang encoder-decoder post, "Approach 2": the ragged call passes
``softcap``; the pages do not define it, so the plainest reading is taken):
with ``softcap > 0`` every scaled score becomes ``softcap * tanh(s /
softcap)`` before the softmax; ``0`` leaves the scores as they are.

Mixed spans ([OMNI] "Attention execution"): a row's tokens fall into causal
and full spans; a causal span ``[s, e)`` is the segment ``Q[s:e]`` over
``K[:e]`` with the causal flag, a full span ``[a, b)`` is ``Q[a:b]`` over
``K[:b]`` without it.  Each segment is then an ordinary request.
"""
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .numerics import to_f64


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool,
           softcap: float = 0.0) -> Tuple[np.ndarray, np.ndarray]:
    """One request.  q ``[n, Hq, Dqk]``, K ``[L, Hkv, Dqk]``, V ``[L, Hkv, Dv]``
    (float64).  Returns out ``[n, Hq, Dv]`` and lse ``[n, Hq]`` (natural log)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, Hq, _ = q.shape
    L, Hkv, _ = K.shape
    Dv = V.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    G = Hq // Hkv
    out = np.zeros((n, Hq, Dv), np.float64)
    lse = np.full((n, Hq), -np.inf, np.float64)
    if L == 0 or n == 0:
        return out, lse
    pos = (L - n) + np.arange(n)  # absolute position of each query (bottom-right)
    visible = (np.arange(L)[None, :] <= pos[:, None]) if causal else np.ones((n, L), bool)
    for g in range(Hkv):
        qg = q[:, g * G:(g + 1) * G, :].reshape(n * G, -1)  # rows (j, h)
        s = scale * (qg @ K[:, g, :].T)  # [n*G, L]
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        s = s.reshape(n, G, L)
        s = np.where(visible[:, None, :], s, -np.inf)
        m = s.max(axis=2, keepdims=True)
        has = np.isfinite(m[..., 0])
        m_safe = np.where(np.isfinite(m), m, 0.0)
        p = np.where(visible[:, None, :], np.exp(s - m_safe), 0.0)
        l = p.sum(axis=2)  # [n, G]
        o = (p.reshape(n * G, L) @ V[:, g, :]).reshape(n, G, Dv)
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(has[..., None], o / np.where(has, l, 1.0)[..., None], 0.0)
            lg = np.where(has, m[..., 0] + np.log(np.where(has, l, 1.0)), -np.inf)
        out[:, g * G:(g + 1) * G, :] = o
        lse[:, g * G:(g + 1) * G] = lg
    return out, lse


def paged_attention(q_raw: np.ndarray, q_lens: Sequence[int], pool_k_raw: np.ndarray,
                    pool_v_raw: Optional[np.ndarray], dtype: str, slot_lists: List[np.ndarray],
                    scale: float, causal, head_dim_v: Optional[int] = None,
                    requests: Optional[Sequence[int]] = None, softcap: float = 0.0):
    """Batch of requests reading K/V through slot lists.

    ``q_raw`` ``[sum(q_lens), Hq, Dqk]`` and the per-token pool views
    ``[slots, Hkv, D]`` hold raw stored values (float32, or uint16 bf16
    bits).  ``slot_lists[i]`` gives the slots of request ``i``'s logical
    tokens ``0..L_i-1`` (from any of the table formats).  A latent pool
    passes ``pool_v_raw=None`` and ``head_dim_v``: V is the first
    ``head_dim_v`` values of each K row.  ``requests`` limits the work to a
    subset; other rows of the result stay NaN.  ``causal`` is one flag for
    every request or a per-request sequence (mixed causal/full segments).

    Returns out ``[sum(q_lens), Hq, Dv]`` and lse ``[sum(q_lens), Hq]``, fp64."""
    q_lens = np.asarray(q_lens, np.int64)
    qo = np.concatenate([[0], np.cumsum(q_lens)])
    Hq = q_raw.shape[1]
    Dv = pool_v_raw.shape[2] if pool_v_raw is not None else int(head_dim_v)
    out = np.full((int(qo[-1]), Hq, Dv), np.nan)
    lse = np.full((int(qo[-1]), Hq), np.nan)
    reqs = range(len(q_lens)) if requests is None else requests
    for i in reqs:
        a, b = int(qo[i]), int(qo[i + 1])
        slots = np.asarray(slot_lists[i], np.int64)
        K = to_f64(pool_k_raw[slots], dtype)
        V = K[..., :Dv] if pool_v_raw is None else to_f64(pool_v_raw[slots], dtype)
        c = bool(causal[i]) if isinstance(causal, (list, tuple, np.ndarray)) else bool(causal)
        o, l = attend(to_f64(q_raw[a:b], dtype), K, V, scale, c, softcap)
        out[a:b] = o
        lse[a:b] = l
    return out, lse


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine attention results over disjoint key subsets into the result
    over their union: ``lse = log sum_s exp(lse_s)``, ``o = sum_s exp(lse_s -
    lse) o_s``.  Subsets with ``lse_s = -inf`` (no keys) contribute nothing;
    if every subset is empty, ``o = 0`` and ``lse = -inf``."""
    L = np.stack([np.asarray(x, np.float64) for x in lses])  # [S, ...]
    O = np.stack([np.asarray(x, np.float64) for x in outs])  # [S, ..., Dv]
    m = L.max(axis=0)
    fin = np.isfinite(m)
    m0 = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - m0[None]), 0.0)
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(fin, m0 + np.log(np.where(fin, tot, 1.0)), -np.inf)
        o = np.where(fin[..., None], (w[..., None] * O).sum(axis=0) / np.where(fin, tot, 1.0)[..., None], 0.0)
    return o, lse


def gather(pool_raw: np.ndarray, slot_lists: List[np.ndarray]) -> np.ndarray:
    """Ragged gather: each request's rows, in logical order, one request after
    another (``index_select`` by packed slots, [XPU] "Approach 2").  Raw
    stored values, bit for bit."""
    if not slot_lists:
        return pool_raw[:0].copy()
    idx = np.concatenate([np.asarray(s, np.int64) for s in slot_lists])
    return pool_raw[idx].copy()


def span_segments(spans: Sequence[Tuple[int, int, bool]]) -> List[Tuple[int, int, int, bool]]:
    """A row's spans ``(start, end, causal)`` as native segments ``(q_start,
    q_end, kv_len, causal)``: both kinds read the row's keys up to the span's
    end ([OMNI] "Attention execution", the segment table)."""
    return [(int(a), int(b), int(b), bool(c)) for a, b, c in spans]
