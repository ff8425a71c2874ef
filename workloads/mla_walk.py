"""Planted-key walk over the MLA latent pool: inputs for structural tests of a
decode kernel that streams many 32-key tiles per workgroup.

What is built here, and nothing more (no attention is computed):

* an MLA-shaped workload (``mla_decode``) whose requests have at most 128
  tiles of 32 keys, so that each of the 128 query rows of a request (heads,
  or heads x drafts for target verification) can own one tile;
* values of unit variance (the pool, the new rows, the queries);
* for each request and each tile, one *planted* key: the row's query is
  ``q_scale * u_row`` and the planted key ``key_scale * u_row`` for a set of
  orthonormal directions ``u`` (one per row), so that the row's attention is
  dominated by that one key (a score margin of about 25 nats over the random
  keys) and its output is, to within bf16 rounding, the planted row's first
  512 values.  Rows of a request with fewer tiles than rows get a query along
  their direction and no planted key.

The offsets inside each tile vary from tile to tile (first, last and middle
positions), and some requests plant their last key in this step's new rows
(the KV append), so the walk covers every tile of every request, and with
it every run boundary, every piece's first and last tile and every LDS ring
slot of a kernel that splits the tile stream into equal runs.

``stream_layout`` restates that split -- the requests' tiles laid end to end,
cut into ``runs`` equal runs -- so that tests can name which tiles fall at a
run's edges or in which ring slot; it is a description of the launch, not
part of the method (any split gives the same attention).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, List

import numpy as np

from .cases import Case, make_values, mla_decode

TILE = 32


@dataclass
class Planted:
    request: int
    row: int  # query row of the request: draft * heads + head
    pos: int  # logical key position
    tile: int  # tile of the request (pos // 32)
    in_append: bool  # the planted key is one of this step's new rows


def stream_layout(kv_lens: np.ndarray, runs: int):
    """Tiles per request, first global tile per request, run length (tiles
    per run) and total tiles, for the requests' tiles laid end to end and cut
    into ``runs`` equal runs."""
    T = (np.asarray(kv_lens, np.int64) + TILE - 1) // TILE
    P = np.concatenate([[0], np.cumsum(T)[:-1]]).astype(np.int64)
    total = int(T.sum())
    Bt = max(1, -(-total // runs))
    return T, P, Bt, total


def tile_roles(kv_lens: np.ndarray, runs: int, ring: int = 4) -> Dict[str, List[tuple]]:
    """(request, tile) pairs that sit at the named places of the split: the
    first and last tile of every piece (a request's tiles inside one run),
    and, per ring slot k, every tile whose index inside its run is k mod
    ``ring``."""
    T, P, Bt, total = stream_layout(kv_lens, runs)
    roles: Dict[str, List[tuple]] = {"piece_first": [], "piece_last": []}
    for k in range(ring):
        roles[f"ring_{k}"] = []
    for i in range(len(T)):
        for j in range(int(T[i])):
            g = int(P[i]) + j
            local = g % Bt
            if j == 0 or local == 0:
                roles["piece_first"].append((i, j))
            if j == int(T[i]) - 1 or local == Bt - 1:
                roles["piece_last"].append((i, j))
            roles[f"ring_{local % ring}"].append((i, j))
    return roles


def mla_walk(seed: int = 0, bs: int = 48, len_range=(1024, 4064), heads: int = 128, num_draft: int = 1,
             q_scale: float = 8.0, key_scale: float = 80.0, device: str = "cpu"):
    """The planted-key walk.  Returns ``(case, vals, planted)``; ``vals`` as
    :func:`workloads.cases.make_values` (bf16 torch tensors on ``device``)
    with the queries and planted keys written in, ``planted`` the list of
    :class:`Planted` keys.  ``heads * num_draft`` must be 128 (one direction
    per row) and every request must have at most 128 tiles."""
    import torch

    rows = heads * num_draft
    assert rows == 128, "one direction per query row"
    assert len_range[1] <= 128 * TILE
    case = mla_decode(seed=seed, bs=bs, len_range=len_range, num_q_heads=heads, num_draft=num_draft)
    case = replace(case, value_scale=1.0, name=case.name + "_walk")
    vals = make_values(case, device=device)
    g = case.geom
    rng = np.random.default_rng(np.random.SeedSequence([38, 4, seed, 977]))
    # orthonormal directions, one per row (columns of a seeded Gaussian's Q)
    u, _ = np.linalg.qr(rng.standard_normal((g.head_dim_qk, rows)))
    U = torch.from_numpy(u.T.copy()).to(torch.float32)  # [rows, 576]
    r = case.regions["self"]
    n = num_draft
    # query row (j, h) sits at q[(i * n + j), h]; rows ordered by visibility:
    # the last draft sees every key, so the last tiles go to its rows
    order = [(j, h) for j in reversed(range(n)) for h in range(heads)]
    q = vals["q"]["self"].view(case.bs, n, heads, g.head_dim_qk)
    q.copy_((q_scale * U).view(n, heads, -1).to(q.dtype).unsqueeze(0).expand(case.bs, -1, -1, -1))
    pool_k = vals["pool_k"]
    k_new = vals["k_new"]
    new_base = 0
    planted: List[Planted] = []
    for i in range(case.bs):
        L = int(r.kv_lens[i])
        T = -(-L // TILE)
        first_new = L - min(n, L)  # positions of this step's new rows
        row_of_table = case.req_to_token[case.req_pool_indices[i]]
        for t in range(T):
            j, h = order[T - 1 - t]
            rho = j * heads + h
            lim = min(L - 1, L - n + j)  # last key row (j, h) sees
            lo, hi = t * TILE, min(t * TILE + TILE - 1, lim)
            # vary the offset: first, last, then a stride through the tile
            k = (t + 3 * i) % 5
            if k == 0:
                pos = lo
            elif k == 1:
                pos = hi
            else:
                pos = lo + (7 * t + 11 * i + 5 * k) % (hi - lo + 1)
            if t == T - 1 and i % 3 == 0:
                pos = hi  # the newest key this row sees
            key = (key_scale * U[rho]).to(pool_k.dtype)
            in_app = pos >= first_new
            if in_app:
                k_new[new_base + (pos - first_new), 0] = key.to(k_new.device)
            else:
                pool_k[int(row_of_table[pos]), 0] = key.to(pool_k.device)
            planted.append(Planted(i, rho, pos, t, in_app))
        new_base += min(n, L)
    return case, vals, planted
