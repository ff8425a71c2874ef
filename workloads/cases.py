"""Seeded synthetic workloads: the world state a serving engine hands to the
attention layer, for the five workload shapes of the paged KV-cache hot path.

What is built here, and nothing more:

* per-request lengths drawn from the stated distributions;
* which physical pages each request owns, popped in request order from a
  free list that is a seeded permutation of the pool's pages -- this module
  plays the part of the paged slot allocator, expanding each page ``p`` into
  its slots ``p*page_size + 0..page_size-1`` the way the paged allocator does
  (SGLang encoder-decoder post, "How SGLang stores the KV cache: two pools
  and a page size");
* the token-granular ``req_to_token`` table those slots are written into, one
  row per request plus a padding row (the *last* row), with every unused
  entry pointing at the padding page;
* the slots that receive this step's new K/V (``out_loc``);
* i.i.d. normal K/V/q values (drawn in fp32, cast to bf16 with
  round-to-nearest-even where the workload is bf16).

No index building, no store, no attention happens here: the oracle and the
HIP path each do those themselves, from these inputs.

Seeds: workload ``c`` with parity seed ``s`` uses
``SeedSequence([38, c, s, *extra])`` spawned into four streams (structure,
page placement, K/V values, queries).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_SEED = 38


def _cdiv(a: int, b: int) -> int:
    return -(-int(a) // int(b))


@dataclass
class Geometry:
    """Pool geometry: ``[num_pages + 1, page_size, num_kv_heads, head_dim]``
    per buffer and layer; page ``num_pages`` is the padding page."""

    dtype: str  # "f32" or "bf16"
    page_size: int
    num_pages: int  # real pages
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    latent: bool  # one buffer; V is the first head_dim_v values of each row
    num_q_heads: int

    @property
    def num_slots(self) -> int:
        return (self.num_pages + 1) * self.page_size

    @property
    def padding_page(self) -> int:
        return self.num_pages

    @property
    def padding_slot(self) -> int:
        return self.num_pages * self.page_size

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclass
class Region:
    """One attention call's view of each request's row: columns
    ``[kv_start, kv_start + kv_len)`` of ``req_to_token``."""

    kv_start: np.ndarray  # int32 [bs]
    kv_lens: np.ndarray  # int32 [bs]
    page_lists: List[np.ndarray]  # physical pages in logical order, per request
    causal: bool
    causal_flags: Optional[np.ndarray] = None  # int32 [bs], per-request mask (mixed causal/full segments)


@dataclass
class Case:
    name: str
    geom: Geometry
    bs: int
    req_to_token: np.ndarray  # int32 [rows, W]; last row = padding row
    req_pool_indices: np.ndarray  # int32 [bs]
    q_lens: np.ndarray  # int32 [bs] new tokens (queries) per request
    regions: Dict[str, Region]
    out_loc: np.ndarray  # int32 [sum(q_lens)] or empty: slots written this step
    sm_scale: float
    value_scale: float
    value_seed: int
    query_seed: int
    free_pages: np.ndarray  # pages no request owns
    tail_slots: np.ndarray  # slots of owned pages that no region covers
    dummy: np.ndarray = field(default_factory=lambda: np.zeros(0, bool))  # [bs] padded-batch dummies
    # requests sharing a prefix: (group_indptr int32 [G + 1], prefix_len int32 [G]) or None
    prefix_groups: Optional[Tuple[np.ndarray, np.ndarray]] = None

    @property
    def padding_row(self) -> int:
        return self.req_to_token.shape[0] - 1

    @property
    def n_new(self) -> int:
        return int(self.out_loc.shape[0])


# ----------------------------------------------------------------------------
# helpers (world construction only)
# ----------------------------------------------------------------------------

def _streams(config_id: int, seed: int, extra=()):
    ss = np.random.SeedSequence([ROOT_SEED, config_id, seed, *extra])
    s_struct, s_place, s_vals, s_q = ss.spawn(4)
    val_seed = int(s_vals.generate_state(1, np.uint64)[0] >> np.uint64(1))
    q_seed = int(s_q.generate_state(1, np.uint64)[0] >> np.uint64(1))
    return np.random.default_rng(s_struct), np.random.default_rng(s_place), val_seed, q_seed


def _expand(pages: np.ndarray, ps: int, n: int) -> np.ndarray:
    """The allocator's page expansion: the slots of the first ``n`` tokens
    living on ``pages`` (each page gives ``ps`` consecutive slots)."""
    pages = np.asarray(pages, dtype=np.int64)
    return (pages[:, None] * ps + np.arange(ps, dtype=np.int64)[None, :]).reshape(-1)[:n]


def _new_table(rows: int, width: int, geom: Geometry) -> np.ndarray:
    # every entry starts on the padding page, keeping in-page contiguity so
    # that even a stray page-granular read of an unused column stays there
    col = np.arange(width, dtype=np.int64) % geom.page_size
    row = geom.padding_page * geom.page_size + col
    return np.broadcast_to(row, (rows, width)).astype(np.int32).copy()


def _tail_slots(page_lists: List[np.ndarray], lens: np.ndarray, ps: int) -> List[np.ndarray]:
    out = []
    for pages, n in zip(page_lists, lens):
        n = int(n)
        if len(pages) == 0:
            continue
        used = n - (len(pages) - 1) * ps
        if used < ps:
            out.append(int(pages[-1]) * ps + np.arange(used, ps, dtype=np.int64))
    return out


def _round32(x: int) -> int:
    return _cdiv(x, 32) * 32


# ----------------------------------------------------------------------------
# the five workload shapes
# ----------------------------------------------------------------------------

def tiny_decode(seed: int = 0, padded: bool = False) -> Case:
    """Tiny paged decode, fp32: 4 requests with post-append KV lengths
    {7, 33, 64, 100}, page_size 16, 64 real pages plus the padding page,
    pages popped from a seeded permutation in request order; 4 query heads,
    2 KV heads, head_dim 64, scale 1/8; one new token per request.

    ``padded`` appends 4 dummy requests that point at the padding row (as a
    padded batch does), each of KV length 1 whose new token goes to the
    padding slot."""
    rs, rp, vseed, qseed = _streams(1, seed)
    ps, num_pages = 16, 64
    geom = Geometry("f32", ps, num_pages, 2, 64, 64, False, 4)
    lens = np.array([7, 33, 64, 100], dtype=np.int32)
    bs_real = len(lens)
    perm = rp.permutation(num_pages)
    pos, page_lists = 0, []
    for n in lens:
        k = _cdiv(n, ps)
        page_lists.append(perm[pos:pos + k].astype(np.int64))
        pos += k
    free = perm[pos:]
    table = _new_table(bs_real + 1, 128, geom)
    rpi = rs.permutation(bs_real).astype(np.int32)
    for i in range(bs_real):
        table[rpi[i], :lens[i]] = _expand(page_lists[i], ps, lens[i])
    out_loc = np.array([table[rpi[i], lens[i] - 1] for i in range(bs_real)], dtype=np.int32)
    tails = _tail_slots(page_lists, lens, ps)
    dummy = np.zeros(bs_real, bool)
    if padded:
        nd = 4
        pad_row = table.shape[0] - 1
        rpi = np.concatenate([rpi, np.full(nd, pad_row, np.int32)])
        lens = np.concatenate([lens, np.ones(nd, np.int32)])
        page_lists += [np.array([geom.padding_page], np.int64) for _ in range(nd)]
        out_loc = np.concatenate([out_loc, np.full(nd, geom.padding_slot, np.int32)])
        dummy = np.concatenate([dummy, np.ones(nd, bool)])
    bs = len(lens)
    region = Region(np.zeros(bs, np.int32), lens.astype(np.int32), page_lists, causal=True)
    return Case(
        name="tiny_decode_f32" + ("_padded" if padded else ""),
        geom=geom, bs=bs, req_to_token=table, req_pool_indices=rpi,
        q_lens=np.ones(bs, np.int32), regions={"self": region}, out_loc=out_loc,
        sm_scale=1.0 / 8.0, value_scale=1.0, value_seed=vseed, query_seed=qseed,
        free_pages=free.astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
        dummy=dummy,
    )


def qwen3_decode(seed: int = 0, bs: int = 64, len_range=(512, 4096),
                 pool_tokens: int = 400_000, max_context: int = 8192) -> Case:
    """Qwen3-0.6B-shaped single-layer decode, bf16: 16 query heads, 8 KV
    heads, head_dim 128, page_size 1 (token-granular table of width 8192);
    KV lengths uniform in [512, 4096]; slots drawn by a seeded shuffle of a
    400k-token pool; one new token per request at position L-1."""
    rs, rp, vseed, qseed = _streams(2, seed)
    geom = Geometry("bf16", 1, pool_tokens, 8, 128, 128, False, 16)
    lens = rs.integers(len_range[0], len_range[1] + 1, size=bs).astype(np.int32)
    assert int(lens.sum()) <= pool_tokens and int(lens.max()) <= max_context
    perm = rp.permutation(pool_tokens)
    table = _new_table(bs + 1, max_context, geom)
    rpi = rs.permutation(bs).astype(np.int32)
    pos, page_lists = 0, []
    for i in range(bs):
        pages = perm[pos:pos + lens[i]].astype(np.int64)
        pos += lens[i]
        page_lists.append(pages)
        table[rpi[i], :lens[i]] = pages  # page_size 1: a page is a slot
    out_loc = np.array([table[rpi[i], lens[i] - 1] for i in range(bs)], dtype=np.int32)
    region = Region(np.zeros(bs, np.int32), lens, page_lists, causal=True)
    return Case(
        name="qwen3_decode_bf16", geom=geom, bs=bs, req_to_token=table, req_pool_indices=rpi,
        q_lens=np.ones(bs, np.int32), regions={"self": region}, out_loc=out_loc,
        sm_scale=1.0 / np.sqrt(128.0), value_scale=1.0, value_seed=vseed, query_seed=qseed,
        free_pages=perm[pos:].astype(np.int64), tail_slots=np.zeros(0, np.int64),
    )


def gqa_prefix_share(page_size: int, seed: int = 0, bs: int = 256, group: int = 8,
                     prefix: int = 2048, median: float = 2048.0, sigma: float = 1.0,
                     clip=(64, 32768), num_q_heads: int = 32) -> Case:
    """Large-batch paged GQA decode with prefix sharing, bf16: 32 query heads,
    8 KV heads, head_dim 128; ln(L) ~ N(ln 2048, sigma), rounded, clipped to
    [64, 32768]; each group of 8 consecutive requests reads the same physical
    pages for its first min(L, 2048) tokens; pool = ceil(1.2 x pages needed)
    real pages in a seeded free-list order. Attention only (no store)."""
    rs, rp, vseed, qseed = _streams(3, seed, (page_size,))
    ps = page_size
    assert prefix % ps == 0 and bs % group == 0
    lens = np.clip(np.rint(np.exp(rs.normal(np.log(median), sigma, size=bs))), clip[0], clip[1]).astype(np.int32)
    ngroups = bs // group
    pre_pages = prefix // ps
    private = [_cdiv(max(int(n) - prefix, 0), ps) for n in lens]
    needed = ngroups * pre_pages + sum(private)
    num_pages = _cdiv(needed * 12, 10)
    geom = Geometry("bf16", ps, num_pages, 8, 128, 128, False, num_q_heads)
    perm = rp.permutation(num_pages)
    width = _round32(int(clip[1]))
    table = _new_table(bs + 1, width, geom)
    rpi = rs.permutation(bs).astype(np.int32)
    pos, page_lists = 0, []
    for g in range(ngroups):
        shared = perm[pos:pos + pre_pages].astype(np.int64)
        pos += pre_pages
        for i in range(g * group, (g + 1) * group):
            n = int(lens[i])
            own = perm[pos:pos + private[i]].astype(np.int64)
            pos += private[i]
            pages = np.concatenate([shared[:_cdiv(min(n, prefix), ps)], own])
            page_lists.append(pages)
            table[rpi[i], :n] = _expand(pages, ps, n)
    # only private last pages have a tail no member reads
    priv = [i for i in range(bs) if int(lens[i]) > prefix]
    tails = _tail_slots([page_lists[i] for i in priv], lens[priv], ps)
    region = Region(np.zeros(bs, np.int32), lens, page_lists, causal=True)
    return Case(
        name=f"gqa_prefix_share_ps{ps}", geom=geom, bs=bs, req_to_token=table, req_pool_indices=rpi,
        q_lens=np.ones(bs, np.int32), regions={"self": region}, out_loc=np.zeros(0, np.int32),
        sm_scale=1.0 / np.sqrt(128.0), value_scale=1.0, value_seed=vseed, query_seed=qseed,
        free_pages=perm[pos:].astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
        prefix_groups=(np.arange(0, bs + 1, group, dtype=np.int32), np.full(ngroups, prefix, np.int32)),
    )


def mla_decode(seed: int = 0, bs: int = 128, len_range=(4096, 16384), num_q_heads: int = 128,
               num_draft: int = 1, fixed_lens: Optional[Dict[int, int]] = None, page_size: int = 64) -> Case:
    """MLA-shaped paged decode, bf16: page_size 64, 128 query heads over one
    latent KV row of 576 values (512 latent + 64 rope); V is the first 512;
    KV lengths uniform in [4096, 16384]; values N(0,1) x 0.1; pool =
    ceil(1.2 x needed) real pages, seeded free-list order, popped in request
    order; one new token per request at position L-1.

    ``num_draft > 1`` is target verification ([BACKEND] init_forward_metadata,
    target-verify branch): each request's last ``num_draft`` tokens are draft
    tokens appended this step (positions L - num_draft .. L - 1, those that
    exist), each with its own queries, attending causally (bottom-right).
    ``fixed_lens`` sets chosen requests' lengths (edge cases in tests);
    ``page_size`` other than 64 is for tests (the streams do not depend on it)."""
    rs, rp, vseed, qseed = _streams(4, seed, (num_draft,) if num_draft > 1 else ())
    ps = page_size
    lens = rs.integers(len_range[0], len_range[1] + 1, size=bs).astype(np.int32)
    for i, n in (fixed_lens or {}).items():
        lens[i] = n
    npg = [_cdiv(n, ps) for n in lens]
    num_pages = _cdiv(sum(npg) * 12, 10)
    geom = Geometry("bf16", ps, num_pages, 1, 576, 512, True, num_q_heads)
    perm = rp.permutation(num_pages)
    width = _round32(int(max(len_range[1], lens.max())))
    table = _new_table(bs + 1, width, geom)
    rpi = rs.permutation(bs).astype(np.int32)
    pos, page_lists = 0, []
    for i in range(bs):
        pages = perm[pos:pos + npg[i]].astype(np.int64)
        pos += npg[i]
        page_lists.append(pages)
        table[rpi[i], :lens[i]] = _expand(pages, ps, lens[i])
    out_loc = np.concatenate([table[rpi[i], max(0, lens[i] - num_draft):lens[i]] for i in range(bs)]).astype(np.int32)
    tails = _tail_slots(page_lists, lens, ps)
    region = Region(np.zeros(bs, np.int32), lens, page_lists, causal=True)
    return Case(
        name="mla_decode_bf16" if num_draft == 1 else f"mla_verify{num_draft}_bf16", geom=geom, bs=bs,
        req_to_token=table, req_pool_indices=rpi, q_lens=np.full(bs, num_draft, np.int32), regions={"self": region},
        out_loc=out_loc,
        sm_scale=1.0 / np.sqrt(576.0), value_scale=0.1, value_seed=vseed, query_seed=qseed,
        free_pages=perm[pos:].astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
    )


def encdec_extend(seed: int = 0, bs: int = 32, enc_len: int = 1500, prefix_range=(0, 448),
                  new_range=(1, 512), num_heads: int = 20, head_dim: int = 64,
                  page_size: int = 16) -> Case:
    """Whisper-shaped encoder-decoder extend, bf16: 20 heads (MHA), head_dim
    64, page_size 16.  Each row holds the encoder's slots in columns
    [0, enc_len) (enc_len 1500 is not page aligned: the last encoder page has
    12 valid tokens) and the decoder's slots from the next page boundary
    (column 1504) on.  Decoder prefix p ~ U{0..448} tokens already cached;
    n ~ U{1..512} new tokens appended this step and attended causally over
    the decoder region ('self'); the same queries' layer also reads the whole
    encoder region non-causally ('cross').  ``enc_len = 0`` is the warm-up
    case with an empty encoder."""
    rs, rp, vseed, qseed = _streams(5, seed, (enc_len,))
    ps = page_size
    p = rs.integers(prefix_range[0], prefix_range[1] + 1, size=bs).astype(np.int32)
    n = rs.integers(new_range[0], new_range[1] + 1, size=bs).astype(np.int32)
    enc_pages = _cdiv(enc_len, ps)
    dec_start = enc_pages * ps  # decoder region begins on the next page boundary
    dec_lens = (p + n).astype(np.int32)
    dec_pages = [_cdiv(d, ps) for d in dec_lens]
    needed = bs * enc_pages + sum(dec_pages)
    num_pages = _cdiv(needed * 12, 10)
    geom = Geometry("bf16", ps, num_pages, num_heads, head_dim, head_dim, False, num_heads)
    perm = rp.permutation(num_pages)
    width = _round32(dec_start + int(dec_lens.max()))
    table = _new_table(bs + 1, width, geom)
    rpi = rs.permutation(bs).astype(np.int32)
    pos = 0
    enc_lists, dec_lists, out_loc = [], [], []
    for i in range(bs):
        ep = perm[pos:pos + enc_pages].astype(np.int64)
        pos += enc_pages
        dp = perm[pos:pos + dec_pages[i]].astype(np.int64)
        pos += dec_pages[i]
        enc_lists.append(ep)
        dec_lists.append(dp)
        r = rpi[i]
        table[r, :enc_len] = _expand(ep, ps, enc_len)
        table[r, dec_start:dec_start + dec_lens[i]] = _expand(dp, ps, dec_lens[i])
        out_loc.append(table[r, dec_start + p[i]:dec_start + dec_lens[i]])
    tails = _tail_slots(enc_lists, np.full(bs, enc_len, np.int32), ps) + _tail_slots(dec_lists, dec_lens, ps)
    regions = {
        "self": Region(np.full(bs, dec_start, np.int32), dec_lens, dec_lists, causal=True),
        "cross": Region(np.zeros(bs, np.int32), np.full(bs, enc_len, np.int32), enc_lists, causal=False),
    }
    return Case(
        name=f"encdec_extend_enc{enc_len}", geom=geom, bs=bs, req_to_token=table, req_pool_indices=rpi,
        q_lens=n, regions=regions, out_loc=np.concatenate(out_loc).astype(np.int32),
        sm_scale=1.0 / np.sqrt(float(head_dim)), value_scale=1.0, value_seed=vseed, query_seed=qseed,
        free_pages=perm[pos:].astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
    )


def mixed_spans(seed: int = 0, rows: int = 4, spans=((128, True), (2048, False)), num_q_heads: int = 32,
                num_kv_heads: int = 8, head_dim: int = 128, page_size: int = 16) -> Case:
    """Rows of mixed causal and full spans, bf16, written once and attended
    as native segments (the vLLM-Omni notes, "Attention execution": a causal
    span [s, e) is Q[s:e] over K[:e] with the causal flag, a full span
    [a, b) is Q[a:b] over K[:b] without it; the first denoising step writes
    the complete sequence once).  Default: 4 rows (two requests, one
    conditional and one unconditional branch each) of a 128-token causal
    text span followed by a 2048-token full image span; GQA 32 / 8 query /
    KV heads, head_dim 128, page_size 16.  The sizes are synthetic choices:
    the notes give none.  Each segment is one request of the batch, every
    segment of a row reading the same table row."""
    rs, rp, vseed, qseed = _streams(6, seed, (rows, len(spans)))
    ps = page_size
    row_len = int(sum(n for n, _ in spans))
    pages_per_row = _cdiv(row_len, ps)
    num_pages = _cdiv(rows * pages_per_row * 12, 10)
    geom = Geometry("bf16", ps, num_pages, num_kv_heads, head_dim, head_dim, False, num_q_heads)
    perm = rp.permutation(num_pages)
    table = _new_table(rows + 1, _round32(row_len), geom)
    row_ids = rs.permutation(rows).astype(np.int32)
    bs = rows * len(spans)
    rpi, q_lens, kv_lens, flags, lists, out_loc = [], [], [], [], [], []
    for r in range(rows):
        pages = perm[r * pages_per_row:(r + 1) * pages_per_row].astype(np.int64)
        tr = row_ids[r]
        table[tr, :row_len] = _expand(pages, ps, row_len)
        out_loc.append(table[tr, :row_len])
        start = 0
        for n, causal in spans:
            end = start + int(n)
            rpi.append(tr)
            q_lens.append(int(n))
            kv_lens.append(end)
            flags.append(1 if causal else 0)
            lists.append(pages[:_cdiv(end, ps)])
            start = end
    tails = _tail_slots([perm[r * pages_per_row:(r + 1) * pages_per_row] for r in range(rows)],
                        np.full(rows, row_len, np.int32), ps)
    region = Region(np.zeros(bs, np.int32), np.asarray(kv_lens, np.int32), lists, causal=True,
                    causal_flags=np.asarray(flags, np.int32))
    return Case(
        name=f"mixed_spans_r{rows}", geom=geom, bs=bs, req_to_token=table, req_pool_indices=np.asarray(rpi, np.int32),
        q_lens=np.asarray(q_lens, np.int32), regions={"self": region},
        out_loc=np.concatenate(out_loc).astype(np.int32), sm_scale=1.0 / np.sqrt(float(head_dim)), value_scale=1.0,
        value_seed=vseed, query_seed=qseed, free_pages=perm[rows * pages_per_row:].astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
    )


def shared_prefix_batch(page_size: int, groups, seed: int = 0, num_q_heads: int = 32, num_kv_heads: int = 8,
                        head_dim: int = 128, dtype: str = "bf16") -> Case:
    """A decode batch with hand-placed prefix sharing, for structural tests.

    ``groups`` lists consecutive runs of requests; each is ``(prefix_pages,
    members)`` with ``members`` a list of ``(L, shared_pages)``: the member
    has ``L`` keys, of which the first ``min(L, shared_pages * page_size)``
    sit on the group's first ``shared_pages`` prefix pages (``shared_pages
    <= prefix_pages``) and the rest on private pages.  A group of one member
    with ``shared_pages = 0`` is a private request.  Pages come from a
    seeded permutation of a pool 1.2x the pages needed; attention only (no
    store)."""
    rs, rp, vseed, qseed = _streams(7, seed, (page_size, len(groups)))
    ps = page_size
    lens, need = [], 0
    for prefix_pages, members in groups:
        need += prefix_pages
        for L, sh in members:
            assert sh <= prefix_pages
            lens.append(int(L))
            need += _cdiv(max(int(L) - sh * ps, 0), ps)
    lens = np.asarray(lens, np.int32)
    bs = len(lens)
    num_pages = _cdiv(max(need, 1) * 12, 10)
    geom = Geometry(dtype, ps, num_pages, num_kv_heads, head_dim, head_dim, False, num_q_heads)
    perm = rp.permutation(num_pages)
    width = _round32(int(lens.max(initial=1)))
    table = _new_table(bs + 1, width, geom)
    rpi = rs.permutation(bs).astype(np.int32)
    pos, i, page_lists = 0, 0, []
    for prefix_pages, members in groups:
        shared = perm[pos:pos + prefix_pages].astype(np.int64)
        pos += prefix_pages
        for L, sh in members:
            L = int(L)
            n_sh = min(_cdiv(L, ps), sh)
            own_n = _cdiv(max(L - sh * ps, 0), ps)
            own = perm[pos:pos + own_n].astype(np.int64)
            pos += own_n
            pages = np.concatenate([shared[:n_sh], own])
            page_lists.append(pages)
            if L:
                table[rpi[i], :L] = _expand(pages, ps, L)
            i += 1
    # unread slots: on each page, those past the last offset any request reads
    used = {}
    for pages, L in zip(page_lists, lens.tolist()):
        for k, pg in enumerate(pages.tolist()):
            used[pg] = max(used.get(pg, 0), min(ps, L - k * ps))
    tails = [pg * ps + np.arange(u, ps, dtype=np.int64) for pg, u in used.items() if u < ps]
    region = Region(np.zeros(bs, np.int32), lens, page_lists, causal=True)
    return Case(
        name=f"shared_prefix_batch_ps{ps}", geom=geom, bs=bs, req_to_token=table, req_pool_indices=rpi,
        q_lens=np.ones(bs, np.int32), regions={"self": region}, out_loc=np.zeros(0, np.int32),
        sm_scale=1.0 / np.sqrt(float(head_dim)), value_scale=1.0, value_seed=vseed, query_seed=qseed,
        free_pages=perm[pos:].astype(np.int64),
        tail_slots=np.concatenate(tails) if tails else np.zeros(0, np.int64),
    )


CONFIG_BUILDERS = {
    1: tiny_decode,
    2: qwen3_decode,
    3: gqa_prefix_share,
    4: mla_decode,
    5: encdec_extend,
    6: mixed_spans,
}


# ----------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------

def make_values(case: Case, device: str = "cpu", canary: bool = False) -> Dict[str, object]:
    """Draw the pool contents, this step's new K/V and the queries as torch
    tensors on ``device`` (i.i.d. N(0,1) x value_scale in fp32, then cast to
    the pool dtype).  Returns a dict with ``pool_k``, ``pool_v`` (None for a
    latent pool), ``k_new``, ``v_new`` (None for latent) and ``q`` (a dict of
    per-region query tensors, ``[sum(q_lens), Hq, Dqk]``).

    ``canary`` writes NaN into every slot no real request may read: the
    padding page, pages no request owns, the unused tail of owned pages, and
    the slots that only become valid once this step's K/V is stored."""
    import torch

    g = case.geom
    dt = torch.float32 if g.dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device=device).manual_seed(case.value_seed)
    qgen = torch.Generator(device=device).manual_seed(case.query_seed)

    def draw(shape, gg):
        x = torch.randn(shape, generator=gg, device=device, dtype=torch.float32)
        if case.value_scale != 1.0:
            x.mul_(case.value_scale)
        return x.to(dt)

    pool_k = draw((g.num_slots, g.num_kv_heads, g.head_dim_qk), gen)
    pool_v = None if g.latent else draw((g.num_slots, g.num_kv_heads, g.head_dim_v), gen)
    nn = case.n_new
    k_new = draw((nn, g.num_kv_heads, g.head_dim_qk), gen)
    v_new = None if g.latent else draw((nn, g.num_kv_heads, g.head_dim_v), gen)
    nq = int(case.q_lens.sum())
    q = {name: draw((nq, g.num_q_heads, g.head_dim_qk), qgen) for name in case.regions}
    if canary:
        ps = g.page_size
        bad_pages = np.concatenate([[g.padding_page], case.free_pages]).astype(np.int64)
        bad = np.concatenate([
            (bad_pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1),
            case.tail_slots.astype(np.int64),
            case.out_loc.astype(np.int64),
        ])
        idx = torch.from_numpy(np.unique(bad)).to(device)
        pool_k.index_fill_(0, idx, float("nan"))
        if pool_v is not None:
            pool_v.index_fill_(0, idx, float("nan"))
    return {"pool_k": pool_k, "pool_v": pool_v, "k_new": k_new, "v_new": v_new, "q": q}


def to_numpy_bits(t) -> Optional[np.ndarray]:
    """Host copy of a torch tensor as raw storage: float32 for f32 tensors,
    uint16 bit patterns for bf16 tensors."""
    import torch

    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
