"""paged_decode_attn on batches whose requests share prefix pages, against the
oracle, through the C ABI.

The decode finds shared prefixes itself: consecutive requests whose keys
start on the same page form a group (within 64-request blocks), the longest
member is the group's reference, and each member's shared keys end at the
first page where its table leaves the reference's.  Those keys are read
once for the whole group; the rest of each request goes through the stream
kernel.  The result is plain attention ([MINI] prefix caching; the oracle
knows nothing of the groups), so every case here is compared with the
oracle: members shorter than the prefix, a reference that is not the first
member, members that leave the prefix at different pages, an empty request
and a dummy on the padding page inside a run of requests, groups cut by the
64-request blocks, and token-table maps at page size 1."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, i32, oracle_region

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


def _mixed_groups(ps):
    """Groups of every shape the detection has to handle (page size ps)."""
    pp = 2048 // ps  # prefix pages of the big group
    g = []
    # members shorter than the prefix, the longest not first, one leaving early
    g.append((pp, [(700, pp), (3000, pp), (2048, pp), (5100, pp), (90, pp), (2049, pp), (1500, pp // 4),
                   (2600, pp)]))
    g.append((0, [(333, 0)]))  # a private request between groups
    # a group whose members leave the prefix at different pages
    g.append((8, [(40 * ps, 8), (30 * ps, 2), (9 * ps, 8), (5 * ps, 5), (8 * ps, 8)]))
    g.append((3, [(0, 0)]))  # an empty request (starts no group)
    g.append((3, [(3 * ps + 1, 3), (6 * ps, 3)]))
    # private requests up to the 64-request block edge, then a group across it
    for L in np.random.default_rng(ps).integers(1, 900, size=40):
        g.append((0, [(int(L), 0)]))
    g.append((12, [(12 * ps + 7, 12)] * 10))
    return g


def _check(case, fmt, what):
    vals = W.make_values(case, device="cuda", canary=True)
    dc = DeviceCase(case, vals)
    out, lse = dc.decode(fmt)
    live = [i for i in range(case.bs) if case.regions["self"].kv_lens[i] > 0]
    ref_o, ref_l = oracle_region(case, vals, "self", requests=list(range(case.bs)))
    assert_attn_close(out, ref_o, case.geom.dtype, what, rows=live)
    assert_lse_close(lse, ref_l, case.geom.dtype, what, rows=live)
    for i in range(case.bs):
        if case.regions["self"].kv_lens[i] == 0:
            assert (out[i].float() == 0).all() and torch.isneginf(lse[i]).all()
    return out, lse


@pytest.mark.parametrize("ps", [16, 64])
@pytest.mark.parametrize("fmt", FMTS)
def test_detected_groups_match_oracle(ps, fmt):
    case = W.shared_prefix_batch(ps, _mixed_groups(ps), seed=ps)
    print(f"shared groups ps {ps} fmt {fmt}: bs {case.bs}", flush=True)
    assert case.bs > 64
    _check(case, fmt, f"shared groups ps{ps} fmt{fmt}")


def test_detected_groups_formats_agree_bitwise():
    case = W.shared_prefix_batch(16, _mixed_groups(16), seed=3)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    outs = [dc.decode(f) for f in FMTS]
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_token_table_sharing_at_page_size_one():
    """Page size 1: the shared keys end at the first differing slot."""
    groups = [(300, [(300, 300), (1000, 300), (150, 300), (800, 137)]), (0, [(500, 0)]),
              (64, [(64, 64), (64, 64), (200, 64)])]
    case = W.shared_prefix_batch(1, groups, seed=5)
    _check(case, P.PKV_MAP_TOKEN_TABLE, "shared groups ps1")


def test_padding_dummies_are_not_grouped():
    """Dummy requests all start on the padding page; they must not form a
    group with each other (their outputs are don't-care but finite) and the
    real requests must be exact."""
    case = W.tiny_decode(seed=0, padded=True)
    case.geom.dtype = "bf16"
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(P.PKV_MAP_CSR)
    real = [i for i in range(case.bs) if not case.dummy[i]]
    ref_o, ref_l = oracle_region(case, vals, "self", requests=real)
    assert_attn_close(out, ref_o, "bf16", "padded batch with dummies", rows=real)
    assert torch.isfinite(out.float()).all()


def test_sharing_and_private_copies_agree_with_the_oracle_at_full_size():
    """The prefix-sharing workload and the same keys copied into private
    pages (no sharing to find) both match the oracle on a sample."""
    case = W.gqa_prefix_share(16, seed=0)
    print("full-size prefix sharing vs private copies", flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    out_s, lse_s = dc.decode(P.PKV_MAP_CSR)
    # private copies: every request's keys moved to its own fresh pages
    r = case.regions["self"]
    ps = case.geom.page_size
    pages = [len(p) for p in r.page_lists]
    tot = int(sum(pages))
    geom = case.geom
    table = case.req_to_token.copy()
    pk = dc.pool.flat("k", 0)
    pv = dc.pool.flat("v", 0)
    base = 0
    src_rows, dst_rows = [], []
    # the copies go to a second pool of exactly the private pages
    for i, pl in enumerate(r.page_lists):
        L = int(r.kv_lens[i])
        own = np.arange(base, base + len(pl), dtype=np.int64)
        base += len(pl)
        src = (np.asarray(pl, np.int64)[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)[:L]
        dst = (own[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)[:L]
        src_rows.append(src)
        dst_rows.append(dst)
        table[case.req_pool_indices[i], :L] = dst
    kb2, vb2 = P.kv_pool_bytes(1, tot, ps, geom.num_kv_heads, geom.head_dim_qk, geom.head_dim_v, torch.bfloat16)
    k2 = torch.zeros(kb2 // 2, dtype=torch.bfloat16, device="cuda")
    v2 = torch.zeros(vb2 // 2, dtype=torch.bfloat16, device="cuda")
    pool2 = P.kv_pool_create(k2, v2, num_layers=1, num_pages=tot, page_size=ps, num_kv_heads=geom.num_kv_heads,
                             head_dim_qk=geom.head_dim_qk, head_dim_v=geom.head_dim_v)
    src = torch.from_numpy(np.concatenate(src_rows)).cuda()
    dst = torch.from_numpy(np.concatenate(dst_rows)).cuda()
    pool2.flat("k", 0)[dst] = pk[src]
    pool2.flat("v", 0)[dst] = pv[src]
    t2 = i32(table)
    kv_lens = i32(r.kv_lens)
    m2 = P.make_kv_map(P.PKV_MAP_TOKEN_TABLE, kv_lens, int(r.kv_lens.max()), req_to_token=t2,
                       req_pool_indices=i32(case.req_pool_indices), kv_start=i32(r.kv_start))
    out_p = torch.empty_like(out_s)
    lse_p = torch.empty_like(lse_s)
    ws = torch.empty(P.paged_decode_workspace_bytes(pool2, case.bs, geom.num_q_heads, m2.max_kv_len),
                     dtype=torch.uint8, device="cuda")
    P.paged_decode_attn(pool2, 0, dc.q["self"], m2, case.sm_scale, out_p, lse_p, ws)
    torch.cuda.synchronize()
    reqs = sorted(set(np.random.default_rng(1).choice(case.bs, 24, replace=False).tolist()) |
                  {int(np.argmin(r.kv_lens)), int(np.argmax(r.kv_lens))})
    ref_o, ref_l = oracle_region(case, vals, "self", requests=reqs)
    assert_attn_close(out_s, ref_o, "bf16", "prefix sharing, shared pages", rows=reqs)
    assert_attn_close(out_p, ref_o, "bf16", "prefix sharing, private copies", rows=reqs)
    assert_lse_close(lse_s, ref_l, "bf16", "shared", rows=reqs)
    assert_lse_close(lse_p, ref_l, "bf16", "private", rows=reqs)
    P.kv_pool_destroy(pool2)


def test_large_batch_with_groups_of_every_size():
    """A thousand requests in groups of 1 to 70 members (groups longer than
    the 64-request blocks split into several), random prefix and total
    lengths, page size 16, CSR: every output against the oracle on a
    sample, and the shared layout against itself in the block-table format
    bit for bit."""
    rng = np.random.default_rng(11)
    groups, bs = [], 0
    while bs < 1000:
        size = int(rng.choice([1, 1, 2, 3, 8, 15, 33, 70]))
        pp = int(rng.integers(1, 40))
        members = []
        for _ in range(size):
            L = int(rng.integers(1, 1800))
            members.append((L, int(rng.integers(0, pp + 1))))
        groups.append((pp, members))
        bs += size
    case = W.shared_prefix_batch(16, groups, seed=11, num_q_heads=16, num_kv_heads=8)
    print(f"large shared batch: bs {case.bs}, {len(groups)} groups", flush=True)
    vals = W.make_values(case, device="cuda", canary=True)
    dc = DeviceCase(case, vals)
    out, lse = dc.decode(P.PKV_MAP_CSR)
    o2, l2 = dc.decode(P.PKV_MAP_BLOCK_TABLE)
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    lens = case.regions["self"].kv_lens
    live = [i for i in range(case.bs) if lens[i] > 0]
    reqs = sorted(set(np.random.default_rng(2).choice(live, 120, replace=False).tolist()))
    ref_o, ref_l = oracle_region(case, vals, "self", requests=reqs)
    assert_attn_close(out, ref_o, "bf16", "large shared batch", rows=reqs)
    assert_lse_close(lse, ref_l, "bf16", "large shared batch", rows=reqs)


SHAPES = [  # (KV heads, query heads per KV head, head_dim): every launch shape, odd query groups
    (1, 1, 64), (1, 16, 128), (2, 3, 128), (3, 5, 128), (4, 4, 64), (8, 1, 64), (2, 7, 64),
]


@pytest.mark.parametrize("hkv,group,d", SHAPES)
def test_detected_groups_head_shapes(hkv, group, d):
    """Detected sharing through the prefix pass at every launch shape (one,
    two and four waves per workgroup), head_dim 64 and 128, and query groups
    that do not divide the pass's 32 rows (3, 5, 7 heads: slices of 10, 6 and
    4 members with padding rows)."""
    ps = 16
    groups = [(20, [(700, 20), (320, 20), (900, 20), (100, 20), (2000, 20), (330, 20), (321, 20), (1200, 20),
                    (640, 20), (500, 20), (800, 20), (350, 20)]),
              (0, [(250, 0)]),
              (12, [(400, 12), (190, 12), (640, 8), (13 * ps, 12)])]
    case = W.shared_prefix_batch(ps, groups, seed=hkv * 100 + group, num_q_heads=hkv * group, num_kv_heads=hkv,
                                 head_dim=d)
    print(f"detected groups shape: {hkv} kv heads x {group}, head_dim {d}", flush=True)
    for fmt in (P.PKV_MAP_CSR, P.PKV_MAP_TOKEN_TABLE):
        _check(case, fmt, f"shape {hkv}x{group} d{d} fmt{fmt}")
