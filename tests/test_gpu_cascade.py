"""GPU parity of the cascade decode over shared prefixes (each group's
shared prefix read once for all members, each request's own keys by the
split-K decode, merged by log-sum-exp) against the oracle, through the C
ABI.  The oracle knows nothing of groups: the result must be plain
attention over each request's keys."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, i32, oracle_region

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


def cascade(dc, fmt, indptr, prefix_len, max_group=None):
    c, g = dc.case, dc.case.geom
    m = dc.kv_map("self", fmt)
    ip, pl = i32(indptr), i32(prefix_len)
    mg = max_group if max_group is not None else int(np.diff(indptr).max(initial=0))
    groups = P.make_prefix_groups(ip, pl, mg, int(np.max(prefix_len, initial=0)))
    out = torch.full((c.bs, g.num_q_heads, g.head_dim_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.bs, g.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    nb = P.paged_decode_cascade_workspace_bytes(dc.pool, c.bs, g.num_q_heads, m.max_kv_len, groups)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    P.paged_decode_attn_cascade(dc.pool, dc.layer, dc.q["self"], m, groups, c.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def small(ps, seed=0, bs=32, group=8, prefix=512, num_q_heads=32):
    return W.gqa_prefix_share(ps, seed=seed, bs=bs, group=group, prefix=prefix, median=prefix, clip=(64, 4 * prefix),
                              num_q_heads=num_q_heads)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("ps", [16, 64])
def test_cascade_matches_oracle(ps, fmt):
    case = small(ps, seed=ps)
    print(f"cascade ps {ps} fmt {fmt}: lens {case.regions['self'].kv_lens.tolist()}", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    out, lse = cascade(dc, fmt, *case.prefix_groups)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"cascade ps {ps} fmt {fmt}")
    assert_lse_close(lse, ref_l, "bf16", f"cascade ps {ps} fmt {fmt}")


@pytest.mark.parametrize("group,heads", [(16, 32), (8, 64), (4, 8)])
def test_cascade_group_slices_and_head_counts(group, heads):
    """Groups with more rows than one wave holds (16 members x 4 heads, 8 x 8)
    and a group of one-head members."""
    case = small(16, seed=group + heads, bs=32, group=group, prefix=256, num_q_heads=heads)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    out, lse = cascade(dc, P.PKV_MAP_CSR, *case.prefix_groups)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"cascade group {group} heads {heads}")
    assert_lse_close(lse, ref_l, "bf16", f"cascade group {group} heads {heads}")


def test_cascade_unaligned_prefix_partial_groups_and_empty_request():
    """prefix_len 48 (not a multiple of the 32-key tile: the cascade splits
    at 32), only the first two groups declared (the rest decode as plain
    requests), and one empty request inside a group."""
    case = small(16, seed=5, bs=32, group=8, prefix=48)
    case.regions["self"].kv_lens[3] = 0
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    indptr, pl = case.prefix_groups
    out, lse = cascade(dc, P.PKV_MAP_TOKEN_TABLE, indptr[:3], pl[:2])
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", "cascade unaligned")
    assert_lse_close(lse, ref_l, "bf16", "cascade unaligned")
    assert (out[3].float() == 0).all() and torch.isneginf(lse[3]).all()


def test_cascade_without_groups_equals_decode_bitwise():
    """With no groups the cascade is the split-K decode plus a merge: on a
    batch where no request shares a page (so paged_decode_attn finds no
    shared prefix either) the two give the same bits."""
    lens = np.random.default_rng(7).integers(1, 2000, size=32)
    case = W.shared_prefix_batch(64, [(0, [(int(L), 0)]) for L in lens], seed=7)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    o1, l1 = dc.decode(P.PKV_MAP_CSR)
    o2, l2 = cascade(dc, P.PKV_MAP_CSR, np.zeros(1, np.int32), np.zeros(0, np.int32), max_group=0)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    ref_o, _ = oracle_region(case, vals, "self")
    assert_attn_close(o2, ref_o, "bf16", "cascade without groups")


def test_cascade_full_size_prefix_share():
    """The 256-request, 2048-token-prefix workload at page_size 16, checked on
    a seeded sample of requests (always the shortest and the longest)."""
    case = W.gqa_prefix_share(16, seed=0)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    out, lse = cascade(dc, P.PKV_MAP_CSR, *case.prefix_groups)
    L = case.regions["self"].kv_lens
    rng = np.random.default_rng(3)
    reqs = sorted(set(rng.choice(case.bs, 30, replace=False).tolist()) | {int(np.argmin(L)), int(np.argmax(L))})
    ref_o, ref_l = oracle_region(case, vals, "self", requests=reqs)
    rows = np.asarray(reqs)
    assert_attn_close(out, ref_o, "bf16", "cascade full size", rows=rows)
    assert_lse_close(lse, ref_l, "bf16", "cascade full size", rows=rows)


@pytest.mark.parametrize("fmt", [P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE])
def test_cascade_empty_and_single_member_groups(fmt):
    """Declared groups that are a sub-division of the shared ones: requests
    before the first group and after the last, empty groups (one at the
    start, one between others), groups of one member, a prefix_len of 0 and
    prefix lengths below the shared length (any split at or below it is
    exact).  Each group's work items are listed after those of the groups
    before it, so empty groups must count for nothing."""
    case = small(16, seed=11, bs=32, group=8, prefix=512)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    indptr = np.array([2, 2, 7, 8, 8, 9, 16, 24], np.int32)
    pl = np.array([512, 512, 300, 0, 0, 200, 512], np.int32)
    print(f"cascade groups {indptr.tolist()} prefix {pl.tolist()} fmt {fmt}", flush=True)
    out, lse = cascade(dc, fmt, indptr, pl, max_group=12)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", "cascade empty/single groups")
    assert_lse_close(lse, ref_l, "bf16", "cascade empty/single groups")


@pytest.mark.parametrize("head_dim,num_kv_heads,num_q_heads",
                         [(64, 8, 32), (64, 2, 8), (128, 1, 4), (64, 1, 16), (64, 2, 6), (128, 3, 15)])
def test_cascade_head_dims_and_kv_head_counts(head_dim, num_kv_heads, num_q_heads):
    """The cascade at head_dim 64 and with one, two or three KV heads
    (workgroups of one or two waves; 16 query heads per KV head give slices
    of two members, 3 and 5 leave padding rows in the 32-row slices), on
    hand-placed groups: members shorter than the prefix, a one-request group
    with nothing shared, and a group whose declared prefix is the shortest
    member's share."""
    ps = 16
    groups = [(20, [(700, 20), (320, 20), (900, 20), (100, 20)]), (1, [(250, 0)]),
              (12, [(400, 12), (190, 12), (640, 8)])]
    case = W.shared_prefix_batch(ps, groups, seed=head_dim + num_kv_heads, num_q_heads=num_q_heads,
                                 num_kv_heads=num_kv_heads, head_dim=head_dim)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    indptr = np.array([0, 4, 5, 8], np.int32)
    pl = np.array([20 * ps, 0, 8 * ps], np.int32)
    print(f"cascade D {head_dim} Hkv {num_kv_heads} Hq {num_q_heads}", flush=True)
    out, lse = cascade(dc, P.PKV_MAP_CSR, indptr, pl)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"cascade D {head_dim} Hkv {num_kv_heads}")
    assert_lse_close(lse, ref_l, "bf16", f"cascade D {head_dim} Hkv {num_kv_heads}")


def test_cascade_group_larger_than_its_bound_stays_in_bounds():
    """A caller whose groups hold more members than max_group_size breaks the
    bounds' promise: the members past the slices the bound sizes get an
    unspecified result, but the call still ends normally with nothing read
    or written out of range, and the members the bound covers are exact."""
    case = small(16, seed=13, bs=32, group=16, prefix=256)  # two groups of 16; 8 members per slice
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    indptr, pl = case.prefix_groups
    print(f"cascade groups {indptr.tolist()} declared at most 8 members", flush=True)
    out, lse = cascade(dc, P.PKV_MAP_CSR, indptr, pl, max_group=8)
    ref_o, ref_l = oracle_region(case, vals, "self")
    covered = list(range(0, 8)) + list(range(16, 24))
    assert_attn_close(out, ref_o, "bf16", "cascade bound too small (covered members)", rows=covered)
    assert_lse_close(lse, ref_l, "bf16", "cascade bound too small (covered members)", rows=covered)
