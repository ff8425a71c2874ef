"""GPU parity of the decode slice -- KV append, index building, ragged gather
and paged decode attention -- against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_38_amd as P
import workloads as W
from workloads.cases import to_numpy_bits

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, i32, offsets, oracle_after_store, oracle_region

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


def small_cases():
    return {
        "tiny_f32": lambda s: W.tiny_decode(seed=s),
        "tiny_f32_padded": lambda s: W.tiny_decode(seed=s, padded=True),
        "qwen3_small": lambda s: W.qwen3_decode(seed=s, bs=8, len_range=(1, 700), pool_tokens=8000, max_context=768),
        "gqa_ps16_small": lambda s: W.gqa_prefix_share(16, seed=s, bs=16, prefix=256, median=300, sigma=0.8,
                                                       clip=(1, 1500)),
        "gqa_ps64_small": lambda s: W.gqa_prefix_share(64, seed=s, bs=16, prefix=256, median=300, sigma=0.8,
                                                       clip=(1, 1500)),
    }


# ---------------------------------------------------------------------------
# KV append: bit exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_padded", "qwen3_small", "mla_small", "encdec_small"])
def test_kv_store_bit_exact(name):
    builders = dict(small_cases())
    builders["mla_small"] = lambda s: W.mla_decode(seed=s, bs=4, len_range=(60, 300))
    builders["encdec_small"] = lambda s: W.encdec_extend(seed=s, bs=4, enc_len=100, prefix_range=(0, 40),
                                                        new_range=(1, 60))
    case = builders[name](0)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals, num_layers=3, layer=1)
    before_other = dc.k_buf.view(3, -1)[[0, 2]].clone()
    dc.store()
    torch.cuda.synchronize()
    pk, pv = oracle_after_store(case, vals)
    got_k = to_numpy_bits(dc.pool.flat("k", 1))
    if case.dummy.any():
        # dummies race on the padding slot: any one of their rows may win there
        pad = case.geom.padding_slot
        ok_rows = to_numpy_bits(vals["k_new"])[case.dummy]
        assert any(np.array_equal(got_k[pad].view(np.uint8), r.view(np.uint8)) for r in ok_rows)
        got_k, pk = np.delete(got_k, pad, 0), np.delete(pk, pad, 0)
    assert np.array_equal(got_k.view(np.uint8), pk.view(np.uint8))
    if pv is not None:
        got_v = to_numpy_bits(dc.pool.flat("v", 1))
        if case.dummy.any():
            got_v, pv = np.delete(got_v, case.geom.padding_slot, 0), np.delete(pv, case.geom.padding_slot, 0)
        assert np.array_equal(got_v.view(np.uint8), pv.view(np.uint8))
    assert torch.equal(dc.k_buf.view(3, -1)[[0, 2]], before_other)  # other layers untouched


# ---------------------------------------------------------------------------
# index building: bit exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_small", "gqa_ps16_small", "gqa_ps64_small", "mla", "encdec"])
def test_build_kv_indices_bit_exact(name):
    builders = dict(small_cases())
    builders["mla"] = lambda s: W.mla_decode(seed=s, bs=6, len_range=(1, 900))
    builders["encdec"] = lambda s: W.encdec_extend(seed=s, bs=6)
    case = builders[name](1)
    ps = case.geom.page_size
    dev_table, dev_rpi = i32(case.req_to_token), i32(case.req_pool_indices)
    for rname, r in case.regions.items():
        maxl = int(r.kv_lens.max())
        per = -(-maxl // ps)
        ks, kl = i32(r.kv_start), i32(r.kv_lens)
        ref_ptr, ref_idx = oracle.build_csr(case.req_to_token, case.req_pool_indices, r.kv_start, r.kv_lens, ps)
        ref_bt = oracle.build_block_table(case.req_to_token, case.req_pool_indices, r.kv_start, r.kv_lens, ps,
                                          per + 3)
        ref_lpl = oracle.last_page_len(r.kv_lens, ps)
        indptr = torch.full((case.bs + 1,), -9, dtype=torch.int32, device="cuda")
        cap = case.bs * per
        indices = torch.full((cap + 5,), -9, dtype=torch.int32, device="cuda")
        lpl = torch.full((case.bs,), -9, dtype=torch.int32, device="cuda")
        P.build_kv_indices(P.PKV_MAP_CSR, dev_table, dev_rpi, ks, kl, ps, maxl, indptr, indices, lpl)
        bt = torch.full((case.bs, per + 3), -9, dtype=torch.int32, device="cuda")
        P.build_kv_indices(P.PKV_MAP_BLOCK_TABLE, dev_table, dev_rpi, ks, kl, ps, maxl, None, bt)
        torch.cuda.synchronize()
        assert np.array_equal(indptr.cpu().numpy(), ref_ptr), rname
        n = int(ref_ptr[-1])
        got = indices.cpu().numpy()
        assert np.array_equal(got[:n], ref_idx), rname
        assert (got[n:] == -9).all(), "wrote past the last page id"
        assert np.array_equal(bt.cpu().numpy(), ref_bt), rname
        assert np.array_equal(lpl.cpu().numpy(), ref_lpl), rname
        # the page lists the allocator handed out come back
        for i in range(case.bs):
            assert np.array_equal(got[ref_ptr[i]:ref_ptr[i + 1]], r.page_lists[i])


def test_build_kv_indices_empty_and_zero_length():
    table = i32(np.arange(64).reshape(4, 16))
    kl = i32([0, 5, 0])
    rpi = i32([0, 1, 2])
    indptr = torch.full((4,), -9, dtype=torch.int32, device="cuda")
    indices = torch.full((6,), -9, dtype=torch.int32, device="cuda")
    lpl = torch.full((3,), -9, dtype=torch.int32, device="cuda")
    P.build_kv_indices(P.PKV_MAP_CSR, table, rpi, None, kl, 4, 5, indptr, indices, lpl)
    torch.cuda.synchronize()
    assert indptr.tolist() == [0, 0, 2, 2]
    assert indices.tolist()[:2] == [4, 5]
    assert lpl.tolist() == [0, 1, 0]
    empty = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    P.build_kv_indices(P.PKV_MAP_CSR, table, rpi[:0], None, kl[:0], 4, 0, empty, indices)
    torch.cuda.synchronize()
    assert empty.tolist() == [0]


# ---------------------------------------------------------------------------
# ragged gather: bit exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_kv_gather_bit_exact(fmt):
    case = W.encdec_extend(seed=2, bs=5, enc_len=300, prefix_range=(0, 90), new_range=(1, 70))
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    pk, pv = oracle_after_store(case, vals)
    for rname, r in case.regions.items():
        m = dc.kv_map(rname, fmt)
        cu = offsets(r.kv_lens)
        tot = int(cu[-1])
        ko = torch.full((tot + 3, case.geom.num_kv_heads, case.geom.head_dim_qk), float("nan"), dtype=dc.dtype,
                        device="cuda")
        vo = torch.full_like(ko, float("nan"))
        P.kv_gather(dc.pool, 0, m, i32(cu), ko, vo)
        torch.cuda.synchronize()
        slots = [oracle.slots_from_token_table(case.req_to_token, case.req_pool_indices[i], r.kv_start[i],
                                               r.kv_lens[i]) for i in range(case.bs)]
        assert np.array_equal(to_numpy_bits(ko[:tot]), oracle.gather(pk, slots))
        assert np.array_equal(to_numpy_bits(vo[:tot]), oracle.gather(pv, slots))
        assert torch.isnan(ko[tot:].float()).all()


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", list(small_cases()))
@pytest.mark.parametrize("seed", [0, 1])
def test_decode_matches_oracle(name, fmt, seed):
    case = small_cases()[name](seed)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(fmt)
    ref_o, ref_l = oracle_region(case, vals, "self")
    real = ~case.dummy if case.dummy.size else np.ones(case.bs, bool)
    assert_attn_close(out, ref_o, case.geom.dtype, f"{name} fmt {fmt}", rows=real)
    assert_lse_close(lse, ref_l, case.geom.dtype, f"{name} fmt {fmt}", rows=real)


STREAM_SHAPES = {
    # runs each cover many whole requests (most written directly, a few cut)
    "many_short": lambda s: W.qwen3_decode(seed=s, bs=1500, len_range=(1, 70), pool_tokens=60000, max_context=128),
    # one request cut into a piece per run (the merge sees 100+ pieces)
    "one_long": lambda s: W.qwen3_decode(seed=s, bs=1, len_range=(60000, 60000), pool_tokens=61000,
                                         max_context=60032),
    # long and short requests side by side, page-granular map
    "mixed_ps64": lambda s: W.gqa_prefix_share(64, seed=s, bs=40, prefix=64, median=200, sigma=2.0,
                                               clip=(1, 30000)),
}


@pytest.mark.parametrize("name", list(STREAM_SHAPES))
def test_decode_stream_split_shapes(name):
    """The bf16 decode cuts the concatenated key tiles of all requests into
    equal runs; these shapes put many requests in one run, one request over
    every run, and both at once."""
    case = STREAM_SHAPES[name](7)
    print(f"stream shape {name}: bs {case.bs}, sum L {int(case.regions['self'].kv_lens.sum())}", flush=True)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    if case.n_new:
        dc.store()
    fmt = P.PKV_MAP_TOKEN_TABLE if case.geom.page_size == 1 else P.PKV_MAP_CSR
    out, lse = dc.decode(fmt)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, case.geom.dtype, name)
    assert_lse_close(lse, ref_l, case.geom.dtype, name)


def test_decode_formats_agree_bitwise_and_repeat():
    """The three table formats resolve to the same slots, and split
    boundaries are logical: all give identical bits, run after run."""
    case = small_cases()["gqa_ps16_small"](3)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    outs = [dc.decode(f) for f in FMTS] + [dc.decode(P.PKV_MAP_CSR)]
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_decode_page_permutation_bitwise_invariant():
    case = W.gqa_prefix_share(16, seed=4, bs=16, prefix=256, median=300, sigma=0.8, clip=(1, 1500))
    vals = W.make_values(case)
    o1, l1 = DeviceCase(case, vals).decode(P.PKV_MAP_CSR)
    g = case.geom
    ps = g.page_size
    pi = np.random.default_rng(5).permutation(g.num_pages)
    pi = np.concatenate([pi, [g.num_pages]])  # padding page stays last
    perm_idx = torch.from_numpy((np.argsort(pi)[:, None] * ps + np.arange(ps)[None, :]).reshape(-1))
    v2 = dict(vals)
    v2["pool_k"] = vals["pool_k"][perm_idx]
    v2["pool_v"] = vals["pool_v"][perm_idx]
    t = case.req_to_token.astype(np.int64)
    case.req_to_token = (pi[t // ps] * ps + t % ps).astype(np.int32)
    o2, l2 = DeviceCase(case, v2).decode(P.PKV_MAP_CSR)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["qwen3_small", "gqa_ps64_small"])
def test_decode_planted_keys_every_position(name):
    """A planted key whose score dwarfs the rest makes the output its value
    row: walking it over every page and offset proves each token is read
    from the right slot."""
    case = small_cases()[name](0)
    vals = W.make_values(case)
    g = case.geom
    r = case.regions["self"]
    q = vals["q"]["self"].float()
    rng = np.random.default_rng(0)
    i = int(np.argmax(r.kv_lens))
    L = int(r.kv_lens[i])
    positions = sorted(set(rng.choice(L, size=min(L, 24), replace=False).tolist() + [0, L - 1]))
    for t in positions:
        v2 = {k: (dict(x) if isinstance(x, dict) else (x.clone() if x is not None else None)) for k, x in vals.items()}
        slot = int(case.req_to_token[case.req_pool_indices[i], t])
        for kvh in range(g.num_kv_heads):
            G = g.num_q_heads // g.num_kv_heads
            qd = q[i, kvh * G:(kvh + 1) * G].sum(0)
            key = (qd / qd.norm() * 60.0).to(v2["pool_k"].dtype)
            if t == L - 1 and case.n_new:
                v2["k_new"][i, kvh] = key
            else:
                v2["pool_k"][slot, kvh] = key
        dc = DeviceCase(case, v2)
        dc.store()
        out, _ = dc.decode(P.PKV_MAP_CSR if g.page_size > 1 else P.PKV_MAP_TOKEN_TABLE)
        ref_o, _ = oracle_region(case, v2, "self", requests=[i])
        assert_attn_close(out[i:i + 1], ref_o[i:i + 1], g.dtype, f"planted t={t}")
        vrow = (v2["v_new"][i] if (t == L - 1 and case.n_new) else v2["pool_v"][slot]).float().cpu().numpy()
        G = g.num_q_heads // g.num_kv_heads
        got = out[i].float().cpu().numpy()
        for h in range(g.num_q_heads):
            np.testing.assert_allclose(got[h], vrow[h // G], atol=3e-2)


def test_decode_empty_request_gives_zero_and_minus_inf():
    case = W.qwen3_decode(seed=0, bs=6, len_range=(1, 300), pool_tokens=4000, max_context=320)
    case.regions["self"].kv_lens[[1, 4]] = 0
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    for fmt in FMTS:
        out, lse = dc.decode(fmt)
        assert (out[[1, 4]].float() == 0).all()
        assert torch.isneginf(lse[[1, 4]]).all()
        ref_o, ref_l = oracle_region(case, vals, "self", requests=[0, 2, 3, 5])
        rows = [0, 2, 3, 5]
        assert_attn_close(out, ref_o, "bf16", "empty-mixed", rows=rows)


# ---------------------------------------------------------------------------
# decode with the step's append in the same call
# ---------------------------------------------------------------------------

APPEND_CASES = {
    "tiny_f32": lambda: W.tiny_decode(seed=3),                      # fp32: separate store launch
    "tiny_f32_padded": lambda: W.tiny_decode(seed=3, padded=True),  # dummy rows on the padding page
    "qwen3_small": lambda: small_cases()["qwen3_small"](3),
    "gqa_ps64_small": lambda: small_cases()["gqa_ps64_small"](3),
    "many_short": lambda: STREAM_SHAPES["many_short"](3),           # 1500 rows: 375 extra planner blocks
    "mla_small": lambda: W.mla_decode(seed=3, bs=6, len_range=(1, 900)),
}


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_decode_append_equals_store_then_decode_bitwise(name, fmt):
    """paged_decode_attn_append gives the bits of kv_store followed by
    paged_decode_attn: outputs, lse and the whole pool."""
    case = APPEND_CASES[name]()
    g = case.geom
    print(f"decode append {name} fmt {fmt}: bs {case.bs}, {len(case.out_loc)} new rows", flush=True)
    vals = W.make_values(case, canary=True)
    a = DeviceCase(case, vals)
    a.store()
    oa, la = a.decode(fmt)
    b = DeviceCase(case, vals)
    m = b.kv_map("self", fmt)
    out = torch.full_like(oa, float("nan"))
    lse = torch.full_like(la, float("nan"))
    nb = P.paged_decode_workspace_bytes(b.pool, case.bs, g.num_q_heads, m.max_kv_len)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    P.paged_decode_attn_append(b.pool, 0, b.q["self"], m, b.k_new, b.v_new, b.out_loc, case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    # dummy requests all write the padding page, in no defined order, and
    # read it back: compare real rows and real pages bit for bit
    real = ~case.dummy if case.dummy.size else np.ones(case.bs, bool)
    rt = torch.from_numpy(real).to("cuda")
    assert torch.equal(_bits(out)[rt], _bits(oa)[rt]) and torch.equal(_bits(lse)[rt], _bits(la)[rt])
    real_slots = g.num_pages * g.page_size
    assert torch.equal(_bits(b.pool.flat("k", 0))[:real_slots], _bits(a.pool.flat("k", 0))[:real_slots])
    if not g.latent:
        assert torch.equal(_bits(b.pool.flat("v", 0))[:real_slots], _bits(a.pool.flat("v", 0))[:real_slots])
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, g.dtype, f"append {name}", rows=real)
    assert_lse_close(lse, ref_l, g.dtype, f"append {name}", rows=real)


def test_decode_append_with_empty_batch_only_stores():
    case = small_cases()["qwen3_small"](4)
    vals = W.make_values(case)
    a = DeviceCase(case, vals)
    a.store()
    b = DeviceCase(case, vals)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    m = P.make_kv_map(P.PKV_MAP_TOKEN_TABLE, empty, 0, req_to_token=b.req_to_token, req_pool_indices=empty,
                      kv_start=empty)
    g = case.geom
    q = torch.empty((0, g.num_q_heads, g.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, g.num_q_heads, g.head_dim_v), dtype=torch.bfloat16, device="cuda")
    P.paged_decode_attn_append(b.pool, 0, q, m, b.k_new, b.v_new, b.out_loc, case.sm_scale, out)
    torch.cuda.synchronize()
    assert torch.equal(_bits(b.pool.flat("k", 0)), _bits(a.pool.flat("k", 0)))
    assert torch.equal(_bits(b.pool.flat("v", 0)), _bits(a.pool.flat("v", 0)))
