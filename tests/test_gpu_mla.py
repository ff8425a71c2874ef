"""GPU parity of the MLA (latent 576/512) paged decode against the oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, oracle_region, run_verify

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [0, 1])
def test_mla_decode_matches_oracle(seed, fmt):
    case = W.mla_decode(seed=seed, bs=5, len_range=(1, 1500))
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(fmt)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"mla fmt {fmt}")
    assert_lse_close(lse, ref_l, "bf16", f"mla fmt {fmt}")


@pytest.mark.parametrize("heads", [16, 64])
def test_mla_decode_fewer_heads(heads):
    case = W.mla_decode(seed=2, bs=3, len_range=(100, 700), num_q_heads=heads)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(P.PKV_MAP_BLOCK_TABLE)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"mla {heads} heads")
    assert_lse_close(lse, ref_l, "bf16", f"mla {heads} heads")


@pytest.mark.parametrize("key_scale", [80.0, 200.0])
def test_mla_planted_key_and_empty_request(key_scale):
    """One key far along the query direction.  At 200 its score sits ~100
    log2 units above the first tile's: the kernel's fixed softmax reference
    would overflow there, so the request goes through the exact fallback."""
    case = W.mla_decode(seed=3, bs=4, len_range=(200, 900))
    case.regions["self"].kv_lens[2] = 0
    vals = W.make_values(case)
    i = 1
    L = int(case.regions["self"].kv_lens[i])
    # every head of request i looks along u; one key lies far along u
    u = torch.randn(576, generator=torch.Generator().manual_seed(5))
    u = u / u.norm()
    vals["q"]["self"][i] = (u * 8.0).to(torch.bfloat16)[None, :].expand(case.geom.num_q_heads, 576)
    key = (u * key_scale).to(torch.bfloat16)
    t = L // 2
    slot = int(case.req_to_token[case.req_pool_indices[i], t])
    vals["pool_k"][slot, 0] = key
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(P.PKV_MAP_CSR)
    assert (out[2].float() == 0).all() and torch.isneginf(lse[2]).all()
    ref_o, ref_l = oracle_region(case, vals, "self", requests=[0, 1, 3])
    assert_attn_close(out, ref_o, "bf16", "mla planted", rows=[0, 1, 3])
    # the planted key dominates: every head returns (nearly) its V part
    np.testing.assert_allclose(out[i].float().cpu().numpy(),
                               np.repeat(key[:512].float().cpu().numpy()[None], case.geom.num_q_heads, 0), atol=0.05)


@pytest.mark.parametrize("heads", [32, 128])
def test_mla_many_short_requests(heads):
    """Many short requests (and empty ones) so that every run of tiles holds
    several requests and many requests are split across runs."""
    case = W.mla_decode(seed=4, bs=48, len_range=(1, 90), num_q_heads=heads)
    for i in (3, 17, 18, 40):
        case.regions["self"].kv_lens[i] = 0
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(P.PKV_MAP_BLOCK_TABLE)
    live = [i for i in range(case.bs) if case.regions["self"].kv_lens[i] > 0]
    ref_o, ref_l = oracle_region(case, vals, "self", requests=live)
    assert_attn_close(out, ref_o, "bf16", f"mla short {heads}", rows=live)
    assert_lse_close(lse, ref_l, "bf16", f"mla short {heads}", rows=live)
    for i in (3, 17, 18, 40):
        assert (out[i].float() == 0).all() and torch.isneginf(lse[i]).all()


def test_mla_formats_agree_bitwise_and_repeat():
    case = W.mla_decode(seed=6, bs=9, len_range=(1, 3000))
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    outs = [dc.decode(f) for f in FMTS] + [dc.decode(P.PKV_MAP_BLOCK_TABLE)]
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


# --------------------------------------------------------------------------
# target verification: drafts folded into heads, bottom-right causal
# --------------------------------------------------------------------------

@pytest.mark.parametrize("heads,n", [(16, 2), (16, 8), (32, 4), (64, 2), (16, 4), (128, 2), (64, 4), (32, 12)])
@pytest.mark.parametrize("fmt", FMTS)
def test_mla_verify_matches_oracle(heads, n, fmt):
    """Short and long requests (pieces cut across runs, drafts straddling a
    tile boundary), one request shorter than its drafts (its first drafts see
    no key)."""
    # request 0 is shorter than its drafts; request 1's drafts straddle the
    # 32-key tile boundary at 64
    case = W.mla_decode(seed=heads + n, bs=6, len_range=(1, 1300), num_q_heads=heads, num_draft=n,
                        fixed_lens={0: max(1, n - 1), 1: 64 + n // 2})
    print(f"mla verify heads {heads} drafts {n} fmt {fmt}", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_verify(dc, fmt, n)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"verify {heads}x{n} fmt {fmt}")
    assert_lse_close(lse, ref_l, "bf16", f"verify {heads}x{n} fmt {fmt}")


@pytest.mark.parametrize("heads,n", [(16, 4), (128, 2)])
def test_mla_verify_planted_key_goes_through_the_exact_fallback(heads, n):
    """A key far along the queries' direction at the last draft's own
    position: only the last draft sees it (its score outruns the fixed
    softmax reference, so the request is recomputed exactly), the earlier
    drafts must not.  At 128 heads x 2 drafts the last draft is the second
    slice of 128 rows: the first slice finishes normally, the second takes
    the fallback."""
    print(f"mla verify planted key heads {heads} drafts {n}", flush=True)
    case = W.mla_decode(seed=9, bs=3, len_range=(300, 900), num_q_heads=heads, num_draft=n)
    vals = W.make_values(case)
    i = 1
    L = int(case.regions["self"].kv_lens[i])
    u = torch.randn(576, generator=torch.Generator().manual_seed(6))
    u = u / u.norm()
    qrows = vals["q"]["self"][i * n:(i + 1) * n]
    qrows[:] = (u * 8.0).to(torch.bfloat16)[None, None, :]
    # the last draft's K row is stored this step: plant it in k_new
    vals["k_new"][(i + 1) * n - 1, 0] = (u * 200.0).to(torch.bfloat16)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_verify(dc, P.PKV_MAP_BLOCK_TABLE, n)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", "verify planted key")
    assert_lse_close(lse, ref_l, "bf16", "verify planted key")
    assert np.isfinite(ref_l[i * n + n - 1]).all() and ref_l[i * n + n - 1, 0] > ref_l[i * n, 0] + 50


def test_mla_decode_256_heads_in_two_slices():
    """256 query heads: two slices of 128 rows over one plan and workspace."""
    case = W.mla_decode(seed=12, bs=5, len_range=(1, 2000), num_q_heads=256)
    print("mla decode 256 heads", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = dc.decode(P.PKV_MAP_BLOCK_TABLE)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", "mla 256 heads")
    assert_lse_close(lse, ref_l, "bf16", "mla 256 heads")


def test_mla_verify_with_one_draft_equals_decode_bitwise():
    case = W.mla_decode(seed=4, bs=4, len_range=(10, 800), num_q_heads=64)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    o1, l1 = dc.decode(P.PKV_MAP_CSR)
    o2, l2 = run_verify(dc, P.PKV_MAP_CSR, 1)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("heads,n", [(16, 4), (128, 2)])
def test_mla_verify_append_equals_store_then_verify_bitwise(heads, n):
    """paged_verify_attn_append gives the bits of kv_store followed by
    paged_verify_attn: outputs, lse and the latent pool."""
    case = W.mla_decode(seed=20 + n, bs=5, len_range=(1, 900), num_q_heads=heads, num_draft=n,
                        fixed_lens={0: max(1, n - 1)})
    print(f"mla verify append heads {heads} drafts {n}", flush=True)
    vals = W.make_values(case, canary=True)
    a = DeviceCase(case, vals)
    a.store()
    oa, la = run_verify(a, P.PKV_MAP_BLOCK_TABLE, n)
    b = DeviceCase(case, vals)
    g = case.geom
    m = b.kv_map("self", P.PKV_MAP_BLOCK_TABLE)
    q = b.q["self"].view(case.bs, n, g.num_q_heads, g.head_dim_qk)
    out = torch.full((case.bs, n, g.num_q_heads, g.head_dim_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.bs, n, g.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    nb = P.paged_decode_workspace_bytes(b.pool, case.bs, n * g.num_q_heads, m.max_kv_len)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    P.paged_verify_attn_append(b.pool, 0, q, m, b.k_new, b.out_loc, case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, g.num_q_heads, g.head_dim_v).view(torch.int16), oa.view(torch.int16))
    assert torch.equal(lse.view(-1, g.num_q_heads).view(torch.int32), la.view(torch.int32))
    assert torch.equal(b.pool.flat("k", 0).view(torch.int16), a.pool.flat("k", 0).view(torch.int16))
