"""bf16 decode over the head shapes the stream kernel accepts beyond the
workloads' 8 KV heads: one, two, three and four KV heads (the one-, two-
and four-wave launch shapes), head_dim 64 and 128, and query groups of 1
to 16 heads per KV head, odd ones included; against the oracle, in the
three map formats, plain and with the append in the call."""
import dataclasses

import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, oracle_region

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]

SHAPES = [  # (KV heads, query heads per KV head, head_dim)
    (1, 1, 64), (1, 16, 128), (2, 8, 64), (2, 3, 128), (3, 5, 128), (4, 4, 64), (4, 16, 128), (8, 1, 64),
]


@pytest.mark.parametrize("hkv,group,d", SHAPES)
def test_decode_head_shapes(hkv, group, d):
    base = W.qwen3_decode(seed=hkv * 100 + group, bs=12, len_range=(1, 900), pool_tokens=12000, max_context=1024)
    g = dataclasses.replace(base.geom, num_kv_heads=hkv, num_q_heads=hkv * group, head_dim_qk=d, head_dim_v=d)
    case = dataclasses.replace(base, geom=g, sm_scale=d ** -0.5)
    print(f"decode shape: {hkv} kv heads x {group}, head_dim {d}", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    ref_o, ref_l = oracle_region(case, vals, "self")
    for fmt in FMTS:
        out, lse = dc.decode(fmt)
        assert_attn_close(out, ref_o, "bf16", f"{hkv}x{group} d{d} fmt {fmt}")
        assert_lse_close(lse, ref_l, "bf16", f"{hkv}x{group} d{d} fmt {fmt}")
    # the same step with the append carried by the decode call
    b = DeviceCase(case, vals)
    m = b.kv_map("self", P.PKV_MAP_TOKEN_TABLE)
    out = torch.full((case.bs, g.num_q_heads, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.bs, g.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    nb = P.paged_decode_workspace_bytes(b.pool, case.bs, g.num_q_heads, m.max_kv_len)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    P.paged_decode_attn_append(b.pool, 0, b.q["self"], m, b.k_new, b.v_new, b.out_loc, case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    assert_attn_close(out, ref_o, "bf16", f"append {hkv}x{group} d{d}")
    assert_lse_close(lse, ref_l, "bf16", f"append {hkv}x{group} d{d}")
