"""paged_decode_attn_noalloc -- the decode for callers that cannot allocate --
against paged_decode_attn with a caller workspace, through the C ABI.

The two calls run the same kernels; only the workspace differs (the
library's own device array instead of the caller's buffer), so the outputs
and lse must agree bit for bit.  Each test makes two calls in a row on the
shared array, the second with a smaller batch, so a call that read what the
previous one left behind would show."""
import dataclasses

import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase

pytestmark = pytest.mark.gpu


def _f32(case):
    return dataclasses.replace(case, geom=dataclasses.replace(case.geom, dtype="f32"))


SEQUENCES = {
    "gqa_bf16": [(lambda: W.gqa_prefix_share(16, seed=0), P.PKV_MAP_CSR),
                 (lambda: W.gqa_prefix_share(16, seed=4, bs=16, prefix=256, median=300, sigma=0.8, clip=(1, 1500)),
                  P.PKV_MAP_CSR)],
    "qwen3_bf16": [(lambda: W.qwen3_decode(seed=0), P.PKV_MAP_TOKEN_TABLE),
                   (lambda: W.qwen3_decode(seed=3, bs=8, len_range=(1, 700), pool_tokens=20000, max_context=1024),
                    P.PKV_MAP_TOKEN_TABLE)],
    "mla_bf16": [(lambda: W.mla_decode(seed=0), P.PKV_MAP_BLOCK_TABLE),
                 (lambda: W.mla_decode(seed=6, bs=9, len_range=(1, 3000)), P.PKV_MAP_BLOCK_TABLE)],
    "f32": [(lambda: _f32(W.qwen3_decode(seed=2, bs=16, len_range=(100, 2000), pool_tokens=40000,
                                         max_context=2048)), P.PKV_MAP_TOKEN_TABLE),
            (lambda: W.tiny_decode(seed=0), P.PKV_MAP_CSR)],
}


@pytest.mark.parametrize("name", list(SEQUENCES))
def test_noalloc_equals_workspace_decode_twice(name):
    for k, (build, fmt) in enumerate(SEQUENCES[name]):
        case = build()
        print(f"noalloc {name} call {k}: bs {case.bs}, max len {int(case.regions['self'].kv_lens.max())}", flush=True)
        dc = DeviceCase(case, W.make_values(case, device="cuda"))
        if case.n_new:
            dc.store()
        ref_o, ref_l = dc.decode(fmt)
        g = case.geom
        m = dc.kv_map("self", fmt)
        out = torch.full((case.bs, g.num_q_heads, g.head_dim_v), float("nan"), dtype=dc.dtype, device="cuda")
        lse = torch.full((case.bs, g.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        P.paged_decode_attn_noalloc(dc.pool, dc.layer, dc.q["self"], m, case.sm_scale, out, lse)
        torch.cuda.synchronize()
        bits = torch.int16 if dc.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(bits), ref_o.view(bits)), f"{name} call {k}: outputs differ"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"{name} call {k}: lse differs"


def test_noalloc_rejects_a_batch_past_its_array():
    """A shape whose workspace exceeds the array is refused before launch."""
    case = W.mla_decode(seed=6, bs=9, len_range=(1, 3000))
    dc = DeviceCase(case, W.make_values(case, device="cuda"))
    g = case.geom
    bs, maxl = 4096, 65536
    assert P.paged_decode_workspace_bytes(dc.pool, bs, g.num_q_heads, maxl) > (128 << 20)
    lens = torch.ones(bs, dtype=torch.int32, device="cuda")
    bt = torch.zeros((bs, maxl // 64), dtype=torch.int32, device="cuda")
    m = P.make_kv_map(P.PKV_MAP_BLOCK_TABLE, lens, maxl, block_table=bt)
    q = torch.zeros((bs, g.num_q_heads, g.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((bs, g.num_q_heads, g.head_dim_v), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.PagedKVError) as e:
        P.paged_decode_attn_noalloc(dc.pool, 0, q, m, case.sm_scale, out)
    assert e.value.status == P._lib.PKV_ECAPACITY
