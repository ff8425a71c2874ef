"""Every attention path reads only the layer it is given.  A three-layer
pool holds the case in layer 2 and NaN in layers 0 and 1; every call must
give the bits of the same call on a one-layer pool (a wrong layer offset
reads NaN or zeros and fails the comparison)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, i32, run_extend, run_verify
from test_gpu_cascade import cascade, small

pytestmark = pytest.mark.gpu


def pair(case, vals):
    one = DeviceCase(case, vals)
    many = DeviceCase(case, vals, num_layers=3, layer=2)
    many.k_buf.view(3, -1)[:2].fill_(float("nan"))
    if many.v_buf is not None:
        many.v_buf.view(3, -1)[:2].fill_(float("nan"))
    one.store()
    many.store()
    return one, many


def same_bits(a, b):
    for x, y in zip(a, b):
        assert x.shape == y.shape
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name", ["qwen3_bf16", "tiny_f32", "mla"])
def test_decode_reads_only_its_layer(name):
    case = {"qwen3_bf16": lambda: W.qwen3_decode(seed=5, bs=8, len_range=(1, 700), pool_tokens=8000,
                                                 max_context=768),
            "tiny_f32": lambda: W.tiny_decode(seed=5),
            "mla": lambda: W.mla_decode(seed=5, bs=5, len_range=(1, 900))}[name]()
    print(f"layer offsets: decode {name}", flush=True)
    vals = W.make_values(case)
    one, many = pair(case, vals)
    for fmt in (P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE):
        same_bits(one.decode(fmt), many.decode(fmt))


def test_decode_append_writes_and_reads_only_its_layer():
    case = W.qwen3_decode(seed=6, bs=8, len_range=(1, 700), pool_tokens=8000, max_context=768)
    vals = W.make_values(case)
    one = DeviceCase(case, vals)
    one.store()
    ref = one.decode(P.PKV_MAP_TOKEN_TABLE)
    many = DeviceCase(case, vals, num_layers=3, layer=2)
    many.k_buf.view(3, -1)[:2].fill_(float("nan"))
    many.v_buf.view(3, -1)[:2].fill_(float("nan"))
    g = case.geom
    m = many.kv_map("self", P.PKV_MAP_TOKEN_TABLE)
    out = torch.full_like(ref[0], float("nan"))
    lse = torch.full_like(ref[1], float("nan"))
    nb = P.paged_decode_workspace_bytes(many.pool, case.bs, g.num_q_heads, m.max_kv_len)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    P.paged_decode_attn_append(many.pool, 2, many.q["self"], m, many.k_new, many.v_new, many.out_loc,
                               case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    same_bits(ref, (out, lse))
    assert torch.isnan(many.k_buf.view(3, -1)[:2].float()).all()  # the append stayed in layer 2


@pytest.mark.parametrize("ragged", [False, True])
def test_extend_reads_only_its_layer(ragged):
    case = W.encdec_extend(seed=5, bs=4, enc_len=100, prefix_range=(0, 40), new_range=(1, 60))
    print(f"layer offsets: extend ragged={ragged}", flush=True)
    vals = W.make_values(case)
    one, many = pair(case, vals)
    for region in ("self", "cross"):
        same_bits(run_extend(one, region, P.PKV_MAP_CSR, contiguous=ragged),
                  run_extend(many, region, P.PKV_MAP_CSR, contiguous=ragged))


def test_verify_and_cascade_read_only_their_layer():
    n = 4
    case = W.mla_decode(seed=7, bs=4, len_range=(8, 700), num_q_heads=16, num_draft=n)
    vals = W.make_values(case)
    one, many = pair(case, vals)
    same_bits(run_verify(one, P.PKV_MAP_BLOCK_TABLE, n), run_verify(many, P.PKV_MAP_BLOCK_TABLE, n))
    case = small(16, seed=3, bs=16, prefix=256)
    vals = W.make_values(case)
    one, many = pair(case, vals)
    ip, pl = case.prefix_groups
    same_bits(cascade(one, P.PKV_MAP_CSR, ip, pl), cascade(many, P.PKV_MAP_CSR, ip, pl))
