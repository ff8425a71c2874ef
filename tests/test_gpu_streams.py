"""Calls on two streams at once share no hidden state: decode of one batch
on one stream and extend of another on a second stream, each with its own
workspace, overlap on the device and still give the bits of the same
calls run one after the other on the default stream."""
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, i32, offsets

pytestmark = pytest.mark.gpu


def test_two_streams_give_the_sequential_bits():
    dcase = W.qwen3_decode(seed=8, bs=32, len_range=(100, 3000), pool_tokens=100000, max_context=3072)
    ecase = W.encdec_extend(seed=8, bs=6, enc_len=400, prefix_range=(0, 100), new_range=(1, 300))
    dd = DeviceCase(dcase, W.make_values(dcase))
    de = DeviceCase(ecase, W.make_values(ecase))
    dd.store()
    de.store()
    dm = dd.kv_map("self", P.PKV_MAP_TOKEN_TABLE)
    em = de.kv_map("cross", P.PKV_MAP_CSR)
    g, ge = dcase.geom, ecase.geom
    d_out = torch.empty((dcase.bs, g.num_q_heads, g.head_dim_v), dtype=torch.bfloat16, device="cuda")
    d_lse = torch.empty((dcase.bs, g.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(P.paged_decode_workspace_bytes(dd.pool, dcase.bs, g.num_q_heads, dm.max_kv_len), 256),
                     dtype=torch.uint8, device="cuda")
    qo = i32(offsets(ecase.q_lens))
    tq = int(ecase.q_lens.sum())
    e_out = torch.empty((tq, ge.num_q_heads, ge.head_dim_v), dtype=torch.bfloat16, device="cuda")
    e_lse = torch.empty((tq, ge.num_q_heads), dtype=torch.float32, device="cuda")

    def run(s1, s2, reps):
        for _ in range(reps):
            P.paged_decode_attn(dd.pool, 0, dd.q["self"], dm, dcase.sm_scale, d_out, d_lse, ws, stream=s1)
            P.paged_extend_attn(de.pool, 0, de.q["cross"], qo, int(ecase.q_lens.max()), em, False, ecase.sm_scale,
                                e_out, e_lse, stream=s2)

    run(None, None, 1)
    torch.cuda.synchronize()
    refs = [t.clone() for t in (d_out, d_lse, e_out, e_lse)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for t in (d_out, d_lse, e_out, e_lse):
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    run(s1, s2, 5)
    torch.cuda.synchronize()
    for t, r in zip((d_out, d_lse, e_out, e_lse), refs):
        assert torch.equal(t.view(torch.uint8), r.view(torch.uint8))
