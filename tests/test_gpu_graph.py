"""The hot-path calls are asynchronous, allocate nothing and issue no memset,
so they may be captured in a HIP graph.  Each case captures one step,
replays it several times with eager work and synchronisations in between,
and checks every replay bit for bit against the eager result."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, i32, run_extend

pytestmark = pytest.mark.gpu


def capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def check_replays(g, outputs, refs, reset, eager):
    for r in range(4):
        for o in outputs:
            reset(o)
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outputs, refs):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"replay {r}"
        eager()
        torch.cuda.synchronize()


def _decode_case(name):
    if name == "qwen3_small":
        return W.qwen3_decode(seed=1, bs=16), P.PKV_MAP_TOKEN_TABLE
    if name == "mla_small":
        return W.mla_decode(seed=1, bs=8, len_range=(100, 900)), P.PKV_MAP_BLOCK_TABLE
    # prefix sharing: the decode's own shared-prefix detection and prefix work
    return W.gqa_prefix_share(16, seed=5, bs=24, group=8, prefix=512, median=600, clip=(64, 2000)), P.PKV_MAP_CSR


# (the prefix-sharing workload stores nothing, so it runs without the append)
@pytest.mark.parametrize("name,append", [("qwen3_small", False), ("qwen3_small", True), ("mla_small", False),
                                         ("mla_small", True), ("prefix_share_small", False)])
def test_decode_step_replays_bitwise(name, append):
    case, fmt = _decode_case(name)
    assert case.n_new or not append
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    g_ = case.geom
    m = dc.kv_map("self", fmt)
    out = torch.empty((case.bs, g_.num_q_heads, g_.head_dim_v), dtype=dc.dtype, device="cuda")
    lse = torch.empty((case.bs, g_.num_q_heads), dtype=torch.float32, device="cuda")
    nb = P.paged_decode_workspace_bytes(dc.pool, case.bs, g_.num_q_heads, m.max_kv_len)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")

    def step():
        if append:  # the append rides in the decode's planner launch
            P.paged_decode_attn_append(dc.pool, 0, dc.q["self"], m, dc.k_new, dc.v_new, dc.out_loc, case.sm_scale,
                                       out, lse, ws)
        else:
            dc.store()
            P.paged_decode_attn(dc.pool, 0, dc.q["self"], m, case.sm_scale, out, lse, ws)

    step()
    torch.cuda.synchronize()
    refs = [out.clone(), lse.clone()]
    g = capture(step)
    check_replays(g, [out, lse], refs, lambda t: t.fill_(float("nan")), step)


def test_cascade_and_extend_replay_bitwise():
    case = W.gqa_prefix_share(16, seed=2, bs=16, group=8, prefix=256, median=256, clip=(64, 1024))
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    g_ = case.geom
    m = dc.kv_map("self", P.PKV_MAP_CSR)
    groups = P.make_prefix_groups(i32(case.prefix_groups[0]), i32(case.prefix_groups[1]), 8, 256)
    out = torch.empty((case.bs, g_.num_q_heads, g_.head_dim_v), dtype=torch.bfloat16, device="cuda")
    nb = P.paged_decode_cascade_workspace_bytes(dc.pool, case.bs, g_.num_q_heads, m.max_kv_len, groups)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")

    def step():
        P.paged_decode_attn_cascade(dc.pool, 0, dc.q["self"], m, groups, case.sm_scale, out, None, ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(step)
    check_replays(g, [out], [ref], lambda t: t.fill_(float("nan")), step)

    ecase = W.encdec_extend(seed=3, bs=4, enc_len=200, prefix_range=(0, 60), new_range=(1, 100))
    evals = W.make_values(ecase)
    edc = DeviceCase(ecase, evals)
    edc.store()
    res = {}

    def estep():
        res["o"], res["l"] = run_extend(edc, "self", P.PKV_MAP_TOKEN_TABLE)

    estep()
    eref = res["o"].clone()
    # run_extend allocates its outputs: capture a step that writes fixed buffers instead
    qo = i32(np.concatenate([[0], np.cumsum(ecase.q_lens)]))
    em = edc.kv_map("self", P.PKV_MAP_TOKEN_TABLE)
    eout = torch.empty_like(eref)

    def estep_fixed():
        P.paged_extend_attn(edc.pool, 0, edc.q["self"], qo, int(ecase.q_lens.max()), em, True, ecase.sm_scale, eout)

    g2 = capture(estep_fixed)
    check_replays(g2, [eout], [eref], lambda t: t.fill_(float("nan")), estep_fixed)


def test_allocator_step_replays():
    """A decode allocation step (alloc, row write, free of the same slots)
    captured once: the free list advances with every replay (freed pages go
    to the back), exactly as a second free list driven by eager calls does."""
    w = __import__("workloads.alloc", fromlist=["serving_alloc"]).serving_alloc(True)
    bs = 256
    seq, rpi = i32(w.seq_lens[:bs]), i32(np.arange(bs))
    pre = i32(w.prefix_lens[:bs])
    last = i32(np.full(bs, -1))
    width = int(w.seq_lens[:bs].max())

    def make():
        fl = P.kv_free_list_create(w.page_size, w.num_pages)
        out = torch.empty(bs, dtype=torch.int32, device="cuda")
        table = torch.zeros((bs, width), dtype=torch.int32, device="cuda")

        def step():
            P.kv_alloc_decode(fl, seq, last, out)
            P.write_req_to_token(table, rpi, pre, seq, out, width)
            P.kv_free(fl, out)
        return fl, out, table, step

    fa, out_a, tab_a, step_a = make()
    fb, out_b, tab_b, step_b = make()
    step_a()
    step_b()
    torch.cuda.synchronize()
    g = capture(step_a)  # the capture's warm-up runs the step once more on list A
    step_b()
    for r in range(4):
        g.replay()
        step_b()
        torch.cuda.synchronize()
        for x, y in ((out_a, out_b), (tab_a, tab_b), (fa.state, fb.state), (fa.pages, fb.pages)):
            assert torch.equal(x, y), f"replay {r}"
        assert int(fa.status.item()) == int(fb.status.item()) == P.PKV_ALLOC_OK
