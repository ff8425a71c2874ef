"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (same builders, seeds, map formats and call sequence).  The oracle
checks every request where that takes seconds and a seeded sample (always
including the shortest and the longest request) where it would take longer;
index building and the KV append are checked bit-exactly in full.

fp32 copies of the Qwen3-shaped and prefix-sharing decode workloads run
against the 1e-5 bound: a dropped or repeated page moves an fp32 output far
more than that, even where bf16 tolerance could hide it."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_38_amd as P
import workloads as W
from workloads.cases import to_numpy_bits

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, i32, oracle_after_store, oracle_region, \
    run_extend, run_verify

pytestmark = pytest.mark.gpu


def _sample(case, k, seed=5):
    """Seeded sample of k requests plus the shortest and the longest."""
    L = case.regions["self"].kv_lens
    if k is None or k >= case.bs:
        return list(range(case.bs))
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(case.bs, size=k, replace=False).tolist())
    pick |= {int(np.argmin(L)), int(np.argmax(L))}
    return sorted(pick)


def _as_f32(case):
    return dataclasses.replace(case, geom=dataclasses.replace(case.geom, dtype="f32"))


DECODE = {
    # name: (builder, map format used by bench.py, requests checked (None = all))
    "qwen3_decode": (lambda: W.qwen3_decode(seed=0), P.PKV_MAP_TOKEN_TABLE, None),
    "gqa_prefix_share_ps16": (lambda: W.gqa_prefix_share(16, seed=0), P.PKV_MAP_CSR, 40),
    "gqa_prefix_share_ps64": (lambda: W.gqa_prefix_share(64, seed=0), P.PKV_MAP_CSR, 40),
    "mla_decode": (lambda: W.mla_decode(seed=0), P.PKV_MAP_BLOCK_TABLE, 24),
    "qwen3_decode_f32": (lambda: _as_f32(W.qwen3_decode(seed=0)), P.PKV_MAP_TOKEN_TABLE, 24),
    "gqa_prefix_share_ps16_f32": (lambda: _as_f32(W.gqa_prefix_share(16, seed=0)), P.PKV_MAP_CSR, 24),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_full_size(name):
    build, fmt, k = DECODE[name]
    case = build()
    print(f"full-size decode {name}: bs {case.bs}, sum L {int(case.regions['self'].kv_lens.sum())}", flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    if case.n_new:
        dc.store()
    out, lse = dc.decode(fmt)
    pk, pv = oracle_after_store(case, vals)
    if case.n_new:  # the append, bit-exact on every stored row
        got = to_numpy_bits(dc.pool.flat("k", 0))[case.out_loc]
        assert np.array_equal(got.view(np.uint8), pk[case.out_loc].view(np.uint8))
    reqs = _sample(case, k)
    ref_o, ref_l = oracle_region(case, vals, "self", pk, pv, requests=reqs)
    rows = np.asarray(reqs)
    assert_attn_close(out, ref_o, case.geom.dtype, name, rows=rows)
    assert_lse_close(lse, ref_l, case.geom.dtype, name, rows=rows)


@pytest.mark.parametrize("name", ["gqa_prefix_share_ps16", "gqa_prefix_share_ps64", "mla_decode"])
def test_build_indices_full_size(name):
    build, fmt, _ = DECODE[name]
    case = build()
    r = case.regions["self"]
    ps = case.geom.page_size
    maxl = int(r.kv_lens.max())
    per = -(-maxl // ps)
    tab, rpi, ks, kl = i32(case.req_to_token), i32(case.req_pool_indices), i32(r.kv_start), i32(r.kv_lens)
    if fmt == P.PKV_MAP_CSR:
        ref_ptr, ref_idx = oracle.build_csr(case.req_to_token, case.req_pool_indices, r.kv_start, r.kv_lens, ps)
        indptr = torch.empty(case.bs + 1, dtype=torch.int32, device="cuda")
        idx = torch.full((case.bs * per,), -7, dtype=torch.int32, device="cuda")
        P.build_kv_indices(fmt, tab, rpi, ks, kl, ps, maxl, indptr, idx)
        torch.cuda.synchronize()
        assert np.array_equal(indptr.cpu().numpy(), ref_ptr)
        assert np.array_equal(idx.cpu().numpy()[:len(ref_idx)], ref_idx)
    else:
        ref = oracle.build_block_table(case.req_to_token, case.req_pool_indices, r.kv_start, r.kv_lens, ps, per)
        bt = torch.full((case.bs, per), -7, dtype=torch.int32, device="cuda")
        P.build_kv_indices(fmt, tab, rpi, ks, kl, ps, maxl, None, bt)
        torch.cuda.synchronize()
        assert np.array_equal(bt.cpu().numpy(), ref)


@pytest.mark.parametrize("ragged", [False, True])
def test_extend_full_size(ragged):
    case = W.encdec_extend(seed=0)
    print(f"full-size encoder-decoder extend (ragged={ragged}): bs {case.bs}, sum n {int(case.q_lens.sum())}",
          flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    dc.store()
    pk, pv = oracle_after_store(case, vals)
    for name in ("self", "cross"):
        out, lse = run_extend(dc, name, P.PKV_MAP_CSR, contiguous=ragged)
        ref_o, ref_l = oracle_region(case, vals, name, pk, pv)
        assert_attn_close(out, ref_o, "bf16", f"extend {name}")
        assert_lse_close(lse, ref_l, "bf16", f"extend {name}")


def test_verify_full_size():
    """Target verification at its benchmark shape: bs 128, L ~ U{4096..16384}
    including the drafts, 32 heads x 4 drafts folded into 128 rows, block
    table; the oracle checks a seeded sample of requests, every draft."""
    n = 4
    case = W.mla_decode(seed=0, num_q_heads=32, num_draft=n)
    print(f"full-size target verification: bs {case.bs}, sum L {int(case.regions['self'].kv_lens.sum())}",
          flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_verify(dc, P.PKV_MAP_BLOCK_TABLE, n)
    pk, pv = oracle_after_store(case, vals)
    got = to_numpy_bits(dc.pool.flat("k", 0))[case.out_loc]  # the drafts' K rows, bit-exact
    assert np.array_equal(got.view(np.uint8), pk[case.out_loc].view(np.uint8))
    reqs = _sample(case, 16)
    ref_o, ref_l = oracle_region(case, vals, "self", pk, pv, requests=reqs)
    rows = np.asarray([i * n + j for i in reqs for j in range(n)])
    assert_attn_close(out, ref_o, "bf16", "verify full size", rows=rows)
    assert_lse_close(lse, ref_l, "bf16", "verify full size", rows=rows)


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_mixed_spans_full_size(softcap):
    """Mixed causal/full spans at their benchmark shape (4 rows of a
    128-token causal span and a 2048-token full span, 32 / 8 heads, D 128,
    CSR map, per-segment flags), every segment checked."""
    case = W.mixed_spans(seed=0)
    print(f"full-size mixed spans (softcap {softcap}): {case.bs} segments, sum n {int(case.q_lens.sum())}",
          flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, "self", P.PKV_MAP_CSR, softcap=softcap)
    pk, pv = oracle_after_store(case, vals)
    ref_o, ref_l = oracle_region(case, vals, "self", pk, pv, softcap=softcap)
    assert_attn_close(out, ref_o, "bf16", f"mixed spans full size, cap {softcap}")
    assert_lse_close(lse, ref_l, "bf16", f"mixed spans full size, cap {softcap}")


def test_extend_full_size_f32():
    """The encoder-decoder extend at full size in fp32 (the vector-ALU
    kernel), every request against the oracle at 1e-5 + 1e-5 |o|: a dropped
    or repeated key tile moves an fp32 output far more than that."""
    case = W.encdec_extend(seed=0)
    case.geom.dtype = "f32"
    print(f"full-size encoder-decoder extend, fp32: bs {case.bs}, sum n {int(case.q_lens.sum())}", flush=True)
    vals = W.make_values(case, device="cuda")
    dc = DeviceCase(case, vals)
    dc.store()
    pk, pv = oracle_after_store(case, vals)
    for name in ("self", "cross"):
        out, lse = run_extend(dc, name, P.PKV_MAP_CSR)
        ref_o, ref_l = oracle_region(case, vals, name, pk, pv)
        assert_attn_close(out, ref_o, "f32", f"extend {name} f32")
        assert_lse_close(lse, ref_l, "f32", f"extend {name} f32")
