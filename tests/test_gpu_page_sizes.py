"""Page sizes beyond the workloads' 1, 16 and 64: decode, cascade decode,
MLA decode and extend (paged and ragged) against the oracle at page sizes
1 to 128, the whole range the pool accepts.  The index math (slot = page * page_size +
offset) and every tile that straddles a page boundary change with it."""
import dataclasses

import numpy as np
import pytest

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, oracle_region, run_extend
from test_gpu_cascade import cascade

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


@pytest.mark.parametrize("ps", [2, 8, 32, 128])
def test_decode_and_cascade_at_page_size(ps):
    case = W.gqa_prefix_share(ps, seed=ps, bs=16, prefix=256, median=300, sigma=0.8, clip=(1, 1500))
    print(f"page size {ps}: decode, cascade", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    ref_o, ref_l = oracle_region(case, vals, "self")
    for fmt in FMTS:
        out, lse = dc.decode(fmt)
        assert_attn_close(out, ref_o, "bf16", f"decode ps {ps} fmt {fmt}")
        assert_lse_close(lse, ref_l, "bf16", f"decode ps {ps} fmt {fmt}")
    ip, pl = case.prefix_groups
    out, lse = cascade(dc, P.PKV_MAP_CSR, ip, pl)
    assert_attn_close(out, ref_o, "bf16", f"cascade ps {ps}")
    assert_lse_close(lse, ref_l, "bf16", f"cascade ps {ps}")


@pytest.mark.parametrize("ps", [1, 4, 32, 128])
def test_extend_at_page_size(ps):
    case = W.encdec_extend(seed=ps, bs=5, enc_len=150, prefix_range=(0, 90), new_range=(1, 200), page_size=ps)
    print(f"page size {ps}: extend", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    for region in ("self", "cross"):
        ref_o, ref_l = oracle_region(case, vals, region)
        for fmt, ragged in ((P.PKV_MAP_CSR, False), (P.PKV_MAP_BLOCK_TABLE, False), (P.PKV_MAP_CSR, True)):
            out, lse = run_extend(dc, region, fmt, contiguous=ragged)
            assert_attn_close(out, ref_o, "bf16", f"extend {region} ps {ps} fmt {fmt} ragged {ragged}")
            assert_lse_close(lse, ref_l, "bf16", f"extend {region} ps {ps} fmt {fmt} ragged {ragged}")


@pytest.mark.parametrize("ps", [1, 16, 128])
def test_mla_decode_at_page_size(ps):
    """The MLA pool (one 576-value latent row per token) at page sizes other
    than the workload's 64, in every map format, with the step's append."""
    # unit-variance values, so the outputs (~1e-1) are far above the tolerance's absolute part
    case = dataclasses.replace(W.mla_decode(seed=ps, bs=6, len_range=(1, 1400), num_q_heads=32, page_size=ps),
                               value_scale=1.0)
    print(f"page size {ps}: mla decode", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    ref_o, ref_l = oracle_region(case, vals, "self")
    for fmt in FMTS:
        out, lse = dc.decode(fmt)
        assert_attn_close(out, ref_o, "bf16", f"mla ps {ps} fmt {fmt}")
        assert_lse_close(lse, ref_l, "bf16", f"mla ps {ps} fmt {fmt}")
