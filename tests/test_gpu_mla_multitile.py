"""GPU parity of the MLA decode and target verification where every
workgroup streams many tiles: the requests' 32-key tiles are cut into one
run per CU, and these workloads give each run 8 or more tiles, so the
kernel's four-deep LDS tile ring turns over several times per run, pieces
start and end at run edges inside requests, and the softmax reference
fixed at a piece's first tile is carried across tiles ([BACKEND]
"AttentionBackend", init_forward_metadata: decode and target-verify
branches of the split metadata).

Two kinds of input:

* unit-variance values at the MLA workload's geometry (128 heads or 32 heads
  x 4 drafts over latent rows of 576 / 512, page size 64, lengths
  U[4096, 16384]): scores of standard deviation ~1, outputs of 1e-2 to
  1e-1, compared with the fp64 oracle on sampled requests;
* the planted-key walk (workloads.mla_walk): every tile of every request
  holds one key that dominates one query row, so that row's output is that
  key's value row.  A dropped, repeated or stale tile, or a zero output,
  moves some output by about its own size (~3), far outside the tolerance;
  tests/test_oracle_mla_walk.py shows on the CPU that these assertions fail
  for each such mistake.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W
from workloads.mla_walk import mla_walk, stream_layout, tile_roles

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, oracle_region, run_verify

pytestmark = pytest.mark.gpu


def _runs() -> int:
    # the kernel cuts the tile stream into one run per compute unit
    return torch.cuda.get_device_properties(0).multi_processor_count


def _sample(lens, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(len(lens), size=min(k, len(lens)), replace=False).tolist())
    pick |= {int(np.argmin(lens)), int(np.argmax(lens))}
    return sorted(pick)


def _run(dc, n, fmt):
    if n == 1:
        return dc.decode(fmt)
    return run_verify(dc, fmt, n)


@pytest.mark.parametrize("n,fmt", [(1, P.PKV_MAP_BLOCK_TABLE), (1, P.PKV_MAP_CSR), (4, P.PKV_MAP_BLOCK_TABLE)])
def test_mla_unit_variance_many_tiles_per_run(n, fmt):
    heads = 128 // n
    case = W.mla_decode(seed=31 + n, bs=24, num_q_heads=heads, num_draft=n)
    case.value_scale = 1.0
    r = case.regions["self"]
    _, _, Bt, total = stream_layout(r.kv_lens, _runs())
    print(f"mla unit variance n {n} fmt {fmt}: {total} tiles, {Bt} per run", flush=True)
    assert Bt >= 8
    vals = W.make_values(case, device="cuda", canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = _run(dc, n, fmt)
    reqs = _sample(r.kv_lens, 8, seed=n)
    ref_o, ref_l = oracle_region(case, vals, "self", requests=reqs)
    rows = np.concatenate([np.arange(i * n, (i + 1) * n) for i in reqs])
    st = assert_attn_close(out, ref_o, "bf16", f"mla unit variance n={n} fmt={fmt} Bt={Bt}", rows=rows)
    assert_lse_close(lse, ref_l, "bf16", "mla unit variance", rows=rows)
    # the outputs are not all below the absolute tolerance: a zero output fails
    assert np.mean(np.abs(ref_o[rows]) > 2e-2 / 0.99) > 0.1
    print(f"  max_abs {st['max_abs']:.3e} max_rel {st['max_rel']} rms {st['rms']:.3e}", flush=True)


@pytest.mark.parametrize("n,fmt", [(1, P.PKV_MAP_BLOCK_TABLE), (1, P.PKV_MAP_TOKEN_TABLE), (4, P.PKV_MAP_CSR)])
def test_mla_planted_walk_every_tile_of_every_run(n, fmt):
    heads = 128 // n
    case, vals, planted = mla_walk(seed=40 + n, heads=heads, num_draft=n, device="cuda")
    r = case.regions["self"]
    runs = _runs()
    _, _, Bt, total = stream_layout(r.kv_lens, runs)
    roles = tile_roles(r.kv_lens, runs)
    print(f"mla planted walk n {n} fmt {fmt}: {len(planted)} planted keys, {total} tiles, {Bt} per run, "
          f"{len(roles['piece_first'])} pieces", flush=True)
    assert Bt >= 8 and len(planted) == total
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = _run(dc, n, fmt)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"mla planted walk n={n} fmt={fmt} Bt={Bt}")
    assert_lse_close(lse, ref_l, "bf16", "mla planted walk")
    # each planted row returns its planted key's value row
    g = out.float().cpu().numpy()
    k_rows = vals["pool_k"].float().cpu().numpy()
    k_new = vals["k_new"].float().cpu().numpy()
    first_new = np.concatenate([[0], np.cumsum(np.minimum(n, r.kv_lens))])
    bad = []
    for p in planted:
        L = int(r.kv_lens[p.request])
        if p.in_append:
            v = k_new[first_new[p.request] + p.pos - (L - min(n, L)), 0, :512]
        else:
            v = k_rows[int(case.req_to_token[case.req_pool_indices[p.request], p.pos]), 0, :512]
        j, h = divmod(p.row, heads)
        got = g[p.request * n + j, h]
        if not np.all(np.abs(got - v) <= 2e-2 + 1e-2 * np.abs(v)):
            bad.append((p.request, p.row, p.pos, p.tile))
    assert not bad, f"{len(bad)} planted rows miss their key, first {bad[:5]}"
