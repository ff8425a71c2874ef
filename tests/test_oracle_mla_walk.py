"""The multi-tile MLA parity assertions can fail (CPU only).

tests/test_gpu_mla_multitile.py compares the MLA decode with the oracle on
workloads where every run of tiles is 8 or more tiles long.  Here the same
assertion (tests/gpu_util.assert_attn_close, the bf16 tolerance
|g - o| <= 2e-2 + 1e-2 |o|) is run on results the oracle computes with a
planted mistake, for each mistake a kernel that streams a ring of tiles
could make: a zero output, a dropped tile, a tile read twice, a stale ring
buffer (the tile four places back), each at the first and last tile of a
piece and in each of the four ring slots.  Every one must fail, or the GPU
test could not catch it.  The runs are those of a 256-CU device."""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.cases import to_numpy_bits
from workloads.mla_walk import TILE, mla_walk, stream_layout, tile_roles

from gpu_util import assert_attn_close, oracle_after_store

RUNS = 256  # one run per compute unit of an MI355X


@pytest.fixture(scope="module")
def walk():
    case, vals, planted = mla_walk(seed=41, heads=128, num_draft=1)  # the GPU test's decode walk
    pk, _ = oracle_after_store(case, vals)
    q = to_numpy_bits(vals["q"]["self"])
    r = case.regions["self"]
    slots = [oracle.slots_from_token_table(case.req_to_token, case.req_pool_indices[i], r.kv_start[i], r.kv_lens[i])
             for i in range(case.bs)]
    return case, pk, q, slots, planted


def _attend(case, pk, q, slots, i, sl=None):
    """Oracle output of request i over slot list sl (default: its own)."""
    s = slots[i] if sl is None else sl
    K = oracle.to_f64(pk[np.asarray(s, np.int64)], "bf16")
    o, _ = oracle.attend(oracle.to_f64(q[i:i + 1], "bf16"), K, K[..., :512], case.sm_scale, True)
    return o


def _fails(got, ref):
    try:
        assert_attn_close(got, ref, "bf16", "planted mistake", record=False)
    except AssertionError:
        return True
    return False


def test_walk_covers_every_tile_and_runs_are_long(walk):
    case, pk, q, slots, planted = walk
    T, P, Bt, total = stream_layout(case.regions["self"].kv_lens, RUNS)
    assert Bt >= 8 and len(planted) == total
    assert {(p.request, p.tile) for p in planted} == {(i, j) for i in range(case.bs) for j in range(int(T[i]))}
    assert any(p.in_append for p in planted)


def test_planted_rows_return_their_value_row(walk):
    """The construction does what it claims: on the oracle, each planted
    row's output is its key's first 512 values."""
    case, pk, q, slots, planted = walk
    for i in (0, 7, 31):
        o = _attend(case, pk, q, slots, i)[0]
        for p in planted:
            if p.request == i:
                v = oracle.to_f64(pk[int(slots[i][p.pos])], "bf16")[0, :512]
                np.testing.assert_allclose(o[p.row], v, rtol=1e-5, atol=1e-5)


ROLES = ["piece_first", "piece_last", "ring_0", "ring_1", "ring_2", "ring_3"]


@pytest.mark.parametrize("role", ROLES)
def test_planted_mistakes_fail_the_assertion(walk, role):
    case, pk, q, slots, planted = walk
    r = case.regions["self"]
    roles = tile_roles(r.kv_lens, RUNS)
    # an example of the role inside a request, with four tiles before it
    # (so the stale-buffer mistake has a tile to read)
    i, j = next((i, j) for i, j in roles[role] if j >= 4)
    ref = _attend(case, pk, q, slots, i)
    assert not _fails(ref, ref)
    assert _fails(np.zeros_like(ref), ref), "zero output"
    s = np.asarray(slots[i])
    lo, hi = j * TILE, min((j + 1) * TILE, len(s))
    dropped = np.concatenate([s[:lo], s[hi:]])
    assert _fails(_attend(case, pk, q, slots, i, dropped), ref), f"tile {j} of request {i} dropped ({role})"
    twice = s.copy()
    twice[lo:hi] = s[lo - TILE:hi - TILE]
    assert _fails(_attend(case, pk, q, slots, i, twice), ref), f"tile {j - 1} read in place of {j} ({role})"
    stale = s.copy()
    stale[lo:hi] = s[lo - 4 * TILE:hi - 4 * TILE]
    assert _fails(_attend(case, pk, q, slots, i, stale), ref), f"stale ring buffer at tile {j} ({role})"


def test_unit_variance_zero_output_fails():
    """At the MLA geometry with unit-variance values the outputs are not all
    inside the absolute tolerance, so a zero output fails there too."""
    case = W.mla_decode(seed=32, bs=24, num_q_heads=128)  # the GPU test's decode case
    case.value_scale = 1.0
    vals = W.make_values(case)
    pk, _ = oracle_after_store(case, vals)
    r = case.regions["self"]
    _, _, Bt, _ = stream_layout(r.kv_lens, RUNS)
    assert Bt >= 8
    i = int(np.argmin(r.kv_lens))
    sl = oracle.slots_from_token_table(case.req_to_token, case.req_pool_indices[i], r.kv_start[i], r.kv_lens[i])
    q = to_numpy_bits(vals["q"]["self"])
    K = oracle.to_f64(pk[np.asarray(sl, np.int64)], "bf16")
    ref, _ = oracle.attend(oracle.to_f64(q[i:i + 1], "bf16"), K, K[..., :512], case.sm_scale, True)
    assert _fails(np.zeros_like(ref), ref)
