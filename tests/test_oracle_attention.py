"""Pins of the oracle's attention against brute force, a library routine,
closed forms and the invariants the pages fix.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.cases import to_numpy_bits


# --------------------------------------------------------------------------
# brute force: pure Python, math.exp / math.fsum, tiny inputs
# --------------------------------------------------------------------------

def brute_attention(q, K, V, scale, causal):
    n, Hq, D = len(q), len(q[0]), len(q[0][0])
    L, Hkv = len(K), (len(K[0]) if len(K) else 1)
    G = Hq // Hkv
    Dv = len(V[0][0]) if L else 0
    out, lse = [], []
    for j in range(n):
        orow, lrow = [], []
        for h in range(Hq):
            g = h // G
            keys = [t for t in range(L) if (not causal) or t <= L - n + j]
            if not keys:
                orow.append([0.0] * max(Dv, 1))
                lrow.append(-math.inf)
                continue
            s = [scale * math.fsum(q[j][h][d] * K[t][g][d] for d in range(D)) for t in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            orow.append([math.fsum(e[a] * V[t][g][d] for a, t in enumerate(keys)) / tot for d in range(Dv)])
            lrow.append(m + math.log(tot))
        out.append(orow)
        lse.append(lrow)
    return out, lse


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [False, True])
def test_attend_matches_brute_force(seed, causal):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 3))
    Hq, D, Dv = Hkv * G, int(rng.integers(1, 5)), int(rng.integers(1, 5))
    L = int(rng.integers(1, 7))
    n = int(rng.integers(1, L + 1))
    q = rng.normal(size=(n, Hq, D))
    K = rng.normal(size=(L, Hkv, D))
    V = rng.normal(size=(L, Hkv, Dv))
    scale = float(rng.uniform(0.2, 1.5))
    o, l = oracle.attend(q, K, V, scale, causal)
    bo, bl = brute_attention(q.tolist(), K.tolist(), V.tolist(), scale, causal)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=0, atol=1e-12)


def test_attend_matches_sdpa_float64():
    """torch's scaled_dot_product_attention (float64, CPU) on the gathered
    buffers, KV heads repeated for GQA, bottom-right causal mask built
    explicitly."""
    rng = np.random.default_rng(11)
    for causal in (False, True):
        n, L, Hq, Hkv, D, Dv = 5, 37, 8, 2, 16, 12
        q = rng.normal(size=(n, Hq, D))
        K = rng.normal(size=(L, Hkv, D))
        V = rng.normal(size=(L, Hkv, Dv))
        o, _ = oracle.attend(q, K, V, 0.3, causal)
        G = Hq // Hkv
        tq = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, n, D]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        mask = None
        if causal:
            mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3)
        np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, K, V = rng.normal(size=(1, 4, 8)), rng.normal(size=(1, 2, 8)), rng.normal(size=(1, 2, 5))
    o, l = oracle.attend(q, K, V, 0.7, True)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[0, h // 2], atol=1e-15)
        assert l[0, h] == pytest.approx(0.7 * q[0, h] @ K[0, h // 2], abs=1e-13)


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(2)
    L = 23
    V = rng.normal(size=(L, 1, 6))
    o, l = oracle.attend(rng.normal(size=(1, 3, 4)), np.zeros((L, 1, 4)), V, 1.0, False)
    np.testing.assert_allclose(o[0], np.repeat(V.mean(axis=0), 3, axis=0), atol=1e-14)
    np.testing.assert_allclose(l, math.log(L), atol=1e-14)


def test_planted_key_dominates():
    rng = np.random.default_rng(3)
    L, D = 50, 16
    K = rng.normal(size=(L, 1, D)) * 0.01
    V = rng.normal(size=(L, 1, 4))
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    for t in (0, 17, L - 1):
        K2 = K.copy()
        K2[t, 0, 0] = 60.0
        o, _ = oracle.attend(q, K2, V, 1.0, False)
        np.testing.assert_allclose(o[0, 0], V[t, 0], atol=1e-12)


def test_empty_kv_gives_zero_and_minus_inf():
    o, l = oracle.attend(np.ones((3, 4, 8)), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 1.0, True)
    assert (o == 0).all() and np.isneginf(l).all()
    o, l = oracle.merge_partials([np.zeros((2, 5))] * 3, [np.full(2, -np.inf)] * 3)
    assert (o == 0).all() and np.isneginf(l).all()


def test_causal_decode_sees_every_key():
    """One new query (decode) under the causal rule sees all L keys."""
    rng = np.random.default_rng(4)
    q, K, V = rng.normal(size=(1, 2, 8)), rng.normal(size=(30, 1, 8)), rng.normal(size=(30, 1, 8))
    a, la = oracle.attend(q, K, V, 0.5, True)
    b, lb = oracle.attend(q, K, V, 0.5, False)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_causal_first_new_query_sees_prefix_plus_itself():
    rng = np.random.default_rng(5)
    p, n = 6, 4
    q, K, V = rng.normal(size=(n, 1, 8)), rng.normal(size=(p + n, 1, 8)), rng.normal(size=(p + n, 1, 3))
    o, _ = oracle.attend(q, K, V, 0.5, True)
    for j in range(n):
        oj, _ = oracle.attend(q[j:j + 1], K[:p + j + 1], V[:p + j + 1], 0.5, False)
        np.testing.assert_allclose(o[j], oj[0], atol=1e-14)


# --------------------------------------------------------------------------
# split / merge identity
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_split_merge_identity(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(5, 200))
    q, K, V = rng.normal(size=(1, 4, 16)), rng.normal(size=(L, 2, 16)), rng.normal(size=(L, 2, 8))
    full, lfull = oracle.attend(q, K, V, 0.25, False)
    cuts = np.sort(rng.choice(np.arange(1, L), size=min(5, L - 1), replace=False))
    parts = np.split(rng.permutation(L), cuts)
    parts.append(np.zeros(0, np.int64))  # an empty split contributes nothing
    outs, lses = [], []
    for idx in parts:
        o, l = oracle.attend(q, K[idx], V[idx], 0.25, False)
        outs.append(o)
        lses.append(l)
    mo, ml = oracle.merge_partials(outs, lses)
    np.testing.assert_allclose(mo, full, atol=1e-13)
    np.testing.assert_allclose(ml, lfull, atol=1e-13)


# --------------------------------------------------------------------------
# invariants over paged layouts (bitwise in the oracle)
# --------------------------------------------------------------------------

def _decode_via_table(case, vals, req_to_token=None, pool_k=None, pool_v=None):
    g = case.geom
    t = case.req_to_token if req_to_token is None else req_to_token
    pk = to_numpy_bits(vals["pool_k"]) if pool_k is None else pool_k
    pv = to_numpy_bits(vals["pool_v"]) if pool_v is None else pool_v
    r = case.regions["self"]
    slots = [oracle.slots_from_token_table(t, case.req_pool_indices[i], r.kv_start[i], r.kv_lens[i])
             for i in range(case.bs)]
    kn, vn = to_numpy_bits(vals["k_new"]), to_numpy_bits(vals["v_new"])
    if case.n_new:
        pk = oracle.store(pk, kn, case.out_loc)
        pv = oracle.store(pv, vn, case.out_loc)
    q = to_numpy_bits(vals["q"]["self"])
    return oracle.paged_attention(q, case.q_lens, pk, pv, g.dtype, slots, case.sm_scale, True)


def test_physical_page_permutation_is_invisible():
    case = W.tiny_decode(seed=1)
    vals = W.make_values(case)
    o1, l1 = _decode_via_table(case, vals)
    g = case.geom
    ps = g.page_size
    pi = np.random.default_rng(9).permutation(g.num_pages + 1)  # includes the padding page
    pk, pv = to_numpy_bits(vals["pool_k"]), to_numpy_bits(vals["pool_v"])
    npk, npv = np.empty_like(pk), np.empty_like(pv)
    for p in range(g.num_pages + 1):
        npk[pi[p] * ps:(pi[p] + 1) * ps] = pk[p * ps:(p + 1) * ps]
        npv[pi[p] * ps:(pi[p] + 1) * ps] = pv[p * ps:(p + 1) * ps]
    t = case.req_to_token.astype(np.int64)
    nt = (pi[t // ps] * ps + t % ps).astype(np.int32)
    case.out_loc = (pi[case.out_loc // ps] * ps + case.out_loc % ps).astype(np.int32)
    o2, l2 = _decode_via_table(case, vals, nt, npk, npv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_is_invisible():
    """The same logical K/V laid out at page sizes 1, 2, 16 and 64 gives
    identical outputs, through the token table and through the CSR form."""
    rng = np.random.default_rng(12)
    bs, Hq, Hkv, D = 5, 4, 2, 8
    lens = rng.integers(1, 150, size=bs)
    Kl = [rng.normal(size=(n, Hkv, D)).astype(np.float32) for n in lens]
    Vl = [rng.normal(size=(n, Hkv, D)).astype(np.float32) for n in lens]
    q = rng.normal(size=(bs, Hq, D)).astype(np.float32)
    results = []
    for ps in (1, 2, 16, 64):
        npages = sum(-(-int(n) // ps) for n in lens) + 3
        perm = rng.permutation(npages)
        pk = np.full((npages * ps, Hkv, D), np.nan, np.float32)
        pv = np.full((npages * ps, Hkv, D), np.nan, np.float32)
        table = np.zeros((bs, 160), np.int32)
        pos = 0
        for i, n in enumerate(lens):
            k = -(-int(n) // ps)
            pg = perm[pos:pos + k]
            pos += k
            slots = np.array([pg[t // ps] * ps + t % ps for t in range(n)])
            pk[slots], pv[slots] = Kl[i], Vl[i]
            table[i, :n] = slots
        s_tab = [oracle.slots_from_token_table(table, i, 0, lens[i]) for i in range(bs)]
        indptr, indices = oracle.build_csr(table, np.arange(bs), None, lens, ps)
        s_csr = [oracle.slots_from_csr(indptr, indices, i, ps, lens[i]) for i in range(bs)]
        a = oracle.paged_attention(q, np.ones(bs), pk, pv, "f32", s_tab, 0.3, True)
        b = oracle.paged_attention(q, np.ones(bs), pk, pv, "f32", s_csr, 0.3, True)
        assert np.array_equal(a[0], b[0])
        results.append(a)
    for r in results[1:]:
        assert np.array_equal(r[0], results[0][0]) and np.array_equal(r[1], results[0][1])
    assert np.isfinite(results[0][0]).all()


def test_shared_prefix_pages_equal_private_copies():
    case = W.gqa_prefix_share(16, bs=16, group=8, prefix=64, median=80, sigma=0.5, clip=(8, 300), num_q_heads=16)
    g = case.geom
    ps = g.page_size
    rng = np.random.default_rng(0)
    pk = rng.normal(size=(g.num_slots, 8, 128)).astype(np.float32)
    pv = rng.normal(size=(g.num_slots, 8, 128)).astype(np.float32)
    q = rng.normal(size=(case.bs, g.num_q_heads, 128)).astype(np.float32)
    r = case.regions["self"]
    slots = [oracle.slots_from_token_table(case.req_to_token, case.req_pool_indices[i], 0, r.kv_lens[i])
             for i in range(case.bs)]
    a = oracle.paged_attention(q, case.q_lens, pk, pv, "f32", slots, 0.1, True)
    # copy every request's pages into private pages of a fresh pool
    tot = sum(len(p) for p in r.page_lists)
    pk2 = np.full((tot * ps, 8, 128), np.nan, np.float32)
    pv2 = np.full_like(pk2, np.nan)
    slots2, pos = [], 0
    for i in range(case.bs):
        n = int(r.kv_lens[i])
        new = np.arange(pos * ps, pos * ps + n)
        pos += len(r.page_lists[i])
        pk2[new], pv2[new] = pk[slots[i]], pv[slots[i]]
        slots2.append(new)
    b = oracle.paged_attention(q, case.q_lens, pk2, pv2, "f32", slots2, 0.1, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # sharing really happened in this case
    firsts = [int(p[0]) for p in r.page_lists[:8]]
    assert len(set(firsts)) == 1


@pytest.mark.parametrize("builder", [
    lambda: W.tiny_decode(seed=2),
    lambda: W.tiny_decode(seed=2, padded=True),
    lambda: W.qwen3_decode(seed=0, bs=4, len_range=(40, 90), pool_tokens=1000, max_context=128),
    lambda: W.mla_decode(seed=0, bs=3, len_range=(60, 200)),
])
def test_nan_canaries_are_never_read(builder):
    case = builder()
    clean = W.make_values(case)
    dirty = W.make_values(case, canary=True)
    g = case.geom
    if g.latent:
        r = case.regions["self"]
        outs = []
        for vals in (clean, dirty):
            pk = oracle.store(to_numpy_bits(vals["pool_k"]), to_numpy_bits(vals["k_new"]), case.out_loc)
            slots = [oracle.slots_from_token_table(case.req_to_token, case.req_pool_indices[i], 0, r.kv_lens[i])
                     for i in range(case.bs)]
            outs.append(oracle.paged_attention(to_numpy_bits(vals["q"]["self"]), case.q_lens, pk, None,
                                               g.dtype, slots, case.sm_scale, True, head_dim_v=g.head_dim_v))
        a, b = outs
    else:
        a = _decode_via_table(case, clean)
        b = _decode_via_table(case, dirty)
    real = ~case.dummy if case.dummy.size else np.ones(case.bs, bool)
    assert np.isfinite(b[0][real]).all()
    assert np.array_equal(a[0][real], b[0][real])
    if case.dummy.any():
        # dummy requests read only the padding slot their own store wrote
        # (one of the racing dummy writes survives): finite, otherwise don't-care
        assert np.isfinite(b[0][case.dummy]).all()


def test_paged_equals_ragged_bitwise():
    case = W.encdec_extend(seed=0, bs=4, enc_len=40, prefix_range=(0, 20), new_range=(1, 30))
    vals = W.make_values(case)
    g = case.geom
    pk, pv = to_numpy_bits(vals["pool_k"]), to_numpy_bits(vals["pool_v"])
    pk = oracle.store(pk, to_numpy_bits(vals["k_new"]), case.out_loc)
    pv = oracle.store(pv, to_numpy_bits(vals["v_new"]), case.out_loc)
    for name, reg in case.regions.items():
        q = to_numpy_bits(vals["q"][name])
        indptr, indices = oracle.build_csr(case.req_to_token, case.req_pool_indices, reg.kv_start, reg.kv_lens,
                                           g.page_size)
        slots = [oracle.slots_from_csr(indptr, indices, i, g.page_size, reg.kv_lens[i]) for i in range(case.bs)]
        paged = oracle.paged_attention(q, case.q_lens, pk, pv, g.dtype, slots, case.sm_scale, reg.causal)
        gk, gv = oracle.gather(pk, slots), oracle.gather(pv, slots)
        cu = oracle.token_indptr(reg.kv_lens)
        rslots = [np.arange(cu[i], cu[i + 1]) for i in range(case.bs)]
        ragged = oracle.paged_attention(q, case.q_lens, gk, gv, g.dtype, rslots, case.sm_scale, reg.causal)
        assert np.array_equal(paged[0], ragged[0]) and np.array_equal(paged[1], ragged[1])
        assert np.isfinite(paged[0]).all()


def test_empty_encoder_warmup_gives_zeros():
    case = W.encdec_extend(seed=0, bs=3, enc_len=0, prefix_range=(0, 5), new_range=(1, 4))
    vals = W.make_values(case)
    reg = case.regions["cross"]
    slots = [np.zeros(0, np.int64)] * case.bs
    o, l = oracle.paged_attention(to_numpy_bits(vals["q"]["cross"]), case.q_lens, to_numpy_bits(vals["pool_k"]),
                                  to_numpy_bits(vals["pool_v"]), "bf16", slots, case.sm_scale, reg.causal)
    assert (o == 0).all() and np.isneginf(l).all()


def test_workload_tables_are_in_page_contiguous_and_match_page_lists():
    """The generator's tables recover its page lists through the pages'
    stride-and-divide, for every workload shape (small variants)."""
    cases = [W.tiny_decode(), W.qwen3_decode(bs=6, len_range=(5, 50), pool_tokens=400, max_context=64),
             W.gqa_prefix_share(16, bs=16, prefix=64, median=80, sigma=0.5, clip=(8, 300)),
             W.gqa_prefix_share(64, bs=16, prefix=128, median=200, sigma=0.5, clip=(8, 600)),
             W.mla_decode(bs=4, len_range=(60, 300)), W.encdec_extend(bs=5)]
    for c in cases:
        for reg in c.regions.values():
            ok = oracle.in_page_contiguous(c.req_to_token, c.req_pool_indices, reg.kv_start, reg.kv_lens,
                                           c.geom.page_size)
            assert all(ok)
            for i in range(c.bs):
                ids = oracle.page_ids_from_token_table(c.req_to_token, c.req_pool_indices[i], reg.kv_start[i],
                                                       reg.kv_lens[i], c.geom.page_size)
                assert np.array_equal(ids, reg.page_lists[i])
                assert not (ids == c.geom.padding_page).any()


# --------------------------------------------------------------------------
# softcap (the encoder-decoder post's ragged call passes it; reading: every
# scaled score s becomes cap * tanh(s / cap))
# --------------------------------------------------------------------------

def test_softcap_closed_form_two_keys():
    """Raw scores cap * atanh(+-1/2) are capped to +-cap/2, so the first key's
    weight is 1 / (1 + e^-cap) and lse = log(2 cosh(cap / 2))."""
    for cap in (0.5, 4.0, 30.0):
        x = cap * math.atanh(0.5)
        q = np.array([[[1.0]]])
        K = np.array([[[x]], [[-x]]])
        V = np.array([[[1.0]], [[0.0]]])
        o, l = oracle.attend(q, K, V, 1.0, False, softcap=cap)
        assert abs(o[0, 0, 0] - 1.0 / (1.0 + math.exp(-cap))) < 1e-14
        assert abs(l[0, 0] - math.log(2.0 * math.cosh(cap / 2.0))) < 1e-12


def test_softcap_vanishes_for_a_huge_cap_and_bounds_the_weights():
    rng = np.random.default_rng(21)
    q = rng.normal(size=(3, 4, 8))
    K = rng.normal(size=(11, 2, 8))
    V = rng.normal(size=(11, 2, 5))
    o0, l0 = oracle.attend(q, K, V, 0.7, True)
    o1, l1 = oracle.attend(q, K, V, 0.7, True, softcap=1e9)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)
    # scores of +-1e4 capped at 2: every weight within e^(2 * 2) of every other
    cap = 2.0
    Kb = np.array([[[1e4]], [[-1e4]], [[0.0]]])
    Vb = np.eye(3)[:, None, :]
    ob, _ = oracle.attend(np.array([[[1.0]]]), Kb, Vb, 1.0, False, softcap=cap)
    w = ob[0, 0]
    assert np.isfinite(w).all() and abs(w.sum() - 1) < 1e-12
    assert w.max() / w.min() <= math.exp(2 * cap) * (1 + 1e-12)


def test_softcap_matches_brute_force():
    rng = np.random.default_rng(22)
    q = rng.normal(size=(2, 2, 3)) * 3
    K = rng.normal(size=(5, 1, 3)) * 3
    V = rng.normal(size=(5, 1, 2))
    cap = 1.5
    o, l = oracle.attend(q, K, V, 0.9, True, softcap=cap)
    for j in range(2):
        for h in range(2):
            keys = [t for t in range(5) if t <= 5 - 2 + j]
            s = [cap * math.tanh(0.9 * math.fsum(q[j, h, d] * K[t, 0, d] for d in range(3)) / cap) for t in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            for d in range(2):
                assert abs(o[j, h, d] - math.fsum(e[a] * V[t, 0, d] for a, t in enumerate(keys)) / tot) < 1e-12
            assert abs(l[j, h] - (m + math.log(tot))) < 1e-12


# --------------------------------------------------------------------------
# mixed causal/full spans (vLLM-Omni notes, "Attention execution")
# --------------------------------------------------------------------------

def test_span_segments_equal_one_dense_masked_row():
    """A row of causal and full spans, run as native segments, equals dense
    attention over the whole row with the mask the spans describe: a
    position in a causal span sees keys up to itself, a position in a full
    span [a, b) sees keys up to b."""
    rng = np.random.default_rng(23)
    spans = [(0, 5, True), (5, 12, False), (12, 15, True), (15, 19, False)]
    T, Hq, Hkv, D = 19, 4, 2, 6
    q = rng.normal(size=(T, Hq, D))
    K = rng.normal(size=(T, Hkv, D))
    V = rng.normal(size=(T, Hkv, D))
    seg_o = np.zeros((T, Hq, D))
    seg_l = np.zeros((T, Hq))
    segs = oracle.span_segments(spans)
    assert [(a, b, kv) for a, b, kv, _ in segs] == [(0, 5, 5), (5, 12, 12), (12, 15, 15), (15, 19, 19)]
    for a, b, kv, causal in segs:
        o, l = oracle.attend(q[a:b], K[:kv], V[:kv], 0.4, causal)
        seg_o[a:b], seg_l[a:b] = o, l
    # dense row: torch SDPA in float64 with the span mask, KV heads repeated
    mask = np.zeros((T, T), bool)
    for a, b, causal in spans:
        for p in range(a, b):
            mask[p, :(p + 1 if causal else b)] = True
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.4)
    np.testing.assert_allclose(seg_o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # lse of the dense row, by hand
    s = np.einsum("phd,thd->pht", q, np.repeat(K, G, axis=1)) * 0.4
    s = np.where(mask[:, None, :], s, -np.inf)
    m = s.max(axis=2)
    np.testing.assert_allclose(seg_l, m + np.log(np.exp(s - m[..., None]).sum(axis=2)), rtol=0, atol=1e-12)


def test_paged_attention_takes_per_request_causal_flags():
    rng = np.random.default_rng(24)
    pool = rng.normal(size=(40, 2, 4)).astype(np.float32)
    q = rng.normal(size=(7, 2, 4)).astype(np.float32)
    slots = [np.arange(0, 9), np.arange(10, 25)]
    o, l = oracle.paged_attention(q, [3, 4], pool, pool, "f32", slots, 0.5, [True, False])
    o0, _ = oracle.paged_attention(q, [3, 4], pool, pool, "f32", slots, 0.5, True, requests=[0])
    o1, _ = oracle.paged_attention(q, [3, 4], pool, pool, "f32", slots, 0.5, False, requests=[1])
    assert np.array_equal(o[:3], o0[:3]) and np.array_equal(o[3:], o1[3:])
