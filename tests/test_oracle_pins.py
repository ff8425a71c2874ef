"""Pins of the oracle's index math, layout and store against values the pages
print (tests/golden/*.json, each citing its page and section) and closed
forms.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# KV pool layout and capacity (mini-sglang KV pool chapter, "What it prints")
# --------------------------------------------------------------------------

def test_kv_bytes_and_capacity_printed_values():
    g = golden("mini_kv_pool_example.json")
    q = g["qwen3_0_6b"]
    per = oracle.kv_bytes_per_token(q["num_layers"], q["num_kv_heads"], q["head_dim"], q["elem_bytes"])
    assert per == g["qwen3_kv_bytes_per_token"]
    assert oracle.tokens_that_fit(4 * 2**30, per) == g["tokens_in_4_gib"]
    assert oracle.tokens_that_fit(40 * 2**30, per) == g["tokens_in_40_gib"]
    l8 = g["llama_3_1_8b"]
    assert oracle.kv_bytes_per_token(l8["num_layers"], l8["num_kv_heads"], l8["head_dim"], l8["elem_bytes"]) \
        == g["llama_kv_bytes_per_token"]


def test_pool_shape_and_flattening_printed_values():
    g = golden("mini_kv_pool_example.json")
    q = g["qwen3_0_6b"]
    shape = oracle.pool_shape(q["num_layers"], g["pool"]["num_pages"], g["pool"]["page_size"],
                              q["num_kv_heads"], q["head_dim"])
    assert list(shape) == g["pool_shape"]
    assert list(shape[2:]) == g["layer_k_shape"]
    assert list(oracle.per_token_shape(*shape[2:])) == g["flattened_per_token"]


def test_token_table_rows_give_printed_pages():
    """Rows of the per-token page table at page_size 16 turn into the pages
    the page names (request 0 on pages 2 and 5, request 1 on page 10)."""
    g = golden("mini_kv_pool_example.json")
    ps = g["pool"]["page_size"]
    table = np.zeros((3, 64), np.int32)
    r0, r1 = g["request0_first20_locations"], g["request1_first5_locations"]
    table[0, :len(r0)] = r0
    table[1, :len(r1)] = r1
    assert oracle.page_ids_from_token_table(table, 0, 0, len(r0), ps).tolist() == g["request0_pages"]
    assert oracle.page_ids_from_token_table(table, 1, 0, len(r1), ps).tolist() == g["request1_pages"]
    # and the pages' slot formula gives the rows back
    assert oracle.slots_from_pages(g["request0_pages"], ps, len(r0)).tolist() == r0
    assert oracle.slots_from_pages(g["request1_pages"], ps, len(r1)).tolist() == r1
    assert oracle.in_page_contiguous(table, [0, 1], [0, 0], [len(r0), len(r1)], ps) == [True, True]


def test_exercise_page_count_and_out_loc_formula():
    g = golden("mini_kv_pool_example.json")
    assert int(oracle.ceil_div(17, 16)) == g["exercise_pages_for_17_tokens_at_ps16"]
    # exercise 2: out_loc = page_ids[pos // ps] * ps + pos % ps for pos in [cached, device)
    pages = np.array([7, 3, 11])
    pos = np.arange(5, 40)
    expect = pages[pos // 16] * 16 + pos % 16
    assert np.array_equal(oracle.slots_from_pages(pages, 16, 40)[5:40], expect)


def test_slot_page_offset_round_trip():
    for ps in (1, 2, 16, 64, 128):
        s = np.arange(0, 5000, dtype=np.int64)
        assert np.array_equal(oracle.page_of(s, ps) * ps + oracle.offset_of(s, ps), s)
        assert (oracle.offset_of(s, ps) < ps).all()


# --------------------------------------------------------------------------
# Store (mini-sglang "Tests": test_kv_pool_layout_and_store)
# --------------------------------------------------------------------------

def test_store_reproduces_page_unit_test():
    g = golden("mini_store_test.json")
    shape = oracle.pool_shape(g["num_layers"], g["num_pages"], g["page_size"], g["num_kv_heads"], g["head_dim"])
    assert list(shape) == g["expected_pool_shape"]
    pool = np.zeros(shape, np.float32)
    k = np.arange(24, dtype=np.float32).reshape(3, 8)
    layer = g["layer"]
    flat_shape = oracle.per_token_shape(g["num_pages"], g["page_size"], g["num_kv_heads"], g["head_dim"])
    pool[0, layer] = oracle.store(pool[0, layer].reshape(flat_shape), k, g["out_loc"]).reshape(pool.shape[2:])
    pool[1, layer] = oracle.store(pool[1, layer].reshape(flat_shape), -k, g["out_loc"]).reshape(pool.shape[2:])
    flat_k = pool[0, layer].reshape(g["flat_rows"], g["num_kv_heads"], g["head_dim"])
    assert np.array_equal(flat_k[9].reshape(-1), k[0])
    assert np.array_equal(flat_k[4].reshape(-1), k[2])
    assert np.array_equal(pool[1, layer][4, 1].reshape(-1), -k[0])
    # nothing else was touched
    touched = np.zeros(g["flat_rows"], bool)
    touched[g["out_loc"]] = True
    assert (flat_k[~touched] == 0).all()
    assert (pool[:, [0, 2]] == 0).all()


def test_store_is_bit_exact_for_bf16_nan_and_signed_zero():
    pool = np.zeros((8, 2, 4), np.uint16)
    rows = np.array([[[0x7FC1, 0x8000, 0x0001, 0xFF80]] * 2, [[0x3F80, 0xC000, 0x7F80, 0x0000]] * 2], np.uint16)
    out = oracle.store(pool, rows, [6, 1])
    assert np.array_equal(out[6], rows[0]) and np.array_equal(out[1], rows[1])
    assert (out[[0, 2, 3, 4, 5, 7]] == 0).all()
    assert (pool == 0).all()  # input untouched


# --------------------------------------------------------------------------
# Index building (SGLang AttentionBackend notes)
# --------------------------------------------------------------------------

def test_csr_example_from_pages():
    g = golden("backend_index_examples.json")["csr_example"]
    ps = 64
    pages = g["pages_per_request"]
    lens = [len(p) * ps - d for p, d in zip(pages, (0, 10, 63))]  # full, and two partial last pages
    table = np.full((4, 1024), 0, np.int32)
    for r, (p, n) in enumerate(zip(pages, lens)):
        table[r, :n] = oracle.slots_from_pages(p, ps, n)
    indptr, indices = oracle.build_csr(table, np.arange(3), None, np.array(lens), ps)
    assert indptr.tolist() == g["kv_indptr"]
    assert indices.tolist() == g["kv_indices"]
    bt = oracle.build_block_table(table, np.arange(3), None, np.array(lens), ps, 5)
    assert bt.tolist() == [[5, 6, 8, -1, -1], [2, 3, -1, -1, -1], [10, 11, 15, 18, -1]]
    assert oracle.last_page_len(lens, ps).tolist() == [64, 54, 1]


def test_extend_example_indptrs():
    g = golden("backend_index_examples.json")["extend_example"]
    seq, pre = np.array(g["seq_lens"]), np.array(g["prefix_lens"])
    assert oracle.token_indptr(seq).tolist() == g["kv_indptr"]
    assert oracle.qo_indptr(seq, pre).tolist() == g["qo_indptr"]
    # at page_size 1 the CSR page pointer is the token pointer, and there are
    # as many kv_indices as tokens
    rng = np.random.default_rng(0)
    table = rng.permutation(1000)[:3 * 16].reshape(3, 16).astype(np.int32)
    indptr, indices = oracle.build_csr(table, np.array(g["req_pool_indices"]), None, seq, g["page_size"])
    assert indptr.tolist() == g["kv_indptr"]
    assert len(indices) == g["kv_indices_count"] == g["paged_kernel_lens_sum"]
    assert np.array_equal(indices, np.concatenate([table[r, :n] for r, n in zip(range(3), seq)]))


def test_alignment_arithmetic():
    g = golden("xpu_alignment.json")
    assert g["whisper_encoder_len"] % g["page_size"] == g["encoder_len_mod_page"]
    assert int(oracle.ceil_align(g["whisper_encoder_len"], g["page_size"])) == g["ceil_align_encoder"]
    xs = np.arange(0, 3000)
    assert np.array_equal(oracle.ceil_align(xs, 1), xs)  # a no-op at page_size 1
    assert int(oracle.ceil_align(1500, 16)) == 1504


def test_csr_and_block_table_brute_force_random():
    """Random tables with in-page contiguity, random kv_start on page
    boundaries; every format resolves every token to the same slot."""
    rng = np.random.default_rng(7)
    for ps in (1, 2, 4, 16, 64):
        bs, npages = 9, 300
        perm = rng.permutation(npages)
        lens = rng.integers(0, 5 * ps + 3, size=bs)
        starts = rng.integers(0, 3, size=bs) * ps
        rows = rng.permutation(bs + 2)[:bs]
        table = np.full((bs + 2, 8 * ps + 8), -7, np.int32)
        pos = 0
        truth = []
        for i in range(bs):
            k = -(-int(lens[i]) // ps)
            pg = perm[pos:pos + k]
            pos += k
            slots = [int(pg[t // ps]) * ps + t % ps for t in range(int(lens[i]))]  # brute force
            truth.append(slots)
            table[rows[i], starts[i]:starts[i] + lens[i]] = slots
        indptr, indices = oracle.build_csr(table, rows, starts, lens, ps)
        maxb = max(1, int(oracle.ceil_div(lens.max(), ps)))
        bt = oracle.build_block_table(table, rows, starts, lens, ps, maxb)
        lpl = oracle.last_page_len(lens, ps)
        for i in range(bs):
            assert oracle.slots_from_token_table(table, rows[i], starts[i], lens[i]).tolist() == truth[i]
            assert oracle.slots_from_csr(indptr, indices, i, ps, lens[i]).tolist() == truth[i]
            assert oracle.slots_from_block_table(bt, i, ps, lens[i]).tolist() == truth[i]
            npg = int(indptr[i + 1] - indptr[i])
            assert npg == -(-int(lens[i]) // ps)
            assert (bt[i, npg:] == -1).all()
            if lens[i]:
                assert 1 <= lpl[i] <= ps and (npg - 1) * ps + lpl[i] == lens[i]
            else:
                assert lpl[i] == 0
        assert all(oracle.in_page_contiguous(table, rows, starts, lens, ps))


def test_in_page_contiguity_detects_violation():
    table = np.array([[32, 33, 34, 36, 80]], np.int32)  # slot 35 skipped inside page 2
    assert oracle.in_page_contiguous(table, [0], [0], [5], 16) == [False]
    table = np.array([[33, 34]], np.int32)  # page entered at offset 1
    assert oracle.in_page_contiguous(table, [0], [0], [2], 16) == [False]


def test_block_table_rejects_negative_entry_inside_length():
    with pytest.raises(AssertionError):
        oracle.slots_from_pages([3, -1], 16, 20)


# ---------------------------------------------------------------------------
# element-format conversions (oracle/numerics.py)
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch_and_closed_forms():
    from oracle.numerics import bf16_bits_to_f64, to_f64
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3F81], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 1 + 2 ** -7]
    got = bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert np.signbit(got[3]) and not np.signbit(got[2])
    assert np.isnan(bf16_bits_to_f64(np.array([0x7FC0], np.uint16)))[0]
    # every finite pattern against torch's own bf16 -> fp64 widening
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    mine = bf16_bits_to_f64(allbits)
    fin = np.isfinite(t)
    assert np.array_equal(mine[fin], t[fin]) and np.array_equal(np.isnan(mine), np.isnan(t))
    assert np.array_equal(to_f64(allbits, "bf16")[fin], t[fin])
    f32 = np.array([1.5, -3.25e-30, 7e37], np.float32)
    assert to_f64(f32, "f32").tolist() == [float(x) for x in f32]
    with pytest.raises(ValueError):
        to_f64(f32, "fp8")


def test_bf16_rounding_is_nearest_even():
    from oracle.numerics import f64_to_bf16_bits
    # ties go to the even mantissa: 1 + 2^-8 -> 1.0, 1 + 3 * 2^-8 -> 1 + 2^-6
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.0, np.nan], np.float64)
    assert f64_to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x7FC0]
    # random binary32 values (ties included) against torch's float32 -> bf16
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    f[:2000] = (f[:2000].view(np.uint32) & np.uint32(0xFFFF8000) | np.uint32(0x8000)).view(np.float32)  # ties
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(f.astype(np.float64)), want)
