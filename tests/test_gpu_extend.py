"""GPU parity of paged extend / prefill attention (causal over a paged
prefix, non-causal cross-attention over an encoder region, and the ragged
gather + contiguous variant) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import paged_kv_cache_38_amd as P
import workloads as W

from gpu_util import DeviceCase, assert_attn_close, assert_lse_close, oracle_region, run_extend

pytestmark = pytest.mark.gpu

FMTS = [P.PKV_MAP_TOKEN_TABLE, P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE]


def encdec(seed, **kw):
    args = dict(bs=5, enc_len=300, prefix_range=(0, 90), new_range=(1, 150))
    args.update(kw)
    return W.encdec_extend(seed=seed, **args)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("region", ["self", "cross"])
def test_extend_matches_oracle(region, seed, fmt):
    case = encdec(seed)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, region, fmt)
    ref_o, ref_l = oracle_region(case, vals, region)
    assert_attn_close(out, ref_o, "bf16", f"{region} fmt {fmt}")
    assert_lse_close(lse, ref_l, "bf16", f"{region} fmt {fmt}")


@pytest.mark.parametrize("region", ["self", "cross"])
def test_ragged_variant_equals_paged_bitwise(region):
    """Gather + contiguous extend gives the same bits as the paged read (the
    same keys in the same order through the same kernel)."""
    case = encdec(3)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    paged = run_extend(dc, region, P.PKV_MAP_CSR)
    ragged = run_extend(dc, region, P.PKV_MAP_TOKEN_TABLE, contiguous=True)
    assert torch.equal(paged[0].view(torch.int16), ragged[0].view(torch.int16))
    assert torch.equal(paged[1], ragged[1])
    ref_o, _ = oracle_region(case, vals, region)
    assert_attn_close(ragged[0], ref_o, "bf16", "ragged")


def test_empty_encoder_warmup_gives_zeros():
    case = encdec(0, enc_len=0, prefix_range=(0, 20), new_range=(1, 40))
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    for fmt in FMTS:
        out, lse = run_extend(dc, "cross", fmt)
        assert (out.float() == 0).all() and torch.isneginf(lse).all()
    out, lse = run_extend(dc, "cross", P.PKV_MAP_TOKEN_TABLE, contiguous=True)
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    # self-attention still works in the same batch
    out, lse = run_extend(dc, "self", P.PKV_MAP_CSR)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", "self after empty encoder")


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 4])
def test_extend_head_dims_and_gqa(head_dim, group):
    case = encdec(5, num_heads=4, head_dim=head_dim, bs=3, enc_len=200, new_range=(1, 130))
    case.geom.num_q_heads = case.geom.num_kv_heads * group
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    for region in ("self", "cross"):
        out, lse = run_extend(dc, region, P.PKV_MAP_CSR)
        ref_o, ref_l = oracle_region(case, vals, region)
        assert_attn_close(out, ref_o, "bf16", f"{region} D={head_dim} G={group}")
        assert_lse_close(lse, ref_l, "bf16", f"{region} D={head_dim} G={group}")


def test_extend_single_new_token_equals_decode():
    """An extend with one new token per request is a decode: both kernels
    agree with the oracle on the same pool."""
    case = encdec(6, new_range=(1, 1), enc_len=150)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    out_e, _ = run_extend(dc, "self", P.PKV_MAP_CSR)
    out_d, _ = dc.decode(P.PKV_MAP_CSR, "self")
    ref_o, _ = oracle_region(case, vals, "self")
    assert_attn_close(out_e, ref_o, "bf16", "extend n=1")
    assert_attn_close(out_d, ref_o, "bf16", "decode")


def test_extend_repeatable_bitwise():
    case = encdec(7)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    a = run_extend(dc, "cross", P.PKV_MAP_BLOCK_TABLE)
    b = run_extend(dc, "cross", P.PKV_MAP_BLOCK_TABLE)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


# --------------------------------------------------------------------------
# mixed causal/full spans and softcap (extend options)
# --------------------------------------------------------------------------

SPANS = ((5, True), (40, False), (17, True), (70, False), (1, True))


@pytest.mark.parametrize("fmt", FMTS)
def test_mixed_span_segments_match_oracle(fmt):
    """Rows of causal and full spans (several not aligned to a tile or a page)
    run as one call whose requests are the segments, each with its flag."""
    case = W.mixed_spans(seed=1, rows=3, spans=SPANS, num_q_heads=8, num_kv_heads=2, head_dim=128)
    print(f"mixed spans fmt {fmt}: {case.bs} segments", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, "self", fmt)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"mixed spans fmt {fmt}")
    assert_lse_close(lse, ref_l, "bf16", f"mixed spans fmt {fmt}")


def test_mixed_spans_flags_equal_separate_calls_bitwise():
    """Per-request flags give the same bits as running the causal and the
    full segments in two calls with one flag each."""
    case = W.mixed_spans(seed=2, rows=2, spans=SPANS, num_q_heads=4, num_kv_heads=4, head_dim=64)
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, "self", P.PKV_MAP_CSR)
    reg = case.regions["self"]
    flags = reg.causal_flags.copy()
    for value in (0, 1):
        reg.causal_flags = None
        reg.causal = bool(value)
        o1, l1 = run_extend(dc, "self", P.PKV_MAP_CSR)
        qo = np.concatenate([[0], np.cumsum(case.q_lens)])
        for i in np.nonzero(flags == value)[0]:
            a, b = int(qo[i]), int(qo[i + 1])
            assert torch.equal(out[a:b].view(torch.int16), o1[a:b].view(torch.int16))
            assert torch.equal(lse[a:b], l1[a:b])
    reg.causal_flags = flags


@pytest.mark.parametrize("softcap", [0.5, 5.0, 30.0])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_softcap_matches_oracle(softcap, head_dim):
    case = encdec(7, num_heads=4, head_dim=head_dim, bs=4, enc_len=260, new_range=(1, 140))
    vals = W.make_values(case, canary=True)
    # larger scores so the cap bites
    vals["q"] = {k: (v.float() * 4).to(v.dtype) for k, v in vals["q"].items()}
    dc = DeviceCase(case, vals)
    dc.store()
    for region in ("self", "cross"):
        out, lse = run_extend(dc, region, P.PKV_MAP_CSR, softcap=softcap)
        ref_o, ref_l = oracle_region(case, vals, region, softcap=softcap)
        assert_attn_close(out, ref_o, "bf16", f"softcap {softcap} {region}")
        assert_lse_close(lse, ref_l, "bf16", f"softcap {softcap} {region}")
        # the ragged variant takes the same options
        out2, _ = run_extend(dc, region, P.PKV_MAP_TOKEN_TABLE, contiguous=True, softcap=softcap)
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("fmt", [P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE])
def test_softcap_long_blocks_match_oracle(head_dim, fmt):
    """Softcapped segments long enough on average (600 query rows per
    request) for the phase-alternating kernel: causal 700-row and full
    500-row segments over a shared row of keys, GQA 4, several query tiles
    per segment and the causal diagonal inside them; every row against the
    oracle, and the ragged variant bit for bit."""
    case = W.mixed_spans(seed=14, rows=2, spans=((700, True), (500, False)), num_q_heads=8, num_kv_heads=2,
                         head_dim=head_dim)
    print(f"softcap long blocks d{head_dim} fmt {fmt}: q rows {int(case.q_lens.sum())}", flush=True)
    vals = W.make_values(case, canary=True)
    vals["q"] = {k: (v.float() * 4).to(v.dtype) for k, v in vals["q"].items()}  # so the cap bites
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, "self", fmt, softcap=20.0)
    ref_o, ref_l = oracle_region(case, vals, "self", softcap=20.0)
    assert_attn_close(out, ref_o, "bf16", f"softcap long blocks d{head_dim}")
    assert_lse_close(lse, ref_l, "bf16", f"softcap long blocks d{head_dim}")
    out2, _ = run_extend(dc, "self", P.PKV_MAP_TOKEN_TABLE, contiguous=True, softcap=20.0)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("head_dim", [64, 128])
def test_long_causal_prefill_matches_oracle(head_dim):
    """One 3000-token causal prefill (16 query tiles of the diagonal, every
    mask boundary) followed by a 1000-token full span over all 4000 keys."""
    case = W.mixed_spans(seed=11, rows=1, spans=((3000, True), (1000, False)), num_q_heads=8, num_kv_heads=2,
                         head_dim=head_dim)
    print(f"long causal prefill, head_dim {head_dim}", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, "self", P.PKV_MAP_CSR)
    ref_o, ref_l = oracle_region(case, vals, "self")
    assert_attn_close(out, ref_o, "bf16", f"long prefill d{head_dim}")
    assert_lse_close(lse, ref_l, "bf16", f"long prefill d{head_dim}")


# ---------------------------------------------------------------------------
# fp32 pools: the vector-ALU extend, against the oracle at the fp32 bound
# ---------------------------------------------------------------------------

def _f32(case):
    case.geom.dtype = "f32"
    return case


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("region", ["self", "cross"])
def test_extend_f32_matches_oracle(region, fmt):
    case = _f32(encdec(7))
    print(f"f32 extend {region} fmt {fmt}", flush=True)
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    out, lse = run_extend(dc, region, fmt)
    ref_o, ref_l = oracle_region(case, vals, region)
    assert_attn_close(out, ref_o, "f32", f"f32 {region} fmt {fmt}")
    assert_lse_close(lse, ref_l, "f32", f"f32 {region} fmt {fmt}")


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 4])
def test_extend_f32_head_dims_gqa_softcap_and_ragged(head_dim, group):
    case = _f32(encdec(8, num_heads=4, head_dim=head_dim, bs=3, enc_len=200, new_range=(1, 130)))
    case.geom.num_q_heads = case.geom.num_kv_heads * group
    vals = W.make_values(case, canary=True)
    dc = DeviceCase(case, vals)
    dc.store()
    for region in ("self", "cross"):
        out, lse = run_extend(dc, region, P.PKV_MAP_CSR)
        ref_o, ref_l = oracle_region(case, vals, region)
        assert_attn_close(out, ref_o, "f32", f"f32 D{head_dim} G{group} {region}")
        assert_lse_close(lse, ref_l, "f32", f"f32 D{head_dim} G{group} {region}")
        ragged = run_extend(dc, region, P.PKV_MAP_TOKEN_TABLE, contiguous=True)
        assert torch.equal(out.view(torch.int32), ragged[0].view(torch.int32))
        assert torch.equal(lse, ragged[1])
        capped, _ = run_extend(dc, region, P.PKV_MAP_CSR, softcap=5.0)
        ref_c, _ = oracle_region(case, vals, region, softcap=5.0)
        assert_attn_close(capped, ref_c, "f32", f"f32 D{head_dim} G{group} {region} softcap 5")


def test_extend_f32_empty_encoder_gives_zeros():
    case = _f32(encdec(0, enc_len=0, prefix_range=(0, 20), new_range=(1, 40)))
    vals = W.make_values(case)
    dc = DeviceCase(case, vals)
    dc.store()
    for fmt in FMTS:
        out, lse = run_extend(dc, "cross", fmt)
        assert (out == 0).all() and torch.isneginf(lse).all()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("region", ["self", "cross"])
@pytest.mark.parametrize("fmt", [P.PKV_MAP_CSR, P.PKV_MAP_BLOCK_TABLE])
def test_key_split_short_blocks_match_oracle(head_dim, region, fmt):
    """Query blocks whose rows fit one wave (48 rows at D = 64, 32 at
    D = 128) run key-split: every wave takes all of the block's rows and a
    16-key slice of each tile, and the partial states are merged at the end.
    Requests of 1 .. 48 (32) new tokens make every block such a block; 193 ..
    240 (129 .. 160) new tokens give a full block followed by a short one.
    Causal self region and full cross region; ragged equals paged bit for
    bit."""
    wr = 48 if head_dim == 64 else 32
    bm = 4 * wr
    for k, new_range in enumerate([(1, wr), (bm + 1, bm + wr)]):
        case = W.encdec_extend(seed=21 + k, bs=6, enc_len=700, prefix_range=(0, 300), new_range=new_range,
                               num_heads=4, head_dim=head_dim)
        vals = W.make_values(case, canary=True)
        dc = DeviceCase(case, vals)
        dc.store()
        out, lse = run_extend(dc, region, fmt)
        ref_o, ref_l = oracle_region(case, vals, region)
        tag = f"D {head_dim} {region} fmt {fmt} n {new_range}"
        assert_attn_close(out, ref_o, "bf16", tag)
        assert_lse_close(lse, ref_l, "bf16", tag)
        ragged = run_extend(dc, region, P.PKV_MAP_TOKEN_TABLE, contiguous=True)
        assert torch.equal(out.view(torch.int16), ragged[0].view(torch.int16)), tag
        assert torch.equal(lse, ragged[1]), tag
