"""GPU parity of the encoder-embedding block cache (scatter write, gather +
merge by position map, fill counts and the fail-loud check) against the
oracle, bit for bit, through the C ABI.  The scratch block is left out of
the comparisons: several padding blocks land there in no set order."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_38_amd as P
from workloads.cases import to_numpy_bits
from workloads.enc_cache import enc_cache_case

pytestmark = pytest.mark.gpu

DEV = "cuda"


def values(case, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(case.value_seed)
    shape = (case.block_size, case.fat_dim)
    buf = torch.randn((case.num_blocks, *shape), generator=g, device=DEV).to(dtype)
    src = torch.randn((len(case.write_ids), *shape), generator=g, device=DEV).to(dtype)
    hidden = torch.randn((case.num_tokens, case.fat_dim), generator=g, device=DEV).to(dtype)
    return buf, src, hidden


def t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def bits(x):
    return to_numpy_bits(x)


def scheduled_rows(case, gather_ids=None) -> np.ndarray:
    """Rows some gathered token of a real block is scheduled to fill (the
    check's input, built here; the oracle's counts are the expected side)."""
    ids = case.gather_ids if gather_ids is None else gather_ids
    mask = np.zeros(case.num_tokens, bool)
    for j, b in enumerate(ids):
        if 0 <= int(b) < case.num_blocks:
            p = np.asarray(case.positions[j], np.int64)
            mask[p[(p >= 0) & (p < case.num_tokens)]] = True
    return mask


def run_step(case, buf, src, hidden, gather_ids=None, fill=True):
    P.enc_cache_write(buf, src, t(case.write_ids, torch.int32))
    ids = case.gather_ids if gather_ids is None else gather_ids
    fc = torch.zeros(case.num_tokens, dtype=torch.int32, device=DEV) if fill else None
    P.enc_cache_merge(buf, t(ids, torch.int32), t(case.positions, torch.int64), hidden, fc)
    torch.cuda.synchronize()
    return fc


@pytest.mark.parametrize("fat,dtype", [(64, torch.bfloat16), (520, torch.bfloat16), (96, torch.float32)])
def test_write_and_merge_bit_exact(fat, dtype):
    case = enc_cache_case(seed=fat, num_blocks=9, block_size=16, fat_dim=fat, n_write=5, n_pad=2, n_cached=2,
                          num_tokens=90, token_range=(1, 16))
    print(f"enc cache fat {fat} {dtype}", flush=True)
    buf, src, hidden = values(case, dtype)
    b0, s0, h0 = bits(buf), bits(src), bits(hidden)
    fc = run_step(case, buf, src, hidden)
    want_buf = oracle.write_blocks(b0, s0, case.write_ids)
    # every block but the scratch block, whose contents are whichever padding
    # block landed last (never read)
    assert np.array_equal(bits(buf)[:-1], want_buf[:-1])
    want_h = oracle.merge_blocks(want_buf, case.gather_ids, case.positions, h0, case.num_tokens)
    assert np.array_equal(bits(hidden), want_h)
    want_c = oracle.fill_counts(case.gather_ids, case.positions, case.num_blocks, case.num_tokens)
    assert np.array_equal(fc.cpu().numpy(), want_c)
    sched = t(want_c > 0, torch.int32)
    st, counts = P.enc_cache_check(fc, sched)
    assert st == P._lib.PKV_OK and counts == [0, 0]


def test_fail_loud_check_reports_missing_and_doubled_rows():
    case = enc_cache_case(seed=1, num_blocks=9, block_size=16, fat_dim=64, n_write=4, n_pad=1, n_cached=2,
                          num_tokens=80, token_range=(4, 16))
    buf, src, hidden = values(case)
    sched_np = scheduled_rows(case)
    ids = case.gather_ids.copy()
    ids[1] = case.num_blocks + 3  # a block the cache does not hold: its rows stay unfilled
    case.positions[2, 1] = case.positions[3, 0]  # two tokens onto one row
    fc = run_step(case, buf, src, hidden, gather_ids=ids)
    want = oracle.check_filled(oracle.fill_counts(ids, case.positions, case.num_blocks, case.num_tokens), sched_np)
    st, counts = P.enc_cache_check(fc, t(sched_np, torch.int32))
    assert st == P._lib.PKV_EINVAL and tuple(counts) == want and want[0] > 0 and want[1] == 1


def test_qwen3_vl_geometry_full_size():
    """The notes' geometry: 33 blocks of 512 tokens x 20480 bf16 (40 KiB rows,
    692 MB), 8 written blocks, 8 gathered onto an 8192-row batch."""
    case = enc_cache_case(seed=0)
    buf, src, hidden = values(case)
    b0, s0, h0 = bits(buf), bits(src), bits(hidden)
    fc = run_step(case, buf, src, hidden)
    want_buf = oracle.write_blocks(b0, s0, case.write_ids)
    assert np.array_equal(bits(buf)[:-1], want_buf[:-1])  # the scratch block aside
    want_h = oracle.merge_blocks(want_buf, case.gather_ids, case.positions, h0, case.num_tokens)
    assert np.array_equal(bits(hidden), want_h)
    sched = scheduled_rows(case)
    assert np.array_equal(sched, oracle.fill_counts(case.gather_ids, case.positions, case.num_blocks,
                                                    case.num_tokens) > 0)
    st, counts = P.enc_cache_check(fc, t(sched, torch.int32))
    assert st == P._lib.PKV_OK and counts == [0, 0]
