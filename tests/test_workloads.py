"""The seeded workload builders keep their promises (CPU only): NaN canaries
sit only in slots no request reads, shared prefixes really share pages, and
page lists, tables and lengths agree."""
import numpy as np
import pytest

import workloads as W


def _read_slots(case):
    r = case.regions["self"]
    return [case.req_to_token[case.req_pool_indices[i], r.kv_start[i]:r.kv_start[i] + r.kv_lens[i]]
            for i in range(case.bs)]


def _canary_slots(case):
    ps = case.geom.page_size
    bad = np.concatenate([[case.geom.padding_page], case.free_pages]).astype(np.int64)
    return set((bad[:, None] * ps + np.arange(ps)[None, :]).reshape(-1).tolist()) | set(case.tail_slots.tolist())


def _groups(ps):
    pp = 256 // ps
    return [(pp, [(100, pp), (300, pp), (256, pp), (40, pp // 2)]), (0, [(77, 0)]), (2, [(0, 0)]),
            (3, [(3 * ps + 1, 3), (6 * ps, 3), (2 * ps, 1)])]


@pytest.mark.parametrize("ps", [1, 16, 64])
def test_shared_prefix_batch_canaries_and_sharing(ps):
    case = W.shared_prefix_batch(ps, _groups(ps), seed=ps)
    r = case.regions["self"]
    bad = _canary_slots(case)
    for i, sl in enumerate(_read_slots(case)):
        assert len(sl) == r.kv_lens[i]
        assert not (set(sl.tolist()) & bad), f"request {i} reads a canary slot"
        pages = np.asarray(r.page_lists[i], np.int64)
        if len(sl):
            assert np.array_equal(sl // ps, np.repeat(pages, ps)[:len(sl)])
    # members of the first group share its first pages
    sl = _read_slots(case)
    assert np.array_equal(sl[0][:100], sl[1][:100]) and np.array_equal(sl[1][:256], sl[2][:256])
    assert np.array_equal(sl[3][:min(40, 128)], sl[1][:min(40, 128)])


@pytest.mark.parametrize("ps", [16, 64])
def test_prefix_share_canaries(ps):
    case = W.gqa_prefix_share(ps, seed=1, bs=16, prefix=256, median=300, sigma=0.8, clip=(40, 1500))
    bad = _canary_slots(case)
    for i, sl in enumerate(_read_slots(case)):
        assert not (set(sl.tolist()) & bad), f"request {i} reads a canary slot"
