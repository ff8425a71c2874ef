"""Host-only checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments with the documented
status codes before touching the device.  No kernel is launched."""
import ctypes as C
import os
import re
import subprocess

import pytest

from paged_kv_cache_38_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|int32_t|int64_t|char\s*\*|char)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libpagedkv.so is not built (run python -m paged_kv_cache_38_amd.build)")
    return L.load()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("kv_pool_create", "kv_store", "build_kv_indices", "paged_decode_attn", "paged_extend_attn",
                 "kv_gather", "kv_validate", "kv_pool_bytes", "paged_decode_workspace_bytes"):
        assert name in fns
    assert set(fns) == set(L.SIGNATURES), (set(fns) ^ set(L.SIGNATURES))


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_arch_and_status_strings(lib):
    assert lib.pkv_abi_version() == 1
    assert lib.pkv_build_arch() == b"gfx950"
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.pkv_status_string(st)
    assert lib.pkv_status_string(-99) == b"unknown status"


def desc(**kw):
    d = dict(num_layers=2, num_pages=64, page_size=16, num_kv_heads=2, head_dim_qk=64, head_dim_v=64, dtype=0, kind=0)
    d.update(kw)
    return L.PoolDesc(*[d[f] for f, _ in L.PoolDesc._fields_])


def pool_bytes(lib, d):
    kb, vb = C.c_size_t(), C.c_size_t()
    st = lib.kv_pool_bytes(C.byref(d), C.byref(kb), C.byref(vb))
    return st, kb.value, vb.value


def test_pool_bytes(lib):
    st, kb, vb = pool_bytes(lib, desc())
    assert st == 0 and kb == vb == 2 * 65 * 16 * 2 * 64 * 4
    # Qwen3-0.6B layout of the mini-sglang chapter: 28 layers, 65 pages of 16 tokens, 8 heads x 128, bf16
    st, kb, vb = pool_bytes(lib, desc(num_layers=28, num_pages=64, page_size=16, num_kv_heads=8, head_dim_qk=128,
                                      head_dim_v=128, dtype=1))
    assert st == 0 and kb == 28 * 65 * 16 * 8 * 128 * 2
    st, kb, vb = pool_bytes(lib, desc(num_kv_heads=1, head_dim_qk=576, head_dim_v=512, dtype=1, kind=1,
                                      page_size=64))
    assert st == 0 and vb == 0 and kb == 2 * 65 * 64 * 576 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=3), L.PKV_EUNSUPPORTED),
    (dict(page_size=256), L.PKV_EUNSUPPORTED),
    (dict(page_size=0), L.PKV_EUNSUPPORTED),
    (dict(num_layers=0), L.PKV_EINVAL),
    (dict(num_kv_heads=-1), L.PKV_EINVAL),
    (dict(dtype=7), L.PKV_EUNSUPPORTED),
    (dict(kind=5), L.PKV_EUNSUPPORTED),
    (dict(head_dim_v=32), L.PKV_EINVAL),
    (dict(kind=1, head_dim_v=128), L.PKV_EINVAL),
    (dict(head_dim_qk=3, head_dim_v=3), L.PKV_EUNSUPPORTED),
])
def test_bad_descriptors(lib, kw, status):
    assert pool_bytes(lib, desc(**kw))[0] == status
    assert lib.pkv_last_error()


def make_pool(lib, d, k=0x10000, v=0x20000):
    h = C.c_void_p()
    st = lib.kv_pool_create(C.byref(d), k, v, C.byref(h))
    return st, h


def test_pool_create_checks(lib):
    assert make_pool(lib, desc(), k=None)[0] == L.PKV_EINVAL
    assert make_pool(lib, desc(), v=None)[0] == L.PKV_EINVAL
    assert make_pool(lib, desc(), k=0x10008)[0] == L.PKV_EALIGN
    assert make_pool(lib, desc(kind=1, head_dim_v=32, num_kv_heads=1))[0] == L.PKV_EINVAL  # latent takes no v
    st, h = make_pool(lib, desc())
    assert st == 0 and h.value
    assert lib.kv_pool_padding_page(h) == 64
    assert lib.kv_pool_token_bytes(h) == 2 * 2 * 64 * 4
    assert lib.kv_pool_destroy(h) == 0
    assert lib.kv_pool_padding_page(None) == L.PKV_EINVAL


def test_call_argument_checks_before_launch(lib):
    st, h = make_pool(lib, desc())
    assert st == 0
    try:
        assert lib.kv_store(h, 5, 0x1000, 0x2000, 0x3000, 4, None) == L.PKV_EINVAL  # bad layer
        assert lib.kv_store(h, 0, 0x1000, 0x2000, 0x3000, -1, None) == L.PKV_EINVAL
        assert lib.kv_store(h, 0, 0x1004, 0x2000, 0x3000, 4, None) == L.PKV_EALIGN
        assert lib.kv_store(h, 0, None, 0x2000, 0x3000, 4, None) == L.PKV_EINVAL
        assert lib.kv_store(h, 0, 0x1000, 0x2000, 0x3000, 0, None) == 0  # nothing to do
        # build_kv_indices: capacity checked against bs * ceil(max_kv_len / ps)
        args = [L.PKV_MAP_CSR, 0x1000, 5, 128, 0x2000, None, 0x3000, 4, 16, 100, 0x4000, 0x5000, 27, None, None]
        assert lib.build_kv_indices(*args) == L.PKV_ECAPACITY
        args[12] = 28
        args[1] = None
        assert lib.build_kv_indices(*args) == L.PKV_EINVAL
        args[1] = 0x1000
        args[8] = 12
        assert lib.build_kv_indices(*args) == L.PKV_EUNSUPPORTED
        args[8], args[0] = 16, 7
        assert lib.build_kv_indices(*args) == L.PKV_EINVAL
        args[0], args[12] = L.PKV_MAP_BLOCK_TABLE, 6
        assert lib.build_kv_indices(*args) == L.PKV_ECAPACITY
        # decode: map checks, head grouping, workspace size
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_TOKEN_TABLE, 4, 0x1000, 100
        m.req_to_token, m.table_rows, m.table_width, m.req_pool_indices = 0x2000, 5, 128, 0x3000
        ws = C.c_size_t()
        assert lib.paged_decode_workspace_bytes(h, 4, 4, 100, C.byref(ws)) == 0
        assert lib.paged_decode_attn(h, 0, 0x4000, 3, C.byref(m), 0.125, 0x5000, None, None, 0, None) == L.PKV_EINVAL
        if ws.value:
            assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), 0.125, 0x5000, None, 0x6000, ws.value - 1,
                                         None) == L.PKV_ECAPACITY
        m.fmt = 9
        assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), 0.125, 0x5000, None, None, 0, None) == L.PKV_EINVAL
        m.fmt = L.PKV_MAP_CONTIGUOUS
        assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), 0.125, 0x5000, None, None, 0, None) \
            == L.PKV_EUNSUPPORTED
        m.fmt, m.block_table, m.block_stride = L.PKV_MAP_BLOCK_TABLE, 0x7000, 6
        assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), 0.125, 0x5000, None, None, 0, None) \
            == L.PKV_ECAPACITY
        m.fmt = L.PKV_MAP_TOKEN_TABLE
        for bad in (0.0, -0.125, float("inf"), float("nan")):  # the kernels take the row max on raw scores
            assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), bad, 0x5000, None, None, 0, None) \
                == L.PKV_EINVAL
        m.bs = 0
        assert lib.paged_decode_attn(h, 0, 0x4000, 4, C.byref(m), 0.125, 0x5000, None, None, 0, None) == 0
        assert lib.pkv_set_kernel_timer(0x1, None) == L.PKV_EINVAL
        assert lib.pkv_set_kernel_timer(None, None) == 0
    finally:
        lib.kv_pool_destroy(h)


def test_unsupported_decode_shapes_are_rejected(lib):
    st, h = make_pool(lib, desc(head_dim_qk=96, head_dim_v=96))
    assert st == 0
    ws = C.c_size_t()
    try:
        assert lib.paged_decode_workspace_bytes(h, 4, 4, 100, C.byref(ws)) == L.PKV_EUNSUPPORTED
    finally:
        lib.kv_pool_destroy(h)


def test_allocator_argument_checks_before_launch(lib):
    ring, state, status, out = 0x1000, 0x2000, 0x3000, 0x4000
    assert lib.kv_free_list_init(None, 8, 0, 8, state, None) == L.PKV_EINVAL
    assert lib.kv_free_list_init(ring, 8, 0, 9, state, None) == L.PKV_ECAPACITY
    assert lib.kv_free_list_init(ring, 0, 0, 0, state, None) == L.PKV_EINVAL
    assert lib.kv_free_list_init(ring, 8, -1, 8, state, None) == L.PKV_EINVAL
    assert lib.kv_free_list_init(ring, 8, 2**31 - 4, 8, state, None) == L.PKV_EINVAL
    # page-aligned alloc: need a multiple of page_size, page_size a power of two
    assert lib.kv_alloc(16, 17, ring, 8, state, out, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc(16, -16, ring, 8, state, out, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc(12, 24, ring, 8, state, out, status, None) == L.PKV_EUNSUPPORTED
    assert lib.kv_alloc(256, 256, ring, 8, state, out, status, None) == L.PKV_EUNSUPPORTED
    assert lib.kv_alloc(16, 32, ring, 8, state, out, None, None) == L.PKV_EINVAL
    assert lib.kv_alloc(16, 32, ring, 8, state, None, status, None) == L.PKV_EINVAL
    # growth paths
    lens = 0x5000
    assert lib.kv_alloc_extend(16, 4, None, lens, lens, ring, 8, state, out, 64, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_extend(16, 4, lens, lens, None, ring, 8, state, out, 64, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_extend(16, 4, lens, lens, lens, ring, 8, state, out, -1, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_extend(16, 4, lens, lens, lens, ring, 8, state, out, 2**31, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_extend(16, 8001, lens, lens, lens, ring, 8, state, out, 64, status, None) \
        == L.PKV_EUNSUPPORTED
    assert lib.kv_alloc_extend(16, 4, lens, lens, lens, ring, 0, state, out, 64, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_decode(16, 4, lens, None, ring, 8, state, out, status, None) == L.PKV_EINVAL
    assert lib.kv_alloc_decode(16, -1, lens, lens, ring, 8, state, out, status, None) == L.PKV_EINVAL
    # free
    assert lib.kv_free(16, 0x6000, 4, 64, ring, 8, state, None, status, None) == L.PKV_EINVAL
    assert lib.kv_free(16, None, 4, 64, ring, 8, state, 0x7000, status, None) == L.PKV_EINVAL
    assert lib.kv_free(16, 0x6000, 4, 0, ring, 8, state, 0x7000, status, None) == L.PKV_EINVAL
    # row writing
    t = 0x8000
    assert lib.write_req_to_token(t, 4, 64, lens, lens, lens, out, 10, None, 2, 65, None) == L.PKV_EINVAL
    assert lib.write_req_to_token(t, 4, 64, None, lens, lens, out, 10, None, 2, 64, None) == L.PKV_EINVAL
    assert lib.write_req_to_token(t, 0, 64, lens, lens, lens, out, 10, None, 2, 64, None) == L.PKV_EINVAL
    assert lib.write_req_to_token(t, 4, 64, lens, lens, lens, None, 10, None, 2, 64, None) == L.PKV_EINVAL
    assert lib.write_req_to_token(t, 4, 2**27, lens, lens, lens, out, 10, None, 2, 2**26 + 1, None) \
        == L.PKV_EUNSUPPORTED


def test_extend_options_checked_before_launch(lib):
    st, h = make_pool(lib, desc(dtype=1))
    assert st == 0
    try:
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_TOKEN_TABLE, 4, 0x1000, 100
        m.req_to_token, m.table_rows, m.table_width, m.req_pool_indices = 0x2000, 5, 128, 0x3000
        args = [h, 0, 0x4000, 40, 0x5000, 4, 10, C.byref(m)]
        assert lib.paged_extend_attn_ex(*args, None, 0.125, 0x6000, None, None) == L.PKV_EINVAL
        for bad in (-1.0, float("inf"), float("nan")):
            opts = L.ExtendOpts(1, None, bad)
            assert lib.paged_extend_attn_ex(*args, C.byref(opts), 0.125, 0x6000, None, None) == L.PKV_EINVAL
        opts = L.ExtendOpts(1, None, 0.0)
        assert lib.paged_extend_attn_ex(*args, C.byref(opts), -1.0, 0x6000, None, None) == L.PKV_EINVAL
        m.bs = 0  # nothing to do, options accepted
        opts = L.ExtendOpts(0, 0x7000, 30.0)
        assert lib.paged_extend_attn_ex(*args, C.byref(opts), 0.125, 0x6000, None, None) == 0
    finally:
        lib.kv_pool_destroy(h)


def test_decode_append_arguments_checked_before_launch(lib):
    st, h = make_pool(lib, desc(dtype=1))
    assert st == 0
    try:
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_TOKEN_TABLE, 4, 0x1000, 100
        m.req_to_token, m.table_rows, m.table_width, m.req_pool_indices = 0x2000, 5, 128, 0x3000
        hq = 2 * desc(dtype=1).num_kv_heads

        def call(k=0x10000, v=0x20000, loc=0x30000, n=4, scale=0.1, ws=0):
            return lib.paged_decode_attn_append(h, 0, 0x4000, hq, C.byref(m), k, v, loc, n, scale, 0x5000, None,
                                                0x60000 if ws else None, ws, None)

        assert call(n=-1) == L.PKV_EINVAL                 # append arguments first
        assert call(k=None) == L.PKV_EINVAL
        assert call(loc=None) == L.PKV_EINVAL
        assert call(v=None) == L.PKV_EINVAL               # a split pool needs v
        assert call(k=0x10008) == L.PKV_EALIGN
        assert call(scale=0.0) == L.PKV_EINVAL            # then the decode's
        assert call() == L.PKV_ECAPACITY                  # no workspace: nothing launched
        assert lib.paged_decode_attn_append(h, 0, 0x4000, 3, C.byref(m), 0x10000, 0x20000, 0x30000, 4, 0.1,
                                            0x5000, None, None, 0, None) == L.PKV_EINVAL  # 3 heads over 2
        assert lib.paged_decode_attn_append(h, 7, 0x4000, hq, C.byref(m), 0x10000, 0x20000, 0x30000, 4, 0.1,
                                            0x5000, None, None, 0, None) == L.PKV_EINVAL  # no layer 7
        m.bs = 0
        assert call(n=0) == 0                             # nothing to store, nothing to attend
    finally:
        lib.kv_pool_destroy(h)


def test_verify_arguments_checked_before_launch(lib):
    st, h = make_pool(lib, desc(dtype=1, kind=1, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64),
                      v=None)  # a latent pool takes no V buffer
    assert st == 0
    st2, hs = make_pool(lib, desc(dtype=1))
    assert st2 == 0
    try:
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_TOKEN_TABLE, 4, 0x1000, 100
        m.req_to_token, m.table_rows, m.table_width, m.req_pool_indices = 0x2000, 5, 128, 0x3000
        call = lambda pool, hq, n, scale=0.04: lib.paged_verify_attn(pool, 0, 0x4000, hq, n, C.byref(m), scale,
                                                                       0x5000, None, None, 0, None)
        assert call(h, 16, 0) == L.PKV_EINVAL
        assert call(h, 16, 2, scale=0.0) == L.PKV_EINVAL
        assert call(h, 16, 9) == L.PKV_EUNSUPPORTED      # 144 rows
        assert call(h, 24, 2) == L.PKV_EUNSUPPORTED      # 48 rows
        assert call(h, 128, 16) == L.PKV_EUNSUPPORTED    # 2048 rows
        assert call(h, 128, 4) == L.PKV_ECAPACITY        # 512 rows (four slices) pass the shape check
        assert call(h, 16, 8) == L.PKV_ECAPACITY         # 128 rows
        assert call(hs, 16, 2) == L.PKV_EUNSUPPORTED     # not a latent pool
        assert call(h, 16, 2) == L.PKV_ECAPACITY         # no workspace

        def app(pool, k=0x10000, loc=0x30000, n=8, scale=0.04):
            return lib.paged_verify_attn_append(pool, 0, 0x4000, 16, 2, C.byref(m), k, loc, n, scale, 0x5000, None,
                                                None, 0, None)
        assert app(h, n=-1) == L.PKV_EINVAL               # the append's arguments first
        assert app(h, k=None) == L.PKV_EINVAL
        assert app(h, loc=None) == L.PKV_EINVAL
        assert app(h, k=0x10004) == L.PKV_EALIGN
        assert app(h, scale=0.0) == L.PKV_EINVAL
        assert app(hs) == L.PKV_EUNSUPPORTED              # not a latent pool
        assert app(h) == L.PKV_ECAPACITY                  # no workspace: nothing launched
        m.bs = 0
        assert call(h, 16, 2) == 0
        assert app(h, n=0) == 0
    finally:
        lib.kv_pool_destroy(h)
        lib.kv_pool_destroy(hs)


def test_encoder_cache_arguments_checked_before_launch(lib):
    buf, src, ids, pos, hid = 0x10000, 0x20000, 0x3000, 0x4000, 0x50000
    assert lib.enc_cache_write(buf, 9, 16, 130, src, 4, ids, None) == L.PKV_EALIGN   # row not a multiple of 16
    assert lib.enc_cache_write(buf, 0, 16, 128, src, 4, ids, None) == L.PKV_EINVAL
    assert lib.enc_cache_write(buf, 9, 16, 128, src, -1, ids, None) == L.PKV_EINVAL
    assert lib.enc_cache_write(buf, 9, 16, 128, None, 4, ids, None) == L.PKV_EINVAL
    assert lib.enc_cache_write(buf + 8, 9, 16, 128, src, 4, ids, None) == L.PKV_EALIGN
    assert lib.enc_cache_write(buf, 9, 16, 128, src, 0, ids, None) == 0
    assert lib.enc_cache_merge(buf, 9, 16, 128, ids, 4, None, hid, 90, None, None) == L.PKV_EINVAL
    assert lib.enc_cache_merge(buf, 9, 16, 128, ids, -1, pos, hid, 90, None, None) == L.PKV_EINVAL
    assert lib.enc_cache_merge(buf, 9, 16, 128, ids, 4, pos, hid + 4, 90, None, None) == L.PKV_EALIGN
    assert lib.enc_cache_merge(buf, 9, 16, 128, ids, 0, pos, hid, 90, None, None) == 0
    counts = (C.c_int64 * 2)()
    assert lib.enc_cache_check(None, None, 10, 0x6000, counts, None) == L.PKV_EINVAL
    assert lib.enc_cache_check(0x7000, None, 0, 0x6000, counts, None) == 0
    assert lib.enc_cache_check(0x7000, None, 10, 0x6000, None, None) == L.PKV_EINVAL


def test_cascade_arguments_checked_before_launch(lib):
    st, h = make_pool(lib, desc(dtype=1, head_dim_qk=128, head_dim_v=128, num_kv_heads=2))
    assert st == 0
    st2, hf = make_pool(lib, desc(dtype=0))  # f32 pool: no cascade kernel
    assert st2 == 0
    try:
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_CSR, 4, 0x1000, 100
        m.kv_indptr, m.kv_indices, m.kv_indices_len = 0x2000, 0x3000, 64
        g = L.PrefixGroups(2, 2, 64, 0x4000, 0x5000)
        ws = C.c_size_t()
        assert lib.paged_decode_cascade_workspace_bytes(h, 4, 8, 100, C.byref(g), C.byref(ws)) == 0 and ws.value > 0
        assert lib.paged_decode_cascade_workspace_bytes(hf, 4, 4, 100, C.byref(g), C.byref(ws)) == L.PKV_EUNSUPPORTED
        assert lib.paged_decode_cascade_workspace_bytes(h, 4, 8, 100, None, C.byref(ws)) == L.PKV_EINVAL
        bad = L.PrefixGroups(2, 2, 64, None, 0x5000)
        assert lib.paged_decode_cascade_workspace_bytes(h, 4, 8, 100, C.byref(bad), C.byref(ws)) == L.PKV_EINVAL
        neg = L.PrefixGroups(-1, 2, 64, 0x4000, 0x5000)
        assert lib.paged_decode_cascade_workspace_bytes(h, 4, 8, 100, C.byref(neg), C.byref(ws)) == L.PKV_EINVAL
        # bounds whose prefix work list would need more than 2^31 items are refused, not truncated
        huge, ws2 = L.PrefixGroups(1 << 30, 1 << 20, 64, 0x4000, 0x5000), C.c_size_t()
        assert lib.paged_decode_cascade_workspace_bytes(h, 4, 8, 100, C.byref(huge), C.byref(ws2)) == \
            L.PKV_EUNSUPPORTED
        assert lib.paged_decode_attn_cascade(h, 0, 0x6000, 8, C.byref(m), C.byref(huge), 0.1, 0x7000, None, 0x8000,
                                             1 << 40, None) == L.PKV_EUNSUPPORTED
        call = lambda ws_ptr, n, scale=0.1: lib.paged_decode_attn_cascade(h, 0, 0x6000, 8, C.byref(m), C.byref(g),
                                                                         scale, 0x7000, None, ws_ptr, n, None)
        assert call(0x8000, ws.value - 1) == L.PKV_ECAPACITY
        assert call(0x8004, ws.value) == L.PKV_EALIGN
        assert call(0x8000, ws.value, scale=float("nan")) == L.PKV_EINVAL
        assert lib.paged_decode_attn_cascade(h, 0, 0x6000, 34, C.byref(m), C.byref(g), 0.1, 0x7000, None, 0x8000,
                                             ws.value, None) == L.PKV_EUNSUPPORTED  # 17 query heads per KV head
        m.bs = 0
        assert call(None, 0) == 0
    finally:
        lib.kv_pool_destroy(h)
        lib.kv_pool_destroy(hf)


def test_slot_ids_must_fit_int32(lib):
    """Every slot id of the pool, the padding page's included, is an int32
    (tables, out_loc and the kernels' slot maps)."""
    big = dict(num_layers=1, num_kv_heads=1, head_dim_qk=8, head_dim_v=8, dtype=1, page_size=128)
    ok_pages = (2**31 - 1) // 128 - 1  # (ok_pages + 1) * 128 <= INT32_MAX
    assert pool_bytes(lib, desc(num_pages=ok_pages, **big))[0] == 0
    assert pool_bytes(lib, desc(num_pages=ok_pages + 1, **big))[0] == L.PKV_EUNSUPPORTED
    assert b"int32" in lib.pkv_last_error()


def _fake_pool(latent=False):
    """A Pool record on host tensors: enough for the binding's shape checks,
    which run before any pointer is taken."""
    import torch
    import paged_kv_cache_38_amd as P
    if latent:
        return P.Pool(0, torch.zeros(8, dtype=torch.bfloat16), None, 1, 4, 64, 1, 576, 512, True)
    return P.Pool(0, torch.zeros(8, dtype=torch.bfloat16), torch.zeros(8, dtype=torch.bfloat16), 1, 4, 16, 2, 64, 64,
                  False)


def _fake_map(bs):
    import paged_kv_cache_38_amd as P
    s = L.KVMapStruct()
    s.bs = bs
    return P.KVMap(s, ())


def test_binding_rejects_short_or_misshapen_tensors():
    """The C ABI takes bare pointers and cannot see a tensor's size: the
    binding checks that sources hold the rows the kernels read and that q /
    out / lse match the batch and the pool's head dims, before any launch."""
    import torch
    import paged_kv_cache_38_amd as P
    bf = torch.bfloat16
    pool, m = _fake_pool(), _fake_map(3)
    loc = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="k must be"):
        P.kv_store(pool, 0, torch.zeros(3, 2, 64, dtype=bf), torch.zeros(4, 2, 64, dtype=bf), loc)
    with pytest.raises(ValueError, match="v must be"):
        P.kv_store(pool, 0, torch.zeros(4, 2, 64, dtype=bf), torch.zeros(4, 2, 32, dtype=bf), loc)
    with pytest.raises(ValueError, match="v is required"):
        P.kv_store(pool, 0, torch.zeros(4, 2, 64, dtype=bf), None, loc)
    q = torch.zeros(3, 4, 64, dtype=bf)
    out = torch.zeros(3, 4, 64, dtype=bf)
    with pytest.raises(ValueError, match="q must be"):
        P.paged_decode_attn(pool, 0, torch.zeros(2, 4, 64, dtype=bf), m, 0.1, out)
    with pytest.raises(ValueError, match="q must be"):
        P.paged_decode_attn(pool, 0, torch.zeros(3, 4, 32, dtype=bf), m, 0.1, out)
    with pytest.raises(ValueError, match="out must be"):
        P.paged_decode_attn(pool, 0, q, m, 0.1, torch.zeros(3, 4, 32, dtype=bf))
    with pytest.raises(ValueError, match="out must be"):
        P.paged_decode_attn(pool, 0, q, m, 0.1, torch.zeros(2, 4, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse"):
        P.paged_decode_attn(pool, 0, q, m, 0.1, out, torch.zeros(5, dtype=torch.float32))
    with pytest.raises(ValueError, match="k_new must be"):
        P.paged_decode_attn_append(pool, 0, q, m, torch.zeros(2, 2, 64, dtype=bf), torch.zeros(3, 2, 64, dtype=bf),
                                   torch.zeros(3, dtype=torch.int32), 0.1, out)
    # extend: rows of q and out, qo_indptr length
    qe = torch.zeros(10, 4, 64, dtype=bf)
    with pytest.raises(ValueError, match="out must be"):
        P.paged_extend_attn(pool, 0, qe, torch.zeros(4, dtype=torch.int32), 5, m, True, 0.1,
                            torch.zeros(9, 4, 64, dtype=bf))
    with pytest.raises(ValueError, match="qo_indptr"):
        P.paged_extend_attn(pool, 0, qe, torch.zeros(3, dtype=torch.int32), 5, m, True, 0.1,
                            torch.zeros(10, 4, 64, dtype=bf))
    # latent pool: verification shapes and the drafts' rows
    lp = _fake_pool(latent=True)
    qv = torch.zeros(3, 2, 16, 576, dtype=bf)
    with pytest.raises(ValueError, match="out must be"):
        P.paged_verify_attn(lp, 0, qv, m, 0.1, torch.zeros(3, 2, 16, 576, dtype=bf))
    with pytest.raises(ValueError, match="q must be"):
        P.paged_verify_attn(lp, 0, torch.zeros(4, 2, 16, 576, dtype=bf), m, 0.1, torch.zeros(4, 2, 16, 512, dtype=bf))
    with pytest.raises(ValueError, match="k_new must be"):
        P.paged_verify_attn_append(lp, 0, qv, m, torch.zeros(6, 1, 512, dtype=bf), torch.zeros(6, dtype=torch.int32),
                                   0.1, torch.zeros(3, 2, 16, 512, dtype=bf))


def test_noalloc_decode_rejects_past_its_array_before_any_device_call(lib):
    """paged_decode_attn_noalloc refuses a batch whose workspace would not fit
    the library's device array (128 MiB) with PKV_ECAPACITY, before it
    touches the device (so this runs without one)."""
    st, h = make_pool(lib, desc(num_layers=1, num_pages=1000, page_size=64, num_kv_heads=1, head_dim_qk=576,
                                head_dim_v=512, dtype=1, kind=1), v=None)
    assert st == 0
    try:
        m = L.KVMapStruct()
        m.fmt, m.bs, m.kv_lens, m.max_kv_len = L.PKV_MAP_BLOCK_TABLE, 4096, 0x1000, 65536
        m.block_table, m.block_stride = 0x2000, 1024
        need = C.c_size_t()
        assert lib.paged_decode_workspace_bytes(h, 4096, 128, 65536, C.byref(need)) == 0
        assert need.value > (128 << 20)
        assert lib.paged_decode_attn_noalloc(h, 0, 0x3000, 128, C.byref(m), 0.05, 0x4000, None, None) == \
            L.PKV_ECAPACITY
        assert b"workspace" in lib.pkv_last_error()
    finally:
        lib.kv_pool_destroy(h)
