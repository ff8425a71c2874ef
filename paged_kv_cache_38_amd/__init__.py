"""Paged KV-cache hot path for AMD MI355X (gfx950).

A thin binding over the C ABI of ``libpagedkv.so`` (``include/pagedkv.h``):
the functions below carry the same names as the C entry points and only
marshal arguments (torch tensors -> device pointers, the caller's current
HIP stream).  Every step of the hot path runs in the library's HIP kernels;
torch provides device memory and streams.  If the library is missing, the
first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib as L
from ._lib import (  # noqa: F401
    PKV_DTYPE_BF16,
    PKV_DTYPE_F32,
    PKV_KIND_LATENT,
    PKV_KIND_SPLIT_KV,
    PKV_MAP_BLOCK_TABLE,
    PKV_MAP_CONTIGUOUS,
    PKV_MAP_CSR,
    PKV_MAP_TOKEN_TABLE,
    PKV_ALLOC_BAD_LENGTHS,
    PKV_ALLOC_NO_SPACE,
    PKV_ALLOC_OK,
    PKV_ALLOC_OUT_CAPACITY,
    PKV_ALLOC_RING_FULL,
    PagedKVError,
)

__all__ = [
    "Pool", "KVMap", "kv_pool_bytes", "kv_pool_create", "kv_pool_destroy", "kv_pool_padding_page",
    "kv_pool_token_bytes", "kv_store", "build_kv_indices", "make_kv_map", "paged_decode_workspace_bytes",
    "paged_decode_attn", "paged_decode_attn_noalloc", "PrefixGroups", "make_prefix_groups", "paged_decode_cascade_workspace_bytes",
    "paged_decode_attn_cascade", "paged_decode_attn_append", "paged_verify_attn", "paged_verify_attn_append", "paged_extend_attn", "paged_extend_attn_ex", "kv_gather",
    "kv_validate",
    "pkv_set_kernel_timer", "library",
    "enc_cache_write", "enc_cache_merge", "enc_cache_check",
    "FreeList", "kv_free_list_create", "kv_free_list_init", "kv_alloc", "kv_alloc_extend", "kv_alloc_decode",
    "kv_free", "write_req_to_token",
]

_DTYPES = {torch.float32: PKV_DTYPE_F32, torch.bfloat16: PKV_DTYPE_BF16}


def library() -> C.CDLL:
    return L.load()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _check_rows(pool: "Pool", t: Optional[torch.Tensor], name: str, n: int, which: str) -> None:
    """``t`` must hold at least ``n`` token rows of the pool's K (or V) row
    size: the kernels read ``n`` rows from it and cannot check."""
    if n <= 0:
        return
    if t is None:
        raise ValueError(f"{name} is required")
    per = pool.num_kv_heads * (pool.head_dim_qk if which == "k" else pool.head_dim_v)
    if t.dim() < 1 or t.shape[0] < n or t.numel() != t.shape[0] * per:
        raise ValueError(f"{name} must be [>= {n}, {pool.num_kv_heads}, "
                         f"{pool.head_dim_qk if which == 'k' else pool.head_dim_v}] rows, got {tuple(t.shape)}")


def _check_attn(pool: "Pool", q: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor], lead: tuple,
                what: str) -> None:
    """q ``[*lead, Hq, head_dim_qk]``, out ``[*lead, Hq, head_dim_v]``, lse
    ``[*lead, Hq]``: the kernels index them by these sizes and cannot check."""
    k = len(lead)
    if q.dim() != k + 2 or tuple(q.shape[:k]) != tuple(lead) or q.shape[-1] != pool.head_dim_qk:
        raise ValueError(f"{what}: q must be [{', '.join(map(str, lead))}, Hq, {pool.head_dim_qk}], "
                         f"got {tuple(q.shape)}")
    want = (*lead, q.shape[k], pool.head_dim_v)
    if tuple(out.shape) != want:
        raise ValueError(f"{what}: out must be {want}, got {tuple(out.shape)}")
    if lse is not None and lse.numel() != q.numel() // q.shape[-1]:
        raise ValueError(f"{what}: lse must have one entry per query row and head")


# ---------------------------------------------------------------------------
# pool
# ---------------------------------------------------------------------------

def _desc(num_layers, num_pages, page_size, num_kv_heads, head_dim_qk, head_dim_v, dtype, latent) -> L.PoolDesc:
    return L.PoolDesc(num_layers, num_pages, page_size, num_kv_heads, head_dim_qk,
                      head_dim_qk if head_dim_v is None else head_dim_v,
                      _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
                      PKV_KIND_LATENT if latent else PKV_KIND_SPLIT_KV)


def kv_pool_bytes(num_layers: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim_qk: int,
                  head_dim_v: Optional[int] = None, dtype=torch.bfloat16, latent: bool = False) -> Tuple[int, int]:
    d = _desc(num_layers, num_pages, page_size, num_kv_heads, head_dim_qk, head_dim_v, dtype, latent)
    kb, vb = C.c_size_t(), C.c_size_t()
    L.check(L.load().kv_pool_bytes(C.byref(d), C.byref(kb), C.byref(vb)), "kv_pool_bytes")
    return kb.value, vb.value


@dataclass
class Pool:
    """Host handle of a pool whose buffers the caller allocated (kept
    referenced here so they outlive the handle)."""
    handle: int
    k: torch.Tensor
    v: Optional[torch.Tensor]
    num_layers: int
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    latent: bool

    @property
    def dtype(self) -> torch.dtype:
        return self.k.dtype

    def flat(self, which: str, layer: int) -> torch.Tensor:
        """One layer's buffer viewed per token ``[(num_pages+1)*page_size, heads, dim]``."""
        buf = self.k if which == "k" else self.v
        dim = self.head_dim_qk if which == "k" else self.head_dim_v
        return buf.view(self.num_layers, (self.num_pages + 1) * self.page_size, self.num_kv_heads, dim)[layer]


def kv_pool_create(k: torch.Tensor, v: Optional[torch.Tensor], *, num_layers: int, num_pages: int, page_size: int,
                   num_kv_heads: int, head_dim_qk: int, head_dim_v: Optional[int] = None,
                   latent: bool = False) -> Pool:
    if k.dtype not in _DTYPES:
        raise TypeError(f"pool dtype {k.dtype} not supported")
    d = _desc(num_layers, num_pages, page_size, num_kv_heads, head_dim_qk, head_dim_v, k.dtype, latent)
    kb, vb = kv_pool_bytes(num_layers, num_pages, page_size, num_kv_heads, head_dim_qk, head_dim_v, k.dtype, latent)
    if k.numel() * k.element_size() < kb or (v is not None and v.numel() * v.element_size() < vb):
        raise ValueError("pool buffers are smaller than kv_pool_bytes")
    h = C.c_void_p()
    L.check(L.load().kv_pool_create(C.byref(d), _dev(k, "k"), _dev(v, "v"), C.byref(h)), "kv_pool_create")
    return Pool(h.value, k, v, num_layers, num_pages, page_size, num_kv_heads, head_dim_qk,
                head_dim_qk if head_dim_v is None else head_dim_v, latent)


def kv_pool_destroy(pool: Pool) -> None:
    if pool.handle:
        L.check(L.load().kv_pool_destroy(pool.handle), "kv_pool_destroy")
        pool.handle = 0


def kv_pool_padding_page(pool: Pool) -> int:
    r = L.load().kv_pool_padding_page(pool.handle)
    L.check(min(r, 0), "kv_pool_padding_page")
    return r


def kv_pool_token_bytes(pool: Pool) -> int:
    r = L.load().kv_pool_token_bytes(pool.handle)
    L.check(int(min(r, 0)), "kv_pool_token_bytes")
    return r


# ---------------------------------------------------------------------------
# store / indices / gather
# ---------------------------------------------------------------------------

def kv_store(pool: Pool, layer: int, k: torch.Tensor, v: Optional[torch.Tensor], out_loc: torch.Tensor,
             stream=None) -> None:
    _check_rows(pool, k, "k", out_loc.numel(), "k")
    if not pool.latent:
        _check_rows(pool, v, "v", out_loc.numel(), "v")
    L.check(L.load().kv_store(pool.handle, layer, _dev(k, "k", pool.dtype), _dev(v, "v", pool.dtype),
                              _dev(out_loc, "out_loc", torch.int32), out_loc.numel(), _stream(stream)), "kv_store")


def build_kv_indices(out_fmt: int, req_to_token: torch.Tensor, req_pool_indices: torch.Tensor,
                     kv_start: Optional[torch.Tensor], kv_lens: torch.Tensor, page_size: int, max_kv_len: int,
                     kv_indptr: Optional[torch.Tensor], out: torch.Tensor,
                     kv_last_page_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """CSR: ``out`` is kv_indices (capacity = ``out.numel()``).  BLOCK_TABLE:
    ``out`` is ``[bs, stride]`` (capacity = stride)."""
    i32 = torch.int32
    rows, width = req_to_token.shape
    cap = out.numel() if out_fmt == PKV_MAP_CSR else out.shape[-1]
    L.check(L.load().build_kv_indices(
        out_fmt, _dev(req_to_token, "req_to_token", i32), rows, width, _dev(req_pool_indices, "req_pool_indices", i32),
        _dev(kv_start, "kv_start", i32), _dev(kv_lens, "kv_lens", i32), kv_lens.numel(), page_size, max_kv_len,
        _dev(kv_indptr, "kv_indptr", i32), _dev(out, "out", i32), cap,
        _dev(kv_last_page_len, "kv_last_page_len", i32), _stream(stream)), "build_kv_indices")


@dataclass
class KVMap:
    """A pkv_kv_map plus the tensors it points at (kept alive here)."""
    struct: L.KVMapStruct
    refs: tuple

    @property
    def bs(self) -> int:
        return self.struct.bs

    @property
    def max_kv_len(self) -> int:
        return self.struct.max_kv_len


def make_kv_map(fmt: int, kv_lens: torch.Tensor, max_kv_len: int, *, req_to_token=None, req_pool_indices=None,
                kv_start=None, kv_indptr=None, kv_indices=None, block_table=None, k=None, v=None,
                cu_seqlens_k=None) -> KVMap:
    i32 = torch.int32
    s = L.KVMapStruct()
    s.fmt = fmt
    s.bs = kv_lens.numel()
    s.kv_lens = _dev(kv_lens, "kv_lens", i32)
    s.max_kv_len = int(max_kv_len)
    if req_to_token is not None:
        s.req_to_token = _dev(req_to_token, "req_to_token", i32)
        s.table_rows, s.table_width = req_to_token.shape
    s.req_pool_indices = _dev(req_pool_indices, "req_pool_indices", i32)
    s.kv_start = _dev(kv_start, "kv_start", i32)
    s.kv_indptr = _dev(kv_indptr, "kv_indptr", i32)
    if kv_indices is not None:
        s.kv_indices = _dev(kv_indices, "kv_indices", i32)
        s.kv_indices_len = kv_indices.numel()
    if block_table is not None:
        s.block_table = _dev(block_table, "block_table", i32)
        s.block_stride = block_table.shape[-1]
    s.k = _dev(k, "k")
    s.v = _dev(v, "v")
    s.cu_seqlens_k = _dev(cu_seqlens_k, "cu_seqlens_k", i32)
    if k is not None:
        s.total_k = k.shape[0]
    return KVMap(s, (kv_lens, req_to_token, req_pool_indices, kv_start, kv_indptr, kv_indices, block_table, k, v,
                     cu_seqlens_k))


def kv_gather(pool: Pool, layer: int, kv_map: KVMap, cu_seqlens_k: torch.Tensor, k_out: torch.Tensor,
              v_out: Optional[torch.Tensor], stream=None) -> None:
    L.check(L.load().kv_gather(pool.handle, layer, C.byref(kv_map.struct), _dev(cu_seqlens_k, "cu_seqlens_k",
                                                                             torch.int32),
                               _dev(k_out, "k_out", pool.dtype), _dev(v_out, "v_out", pool.dtype), k_out.shape[0],
                               _stream(stream)), "kv_gather")


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def paged_decode_workspace_bytes(pool: Pool, bs: int, num_q_heads: int, max_kv_len: int) -> int:
    n = C.c_size_t()
    L.check(L.load().paged_decode_workspace_bytes(pool.handle, bs, num_q_heads, max_kv_len, C.byref(n)),
            "paged_decode_workspace_bytes")
    return n.value


def paged_decode_attn(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, sm_scale: float, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """q ``[bs, Hq, Dqk]`` -> out ``[bs, Hq, Dv]`` (pool dtype); workspace a
    uint8 device tensor of at least paged_decode_workspace_bytes() bytes."""
    _check_attn(pool, q, out, lse, (kv_map.bs,), "paged_decode_attn")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().paged_decode_attn(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[1],
                                       C.byref(kv_map.struct), float(sm_scale), _dev(out, "out", pool.dtype),
                                       _dev(lse, "lse", torch.float32), ws_ptr, ws_bytes, _stream(stream)),
            "paged_decode_attn")


def paged_decode_attn_noalloc(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, sm_scale: float,
                              out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """paged_decode_attn with its workspace in the library's own device
    array (no allocation; calls overlapping on one device race)."""
    _check_attn(pool, q, out, lse, (kv_map.bs,), "paged_decode_attn_noalloc")
    L.check(L.load().paged_decode_attn_noalloc(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[1],
                                               C.byref(kv_map.struct), float(sm_scale), _dev(out, "out", pool.dtype),
                                               _dev(lse, "lse", torch.float32), _stream(stream)),
            "paged_decode_attn_noalloc")


def paged_decode_attn_append(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, k_new: torch.Tensor,
                             v_new: Optional[torch.Tensor], out_loc: torch.Tensor, sm_scale: float,
                             out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kv_store(pool, layer, k_new, v_new, out_loc) then paged_decode_attn,
    as one call whose append rides in the decode's planner launch."""
    _check_attn(pool, q, out, lse, (kv_map.bs,), "paged_decode_attn_append")
    _check_rows(pool, k_new, "k_new", out_loc.numel(), "k")
    if not pool.latent:
        _check_rows(pool, v_new, "v_new", out_loc.numel(), "v")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().paged_decode_attn_append(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[1],
                                              C.byref(kv_map.struct), _dev(k_new, "k_new", pool.dtype),
                                              _dev(v_new, "v_new", pool.dtype), _dev(out_loc, "out_loc", torch.int32),
                                              out_loc.numel(), float(sm_scale), _dev(out, "out", pool.dtype),
                                              _dev(lse, "lse", torch.float32), ws_ptr, ws_bytes, _stream(stream)),
            "paged_decode_attn_append")


@dataclass
class PrefixGroups:
    """A pkv_prefix_groups plus the device tensors it points at."""
    struct: L.PrefixGroups
    refs: tuple


def make_prefix_groups(group_indptr: torch.Tensor, prefix_len: torch.Tensor, max_group_size: int,
                       max_prefix_len: int) -> PrefixGroups:
    """group_indptr device int32[G + 1] (group g = requests indptr[g] ..
    indptr[g+1] - 1), prefix_len device int32[G]; host bounds."""
    i32 = torch.int32
    st = L.PrefixGroups(prefix_len.numel(), int(max_group_size), int(max_prefix_len),
                        _dev(group_indptr, "group_indptr", i32), _dev(prefix_len, "prefix_len", i32))
    return PrefixGroups(st, (group_indptr, prefix_len))


def paged_decode_cascade_workspace_bytes(pool: Pool, bs: int, num_q_heads: int, max_kv_len: int,
                                         groups: PrefixGroups) -> int:
    n = C.c_size_t()
    L.check(L.load().paged_decode_cascade_workspace_bytes(pool.handle, bs, num_q_heads, max_kv_len,
                                                          C.byref(groups.struct), C.byref(n)),
            "paged_decode_cascade_workspace_bytes")
    return n.value


def paged_decode_attn_cascade(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, groups: PrefixGroups,
                              sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_attn(pool, q, out, lse, (kv_map.bs,), "paged_decode_attn_cascade")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().paged_decode_attn_cascade(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[1],
                                               C.byref(kv_map.struct), C.byref(groups.struct), float(sm_scale),
                                               _dev(out, "out", pool.dtype), _dev(lse, "lse", torch.float32), ws_ptr,
                                               ws_bytes, _stream(stream)), "paged_decode_attn_cascade")


def paged_verify_attn(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, sm_scale: float, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Target verification over a latent pool: q ``[bs, num_draft, Hq, 576]``
    -> out ``[bs, num_draft, Hq, 512]``; workspace of at least
    paged_decode_workspace_bytes(pool, bs, num_draft * Hq, max_kv_len) bytes."""
    if q.dim() != 4:
        raise ValueError("q must be [bs, num_draft, Hq, 576] and out [bs, num_draft, Hq, 512]")
    _check_attn(pool, q, out, lse, (kv_map.bs, q.shape[1]), "paged_verify_attn")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().paged_verify_attn(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[2], q.shape[1],
                                       C.byref(kv_map.struct), float(sm_scale), _dev(out, "out", pool.dtype),
                                       _dev(lse, "lse", torch.float32), ws_ptr, ws_bytes, _stream(stream)),
            "paged_verify_attn")


def paged_verify_attn_append(pool: Pool, layer: int, q: torch.Tensor, kv_map: KVMap, k_new: torch.Tensor,
                             out_loc: torch.Tensor, sm_scale: float, out: torch.Tensor,
                             lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    """kv_store(pool, layer, k_new, None, out_loc) then paged_verify_attn, as
    one call whose append rides in the verification's planner launch."""
    _check_rows(pool, k_new, "k_new", out_loc.numel(), "k")
    if q.dim() != 4:
        raise ValueError("q must be [bs, num_draft, Hq, 576] and out [bs, num_draft, Hq, 512]")
    _check_attn(pool, q, out, lse, (kv_map.bs, q.shape[1]), "paged_verify_attn")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.load().paged_verify_attn_append(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[2], q.shape[1],
                                              C.byref(kv_map.struct), _dev(k_new, "k_new", pool.dtype),
                                              _dev(out_loc, "out_loc", torch.int32), out_loc.numel(),
                                              float(sm_scale), _dev(out, "out", pool.dtype),
                                              _dev(lse, "lse", torch.float32), ws_ptr, ws_bytes, _stream(stream)),
            "paged_verify_attn_append")


def paged_extend_attn(pool: Pool, layer: int, q: torch.Tensor, qo_indptr: torch.Tensor, max_q_len: int,
                      kv_map: KVMap, causal: bool, sm_scale: float, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_attn(pool, q, out, lse, (q.shape[0],), "paged_extend_attn")
    if qo_indptr.numel() != kv_map.bs + 1:
        raise ValueError("qo_indptr must have bs + 1 entries")
    L.check(L.load().paged_extend_attn(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[0],
                                       _dev(qo_indptr, "qo_indptr", torch.int32), q.shape[1], int(max_q_len),
                                       C.byref(kv_map.struct), 1 if causal else 0, float(sm_scale),
                                       _dev(out, "out", pool.dtype), _dev(lse, "lse", torch.float32),
                                       _stream(stream)), "paged_extend_attn")


def paged_extend_attn_ex(pool: Pool, layer: int, q: torch.Tensor, qo_indptr: torch.Tensor, max_q_len: int,
                         kv_map: KVMap, sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                         causal: bool = True, causal_flags: Optional[torch.Tensor] = None, softcap: float = 0.0,
                         stream=None) -> None:
    """paged_extend_attn with per-request causal flags (device int32[bs],
    nonzero = causal) and softcap (0 = off)."""
    _check_attn(pool, q, out, lse, (q.shape[0],), "paged_extend_attn")
    if qo_indptr.numel() != kv_map.bs + 1:
        raise ValueError("qo_indptr must have bs + 1 entries")
    if causal_flags is not None and causal_flags.numel() != kv_map.bs:
        raise ValueError("causal_flags must have one entry per request")
    opts = L.ExtendOpts(1 if causal else 0, _dev(causal_flags, "causal_flags", torch.int32), float(softcap))
    L.check(L.load().paged_extend_attn_ex(pool.handle, layer, _dev(q, "q", pool.dtype), q.shape[0],
                                          _dev(qo_indptr, "qo_indptr", torch.int32), q.shape[1], int(max_q_len),
                                          C.byref(kv_map.struct), C.byref(opts), float(sm_scale),
                                          _dev(out, "out", pool.dtype), _dev(lse, "lse", torch.float32),
                                          _stream(stream)), "paged_extend_attn_ex")


# ---------------------------------------------------------------------------
# encoder-embedding block cache
# ---------------------------------------------------------------------------

def _enc_geometry(buffer: torch.Tensor):
    if buffer.dim() < 2:
        raise ValueError("buffer must be [num_blocks, block_size, ...]")
    row_bytes = buffer[0, 0].numel() * buffer.element_size()
    return buffer.shape[0], buffer.shape[1], row_bytes


def enc_cache_write(buffer: torch.Tensor, src: torch.Tensor, block_ids: torch.Tensor, stream=None) -> None:
    """buffer [num_blocks, block_size, ...]; src [n, block_size, ...] of the
    same dtype and row shape; block_ids device int32[n]."""
    nb, bsz, rb = _enc_geometry(buffer)
    if src.dtype != buffer.dtype or src.shape[1:] != buffer.shape[1:] or block_ids.numel() != src.shape[0]:
        raise ValueError("src must be [n, block_size, ...] like buffer, with one block id per block")
    L.check(L.load().enc_cache_write(_dev(buffer, "buffer"), nb, bsz, rb, _dev(src, "src"), src.shape[0],
                                     _dev(block_ids, "block_ids", torch.int32), _stream(stream)), "enc_cache_write")


def enc_cache_merge(buffer: torch.Tensor, block_ids: torch.Tensor, positions: torch.Tensor, hidden: torch.Tensor,
                    fill_count: Optional[torch.Tensor] = None, stream=None) -> None:
    """positions device int64 [max_blocks, block_size]; hidden [num_tokens,
    ...] rows like the buffer's; fill_count optional int32[num_tokens]."""
    nb, bsz, rb = _enc_geometry(buffer)
    if positions.dim() != 2 or positions.shape[1] != bsz or block_ids.numel() != positions.shape[0]:
        raise ValueError("positions must be [max_blocks, block_size] with one block id per row")
    if hidden.dtype != buffer.dtype or hidden[0].numel() * hidden.element_size() != rb:
        raise ValueError("hidden rows must match the buffer's rows")
    L.check(L.load().enc_cache_merge(_dev(buffer, "buffer"), nb, bsz, rb, _dev(block_ids, "block_ids", torch.int32),
                                     positions.shape[0], _dev(positions, "positions", torch.int64),
                                     _dev(hidden, "hidden"), hidden.shape[0],
                                     _dev(fill_count, "fill_count", torch.int32), _stream(stream)),
            "enc_cache_merge")


def enc_cache_check(fill_count: torch.Tensor, scheduled: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[int, list]:
    """Returns (status, [unfilled scheduled rows, rows filled twice]);
    synchronises the stream."""
    scratch = torch.empty(2, dtype=torch.int64, device=fill_count.device)
    counts = (C.c_int64 * 2)()
    st = L.load().enc_cache_check(_dev(fill_count, "fill_count", torch.int32),
                                  _dev(scheduled, "scheduled", torch.int32), fill_count.numel(),
                                  _dev(scratch, "scratch", torch.int64), counts, _stream(stream))
    if st not in (L.PKV_OK, L.PKV_EINVAL):
        L.check(st, "enc_cache_check")
    return st, list(counts)


# ---------------------------------------------------------------------------
# slot allocation and row writing
# ---------------------------------------------------------------------------

@dataclass
class FreeList:
    """The device tensors of one free list of pages: the ring of page ids,
    its {head, size} state, the status word every call writes, and the page
    bitmap kv_free uses as scratch."""
    page_size: int
    num_pages: int
    pages: torch.Tensor   # int32[capacity]
    state: torch.Tensor   # int32[2]
    status: torch.Tensor  # int32[1]
    bitmap: torch.Tensor  # int32[(num_pages + 31) // 32], read as uint32

    @property
    def capacity(self) -> int:
        return self.pages.numel()

    def _ptrs(self):
        i32 = torch.int32
        return (_dev(self.pages, "free_pages", i32), self.capacity, _dev(self.state, "free_state", i32))


def kv_free_list_create(page_size: int, num_pages: int, capacity: Optional[int] = None, first: int = 0,
                        count: Optional[int] = None, device="cuda", stream=None) -> FreeList:
    """Allocate the tensors of a free list (capacity defaults to num_pages)
    and initialise it to pages first .. first + count - 1 (count defaults to
    num_pages)."""
    cap = num_pages if capacity is None else capacity
    i32 = torch.int32
    fl = FreeList(page_size, num_pages, torch.empty(cap, dtype=i32, device=device),
                  torch.empty(2, dtype=i32, device=device), torch.zeros(1, dtype=i32, device=device),
                  torch.empty((num_pages + 31) // 32, dtype=i32, device=device))
    kv_free_list_init(fl, first, num_pages if count is None else count, stream)
    return fl


def kv_free_list_init(fl: FreeList, first: int, count: int, stream=None) -> None:
    L.check(L.load().kv_free_list_init(_dev(fl.pages, "free_pages", torch.int32), fl.capacity, int(first),
                                       int(count), _dev(fl.state, "free_state", torch.int32), _stream(stream)),
            "kv_free_list_init")


def kv_alloc(fl: FreeList, need: int, out: torch.Tensor, stream=None) -> None:
    if out.numel() < need:
        raise ValueError("out holds fewer than need slots")
    L.check(L.load().kv_alloc(fl.page_size, int(need), *fl._ptrs(), _dev(out, "out", torch.int32),
                              _dev(fl.status, "status", torch.int32), _stream(stream)), "kv_alloc")


def kv_alloc_extend(fl: FreeList, prefix_lens: torch.Tensor, seq_lens: torch.Tensor,
                    last_loc: Optional[torch.Tensor], out_cache_loc: torch.Tensor, stream=None) -> None:
    i32 = torch.int32
    bs = seq_lens.numel()
    if prefix_lens.numel() != bs or (last_loc is not None and last_loc.numel() != bs):
        raise ValueError("prefix_lens, seq_lens and last_loc must have bs entries")
    L.check(L.load().kv_alloc_extend(fl.page_size, bs, _dev(prefix_lens, "prefix_lens", i32),
                                     _dev(seq_lens, "seq_lens", i32), _dev(last_loc, "last_loc", i32), *fl._ptrs(),
                                     _dev(out_cache_loc, "out_cache_loc", i32), out_cache_loc.numel(),
                                     _dev(fl.status, "status", i32), _stream(stream)), "kv_alloc_extend")


def kv_alloc_decode(fl: FreeList, seq_lens: torch.Tensor, last_loc: Optional[torch.Tensor],
                    out_cache_loc: torch.Tensor, stream=None) -> None:
    i32 = torch.int32
    bs = seq_lens.numel()
    if out_cache_loc.numel() < bs or (last_loc is not None and last_loc.numel() != bs):
        raise ValueError("out_cache_loc and last_loc must have bs entries")
    L.check(L.load().kv_alloc_decode(fl.page_size, bs, _dev(seq_lens, "seq_lens", i32),
                                     _dev(last_loc, "last_loc", i32), *fl._ptrs(),
                                     _dev(out_cache_loc, "out_cache_loc", i32), _dev(fl.status, "status", i32),
                                     _stream(stream)), "kv_alloc_decode")


def kv_free(fl: FreeList, slots: torch.Tensor, stream=None) -> None:
    i32 = torch.int32
    L.check(L.load().kv_free(fl.page_size, _dev(slots, "slots", i32), slots.numel(), fl.num_pages, *fl._ptrs(),
                             _dev(fl.bitmap, "page_bitmap", i32), _dev(fl.status, "status", i32),
                             _stream(stream)), "kv_free")


def write_req_to_token(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor, prefix_lens: torch.Tensor,
                       seq_lens: torch.Tensor, out_cache_loc: torch.Tensor, max_seq_len: int,
                       prefix_ptrs=None, stream=None) -> None:
    """prefix_ptrs: None, a device int64 tensor of bs pointers, or a list of
    bs int32 device tensors / None (their addresses are copied to the
    device here; the tensors must stay alive until the work is done)."""
    i32 = torch.int32
    bs = req_pool_indices.numel()
    ptrs = prefix_ptrs
    if isinstance(prefix_ptrs, (list, tuple)):
        if len(prefix_ptrs) != bs:
            raise ValueError("prefix_ptrs must have bs entries")
        addrs = [0 if t is None else _dev(t, "prefix slots", i32) for t in prefix_ptrs]
        ptrs = torch.tensor(addrs, dtype=torch.int64).to(req_to_token.device)
        if stream is not None:  # keep the pointer array alive for the kernel's stream
            ptrs.record_stream(torch.cuda.ExternalStream(_stream(stream)))
    rows, width = req_to_token.shape
    L.check(L.load().write_req_to_token(
        _dev(req_to_token, "req_to_token", i32), rows, width, _dev(req_pool_indices, "req_pool_indices", i32),
        _dev(prefix_lens, "prefix_lens", i32), _dev(seq_lens, "seq_lens", i32),
        _dev(out_cache_loc, "out_cache_loc", i32), out_cache_loc.numel(),
        _dev(ptrs, "prefix_ptrs", torch.int64), bs, int(max_seq_len), _stream(stream)), "write_req_to_token")


# ---------------------------------------------------------------------------
# debug / measurement
# ---------------------------------------------------------------------------

def kv_validate(pool: Pool, kv_map: KVMap, is_dummy: Optional[torch.Tensor] = None,
                scratch: Optional[torch.Tensor] = None, stream=None) -> Tuple[int, list]:
    """Returns (status, counts[8]); synchronises the stream."""
    if scratch is None:
        scratch = torch.empty(max(kv_map.bs, 1) * 8, dtype=torch.int64, device=kv_map.refs[0].device)
    counts = (C.c_int64 * 8)()
    st = L.load().kv_validate(pool.handle, C.byref(kv_map.struct), _dev(is_dummy, "is_dummy", torch.int32),
                              _dev(scratch, "scratch", torch.int64), counts, _stream(stream))
    if st not in (L.PKV_OK, L.PKV_EINVAL, L.PKV_EALIGN):
        L.check(st, "kv_validate")
    return st, list(counts)


def pkv_set_kernel_timer(start_event: Optional[int], stop_event: Optional[int]) -> None:
    """Raw hipEvent_t handles (ints) or None."""
    L.check(L.load().pkv_set_kernel_timer(start_event, stop_event), "pkv_set_kernel_timer")
