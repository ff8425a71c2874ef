// The C ABI (include/pagedkv.h): argument validation, descriptor checks and
// dispatch to the kernel launchers.  No device allocation, no host sync
// (except kv_validate, which is documented as synchronising).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <new>
#include <string>

#include "pagedkv.h"
#include "pkv_alloc.h"
#include "pkv_enc.h"
#include "pkv_launch.h"

struct pkv_pool {
  pkv_pool_desc desc;
  pkv::PoolInfo info;
};

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_timer_start = nullptr;
thread_local hipEvent_t g_timer_stop = nullptr;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() { return PKV_OK; }

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
int32_t ilog2(int32_t x) {
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

int check_desc(const pkv_pool_desc* d) {
  if (!d) return fail(PKV_EINVAL, "null pool descriptor");
  if (d->num_layers <= 0 || d->num_pages < 0 || d->num_kv_heads <= 0 || d->head_dim_qk <= 0 || d->head_dim_v <= 0)
    return fail(PKV_EINVAL, "pool dims must be positive (layers %d, pages %d, kv_heads %d, dims %d/%d)",
                d->num_layers, d->num_pages, d->num_kv_heads, d->head_dim_qk, d->head_dim_v);
  if (!pow2(d->page_size) || d->page_size > 128)
    return fail(PKV_EUNSUPPORTED, "page_size %d: must be a power of two in [1, 128]", d->page_size);
  if (d->dtype != PKV_DTYPE_F32 && d->dtype != PKV_DTYPE_BF16) return fail(PKV_EUNSUPPORTED, "dtype %d", d->dtype);
  if (d->kind == PKV_KIND_SPLIT_KV) {
    if (d->head_dim_qk != d->head_dim_v)
      return fail(PKV_EINVAL, "split K/V pool needs head_dim_qk == head_dim_v (%d vs %d)", d->head_dim_qk,
                  d->head_dim_v);
  } else if (d->kind == PKV_KIND_LATENT) {
    if (d->head_dim_v > d->head_dim_qk) return fail(PKV_EINVAL, "latent pool needs head_dim_v <= head_dim_qk");
  } else {
    return fail(PKV_EUNSUPPORTED, "pool kind %d", d->kind);
  }
  // slot ids are int32 everywhere (tables, out_loc, the kernels' slot maps):
  // every slot of the pool, the padding page's included, must fit
  if (((int64_t)d->num_pages + 1) * d->page_size > (int64_t)INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "pool of %lld slots: slot ids must fit in int32",
                (long long)(((int64_t)d->num_pages + 1) * d->page_size));
  const int eb = d->dtype == PKV_DTYPE_F32 ? 4 : 2;
  if (((int64_t)d->num_kv_heads * d->head_dim_qk * eb) % 16 != 0 ||
      ((int64_t)d->num_kv_heads * d->head_dim_v * eb) % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "token rows must be a multiple of 16 bytes");
  return PKV_OK;
}

void fill_info(const pkv_pool_desc* d, void* k, void* v, pkv::PoolInfo* p) {
  p->num_layers = d->num_layers;
  p->num_pages = d->num_pages;
  p->page_size = d->page_size;
  p->page_shift = ilog2(d->page_size);
  p->num_kv_heads = d->num_kv_heads;
  p->head_dim_qk = d->head_dim_qk;
  p->head_dim_v = d->head_dim_v;
  p->dtype = d->dtype;
  p->kind = d->kind;
  p->elem_bytes = d->dtype == PKV_DTYPE_F32 ? 4 : 2;
  p->k_base = static_cast<char*>(k);
  p->v_base = static_cast<char*>(v);
  p->num_slots = ((int64_t)d->num_pages + 1) * d->page_size;
  p->pad_slot = (int64_t)d->num_pages * d->page_size;
  p->k_row_bytes = (int64_t)d->num_kv_heads * d->head_dim_qk * p->elem_bytes;
  p->v_row_bytes = d->kind == PKV_KIND_LATENT ? 0 : (int64_t)d->num_kv_heads * d->head_dim_v * p->elem_bytes;
  p->k_layer_bytes = p->num_slots * p->k_row_bytes;
  p->v_layer_bytes = p->num_slots * p->v_row_bytes;
}

int check_pool(const pkv_pool* pool) {
  if (!pool) return fail(PKV_EINVAL, "null pool handle");
  return PKV_OK;
}

int check_layer(const pkv_pool* pool, int32_t layer) {
  if (layer < 0 || layer >= pool->desc.num_layers)
    return fail(PKV_EINVAL, "layer %d outside [0, %d)", layer, pool->desc.num_layers);
  return PKV_OK;
}

// Validate a kv map's host-visible fields and turn it into the device view.
int make_devmap(const pkv_pool* pool, const pkv_kv_map* m, bool allow_contiguous, pkv::DevMap* out) {
  if (!m) return fail(PKV_EINVAL, "null kv map");
  if (m->bs < 0 || m->max_kv_len < 0) return fail(PKV_EINVAL, "negative bs or max_kv_len");
  if (m->bs > 0 && !m->kv_lens) return fail(PKV_EINVAL, "null kv_lens");
  memset(out, 0, sizeof(*out));
  out->fmt = m->fmt;
  out->page_shift = pool->info.page_shift;
  out->kv_lens = m->kv_lens;
  out->num_slots = pool->info.num_slots;
  out->pad_slot = pool->info.pad_slot;
  switch (m->fmt) {
    case PKV_MAP_TOKEN_TABLE:
      if (m->bs > 0 && (!m->req_to_token || !m->req_pool_indices))
        return fail(PKV_EINVAL, "token table map needs req_to_token and req_pool_indices");
      if (m->table_rows <= 0 || m->table_width <= 0) return fail(PKV_EINVAL, "token table dims must be positive");
      out->req_to_token = m->req_to_token;
      out->table_rows = m->table_rows;
      out->table_width = m->table_width;
      out->req_pool_indices = m->req_pool_indices;
      out->kv_start = m->kv_start;
      break;
    case PKV_MAP_CSR:
      if (m->bs > 0 && (!m->kv_indptr || !m->kv_indices)) return fail(PKV_EINVAL, "CSR map needs kv_indptr, kv_indices");
      if (m->kv_indices_len < 0) return fail(PKV_EINVAL, "negative kv_indices_len");
      out->kv_indptr = m->kv_indptr;
      out->kv_indices = m->kv_indices;
      out->kv_indices_len = m->kv_indices_len;
      break;
    case PKV_MAP_BLOCK_TABLE: {
      if (m->bs > 0 && !m->block_table) return fail(PKV_EINVAL, "block table map needs block_table");
      const int64_t need = ((int64_t)m->max_kv_len + pool->desc.page_size - 1) / pool->desc.page_size;
      if (m->block_stride < need)
        return fail(PKV_ECAPACITY, "block_stride %lld < ceil(max_kv_len / page_size) = %lld",
                    (long long)m->block_stride, (long long)need);
      out->block_table = m->block_table;
      out->block_stride = m->block_stride;
      break;
    }
    case PKV_MAP_CONTIGUOUS:
      if (!allow_contiguous) return fail(PKV_EUNSUPPORTED, "contiguous map not accepted by this call");
      if (m->bs > 0 && !m->cu_seqlens_k) return fail(PKV_EINVAL, "contiguous map needs cu_seqlens_k");
      if (m->total_k > 0 && (!m->k || (pool->desc.kind == PKV_KIND_SPLIT_KV && !m->v)))
        return fail(PKV_EINVAL, "contiguous map with rows needs k (and v for a split K/V pool)");
      if (m->total_k < 0) return fail(PKV_EINVAL, "negative total_k");
      if (!aligned16(m->k) || !aligned16(m->v)) return fail(PKV_EALIGN, "contiguous k/v not 16-byte aligned");
      out->cu_seqlens_k = m->cu_seqlens_k;
      out->total_k = m->total_k;
      out->contig_k = m->k;
      out->contig_v = pool->desc.kind == PKV_KIND_LATENT ? m->k : m->v;
      out->num_slots = m->total_k;
      out->pad_slot = 0;
      break;
    default:
      return fail(PKV_EINVAL, "unknown map format %d", m->fmt);
  }
  return PKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// paged_decode_attn without a workspace argument, for callers that cannot
// allocate device memory.  The decode workspace (split plan, tile slot
// lists, partial results) lives in this file-scope device array, one copy
// per device, held until the process ends.  Host code never uses the
// array's name as an address: its device address is looked up once per
// device with hipGetSymbolAddress and kept.  Every call on a device shares
// that device's copy: calls that overlap on one device race.  Nothing in the
// workspace has to start at zero (each launch's planner writes everything
// its main kernel and merge read), so no call clears it.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
int scratch_for_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "device %d past %d", dev, kMaxDevices);
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
      if (!a) return fail(PKV_EDEVICE, "hipGetSymbolAddress(scratch) returned a null address");
      p = static_cast<char*>(a);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}
}  // namespace


namespace pkv {
void timer_before(hipStream_t s) {
  if (g_timer_start) (void)hipEventRecord(g_timer_start, s);
}
void timer_after(hipStream_t s) {
  if (g_timer_stop) (void)hipEventRecord(g_timer_stop, s);
  g_timer_start = nullptr;
  g_timer_stop = nullptr;
}
}  // namespace pkv

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported configuration";
    case PKV_EALIGN: return "misaligned pointer or kv_start";
    case PKV_ECAPACITY: return "capacity or workspace too small";
    case PKV_EDEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_build_arch(void) { return "gfx950"; }

int kv_pool_bytes(const pkv_pool_desc* desc, size_t* k_bytes, size_t* v_bytes) {
  int st = check_desc(desc);
  if (st) return st;
  if (!k_bytes || !v_bytes) return fail(PKV_EINVAL, "null output pointer");
  pkv::PoolInfo p;
  fill_info(desc, nullptr, nullptr, &p);
  *k_bytes = (size_t)p.k_layer_bytes * desc->num_layers;
  *v_bytes = (size_t)p.v_layer_bytes * desc->num_layers;
  return ok();
}

int kv_pool_create(const pkv_pool_desc* desc, void* k_base, void* v_base, pkv_pool** out) {
  int st = check_desc(desc);
  if (st) return st;
  if (!out) return fail(PKV_EINVAL, "null output handle");
  if (!k_base) return fail(PKV_EINVAL, "null k_base");
  if (desc->kind == PKV_KIND_SPLIT_KV && !v_base) return fail(PKV_EINVAL, "null v_base for a split K/V pool");
  if (desc->kind == PKV_KIND_LATENT && v_base) return fail(PKV_EINVAL, "latent pool takes no v_base");
  if (!aligned16(k_base) || !aligned16(v_base)) return fail(PKV_EALIGN, "pool buffers must be 16-byte aligned");
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return fail(PKV_EINVAL, "out of host memory");
  p->desc = *desc;
  fill_info(desc, k_base, v_base, &p->info);
  *out = p;
  return ok();
}

int kv_pool_destroy(pkv_pool* pool) {
  delete pool;
  return ok();
}

int32_t kv_pool_padding_page(const pkv_pool* pool) {
  if (int st = check_pool(pool)) return st;
  return pool->desc.num_pages;
}

int64_t kv_pool_token_bytes(const pkv_pool* pool) {
  if (int st = check_pool(pool)) return st;
  return pool->info.k_row_bytes + pool->info.v_row_bytes;
}

}  // extern "C"

namespace {
// Arguments of a KV append (kv_store, or the append a decode call carries);
// a latent pool's v is dropped.
int check_store(const pkv_pool* pool, const void* k, const void** v, const int32_t* out_loc, int64_t n) {
  if (n < 0) return fail(PKV_EINVAL, "negative n");
  if (n == 0) return PKV_OK;
  if (!k || !out_loc) return fail(PKV_EINVAL, "null k or out_loc");
  if (pool->desc.kind == PKV_KIND_SPLIT_KV && !*v) return fail(PKV_EINVAL, "null v for a split K/V pool");
  if (pool->desc.kind == PKV_KIND_LATENT) *v = nullptr;
  if (!aligned16(k) || !aligned16(*v)) return fail(PKV_EALIGN, "k/v must be 16-byte aligned");
  return PKV_OK;
}
}  // namespace

extern "C" {

int kv_store(const pkv_pool* pool, int32_t layer, const void* k, const void* v, const int32_t* out_loc, int64_t n,
             void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  if (int st = check_store(pool, k, &v, out_loc, n)) return st;
  if (n == 0) return ok();
  return device_status(pkv::launch_store(pool->info, layer, k, v, out_loc, n, (hipStream_t)stream), "kv_store");
}

int build_kv_indices(int32_t out_fmt, const int32_t* req_to_token, int64_t table_rows, int64_t table_width,
                     const int32_t* req_pool_indices, const int32_t* kv_start, const int32_t* kv_lens, int32_t bs,
                     int32_t page_size, int32_t max_kv_len, int32_t* kv_indptr, int32_t* out, int64_t capacity,
                     int32_t* kv_last_page_len, void* stream) {
  if (out_fmt != PKV_MAP_CSR && out_fmt != PKV_MAP_BLOCK_TABLE)
    return fail(PKV_EINVAL, "out_fmt must be CSR or BLOCK_TABLE");
  if (bs < 0 || max_kv_len < 0 || capacity < 0) return fail(PKV_EINVAL, "negative bs, max_kv_len or capacity");
  if (!pow2(page_size) || page_size > 128) return fail(PKV_EUNSUPPORTED, "page_size %d", page_size);
  if (out_fmt == PKV_MAP_CSR && !kv_indptr) return fail(PKV_EINVAL, "CSR output needs kv_indptr");
  if (bs > 0 && (!req_to_token || !req_pool_indices || !kv_lens || !out))
    return fail(PKV_EINVAL, "null table, indices, lengths or output");
  if (table_rows <= 0 || table_width <= 0) return fail(PKV_EINVAL, "token table dims must be positive");
  const int64_t per_req = ((int64_t)max_kv_len + page_size - 1) / page_size;
  if (out_fmt == PKV_MAP_CSR && capacity < per_req * bs)
    return fail(PKV_ECAPACITY, "kv_indices capacity %lld < bs * ceil(max_kv_len / page_size) = %lld",
                (long long)capacity, (long long)(per_req * bs));
  if (out_fmt == PKV_MAP_BLOCK_TABLE && capacity < per_req)
    return fail(PKV_ECAPACITY, "block table stride %lld < ceil(max_kv_len / page_size) = %lld", (long long)capacity,
                (long long)per_req);
  return device_status(pkv::launch_build_indices(out_fmt, req_to_token, table_rows, table_width, req_pool_indices,
                                                  kv_start, kv_lens, bs, ilog2(page_size), kv_indptr, out, capacity,
                                                  kv_last_page_len, (hipStream_t)stream),
                       "build_kv_indices");
}

int paged_decode_workspace_bytes(const pkv_pool* pool, int32_t bs, int32_t num_q_heads, int32_t max_kv_len,
                                 size_t* bytes) {
  if (int st = check_pool(pool)) return st;
  if (!bytes || bs < 0 || max_kv_len < 0 || num_q_heads <= 0) return fail(PKV_EINVAL, "bad workspace query");
  if (!pkv::decode_supported(pool->info, num_q_heads))
    return fail(PKV_EUNSUPPORTED, "no decode kernel for this pool (dtype %d, dims %d/%d, %d q heads over %d kv heads)",
                pool->desc.dtype, pool->desc.head_dim_qk, pool->desc.head_dim_v, num_q_heads,
                pool->desc.num_kv_heads);
  const pkv::DecodePlan plan = pkv::plan_decode(pool->info, bs, num_q_heads, max_kv_len);
  *bytes = pkv::decode_workspace_bytes(pool->info, plan, bs, num_q_heads);
  return ok();
}

}  // extern "C"

namespace {
// paged_decode_attn with an optional KV append (st.n == 0: none), checked
// before anything is launched.
int decode_call(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads, const pkv_kv_map* map,
                float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes, void* stream,
                const pkv::StoreArgs& st, const char* what) {
  pkv::DevMap dm;
  if (int e = make_devmap(pool, map, false, &dm)) return e;
  if (num_q_heads <= 0 || num_q_heads % pool->desc.num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads %d not a positive multiple of num_kv_heads %d", num_q_heads,
                pool->desc.num_kv_heads);
  if (!pkv::decode_supported(pool->info, num_q_heads))
    return fail(PKV_EUNSUPPORTED, "no decode kernel for this pool (dtype %d, dims %d/%d, %d q heads over %d kv heads)",
                pool->desc.dtype, pool->desc.head_dim_qk, pool->desc.head_dim_v, num_q_heads,
                pool->desc.num_kv_heads);
  if (!(sm_scale > 0.0f) || std::isinf(sm_scale)) return fail(PKV_EINVAL, "sm_scale must be positive and finite");
  if (map->bs == 0) {
    if (st.n == 0) return ok();
    return device_status(pkv::launch_store_args(st, (hipStream_t)stream), what);
  }
  if (!q || !out) return fail(PKV_EINVAL, "null q or out");
  if (!aligned16(q)) return fail(PKV_EALIGN, "q must be 16-byte aligned");
  const pkv::DecodePlan plan = pkv::plan_decode(pool->info, map->bs, num_q_heads, map->max_kv_len);
  const size_t need = pkv::decode_workspace_bytes(pool->info, plan, map->bs, num_q_heads);
  if (ws_bytes < need) return fail(PKV_ECAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return fail(PKV_EALIGN, "workspace must be non-null and 256-byte aligned");
  return device_status(pkv::launch_decode(pool->info, layer, q, num_q_heads, dm, map->bs, plan, sm_scale, out, lse,
                                          workspace, (hipStream_t)stream, st.n > 0 ? &st : nullptr),
                       what);
}
}  // namespace

extern "C" {

int paged_decode_attn_append(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                             const pkv_kv_map* map, const void* k_new, const void* v_new, const int32_t* out_loc,
                             int64_t n_new, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  if (int st = check_store(pool, k_new, &v_new, out_loc, n_new)) return st;
  const pkv::StoreArgs sa = pkv::make_store_args(pool->info, layer, k_new, v_new, out_loc, n_new);
  return decode_call(pool, layer, q, num_q_heads, map, sm_scale, out, lse, workspace, ws_bytes, stream, sa,
                     "paged_decode_attn_append");
}

int paged_decode_attn(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads, const pkv_kv_map* map,
                      float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  pkv::StoreArgs none{};
  return decode_call(pool, layer, q, num_q_heads, map, sm_scale, out, lse, workspace, ws_bytes, stream, none,
                     "paged_decode_attn");
}

int paged_decode_attn_noalloc(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                              const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  if (!map) return fail(PKV_EINVAL, "null map");
  // the size is checked before any device call, so an oversized batch is
  // rejected the same way with or without a device
  if (num_q_heads > 0 && map->bs >= 0 && map->max_kv_len >= 0 && pkv::decode_supported(pool->info, num_q_heads)) {
    const pkv::DecodePlan plan = pkv::plan_decode(pool->info, map->bs, num_q_heads, map->max_kv_len);
    const size_t need = pkv::decode_workspace_bytes(pool->info, plan, map->bs, num_q_heads);
    if (need > kNoAllocScratchBytes)
      return fail(PKV_ECAPACITY, "this decode needs %zu bytes of workspace; paged_decode_attn_noalloc holds %zu "
                                 "(pass a workspace to paged_decode_attn instead)",
                  need, kNoAllocScratchBytes);
  }
  char* ws = nullptr;
  if (map->bs > 0)
    if (int st = scratch_for_current_device(&ws)) return st;
  pkv::StoreArgs none{};
  return decode_call(pool, layer, q, num_q_heads, map, sm_scale, out, lse, ws, kNoAllocScratchBytes, stream, none,
                     "paged_decode_attn_noalloc");
}

namespace {
int check_groups(const pkv_pool* pool, int32_t num_q_heads, const pkv_prefix_groups* g) {
  if (!g) return fail(PKV_EINVAL, "null prefix groups");
  if (g->num_groups < 0 || g->max_group_size < 0 || g->max_prefix_len < 0)
    return fail(PKV_EINVAL, "negative group count or bound");
  if (g->num_groups > 0 && (!g->group_indptr || !g->prefix_len))
    return fail(PKV_EINVAL, "prefix groups need group_indptr and prefix_len");
  if (pool->desc.kind != PKV_KIND_SPLIT_KV || pool->desc.dtype != PKV_DTYPE_BF16 ||
      !pkv::decode_supported(pool->info, num_q_heads) || num_q_heads % pool->desc.num_kv_heads != 0 ||
      num_q_heads / pool->desc.num_kv_heads > 16)
    return fail(PKV_EUNSUPPORTED, "cascade decode needs a bf16 split K/V pool, head_dim 64 or 128, at most 16 query "
                                  "heads per KV head");
  return ok();
}
}  // namespace

int paged_decode_cascade_workspace_bytes(const pkv_pool* pool, int32_t bs, int32_t num_q_heads, int32_t max_kv_len,
                                         const pkv_prefix_groups* groups, size_t* bytes) {
  if (int st = check_pool(pool)) return st;
  if (!bytes || bs < 0 || max_kv_len < 0 || num_q_heads <= 0) return fail(PKV_EINVAL, "bad workspace query");
  if (int st = check_groups(pool, num_q_heads, groups)) return st;
  const pkv::CascadePlan cp = pkv::plan_cascade(pool->info, bs, num_q_heads, max_kv_len, groups->num_groups,
                                                groups->max_group_size, groups->max_prefix_len);
  if (cp.cap > INT32_MAX) return fail(PKV_EUNSUPPORTED, "too many prefix work items (%lld)", (long long)cp.cap);
  *bytes = pkv::cascade_ws_layout(pool->info, cp, bs, num_q_heads, nullptr, nullptr);
  return ok();
}

int paged_decode_attn_cascade(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                              const pkv_kv_map* map, const pkv_prefix_groups* groups, float sm_scale, void* out,
                              float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  pkv::DevMap dm;
  if (int st = make_devmap(pool, map, false, &dm)) return st;
  if (num_q_heads <= 0) return fail(PKV_EINVAL, "num_q_heads must be positive");
  if (int st = check_groups(pool, num_q_heads, groups)) return st;
  if (!(sm_scale > 0.0f) || std::isinf(sm_scale)) return fail(PKV_EINVAL, "sm_scale must be positive and finite");
  if (map->bs == 0) return ok();
  if (!q || !out) return fail(PKV_EINVAL, "null q or out");
  if (!aligned16(q)) return fail(PKV_EALIGN, "q must be 16-byte aligned");
  const pkv::CascadePlan cp = pkv::plan_cascade(pool->info, map->bs, num_q_heads, map->max_kv_len,
                                                groups->num_groups, groups->max_group_size, groups->max_prefix_len);
  if (cp.cap > INT32_MAX) return fail(PKV_EUNSUPPORTED, "too many prefix work items (%lld)", (long long)cp.cap);
  const size_t need = pkv::cascade_ws_layout(pool->info, cp, map->bs, num_q_heads, nullptr, nullptr);
  if (ws_bytes < need) return fail(PKV_ECAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(PKV_EALIGN, "workspace must be non-null and 256-byte aligned");
  return device_status(pkv::launch_decode_cascade(pool->info, layer, q, num_q_heads, dm, map->bs, cp,
                                                  groups->group_indptr, groups->prefix_len, groups->num_groups,
                                                  sm_scale, out, lse, workspace, (hipStream_t)stream),
                       "paged_decode_attn_cascade");
}

}  // extern "C"

namespace {
// paged_verify_attn with an optional append of the drafts' K rows (st.n ==
// 0: none), checked before anything is launched.
int verify_call(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads, int32_t num_draft,
                const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                void* stream, const pkv::StoreArgs& st, const char* what) {
  pkv::DevMap dm;
  if (int e = make_devmap(pool, map, false, &dm)) return e;
  if (num_q_heads <= 0 || num_draft <= 0) return fail(PKV_EINVAL, "num_q_heads and num_draft must be positive");
  if (!(sm_scale > 0.0f) || std::isinf(sm_scale)) return fail(PKV_EINVAL, "sm_scale must be positive and finite");
  const int64_t rows = (int64_t)num_q_heads * num_draft;
  if (pool->desc.kind != PKV_KIND_LATENT || rows > 1024 || !pkv::decode_supported(pool->info, (int32_t)rows))
    return fail(PKV_EUNSUPPORTED,
                "target verification needs a latent bf16 576/512 pool and num_draft * num_q_heads in {16, 32, 64} "
                "or a multiple of 128 up to 1024 (got %d x %d)", num_draft, num_q_heads);
  if (map->bs == 0) {
    if (st.n == 0) return ok();
    return device_status(pkv::launch_store_args(st, (hipStream_t)stream), what);
  }
  if (!q || !out) return fail(PKV_EINVAL, "null q or out");
  if (!aligned16(q)) return fail(PKV_EALIGN, "q must be 16-byte aligned");
  const pkv::DecodePlan plan = pkv::plan_decode(pool->info, map->bs, (int32_t)rows, map->max_kv_len);
  const size_t need = pkv::decode_workspace_bytes(pool->info, plan, map->bs, (int32_t)rows);
  if (ws_bytes < need) return fail(PKV_ECAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return fail(PKV_EALIGN, "workspace must be non-null and 256-byte aligned");
  return device_status(pkv::launch_mla_verify(pool->info, layer, q, (int32_t)rows, num_draft, dm, map->bs, plan,
                                              sm_scale * pkv::kLog2e, out, lse, workspace, (hipStream_t)stream,
                                              st.n > 0 ? &st : nullptr),
                       what);
}
}  // namespace

extern "C" {

int paged_verify_attn(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads, int32_t num_draft,
                      const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                      void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  pkv::StoreArgs none{};
  return verify_call(pool, layer, q, num_q_heads, num_draft, map, sm_scale, out, lse, workspace, ws_bytes, stream,
                     none, "paged_verify_attn");
}

int paged_verify_attn_append(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                             int32_t num_draft, const pkv_kv_map* map, const void* k_new, const int32_t* out_loc,
                             int64_t n_new, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  const void* v_new = nullptr;  // a latent pool keeps one row per token
  if (pool->desc.kind == PKV_KIND_LATENT)
    if (int st = check_store(pool, k_new, &v_new, out_loc, n_new)) return st;
  const pkv::StoreArgs sa = pkv::make_store_args(pool->info, layer, k_new, nullptr, out_loc,
                                                 pool->desc.kind == PKV_KIND_LATENT ? n_new : 0);
  return verify_call(pool, layer, q, num_q_heads, num_draft, map, sm_scale, out, lse, workspace, ws_bytes, stream,
                     sa, "paged_verify_attn_append");
}

namespace {
int extend_call(const char* call, const pkv_pool* pool, int32_t layer, const void* q, int64_t total_q,
                const int32_t* qo_indptr, int32_t num_q_heads, int32_t max_q_len, const pkv_kv_map* map,
                int32_t causal, const int32_t* causal_flags, float softcap, float sm_scale, void* out, float* lse,
                void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  pkv::DevMap dm;
  if (int st = make_devmap(pool, map, true, &dm)) return st;
  if (num_q_heads <= 0 || num_q_heads % pool->desc.num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads %d not a positive multiple of num_kv_heads %d", num_q_heads,
                pool->desc.num_kv_heads);
  if (max_q_len < 0 || total_q < 0) return fail(PKV_EINVAL, "negative max_q_len or total_q");
  if (!(sm_scale > 0.0f) || std::isinf(sm_scale)) return fail(PKV_EINVAL, "sm_scale must be positive and finite");
  if (!(softcap >= 0.0f) || std::isinf(softcap))
    return fail(PKV_EINVAL, "softcap must be 0 (off) or positive and finite");
  if (!pkv::extend_supported(pool->info, num_q_heads))
    return fail(PKV_EUNSUPPORTED, "no extend kernel for this pool (dtype %d, dims %d/%d)", pool->desc.dtype,
                pool->desc.head_dim_qk, pool->desc.head_dim_v);
  if (map->bs == 0 || max_q_len == 0 || total_q == 0) return ok();
  if (!q || !out || !qo_indptr) return fail(PKV_EINVAL, "null q, out or qo_indptr");
  if (!aligned16(q)) return fail(PKV_EALIGN, "q must be 16-byte aligned");
  return device_status(pkv::launch_extend(pool->info, layer, q, total_q, qo_indptr, num_q_heads, max_q_len, dm, map->bs,
                                          map->max_kv_len, causal, causal_flags, softcap, sm_scale, out, lse,
                                          (hipStream_t)stream),
                       call);
}
}  // namespace

int paged_extend_attn(const pkv_pool* pool, int32_t layer, const void* q, int64_t total_q, const int32_t* qo_indptr,
                      int32_t num_q_heads, int32_t max_q_len, const pkv_kv_map* map, int32_t causal, float sm_scale,
                      void* out, float* lse, void* stream) {
  return extend_call("paged_extend_attn", pool, layer, q, total_q, qo_indptr, num_q_heads, max_q_len, map, causal,
                     nullptr, 0.0f, sm_scale, out, lse, stream);
}

int paged_extend_attn_ex(const pkv_pool* pool, int32_t layer, const void* q, int64_t total_q,
                         const int32_t* qo_indptr, int32_t num_q_heads, int32_t max_q_len, const pkv_kv_map* map,
                         const pkv_extend_opts* opts, float sm_scale, void* out, float* lse, void* stream) {
  if (!opts) return fail(PKV_EINVAL, "null extend options");
  return extend_call("paged_extend_attn_ex", pool, layer, q, total_q, qo_indptr, num_q_heads, max_q_len, map,
                     opts->causal, opts->causal_flags, opts->softcap, sm_scale, out, lse, stream);
}

int kv_gather(const pkv_pool* pool, int32_t layer, const pkv_kv_map* map, const int32_t* cu_seqlens_k, void* k_out,
              void* v_out, int64_t out_rows, void* stream) {
  if (int st = check_pool(pool)) return st;
  if (int st = check_layer(pool, layer)) return st;
  pkv::DevMap dm;
  if (int st = make_devmap(pool, map, false, &dm)) return st;
  if (out_rows < 0) return fail(PKV_EINVAL, "negative out_rows");
  if (map->bs == 0) return ok();
  if (!cu_seqlens_k || !k_out) return fail(PKV_EINVAL, "null cu_seqlens_k or k_out");
  if (pool->desc.kind == PKV_KIND_SPLIT_KV && !v_out) return fail(PKV_EINVAL, "null v_out for a split K/V pool");
  if (pool->desc.kind == PKV_KIND_LATENT) v_out = nullptr;
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(PKV_EALIGN, "k_out/v_out must be 16-byte aligned");
  return device_status(pkv::launch_gather(pool->info, layer, dm, map->bs, map->max_kv_len, cu_seqlens_k, k_out, v_out,
                                          out_rows, (hipStream_t)stream),
                       "kv_gather");
}

int kv_free_list_init(int32_t* free_pages, int32_t capacity, int32_t first, int32_t count, int32_t* free_state,
                      void* stream) {
  if (!free_pages || !free_state) return fail(PKV_EINVAL, "null free list or state");
  if (capacity <= 0 || count < 0 || first < 0) return fail(PKV_EINVAL, "capacity must be positive, count and first >= 0");
  if (count > capacity) return fail(PKV_ECAPACITY, "count %d > capacity %d", count, capacity);
  if ((int64_t)first + count > INT32_MAX) return fail(PKV_EINVAL, "page ids past INT32_MAX");
  return device_status(pkv::launch_free_list_init(free_pages, first, count, free_state, (hipStream_t)stream),
                       "kv_free_list_init");
}

namespace {
int check_ring(int32_t page_size, const int32_t* free_pages, int32_t capacity, const int32_t* free_state,
               const int32_t* status) {
  if (!pow2(page_size) || page_size > 128) return fail(PKV_EUNSUPPORTED, "page_size %d", page_size);
  if (!free_pages || !free_state || !status) return fail(PKV_EINVAL, "null free list, state or status");
  if (capacity <= 0) return fail(PKV_EINVAL, "free list capacity must be positive");
  return ok();
}
}  // namespace

int kv_alloc(int32_t page_size, int64_t need, int32_t* free_pages, int32_t capacity, int32_t* free_state,
             int32_t* out, int32_t* status, void* stream) {
  if (int st = check_ring(page_size, free_pages, capacity, free_state, status)) return st;
  if (need < 0 || need % page_size != 0)
    return fail(PKV_EINVAL, "need %lld is not a non-negative multiple of page_size %d", (long long)need, page_size);
  if (need > INT32_MAX) return fail(PKV_EINVAL, "need %lld past INT32_MAX", (long long)need);
  if (need > 0 && !out) return fail(PKV_EINVAL, "null out");
  return device_status(pkv::launch_alloc_pages(ilog2(page_size), need / page_size, free_pages, capacity, free_state,
                                               out, status, (hipStream_t)stream),
                       "kv_alloc");
}

namespace {
int alloc_growth(const char* call, int32_t page_size, int32_t bs, const int32_t* prefix_lens, const int32_t* seq_lens,
                 const int32_t* last_loc, int32_t* free_pages, int32_t capacity, int32_t* free_state,
                 int32_t* out_cache_loc, int64_t out_capacity, int32_t* status, void* stream) {
  if (int st = check_ring(page_size, free_pages, capacity, free_state, status)) return st;
  if (bs < 0 || out_capacity < 0) return fail(PKV_EINVAL, "negative bs or out_capacity");
  if (bs > pkv::kMaxAllocBatch) return fail(PKV_EUNSUPPORTED, "bs %d > %d", bs, pkv::kMaxAllocBatch);
  if (out_capacity > INT32_MAX) return fail(PKV_EINVAL, "out_capacity past INT32_MAX");
  if (bs > 0 && (!seq_lens || !out_cache_loc)) return fail(PKV_EINVAL, "null seq_lens or out_cache_loc");
  if (bs > 0 && page_size > 1 && !last_loc) return fail(PKV_EINVAL, "page_size > 1 needs last_loc");
  return device_status(pkv::launch_alloc_extend(ilog2(page_size), bs, prefix_lens, seq_lens, last_loc, free_pages,
                                                capacity, free_state, out_cache_loc, out_capacity, status,
                                                (hipStream_t)stream),
                       call);
}
}  // namespace

int kv_alloc_extend(int32_t page_size, int32_t bs, const int32_t* prefix_lens, const int32_t* seq_lens,
                    const int32_t* last_loc, int32_t* free_pages, int32_t capacity, int32_t* free_state,
                    int32_t* out_cache_loc, int64_t out_capacity, int32_t* status, void* stream) {
  if (bs > 0 && !prefix_lens) return fail(PKV_EINVAL, "null prefix_lens");
  return alloc_growth("kv_alloc_extend", page_size, bs, prefix_lens, seq_lens, last_loc, free_pages, capacity,
                      free_state, out_cache_loc, out_capacity, status, stream);
}

int kv_alloc_decode(int32_t page_size, int32_t bs, const int32_t* seq_lens, const int32_t* last_loc,
                    int32_t* free_pages, int32_t capacity, int32_t* free_state, int32_t* out_cache_loc,
                    int32_t* status, void* stream) {
  return alloc_growth("kv_alloc_decode", page_size, bs, nullptr, seq_lens, last_loc, free_pages, capacity, free_state,
                      out_cache_loc, bs, status, stream);
}

int kv_free(int32_t page_size, const int32_t* slots, int64_t n, int32_t num_pages, int32_t* free_pages,
            int32_t capacity, int32_t* free_state, uint32_t* page_bitmap, int32_t* status, void* stream) {
  if (int st = check_ring(page_size, free_pages, capacity, free_state, status)) return st;
  if (n < 0 || num_pages <= 0) return fail(PKV_EINVAL, "negative n or non-positive num_pages");
  if (n > 0 && !slots) return fail(PKV_EINVAL, "null slots");
  if (!page_bitmap) return fail(PKV_EINVAL, "null page_bitmap");
  return device_status(pkv::launch_free(ilog2(page_size), slots, n, num_pages, free_pages, capacity, free_state,
                                        page_bitmap, status, (hipStream_t)stream),
                       "kv_free");
}

int write_req_to_token(int32_t* req_to_token, int64_t table_rows, int64_t table_width,
                       const int32_t* req_pool_indices, const int32_t* prefix_lens, const int32_t* seq_lens,
                       const int32_t* out_cache_loc, int64_t n_out, const int32_t* const* prefix_ptrs, int32_t bs,
                       int32_t max_seq_len, void* stream) {
  if (bs < 0 || max_seq_len < 0 || n_out < 0) return fail(PKV_EINVAL, "negative bs, max_seq_len or n_out");
  if (table_rows <= 0 || table_width <= 0) return fail(PKV_EINVAL, "token table dims must be positive");
  if (bs > 0 && (!req_to_token || !req_pool_indices || !prefix_lens || !seq_lens))
    return fail(PKV_EINVAL, "null table, indices or lengths");
  if (n_out > 0 && !out_cache_loc) return fail(PKV_EINVAL, "null out_cache_loc");
  if (max_seq_len > table_width) return fail(PKV_EINVAL, "max_seq_len %d > table_width %lld", max_seq_len,
                                             (long long)table_width);
  if (((int64_t)max_seq_len + 1023) / 1024 > 65535) return fail(PKV_EUNSUPPORTED, "max_seq_len %d", max_seq_len);
  return device_status(pkv::launch_write_rows(req_to_token, table_rows, table_width, req_pool_indices, prefix_lens,
                                              seq_lens, out_cache_loc, n_out, prefix_ptrs, bs, max_seq_len,
                                              (hipStream_t)stream),
                       "write_req_to_token");
}

int kv_validate(const pkv_pool* pool, const pkv_kv_map* map, const int32_t* is_dummy, int64_t* scratch,
                int64_t counts[8], void* stream) {
  if (int st = check_pool(pool)) return st;
  pkv::DevMap dm;
  if (int st = make_devmap(pool, map, false, &dm)) return st;
  if (!counts) return fail(PKV_EINVAL, "null counts");
  for (int k = 0; k < 8; ++k) counts[k] = 0;
  if (map->bs == 0) return ok();
  if (!scratch) return fail(PKV_EINVAL, "null scratch");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = pkv::launch_validate(pool->info, dm, map->bs, map->max_kv_len, is_dummy,
                                      reinterpret_cast<long long*>(scratch), s);
  if (e != hipSuccess) return device_status(e, "kv_validate launch");
  const size_t n = (size_t)map->bs * 8;
  long long* host = new (std::nothrow) long long[n];
  if (!host) return fail(PKV_EINVAL, "out of host memory");
  e = hipMemcpyAsync(host, scratch, n * sizeof(long long), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete[] host;
    return device_status(e, "kv_validate copy");
  }
  for (size_t r = 0; r < (size_t)map->bs; ++r)
    for (int k = 0; k < 8; ++k) counts[k] += host[r * 8 + k];
  delete[] host;
  bool any = false, only_align = true;
  for (int k = 0; k < 8; ++k) {
    if (counts[k]) {
      any = true;
      if (k != 3) only_align = false;
    }
  }
  if (!any) return ok();
  if (only_align) return fail(PKV_EALIGN, "kv_start not a multiple of page_size for %lld requests", (long long)counts[3]);
  return fail(PKV_EINVAL, "map violations: range %lld, padding %lld, neg %lld, align %lld, contig %lld, len %lld",
              (long long)counts[0], (long long)counts[1], (long long)counts[2], (long long)counts[3],
              (long long)counts[4], (long long)counts[5]);
}

namespace {
int check_enc_geometry(int32_t num_blocks, int32_t block_size, int64_t row_bytes) {
  if (num_blocks <= 0 || block_size <= 0) return fail(PKV_EINVAL, "num_blocks and block_size must be positive");
  if (row_bytes <= 0 || row_bytes % 16 != 0) return fail(PKV_EALIGN, "row_bytes must be a positive multiple of 16");
  return ok();
}
}  // namespace

int enc_cache_write(void* buffer, int32_t num_blocks, int32_t block_size, int64_t row_bytes, const void* src,
                    int32_t n, const int32_t* block_ids, void* stream) {
  if (int st = check_enc_geometry(num_blocks, block_size, row_bytes)) return st;
  if (n < 0) return fail(PKV_EINVAL, "negative n");
  if (n == 0) return ok();
  if (!buffer || !src || !block_ids) return fail(PKV_EINVAL, "null buffer, src or block_ids");
  if (!aligned16(buffer) || !aligned16(src)) return fail(PKV_EALIGN, "buffer and src must be 16-byte aligned");
  if ((int64_t)n * block_size > INT32_MAX) return fail(PKV_EUNSUPPORTED, "too many rows in one call");
  return device_status(pkv::launch_enc_write(static_cast<char*>(buffer), num_blocks, block_size, row_bytes / 16,
                                             static_cast<const char*>(src), n, block_ids, (hipStream_t)stream),
                       "enc_cache_write");
}

int enc_cache_merge(const void* buffer, int32_t num_blocks, int32_t block_size, int64_t row_bytes,
                    const int32_t* block_ids, int32_t max_blocks, const int64_t* positions, void* hidden,
                    int64_t num_tokens, int32_t* fill_count, void* stream) {
  if (int st = check_enc_geometry(num_blocks, block_size, row_bytes)) return st;
  if (max_blocks < 0 || num_tokens < 0) return fail(PKV_EINVAL, "negative max_blocks or num_tokens");
  if (max_blocks == 0) return ok();
  if (!buffer || !block_ids || !positions || (num_tokens > 0 && !hidden))
    return fail(PKV_EINVAL, "null buffer, block_ids, positions or hidden");
  if (!aligned16(buffer) || !aligned16(hidden)) return fail(PKV_EALIGN, "buffer and hidden must be 16-byte aligned");
  if ((int64_t)max_blocks * block_size > INT32_MAX) return fail(PKV_EUNSUPPORTED, "too many rows in one call");
  return device_status(pkv::launch_enc_merge(static_cast<const char*>(buffer), num_blocks, block_size, row_bytes / 16,
                                             block_ids, max_blocks, positions, static_cast<char*>(hidden),
                                             num_tokens, fill_count, (hipStream_t)stream),
                       "enc_cache_merge");
}

int enc_cache_check(const int32_t* fill_count, const int32_t* scheduled, int64_t num_tokens, int64_t* scratch,
                    int64_t counts[2], void* stream) {
  if (!counts) return fail(PKV_EINVAL, "null counts");
  counts[0] = counts[1] = 0;
  if (num_tokens < 0) return fail(PKV_EINVAL, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!fill_count || !scratch) return fail(PKV_EINVAL, "null fill_count or scratch");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = pkv::launch_enc_check(fill_count, scheduled, num_tokens, reinterpret_cast<long long*>(scratch), s);
  if (e != hipSuccess) return device_status(e, "enc_cache_check launch");
  long long host[2] = {0, 0};
  e = hipMemcpyAsync(host, scratch, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_status(e, "enc_cache_check copy");
  counts[0] = host[0];
  counts[1] = host[1];
  if (host[0] == 0 && host[1] == 0) return ok();
  return fail(PKV_EINVAL, "encoder positions: %lld scheduled rows unfilled, %lld rows filled more than once",
              host[0], host[1]);
}

int pkv_set_kernel_timer(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return fail(PKV_EINVAL, "pass both events or neither");
  g_timer_start = static_cast<hipEvent_t>(start_event);
  g_timer_stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

}  // extern "C"
