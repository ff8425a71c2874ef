// Host-side launch interface between the C ABI (pkv_api.hip) and the kernel
// translation units.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

// Everything a launcher needs to know about the pool, resolved once by
// kv_pool_create.
struct PoolInfo {
  int32_t num_layers, num_pages, page_size, page_shift;
  int32_t num_kv_heads, head_dim_qk, head_dim_v;
  int32_t dtype;  // 0 f32, 1 bf16
  int32_t kind;   // 0 split K/V, 1 latent
  int32_t elem_bytes;
  char* k_base;
  char* v_base;  // null for latent
  int64_t num_slots;   // (num_pages + 1) * page_size
  int64_t pad_slot;    // num_pages * page_size
  int64_t k_row_bytes;  // one token, all KV heads
  int64_t v_row_bytes;
  int64_t k_layer_bytes;
  int64_t v_layer_bytes;

  const char* k_layer(int32_t layer) const { return k_base + (int64_t)layer * k_layer_bytes; }
  const char* v_layer(int32_t layer) const { return v_base ? v_base + (int64_t)layer * v_layer_bytes : nullptr; }
};

// Kernel timer hook (pkv_set_kernel_timer): launchers call these around the
// main attention kernel.
void timer_before(hipStream_t s);
void timer_after(hipStream_t s);

hipError_t launch_store(const PoolInfo& p, int32_t layer, const void* k, const void* v, const int32_t* out_loc,
                        int64_t n, hipStream_t s);

// A KV append carried by another launch (the decode planner runs it in
// blocks of its own: the planner reads only tables, so the two are
// independent, and the attention kernel after them reads the stored rows).
struct StoreArgs {
  char* k_dst;
  char* v_dst;  // null for a latent pool
  const char* k_src;
  const char* v_src;
  const int32_t* out_loc;
  int64_t n;  // rows; 0: nothing to store
  int64_t num_slots;
  int32_t k_units, v_units;  // 16-byte units per row
};
StoreArgs make_store_args(const PoolInfo& p, int32_t layer, const void* k, const void* v, const int32_t* out_loc,
                          int64_t n);
constexpr int kStoreRowsPerBlock = 4;  // one wavefront per row, 256-thread blocks
hipError_t launch_store_args(const StoreArgs& a, hipStream_t s);  // the append on its own

// Row `row` of a store, by one wavefront (lanes stride over its 16-byte
// units); slots outside the pool are skipped.
__device__ __forceinline__ void store_one_row(const StoreArgs& a, int64_t row, int lane) {
  if (row >= a.n) return;
  const int64_t slot = a.out_loc[row];
  if (slot < 0 || slot >= a.num_slots) return;
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.k_src) + row * a.k_units;
    u32x4* dst = reinterpret_cast<u32x4*>(a.k_dst) + slot * a.k_units;
    for (int c = lane; c < a.k_units; c += 64) dst[c] = src[c];
  }
  if (a.v_dst) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.v_src) + row * a.v_units;
    u32x4* dst = reinterpret_cast<u32x4*>(a.v_dst) + slot * a.v_units;
    for (int c = lane; c < a.v_units; c += 64) dst[c] = src[c];
  }
}

hipError_t launch_gather(const PoolInfo& p, int32_t layer, const DevMap& m, int32_t bs, int32_t max_kv_len,
                         const int32_t* cu_seqlens_k, void* k_out, void* v_out, int64_t out_rows, hipStream_t s);

hipError_t launch_build_indices(int32_t out_fmt, const int32_t* req_to_token, int64_t table_rows,
                                int64_t table_width, const int32_t* req_pool_indices, const int32_t* kv_start,
                                const int32_t* kv_lens, int32_t bs, int32_t page_shift, int32_t* kv_indptr,
                                int32_t* out, int64_t capacity, int32_t* kv_last_page_len, hipStream_t s);

// Split plan for decode: chunk of logical tokens per split and the number
// of split slots reserved per request in the workspace.
struct DecodePlan {
  int32_t chunk;
  int32_t max_splits;
  int32_t kind;  // which kernel family
};

constexpr int kMaxSplits = 1024;  // per request

// One live (request, split) of a decode launch, written by the planner
// kernel: what a split needs to start streaming at once.
struct __attribute__((aligned(16))) WorkItem {
  int32_t i;      // request
  int32_t s;      // split
  int32_t ns;     // splits of request i (0: empty request)
  int32_t t_end;  // exclusive end of the split's keys (it starts at s * chunk)
  int32_t limit;  // readable table entries (0: malformed row, read as padding)
  int32_t off_lo, off_hi;  // element offset of the request's table row / page list
  int32_t pad;
};

__device__ __forceinline__ ReqView item_view(const WorkItem& w) {
  ReqView v;
  v.off = ((int64_t)w.off_hi << 32) | (uint32_t)w.off_lo;
  v.limit = w.limit;
  return v;
}

// decode workspace: [item count | items[bs * max_splits] | partial o | partial lse]
struct DecodeWs {
  int32_t* count;
  WorkItem* items;
  float* o;
  float* lse;
};
size_t decode_ws_layout(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t Hq, void* base, DecodeWs* w);

bool mla_decode_supported(const PoolInfo& p, int32_t num_q_heads);
// Rows one MLA main-kernel launch covers (more run as consecutive slices).
int32_t mla_slice_rows(int32_t num_q_heads);
// MLA plan: chunk = tiles (32 tokens) per request at most, max_splits = main
// grid (one workgroup per CU)
DecodePlan plan_mla_decode(const PoolInfo& p, int32_t bs, int32_t num_q_heads, int32_t max_kv_len);
// Stream-split decode (pkv_stream.hip): tiles of kStreamT logical positions
// laid end to end and cut into equal runs; per tile the planner writes
// kStreamMetaWords words: 32 slot ids + {request, tile, tiles of request,
// tile prefix, valid keys, 0, 0, 0}.
constexpr int kStreamT = 32;
constexpr int kStreamMetaWords = 40;
struct StreamWs {
  int32_t* header;    // run length (tiles per run), total tiles
  int32_t* prefix;    // per request: first tile
  int32_t* ntiles;    // per request: tiles
  int32_t* fallback;  // requests to recompute exactly (set by a main kernel)
  int32_t* meta;
  float* o;           // pieces: [(runs + bs)][Hq][Dv], id run + request
  float* lse;
};
size_t stream_ws_layout(int32_t bs, int32_t max_tiles, int32_t runs, int32_t Hq, int32_t Dv, void* base,
                        StreamWs* w);
// One work item of a shared-prefix pass: members [i0, i1) of one group
// against tiles [t0, t1) of the prefix keys [0, E), read through member
// ref's table; its partial results go to chunk slot c.  i0 < 0: no work.
// The planner also stores ref's table view (row offset, readable entries),
// so a work item reaches its table entries with no lookup of its own.
struct __attribute__((aligned(16))) PrefixItem {
  int32_t i0, i1, ref, E, t0, t1, c, limit;
  int32_t off_lo, off_hi, pad0, pad1;
};

__device__ __forceinline__ ReqView prefix_item_view(const PrefixItem& it) {
  ReqView v;
  v.off = ((int64_t)it.off_hi << 32) | (uint32_t)it.off_lo;
  v.limit = it.limit;
  return v;
}

// Shared prefixes found by paged_decode_attn itself (share_detect_kernel):
// per request the keys it shares with its group's reference member (s >= 0),
// or -1 for the reference, and the group's bounds; the planner turns them
// into each request's skip and the prefix pass's work items.
struct ShareArgs {
  const int32_t* s;   // [bs]: shared keys (a multiple of the tile, or the whole request), -1: reference
  const int32_t* gs;  // [bs]: first member of the request's group
  const int32_t* ge;  // [bs]: one past its last member
  int32_t* skip;      // out [bs]: keys the prefix pass covers (0: none)
  PrefixItem* items;  // out: the prefix pass's work, group after group in batch order
  int32_t* count;     // out [1]: items listed
  int32_t ms;         // members per slice
  int32_t ch;         // chunks of a group's prefix
};

// skip (nullable, device int32[bs]): keys left out at the start of each
// request, a multiple of kStreamT (cascade decode reads them elsewhere).
// st (nullable): a KV append run by extra blocks of the same launch.
// share (nullable): shared prefixes found by the decode itself; the planner
// computes each request's skip from them (and writes it and the prefix
// pass's work items).
hipError_t launch_stream_plan(const DevMap& m, int32_t bs, int32_t max_tiles, int32_t runs, const StreamWs& w,
                              hipStream_t s, const int32_t* skip = nullptr, const StoreArgs* st = nullptr,
                              const ShareArgs* share = nullptr);
int32_t device_cu_count();
hipError_t launch_mla_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t num_q_heads, const DevMap& m,
                             int32_t bs, const DecodePlan& plan, float scale_log2, void* out, float* lse, void* ws,
                             hipStream_t s, const StoreArgs* st = nullptr);
// Target verification over a latent pool: n_draft query tokens per request,
// folded into Hq = n_draft * heads rows, bottom-right causal among the drafts.
hipError_t launch_mla_verify(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, int32_t n_draft,
                             const DevMap& m, int32_t bs, const DecodePlan& plan, float sl2, void* out, float* lse,
                             void* ws, hipStream_t s, const StoreArgs* st = nullptr);
DecodePlan plan_decode(const PoolInfo& p, int32_t bs, int32_t num_q_heads, int32_t max_kv_len);
size_t decode_workspace_bytes(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t num_q_heads);
bool decode_supported(const PoolInfo& p, int32_t num_q_heads);

// st (nullable): the step's KV append, stored before the attention reads
// the pool (inside the planner launch where there is one).
hipError_t launch_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t num_q_heads, const DevMap& m,
                         int32_t bs, const DecodePlan& plan, float sm_scale, void* out, float* lse, void* ws,
                         hipStream_t s, const StoreArgs* st = nullptr);

// Cascade decode over shared prefixes (pkv_decode.hip): the stream decode of
// each request's own keys plus one pass per group over the shared ones.
struct CascadePlan {
  DecodePlan dp;   // the stream plan of the own (suffix) keys
  int32_t ms;      // members per slice (32 query rows per wave)
  int32_t slices;  // slices per group, at most
  int32_t chunks;  // prefix chunks per group
  int64_t cap;     // prefix work items, at most: groups x slices x chunks (at least 1)
};
struct CascadeWs {
  StreamWs stream;
  int32_t* skip;       // per request: keys read by the prefix pass
  int32_t* count;      // prefix work items listed
  PrefixItem* items;   // [cap]
  float* po;           // prefix partials [chunks][bs][Hq][Dv]
  float* plse;         // [chunks][bs][Hq]
};
CascadePlan plan_cascade(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len, int32_t num_groups,
                         int32_t max_group_size, int32_t max_prefix_len);
size_t cascade_ws_layout(const PoolInfo& p, const CascadePlan& cp, int32_t bs, int32_t Hq, void* base,
                         CascadeWs* w);
hipError_t launch_decode_cascade(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m,
                                 int32_t bs, const CascadePlan& cp, const int32_t* group_indptr,
                                 const int32_t* prefix_len, int32_t num_groups, float sm_scale, void* out, float* lse,
                                 void* ws, hipStream_t s);

bool extend_supported(const PoolInfo& p, int32_t num_q_heads);
hipError_t launch_extend(const PoolInfo& p, int32_t layer, const void* q, int64_t total_q, const int32_t* qo_indptr,
                         int32_t num_q_heads, int32_t max_q_len, const DevMap& m, int32_t bs, int32_t max_kv_len,
                         int32_t causal, const int32_t* causal_flags, float softcap, float sm_scale, void* out,
                         float* lse, hipStream_t s);

hipError_t launch_validate(const PoolInfo& p, const DevMap& m, int32_t bs, int32_t max_kv_len,
                           const int32_t* is_dummy, long long* counts_dev, hipStream_t s);

}  // namespace pkv
