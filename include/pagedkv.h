/*
 * pagedkv.h -- C ABI of the paged KV-cache hot path for AMD MI355X (gfx950).
 *
 * Attention that reads keys and values through a page table out of one
 * shared, preallocated, paged KV pool: the pool geometry, the KV append
 * (scatter of new tokens' K/V into their slots), index building (token table
 * -> page-granular CSR or padded block table), paged decode attention
 * (split-K over pages with a log-sum-exp merge), paged extend/prefill over a
 * paged prefix, and the ragged gather; plus the device-side slot
 * allocator (a free list of pages) and the writing of request rows.
 *
 * Sources, cited by short name:
 *   [XPU]     "Enabling Encoder-Decoder Models on Intel XPU in SGLang: A KV-Cache Story"
 *   [OMNI]    "Scheduler-Managed Paged KV Cache" (vLLM-Omni design documents)
 *   [MINI]    "The KV pool, the page table and the token pool" (mini-sglang from Scratch)
 *   [BACKEND] "AttentionBackend" (SGLang FlashInfer-MLA / FlashMLA backend notes)
 *
 * Conventions for every call:
 *   - Ownership: the library allocates no device memory and frees none.  The
 *     caller owns the pool buffers, tables, outputs and workspace, and keeps
 *     them alive until the work queued on `stream` has finished.  The only
 *     object the library owns is the immutable host-side pool handle.
 *   - Execution: every call that launches work is asynchronous on `stream`
 *     (a hipStream_t; NULL = the default stream) and never synchronises the
 *     host.  Host-known maxima (max_kv_len, max_q_len, capacities) are passed
 *     in by the caller.
 *   - Pointers named "device" must point to device (or managed) memory;
 *     "host" pointers are read before the call returns.
 *   - Errors: each call returns 0 (PKV_OK) or a negative status; no C++
 *     exception crosses this boundary; nothing falls back silently.  The
 *     message of the last failing call on the calling thread is
 *     pkv_last_error().
 *   - Index contents (slots, page ids, lengths) live in device memory and are
 *     not validated on the hot path; every kernel range-checks what it reads
 *     and treats an out-of-range entry as the padding slot, so a corrupt
 *     table gives an unspecified result but no out-of-bounds access.
 *     kv_validate() checks contents (off the hot path, synchronising).
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

/* status codes */
#define PKV_OK 0
#define PKV_EINVAL (-1)       /* null/negative argument, or dims inconsistent with the pool */
#define PKV_EUNSUPPORTED (-2) /* page_size, head_dim, dtype or head grouping not instantiated */
#define PKV_EALIGN (-3)       /* base pointer not 16-byte aligned; kv_start not page aligned */
#define PKV_ECAPACITY (-4)    /* output capacity or workspace too small */
#define PKV_EDEVICE (-5)      /* HIP launch/runtime error (details in pkv_last_error) */

/* element types */
#define PKV_DTYPE_F32 0
#define PKV_DTYPE_BF16 1

/* pool kinds */
#define PKV_KIND_SPLIT_KV 0 /* separate K and V buffers */
#define PKV_KIND_LATENT 1   /* one buffer; V is the first head_dim_v values of each K row (MLA) */

/* KV map formats */
#define PKV_MAP_TOKEN_TABLE 0 /* token-granular req_to_token rows ([XPU] "two pools"; [MINI] page table) */
#define PKV_MAP_CSR 1         /* kv_indptr / kv_indices page ids ([BACKEND] "kv_indptr 和 kv_indices") */
#define PKV_MAP_BLOCK_TABLE 2 /* [bs, block_stride] page ids padded with -1 ([BACKEND] init_forward_metadata) */
#define PKV_MAP_CONTIGUOUS 3  /* gathered K/V addressed by cu_seqlens_k ([XPU] "Approach 2") */

/*
 * Pool geometry ([MINI] "The KV pool: one preallocated block of memory";
 * [XPU] "two pools and a page size").  Each buffer is laid out
 *   [num_layers][num_pages + 1][page_size][num_kv_heads][head_dim]
 * (row-major, token-major inside a page), so that one layer's buffer viewed
 * per token is [(num_pages + 1) * page_size][num_kv_heads][head_dim] and
 * slot s lives at page s / page_size, offset s % page_size.  Page num_pages
 * is the padding page: dummy requests of a padded batch read and write it,
 * real requests never do ([MINI] "Why the extra page?").
 *   page_size: a power of two, 1..128.
 *   head_dim_qk / head_dim_v: K row and V row lengths.  SPLIT_KV requires
 *     head_dim_qk == head_dim_v; LATENT requires head_dim_v <= head_dim_qk.
 */
typedef struct pkv_pool_desc {
  int32_t num_layers;
  int32_t num_pages; /* real pages */
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t dtype; /* PKV_DTYPE_* */
  int32_t kind;  /* PKV_KIND_* */
} pkv_pool_desc;

typedef struct pkv_pool pkv_pool; /* opaque, immutable host-side handle */

/*
 * Where each request's keys live (one attention call's view).
 *   bs          requests in the batch.
 *   kv_lens     device int32[bs]: keys request i attends over, including the
 *               tokens appended this step.
 *   max_kv_len  host bound >= every kv_lens[i] (sizes the launch).
 * TOKEN_TABLE: req_to_token device int32[table_rows][table_width] (row
 *   stride = table_width) holding slots; req_pool_indices device int32[bs]
 *   picks each request's row; kv_start device int32[bs] (NULL = all 0) is the
 *   first column of the region (e.g. the decoder region of an
 *   encoder-decoder row, [XPU] "two KV regions in one row").  Works for
 *   every page size: slot(t) = row[kv_start + t].
 * CSR: kv_indptr device int32[bs+1], kv_indices device int32[kv_indices_len]
 *   of page ids; slot(t) = kv_indices[kv_indptr[i] + t/ps]*ps + t%ps.
 * BLOCK_TABLE: block_table device int32[bs][block_stride] of page ids,
 *   -1 past each request's last page.
 * CONTIGUOUS: k, v device buffers [total_k][num_kv_heads][head_dim]
 *   (v ignored for a LATENT pool) and cu_seqlens_k device int32[bs+1];
 *   request i's keys are rows cu_seqlens_k[i] .. + kv_lens[i].
 */
typedef struct pkv_kv_map {
  int32_t fmt;
  int32_t bs;
  const int32_t* kv_lens;
  int32_t max_kv_len;
  const int32_t* req_to_token;
  int64_t table_rows;
  int64_t table_width;
  const int32_t* req_pool_indices;
  const int32_t* kv_start;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int64_t kv_indices_len;
  const int32_t* block_table;
  int64_t block_stride;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens_k;
  int64_t total_k;
} pkv_kv_map;

/* ---- library ----------------------------------------------------------- */

/* PKV_ABI_VERSION of the built library. */
int pkv_abi_version(void);
/* Static description of a status code. */
const char* pkv_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);
/* Device and gfx architecture the library was built for, e.g. "gfx950". */
const char* pkv_build_arch(void);

/* ---- pool (a1) ---------------------------------------------------------- */

/* Bytes of the K and V buffers for `desc` (v_bytes = 0 for LATENT). */
int kv_pool_bytes(const pkv_pool_desc* desc, size_t* k_bytes, size_t* v_bytes);

/* Describe a caller-allocated pool.  k_base (and v_base for SPLIT_KV) are
 * device pointers to kv_pool_bytes() bytes, 16-byte aligned; v_base must be
 * NULL for LATENT.  *out receives a handle the caller releases with
 * kv_pool_destroy(); the buffers stay the caller's. */
int kv_pool_create(const pkv_pool_desc* desc, void* k_base, void* v_base, pkv_pool** out);
int kv_pool_destroy(pkv_pool* pool);
/* Index of the padding page (== num_pages), or a negative status. */
int32_t kv_pool_padding_page(const pkv_pool* pool);
/* Bytes of one token's K+V in one layer (the [MINI] per-token figure / layers). */
int64_t kv_pool_token_bytes(const pkv_pool* pool);

/* ---- KV append (a2) ----------------------------------------------------- */

/* pool[layer][out_loc[j]] = k[j] (and v[j]) for j < n: a bit-exact scatter
 * of whole token rows ([MINI] store_kv; [OMNI] "Attention execution": the
 * current K/V span is written once per layer before any attention).
 *   k, v: device [n][num_kv_heads][head_dim] contiguous, pool dtype, 16-byte
 *     aligned (v NULL for LATENT).
 *   out_loc: device int32[n], slots in [0, (num_pages+1)*page_size); an
 *     out-of-range slot is skipped.  Duplicate slots race (only meaningful
 *     for dummy writes to the padding page). */
int kv_store(const pkv_pool* pool, int32_t layer, const void* k, const void* v, const int32_t* out_loc,
             int64_t n, void* stream);

/* ---- index building (a3) ------------------------------------------------ */

/* Turn token-table rows into page-granular indices ([XPU] "From slots to a
 * page table": every page_size-th column divided by page_size; [BACKEND]
 * "kv_indptr 和 kv_indices" and init_forward_metadata).
 *   out_fmt: PKV_MAP_CSR or PKV_MAP_BLOCK_TABLE.
 *   req_to_token, req_pool_indices, kv_start (nullable), kv_lens: as in
 *     pkv_kv_map (device).  kv_start[i] must be a multiple of page_size
 *     (the [XPU] page-alignment seam; kv_validate reports PKV_EALIGN).
 *   max_kv_len: host bound >= every kv_lens[i].
 *   CSR: kv_indptr device int32[bs+1] receives the prefix sum of
 *     ceil(kv_lens/page_size); out = kv_indices device int32[capacity].
 *     capacity must be >= bs * ceil(max_kv_len / page_size) (PKV_ECAPACITY).
 *   BLOCK_TABLE: out = device int32[bs][capacity] (capacity = row stride),
 *     capacity >= ceil(max_kv_len / page_size); entries past each request's
 *     last page are -1.  kv_indptr is ignored (may be NULL).
 *   kv_last_page_len: nullable device int32[bs]; receives
 *     kv_lens - (ceil(kv_lens/page_size) - 1) * page_size (0 if empty). */
int build_kv_indices(int32_t out_fmt, const int32_t* req_to_token, int64_t table_rows, int64_t table_width,
                     const int32_t* req_pool_indices, const int32_t* kv_start, const int32_t* kv_lens, int32_t bs,
                     int32_t page_size, int32_t max_kv_len, int32_t* kv_indptr, int32_t* out, int64_t capacity,
                     int32_t* kv_last_page_len, void* stream);

/* ---- paged decode (a4, a5, a6) ------------------------------------------ */

/* Workspace bytes paged_decode_attn needs for this batch shape. */
int paged_decode_workspace_bytes(const pkv_pool* pool, int32_t bs, int32_t num_q_heads, int32_t max_kv_len,
                                 size_t* bytes);

/* One query token per request attends over its kv_lens[i] keys read through
 * `map` ([XPU] "From slots to a page table"; [BACKEND] init_forward_metadata
 * with its split plan).  Query head h reads KV head h / (num_q_heads /
 * num_kv_heads).  The keys are split at logical positions that depend only
 * on kv_lens (bf16: the requests' 32-key tiles laid end to end and cut into
 * equal runs, one per workgroup; f32: fixed-size chunks per request); each
 * piece's partial result is merged by log-sum-exp, so the output does not
 * depend on where pages live.
 *   q: device [bs][num_q_heads][head_dim_qk], pool dtype.
 *   out: device [bs][num_q_heads][head_dim_v], pool dtype (round to nearest
 *     even for bf16).
 *   lse: nullable device float[bs][num_q_heads], natural-log log-sum-exp of
 *     the scaled scores; kv_lens[i] == 0 gives out = 0 and lse = -inf.
 *   sm_scale: the score scale, positive and finite (else PKV_EINVAL).
 *   workspace: device, >= paged_decode_workspace_bytes(), 256-byte aligned.
 *   map->fmt: TOKEN_TABLE, CSR or BLOCK_TABLE.
 * Supported: SPLIT_KV f32 or bf16 with head_dim 64 or 128 and
 * num_q_heads/num_kv_heads <= 16; LATENT bf16 with head_dim_qk 576,
 * head_dim_v 512, one KV head and num_q_heads in {16, 32, 64} or a multiple
 * of 128 up to 1024 (more than 128 heads run as slices of 128). */
int paged_decode_attn(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                      const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* workspace,
                      size_t ws_bytes, void* stream);

/* paged_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the workspace taken
 * from a device array the library holds (128 MiB per device, kept until the
 * process ends) instead of a caller's buffer.  The caller still passes q,
 * out and lse as for paged_decode_attn.
 *   Returns PKV_ECAPACITY, before touching the device, when this batch
 *   shape needs more workspace than the array holds
 *   (paged_decode_workspace_bytes() > 128 MiB); use paged_decode_attn with
 *   a workspace then.
 *   Every call on one device shares that device's array: calls that overlap
 *   on one device (two streams, two threads) race and must be ordered by
 *   the caller.  Allocates nothing and issues no memset. */
int paged_decode_attn_noalloc(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                              const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* stream);

/* paged_decode_attn with the step's KV append in the same call ([MINI]
 * "The KV pool: one preallocated block of memory": the attention backend
 * stores the step's new K/V by out_loc before it computes attention).  The
 * result is that of kv_store(pool, layer, k_new, v_new, out_loc, n_new)
 * followed by paged_decode_attn(...) on the same stream, bit for bit; the
 * append runs inside the decode's planner launch (bf16 and latent pools),
 * which reads only the tables, so a step launches one kernel fewer.
 *   k_new, v_new, out_loc, n_new: as kv_store (v_new ignored for a latent
 *     pool); n_new = 0 stores nothing.  map->kv_lens count the new tokens.
 *   Other arguments and errors: as paged_decode_attn, and as kv_store for
 *   the append's arguments (all checked before anything is launched).  With
 *   map->bs = 0 only the append runs. */
int paged_decode_attn_append(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                             const pkv_kv_map* map, const void* k_new, const void* v_new, const int32_t* out_loc,
                             int64_t n_new, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream);

/* Target verification over a latent (MLA) pool ([BACKEND]
 * init_forward_metadata, the target-verify branch: the sequence lengths
 * include the draft tokens and the drafts multiply the head count).  Each
 * request's num_draft draft tokens are checked in one pass: map->kv_lens
 * counts the keys including the drafts (stored by kv_store first), and the
 * drafts' heads are folded into the head dimension of the decode kernel.
 * Draft j of request i sits at position kv_lens[i] - num_draft + j and sees
 * keys 0 .. that position (bottom-right, as paged_extend_attn's causal mode).
 *   q: device [bs][num_draft][num_q_heads][576] bf16.
 *   out: device [bs][num_draft][num_q_heads][512] bf16; lse nullable float
 *     [bs][num_draft][num_q_heads].  A draft that sees no key
 *     (kv_lens[i] < num_draft) gets out = 0 and lse = -inf.
 *   workspace: device, >= paged_decode_workspace_bytes(pool, bs,
 *     num_draft * num_q_heads, max_kv_len), 256-byte aligned.
 * Supported: LATENT bf16 576/512 pools with num_draft * num_q_heads in
 * {16, 32, 64} or a multiple of 128 up to 1024 (else PKV_EUNSUPPORTED);
 * sm_scale positive and finite.  More than 128 rows run as slices of 128
 * rows, one after another on the stream, sharing the workspace. */
int paged_verify_attn(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads, int32_t num_draft,
                      const pkv_kv_map* map, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                      void* stream);

/* paged_verify_attn with the drafts' latent rows stored in the same call
 * ([BACKEND] target verify: the drafts' keys are written to the pool and
 * attended in one step; [MINI] "The KV pool: one preallocated block of
 * memory": the backend stores before it attends).  Bits equal kv_store(pool,
 * layer, k_new, NULL, out_loc, n_new) followed by paged_verify_attn(...);
 * the append runs inside the verification's planner launch.
 *   k_new, out_loc, n_new: as kv_store on a latent pool.
 *   Other arguments and errors: as paged_verify_attn, and as kv_store for
 *   the append's arguments (all checked before anything is launched).  With
 *   map->bs = 0 only the append runs. */
int paged_verify_attn_append(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                             int32_t num_draft, const pkv_kv_map* map, const void* k_new, const int32_t* out_loc,
                             int64_t n_new, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream);

/* Groups of requests that share a prefix ([XPU] introduction: requests
 * sharing a prefix share its pages; [MINI]'s prefix cache).  Group g is the
 * requests group_indptr[g] .. group_indptr[g+1] - 1 of the batch (groups
 * increasing and disjoint; requests in no group are allowed); the first
 * min(kv_lens[i], prefix_len[g]) keys of every member read the same slots.
 *   num_groups, max_group_size, max_prefix_len: host; the bounds size the
 *     launch and must hold every group's member count and prefix_len.
 *   group_indptr: device int32[num_groups + 1]; prefix_len: device
 *     int32[num_groups] (tokens). */
typedef struct pkv_prefix_groups {
  int32_t num_groups;
  int32_t max_group_size;
  int32_t max_prefix_len;
  const int32_t* group_indptr;
  const int32_t* prefix_len;
} pkv_prefix_groups;

/* Workspace bytes paged_decode_attn_cascade needs. */
int paged_decode_cascade_workspace_bytes(const pkv_pool* pool, int32_t bs, int32_t num_q_heads, int32_t max_kv_len,
                                         const pkv_prefix_groups* groups, size_t* bytes);

/* The result of paged_decode_attn (same arguments and outputs), computed as
 * a cascade: each group's shared prefix (prefix_len rounded down to 32 keys)
 * is read once per KV head and scored against all members' queries, each
 * request's remaining keys go through the split-K decode, and the parts
 * are merged by log-sum-exp.  A caller whose groups break the sharing
 * promise gets an unspecified result (never an out-of-range access).
 *   groups: host struct (see pkv_prefix_groups); num_groups 0 is plain decode.
 *   workspace: >= paged_decode_cascade_workspace_bytes(), 256-byte aligned.
 * Supported: SPLIT_KV bf16, head_dim 64 or 128, num_q_heads / num_kv_heads
 * <= 16; map TOKEN_TABLE, CSR or BLOCK_TABLE. */
int paged_decode_attn_cascade(const pkv_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                              const pkv_kv_map* map, const pkv_prefix_groups* groups, float sm_scale, void* out,
                              float* lse, void* workspace, size_t ws_bytes, void* stream);

/* ---- paged extend / prefill (a7, a8, a9) -------------------------------- */

/* Each request's qo_indptr[i+1] - qo_indptr[i] new query tokens attend over
 * its kv_lens[i] keys ([BACKEND] "例子": qo_indptr / kv_indptr; [OMNI]
 * "Attention execution": causal and full segments).  causal != 0 aligns the
 * queries bottom-right: the j-th of n new queries sees keys 0 .. L - n + j;
 * causal == 0 lets every query see every key (encoder cross-attention).
 *   q: device [total_q][num_q_heads][head_dim_qk]; total_q (host) is the row
 *     count of q and out, >= qo_indptr[bs] (rows past it are never touched).
 *   qo_indptr: device int32[bs+1].
 *   max_q_len: host bound >= every new-token count.
 *   out: device [total_q][num_q_heads][head_dim_v]; lse nullable float
 *     [total_q][num_q_heads].  An empty key set gives out = 0, lse = -inf
 *     ([XPU] "Approach 2" empty-KV guard).
 *   sm_scale: the score scale, positive and finite (else PKV_EINVAL).
 *   map->fmt: any; CONTIGUOUS is the ragged (varlen) variant.
 * Supported: SPLIT_KV bf16 (MFMA kernel) or f32 (vector-ALU kernel, fp32
 * throughout), head_dim 64 or 128, num_q_heads a multiple of
 * num_kv_heads. */
int paged_extend_attn(const pkv_pool* pool, int32_t layer, const void* q, int64_t total_q, const int32_t* qo_indptr,
                      int32_t num_q_heads, int32_t max_q_len, const pkv_kv_map* map, int32_t causal,
                      float sm_scale, void* out, float* lse, void* stream);

/* Options of paged_extend_attn_ex.
 *   causal: the mask of every request when causal_flags is NULL (as in
 *     paged_extend_attn).
 *   causal_flags: nullable device int32[bs], one flag per request: nonzero
 *     = causal (bottom-right), 0 = full.  A row of mixed causal and full spans
 *     ([OMNI] "Attention execution": causal [s, e) is Q[s:e] over K[:e] with
 *     the causal flag, full [a, b) is Q[a:b] over K[:b] without it) runs as
 *     one call whose requests are its segments: several requests may read
 *     the same table row, each with its own kv_lens and query rows.
 *   softcap: 0 = off; > 0 (finite) replaces every scaled score s by
 *     softcap * tanh(s / softcap) before the softmax ([XPU] "Approach 2":
 *     the ragged call passes softcap). */
typedef struct pkv_extend_opts {
  int32_t causal;
  const int32_t* causal_flags;
  float softcap;
} pkv_extend_opts;

/* paged_extend_attn with per-request causal flags and softcap (opts, host,
 * required).  Everything else as paged_extend_attn; negative or infinite
 * softcap gives PKV_EINVAL. */
int paged_extend_attn_ex(const pkv_pool* pool, int32_t layer, const void* q, int64_t total_q,
                         const int32_t* qo_indptr, int32_t num_q_heads, int32_t max_q_len, const pkv_kv_map* map,
                         const pkv_extend_opts* opts, float sm_scale, void* out, float* lse, void* stream);

/* ---- ragged gather (a9) ------------------------------------------------- */

/* Copy each request's first kv_lens[i] K (and V) rows, in logical order,
 * to rows cu_seqlens_k[i] .. of k_out / v_out ([XPU] "Approach 2": the
 * index_select gather feeding the varlen kernel).  Bit exact.
 *   map->fmt: TOKEN_TABLE, CSR or BLOCK_TABLE.
 *   cu_seqlens_k: device int32[bs+1]; out_rows: capacity of k_out / v_out
 *     in rows (rows past it are not written).
 *   k_out, v_out: device [out_rows][num_kv_heads][head_dim] (v_out NULL for
 *     LATENT), 16-byte aligned. */
int kv_gather(const pkv_pool* pool, int32_t layer, const pkv_kv_map* map, const int32_t* cu_seqlens_k,
              void* k_out, void* v_out, int64_t out_rows, void* stream);

/* ---- slot allocation and row writing ------------------------------------ */

/* Device free list of pages ([XPU] "How SGLang stores the KV cache: two
 * pools and a page size": the token allocator's free list of slots and the
 * paged allocator's free list of page ids; at page_size 1 a page is a slot).
 * It is a ring the caller owns:
 *   free_pages: device int32[capacity] of page ids.
 *   free_state: device int32[2] = {head, size}; the free entries, front
 *     first, are free_pages[(head + k) % capacity] for k < size.
 *   status: device int32, written by every call below (PKV_ALLOC_*).  A call
 *     that is not granted changes neither the ring nor its outputs.
 * Allocation takes entries from the front in order; freeing appends at the
 * back.  Calls on one ring must be ordered on one stream (overlapping calls
 * race).  Each call is a fixed sequence of kernel launches with no host
 * synchronisation and no memset, so it may be captured in a graph; the
 * caller reads `status` when it next synchronises. */
#define PKV_ALLOC_OK 0
#define PKV_ALLOC_NO_SPACE 1     /* fewer free pages than needed (the pages' None) */
#define PKV_ALLOC_OUT_CAPACITY 2 /* more new tokens than out_capacity */
#define PKV_ALLOC_BAD_LENGTHS 3  /* some prefix_len < 0 or seq_len < prefix_len */
#define PKV_ALLOC_RING_FULL 4    /* free: the pages do not fit in the ring */

/* free_pages[k] = first + k for k < count, free_state = {0, count} (the
 * pages' clear(): at page_size 1 the free list 1 .. size skips slot 0;
 * with this library's pool, whose padding page is the last one, first = 0
 * and count = num_pages).  count <= capacity (PKV_ECAPACITY). */
int kv_free_list_init(int32_t* free_pages, int32_t capacity, int32_t first, int32_t count, int32_t* free_state,
                      void* stream);

/* Page-aligned alloc ([XPU] paged allocator alloc(); [BACKEND] opening
 * table, page-aligned allocation row): the first need / page_size free pages,
 * page p expanded to slots p * page_size + 0 .. page_size - 1, written to
 * out (device int32[need]).  need must be a multiple of page_size
 * (PKV_EINVAL); page_size a power of two <= 128. */
int kv_alloc(int32_t page_size, int64_t need, int32_t* free_pages, int32_t capacity, int32_t* free_state,
             int32_t* out, int32_t* status, void* stream);

/* Growth path ([XPU] paged allocator alloc_extend): request i grows from
 * prefix_lens[i] to seq_lens[i] tokens.  Its new tokens first fill the rest
 * of its partly used last page (the slots after last_loc[i], the slot of
 * its last cached token), then take whole pages from the front of the free
 * list, request after request, so every page holds consecutive logical
 * positions.  out_cache_loc (device int32[out_capacity]) receives the new
 * slots of request 0, then request 1, ...; entries past the total are not
 * written.
 *   prefix_lens, seq_lens: device int32[bs]; bs <= 8000 (PKV_EUNSUPPORTED).
 *   last_loc: device int32[bs], read only for requests whose prefix ends
 *     inside a page; may be NULL when page_size == 1.
 * Denied (status set, nothing written) when the batch needs more pages than
 * are free, more slots than out_capacity, or has invalid lengths. */
int kv_alloc_extend(int32_t page_size, int32_t bs, const int32_t* prefix_lens, const int32_t* seq_lens,
                    const int32_t* last_loc, int32_t* free_pages, int32_t capacity, int32_t* free_state,
                    int32_t* out_cache_loc, int64_t out_capacity, int32_t* status, void* stream);

/* Decode growth ([XPU] paged allocator alloc_decode): kv_alloc_extend with
 * prefix_lens = seq_lens - 1, one slot per request into out_cache_loc
 * (device int32[bs]).  seq_lens[i] >= 1 (else PKV_ALLOC_BAD_LENGTHS). */
int kv_alloc_decode(int32_t page_size, int32_t bs, const int32_t* seq_lens, const int32_t* last_loc,
                    int32_t* free_pages, int32_t capacity, int32_t* free_state, int32_t* out_cache_loc,
                    int32_t* status, void* stream);

/* Free ([XPU] paged allocator free): the distinct pages slots[0 .. n) lie on
 * (slot / page_size), in increasing page order, are appended to the back of
 * the free list.  Negative slots and pages >= num_pages (the padding page)
 * are ignored.  page_bitmap: device uint32[(num_pages + 31) / 32] the call
 * uses as scratch (its contents on entry do not matter).  Denied with
 * PKV_ALLOC_RING_FULL when the pages do not fit in the ring. */
int kv_free(int32_t page_size, const int32_t* slots, int64_t n, int32_t num_pages, int32_t* free_pages,
            int32_t capacity, int32_t* free_state, uint32_t* page_bitmap, int32_t* status, void* stream);

/* write_cache_indices ([XPU] "How SGLang stores the KV cache", the two
 * writes per request and the one-program-per-request kernel): row
 * req_pool_indices[i] of req_to_token (device int32[table_rows][table_width])
 * gets prefix slots in columns [0, prefix_lens[i]) and its new slots in
 * [prefix_lens[i], seq_lens[i]), the latter from out_cache_loc (device
 * int32[n_out]) after the new tokens of requests 0 .. i-1.
 *   prefix_ptrs: nullable device array of bs device pointers; entry i (may be
 *     NULL) points at request i's int32[prefix_lens[i]] prefix slots.  A NULL
 *     array or entry leaves those columns as they are (e.g. a chunked prefill
 *     continuing its own row, or decode).
 *   max_seq_len: host bound >= every seq_lens[i], <= table_width.
 * A request whose lengths are invalid (prefix < 0, seq < prefix) writes
 * nothing and counts no new tokens; one whose row is out of range or whose
 * seq_len exceeds table_width writes nothing; reads of out_cache_loc past
 * n_out are skipped. */
int write_req_to_token(int32_t* req_to_token, int64_t table_rows, int64_t table_width,
                       const int32_t* req_pool_indices, const int32_t* prefix_lens, const int32_t* seq_lens,
                       const int32_t* out_cache_loc, int64_t n_out, const int32_t* const* prefix_ptrs, int32_t bs,
                       int32_t max_seq_len, void* stream);

/* ---- encoder-embedding block cache ------------------------------------ */

/* One preallocated buffer of encoder embeddings (the AWS Neuron on-device
 * encoder cache notes, "Buffer Layout"): device [num_blocks][block_size]
 * [row_bytes], one multimodal item per block, the last block a scratch block
 * that only padding writes reach.  row_bytes (fat_dim x element size, 40960
 * at the notes' Qwen3-VL geometry) must be a positive multiple of 16
 * (PKV_EALIGN); buffer, src and hidden 16-byte aligned.  The copies are bit
 * exact and element-type agnostic. */

/* Write path ("Write Path": the encoder scatter-writes its output into the
 * allocated blocks): src device [n][block_size][row_bytes] block k goes to
 * block block_ids[k] (device int32[n]); padding blocks carry the scratch
 * block's id; ids outside [0, num_blocks) are dropped. */
int enc_cache_write(void* buffer, int32_t num_blocks, int32_t block_size, int64_t row_bytes, const void* src,
                    int32_t n, const int32_t* block_ids, void* stream);

/* Read path and merge ("Read Path", "Merge Inside Compiled Graph"): token t
 * of gathered block j (block id block_ids[j], device int32[max_blocks]) is
 * copied to row positions[j][t] of hidden (device [num_tokens][row_bytes])
 * when 0 <= positions[j][t] < num_tokens.  positions: device int64
 * [max_blocks][block_size]; the sentinel num_tokens (or any position
 * outside the rows) marks a don't-care token and writes nothing, so hidden
 * needs no dummy row.  Blocks whose id is outside the buffer write nothing.
 *   fill_count: nullable device int32[num_tokens], zeroed by the caller;
 *     each written row's count is incremented (for enc_cache_check).
 * Sequence parallelism: pass a rank its local positions (global positions
 * outside its range become its sentinel) and its own hidden rows. */
int enc_cache_merge(const void* buffer, int32_t num_blocks, int32_t block_size, int64_t row_bytes,
                    const int32_t* block_ids, int32_t max_blocks, const int64_t* positions, void* hidden,
                    int64_t num_tokens, int32_t* fill_count, void* stream);

/* The fail-loud check ("Read Path": every scheduled encoder position must be
 * filled) over enc_cache_merge's fill counts; SYNCHRONISES `stream`.
 *   scheduled: nullable device int32[num_tokens], nonzero = a row that must
 *     be filled (NULL = every row).
 *   scratch: device int64[2]; counts: host int64[2] receives [0] scheduled
 *     rows never filled, [1] rows filled more than once.
 * Returns PKV_OK when both are zero, else PKV_EINVAL. */
int enc_cache_check(const int32_t* fill_count, const int32_t* scheduled, int64_t num_tokens, int64_t* scratch,
                    int64_t counts[2], void* stream);

/* ---- debug / measurement (off the hot path) ------------------------------ */

/* Check a map's contents on the device and SYNCHRONISE `stream`: slots and
 * page ids in range, -1 only after a request's last page, no real request on
 * the padding page, kv_start page aligned for page-granular use, tokens
 * contiguous inside each page.  The invariants are the pages': the paged
 * allocator hands out whole pages and keeps a request's tokens contiguous
 * inside each page, so a page id is slot // page_size ([XPU] "How SGLang
 * stores the KV cache: two pools and a page size"; the page-aligned encoder
 * start of [XPU] "Approach 1: page-align the encoder"); the extra last page
 * is a padding page that only dummy requests of a padded batch point at
 * ([MINI] "Why the extra page?").  A debug call, off the hot path.
 *   is_dummy: nullable device int32[bs], nonzero marks padded-batch dummies.
 *   scratch: device int64[bs * 8] the kernel writes per-request counts to
 *     (the library allocates nothing).
 *   counts: host int64[8] receives the totals of each kind: [0] slot/page
 *     out of range, [1] padding page used by a real request, [2] -1 inside a
 *     length or a real id after it, [3] misaligned kv_start, [4] in-page
 *     contiguity broken, [5] length beyond the table or a bad indptr.
 * Returns PKV_OK when every count is zero, PKV_EALIGN when only kv_start
 * alignment fails, else PKV_EINVAL. */
int kv_validate(const pkv_pool* pool, const pkv_kv_map* map, const int32_t* is_dummy, int64_t* scratch,
                int64_t counts[8], void* stream);

/* Record hipEvent_t `start` before and `stop` after the main attention
 * kernel of the next paged_decode_attn / paged_extend_attn call made on
 * this thread (the split-K kernel for decode), then forget them.
 * Pass NULLs to clear.  For measuring one kernel inside a call. */
int pkv_set_kernel_timer(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
