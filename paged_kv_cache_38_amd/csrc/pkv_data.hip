// Data-movement and index kernels of the paged KV cache: the KV append
// (scatter), the ragged gather, index building and the debug validator.
//
// All three movement/index kernels are HBM- or latency-bound integer work:
// whole token rows move as 16-byte vectors, one wavefront per row, so every
// row's bytes go out as fully coalesced 1 KiB wave transactions.
#include "pkv_launch.h"

namespace pkv {

// ---------------------------------------------------------------------------
// KV append ([MINI] "The KV pool": store_kv writes each new token's K and V
// at its out_loc slot; [OMNI] "Attention execution": once per layer, before
// any attention reads the pool).
// One wavefront per new token: lanes stride over the row's 16-byte units.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) store_rows_kernel(StoreArgs a) {
  store_one_row(a, (int64_t)blockIdx.x * kStoreRowsPerBlock + (threadIdx.x >> 6), threadIdx.x & 63);
}

StoreArgs make_store_args(const PoolInfo& p, int32_t layer, const void* k, const void* v, const int32_t* out_loc,
                          int64_t n) {
  StoreArgs a;
  a.k_dst = const_cast<char*>(p.k_layer(layer));
  a.v_dst = const_cast<char*>(p.v_layer(layer));
  a.k_src = static_cast<const char*>(k);
  a.v_src = static_cast<const char*>(v);
  a.out_loc = out_loc;
  a.n = n;
  a.num_slots = p.num_slots;
  a.k_units = (int32_t)(p.k_row_bytes / 16);
  a.v_units = (int32_t)(p.v_row_bytes / 16);
  return a;
}

hipError_t launch_store_args(const StoreArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (a.n + kStoreRowsPerBlock - 1) / kStoreRowsPerBlock;
  hipLaunchKernelGGL(store_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_store(const PoolInfo& p, int32_t layer, const void* k, const void* v, const int32_t* out_loc,
                        int64_t n, hipStream_t s) {
  return launch_store_args(make_store_args(p, layer, k, v, out_loc, n), s);
}

// ---------------------------------------------------------------------------
// Ragged gather ([XPU] "Approach 2: gather and go ragged": the index_select
// of each request's slots into one contiguous buffer at cu_seqlens_k).
// Block (request i, group of 16 logical tokens); one wavefront per 4 rows.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gather_rows_kernel(DevMap m, const char* __restrict__ k_pool,
                                                          const char* __restrict__ v_pool,
                                                          const int32_t* __restrict__ cu, char* __restrict__ k_out,
                                                          char* __restrict__ v_out, int64_t out_rows,
                                                          int32_t k_units, int32_t v_units) {
  const int32_t i = blockIdx.y;
  const int32_t L = m.kv_lens[i];
  const int32_t t_base = blockIdx.x * 16 + (threadIdx.x >> 6) * 4;
  if (t_base >= L) return;
  const Resolver r = make_resolver(m, i);
  const int64_t dst0 = cu[i];
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int32_t t = t_base + q;
    if (t >= L) break;
    const int64_t d = dst0 + t;
    if (d < 0 || d >= out_rows) continue;
    const int64_t slot = r.slot(t);
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(k_pool) + slot * k_units;
      u32x4* dst = reinterpret_cast<u32x4*>(k_out) + d * k_units;
      for (int c = lane; c < k_units; c += 64) dst[c] = src[c];
    }
    if (v_out) {
      const u32x4* src = reinterpret_cast<const u32x4*>(v_pool) + slot * v_units;
      u32x4* dst = reinterpret_cast<u32x4*>(v_out) + d * v_units;
      for (int c = lane; c < v_units; c += 64) dst[c] = src[c];
    }
  }
}

hipError_t launch_gather(const PoolInfo& p, int32_t layer, const DevMap& m, int32_t bs, int32_t max_kv_len,
                         const int32_t* cu_seqlens_k, void* k_out, void* v_out, int64_t out_rows, hipStream_t s) {
  if (bs == 0 || max_kv_len == 0) return hipSuccess;
  dim3 grid((unsigned)((max_kv_len + 15) / 16), (unsigned)bs);
  hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, s, m, p.k_layer(layer), p.v_layer(layer), cu_seqlens_k,
                     static_cast<char*>(k_out), static_cast<char*>(v_out), out_rows,
                     (int32_t)(p.k_row_bytes / 16), (int32_t)(p.v_row_bytes / 16));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Index building ([XPU] "From slots to a page table": page ids are every
// page_size-th column of the token-granular row divided by page_size;
// [BACKEND] "kv_indptr 和 kv_indices": kv_indptr is the prefix sum of the
// per-request page counts and kv_indices lists the ids; init_forward_metadata:
// the padded block table is filled with -1 past each request's pages).
// One block per request.  The request's CSR offset is the sum of the page
// counts of the requests before it, summed by the block itself (bs is at
// most a few thousand, so the O(bs) reduction per block costs less than a
// separate scan launch).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t page_count(int32_t L, int32_t shift) {
  return L > 0 ? ((L - 1) >> shift) + 1 : 0;
}

__global__ void __launch_bounds__(256) build_indices_kernel(int32_t fmt, const int32_t* __restrict__ table,
                                                            int64_t rows, int64_t width,
                                                            const int32_t* __restrict__ rpi,
                                                            const int32_t* __restrict__ kv_start,
                                                            const int32_t* __restrict__ kv_lens, int32_t shift,
                                                            int32_t* __restrict__ kv_indptr, int32_t* __restrict__ out,
                                                            int64_t capacity, int32_t* __restrict__ last_len) {
  __shared__ int32_t red[4];
  const int32_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t L = max(kv_lens[i], 0);
  const int32_t cnt = page_count(L, shift);
  const int64_t row = rpi[i];
  const int64_t start = kv_start ? (int64_t)kv_start[i] : 0;
  const bool row_ok = row >= 0 && row < rows && start >= 0;
  const int32_t* rowp = table + (row_ok ? row : 0) * width;

  // kBatch entries per thread are loaded before any is stored, so a long
  // request's block waits for one load latency per 256 * kBatch pages
  // rather than one per 256; the first batch goes out before the CSR
  // offset sum, which only the stores need
  constexpr int kBatch = 8;
  int32_t v[kBatch];
  auto load_batch = [&](int32_t k0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int32_t k = k0 + u * 256 + tid;
      const int64_t col = start + ((int64_t)k << shift);
      v[u] = (k < cnt && row_ok && col < width) ? rowp[col] : -1;
    }
  };
  load_batch(0);

  int64_t base = 0;
  if (fmt == MAP_CSR) {
    int32_t acc = 0;
    for (int32_t j = tid; j < i; j += 256) acc += page_count(max(kv_lens[j], 0), shift);
    // wavefront reduction then across the 4 waves
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    base = (int64_t)red[0] + red[1] + red[2] + red[3];
    if (tid == 0) {
      if (i == 0) kv_indptr[0] = 0;
      kv_indptr[i + 1] = (int32_t)(base + cnt);
    }
  }
  for (int32_t k0 = 0; k0 < cnt; k0 += 256 * kBatch) {
    if (k0 > 0) load_batch(k0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int32_t k = k0 + u * 256 + tid;
      if (k >= cnt) break;
      const int32_t page = v[u] >= 0 ? (v[u] >> shift) : -1;
      if (fmt == MAP_CSR) {
        if (base + k < capacity) out[base + k] = page;
      } else if (k < capacity) {
        out[(int64_t)i * capacity + k] = page;
      }
    }
  }
  if (fmt == MAP_BLOCK_TABLE) {
    for (int64_t k = cnt + tid; k < capacity; k += 256) out[(int64_t)i * capacity + k] = -1;
  }
  if (last_len && tid == 0) last_len[i] = L > 0 ? L - ((cnt - 1) << shift) : 0;
}

__global__ void zero_first_kernel(int32_t* p) {
  if (threadIdx.x == 0) p[0] = 0;
}

hipError_t launch_build_indices(int32_t out_fmt, const int32_t* req_to_token, int64_t table_rows,
                                int64_t table_width, const int32_t* req_pool_indices, const int32_t* kv_start,
                                const int32_t* kv_lens, int32_t bs, int32_t page_shift, int32_t* kv_indptr,
                                int32_t* out, int64_t capacity, int32_t* kv_last_page_len, hipStream_t s) {
  if (bs == 0) {
    // an empty batch still gets kv_indptr[0] = 0 (a kernel, not a memset, so
    // the call stays safe to capture in a graph)
    if (out_fmt == MAP_CSR) hipLaunchKernelGGL(zero_first_kernel, dim3(1), dim3(64), 0, s, kv_indptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(build_indices_kernel, dim3((unsigned)bs), dim3(256), 0, s, out_fmt, req_to_token, table_rows,
                     table_width, req_pool_indices, kv_start, kv_lens, page_shift, kv_indptr, out, capacity,
                     kv_last_page_len);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Debug validator (off the hot path): counts violations of the invariants the
// page-granular formats rely on ([XPU] "How SGLang stores the KV cache": a
// request's tokens are contiguous inside each page; [MINI] "Why the extra
// page?": only dummy requests touch the padding page).
// One block per request, threads over logical tokens.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) validate_kernel(DevMap m, int32_t page_size, int32_t num_pages,
                                                       const int32_t* __restrict__ is_dummy,
                                                       long long* __restrict__ counts) {
  __shared__ int red[8];
  if (threadIdx.x < 8) red[threadIdx.x] = 0;
  __syncthreads();
  const int32_t i = blockIdx.x;
  const int32_t L = m.kv_lens[i];
  const bool dummy = is_dummy && is_dummy[i] != 0;
  const int32_t shift = m.page_shift;
  int c_range = 0, c_pad = 0, c_neg = 0, c_align = 0, c_contig = 0, c_len = 0;
  const int64_t pad_lo = (int64_t)num_pages * page_size;
  if (threadIdx.x == 0 && L < 0) c_len++;
  if (m.fmt == MAP_TOKEN_TABLE) {
    const int64_t row = m.req_pool_indices[i];
    const int64_t start = m.kv_start ? (int64_t)m.kv_start[i] : 0;
    if (row < 0 || row >= m.table_rows || start < 0 || start + L > m.table_width) {
      if (threadIdx.x == 0) c_len++;
    } else {
      const int32_t* rp = m.req_to_token + row * m.table_width + start;
      if (threadIdx.x == 0 && page_size > 1 && (start & (page_size - 1)) != 0) c_align++;
      for (int32_t t = threadIdx.x; t < L; t += 256) {
        const int64_t s = rp[t];
        if (s < 0 || s >= m.num_slots) { c_range++; continue; }
        if (!dummy && s >= pad_lo) c_pad++;
        if ((t & (page_size - 1)) != 0) {
          if (s != (int64_t)rp[t - 1] + 1) c_contig++;
        } else if ((s & (page_size - 1)) != 0) {
          c_contig++;
        }
      }
    }
  } else if (m.fmt == MAP_CSR || m.fmt == MAP_BLOCK_TABLE) {
    const int32_t* lst = nullptr;
    int64_t cnt = -1;
    if (m.fmt == MAP_CSR) {
      const int64_t a = m.kv_indptr[i], b = m.kv_indptr[i + 1];
      if (a < 0 || b < a || b > m.kv_indices_len) {
        if (threadIdx.x == 0) c_len++;
      } else {
        lst = m.kv_indices + a;
        cnt = b - a;
      }
    } else {
      lst = m.block_table + (int64_t)i * m.block_stride;
      cnt = m.block_stride;
    }
    if (cnt >= 0) {
      const int64_t need = L > 0 ? ((int64_t)(L - 1) >> shift) + 1 : 0;
      if (threadIdx.x == 0 && need > cnt) c_len++;
      for (int64_t k = threadIdx.x; k < cnt; k += 256) {
        const int64_t pg = lst[k];
        if (k < need) {
          if (pg < 0) c_neg++;
          else if (pg > num_pages) c_range++;
          else if (!dummy && pg == num_pages) c_pad++;
        } else if (m.fmt == MAP_BLOCK_TABLE && pg != -1) {
          c_neg++;  // a real id after the request's last page
        }
      }
    }
  }
  // block totals through LDS atomics; thread 0 writes this request's row
  atomicAdd(&red[0], c_range);
  atomicAdd(&red[1], c_pad);
  atomicAdd(&red[2], c_neg);
  atomicAdd(&red[3], c_align);
  atomicAdd(&red[4], c_contig);
  atomicAdd(&red[5], c_len);
  __syncthreads();
  if (threadIdx.x < 8) counts[(int64_t)i * 8 + threadIdx.x] = red[threadIdx.x];
}

hipError_t launch_validate(const PoolInfo& p, const DevMap& m, int32_t bs, int32_t max_kv_len,
                           const int32_t* is_dummy, long long* counts_dev, hipStream_t s) {
  (void)max_kv_len;
  if (bs == 0) return hipSuccess;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)bs), dim3(256), 0, s, m, p.page_size, p.num_pages, is_dummy,
                     counts_dev);
  return hipGetLastError();
}

}  // namespace pkv
