// Slot allocation and request-row writing on the device ([XPU] "How SGLang
// stores the KV cache: two pools and a page size": the token and paged
// allocators, alloc_extend / alloc_decode, free, and write_cache_indices;
// [BACKEND] opening table, page-aligned allocation row).
//
// The free list is a ring of page ids in device memory (slots when
// page_size is 1) with a two-word state {head, size}: the free entries are
// ring[(head + k) % capacity] for k < size, front first.  Every call is
// asynchronous and reports through a device status word, so a serving loop
// never waits on the host: allocation takes from the front, freeing appends
// at the back, and a call that cannot be satisfied changes nothing.
//
// All of this is small integer work bound by launch latency, not by HBM:
// each call is a fixed number of launches (no host synchronisation, no
// memset, so it may be captured in a graph), and the batch-wide prefix sums
// are block scans in LDS rather than a separate scan pass.
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kAllocThreads = 256;
constexpr int kAllocMaxBlocks = 256;
constexpr int kRowChunk = 1024;  // table columns per write block
constexpr int kCompactThreads = 1024;

__device__ __forceinline__ int32_t pages_spanned(int64_t L, int32_t shift) {
  return L > 0 ? (int32_t)(((L - 1) >> shift) + 1) : 0;
}

// Request j grows from p to s tokens; decode batches (prefix == nullptr)
// grow by one token.
struct Growth {
  int64_t p, s;
  __device__ __forceinline__ bool ok() const { return p >= 0 && s >= p; }
};

__device__ __forceinline__ Growth growth(const int32_t* prefix, const int32_t* seq, int32_t j) {
  const int64_t s = seq[j];
  return {prefix ? (int64_t)prefix[j] : s - 1, s};
}

__device__ __forceinline__ int64_t ring_index(int64_t x, int64_t cap) {
  const int64_t r = x % cap;
  return r < 0 ? r + cap : r;
}

// Exclusive prefix sums of a and b over the block (kAllocThreads threads);
// the block totals come back in ta, tb.  `sh` holds 2 * waves entries.
__device__ __forceinline__ void block_scan2(int64_t& a, int64_t& b, int64_t& ta, int64_t& tb, int64_t* sh) {
  constexpr int W = kAllocThreads / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t ia = a, ib = b;
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t xa = __shfl_up(ia, d, 64), xb = __shfl_up(ib, d, 64);
    if (lane >= d) {
      ia += xa;
      ib += xb;
    }
  }
  if (lane == 63) {
    sh[w] = ia;
    sh[W + w] = ib;
  }
  __syncthreads();
  int64_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    if (k < w) {
      pa += sh[k];
      pb += sh[W + k];
    }
    ta += sh[k];
    tb += sh[W + k];
  }
  a = pa + ia - a;
  b = pb + ib - b;
  __syncthreads();
}

// Batch totals: new tokens, new pages, and whether every request's lengths
// are valid.  Every block of a call computes the same values from the same
// inputs, so all of them reach the same decision.
struct GrowthTotals {
  int64_t tokens, pages;
  bool bad;
};

__device__ GrowthTotals growth_totals(const int32_t* prefix, const int32_t* seq, int32_t bs, int32_t shift,
                                      int64_t* sh) {
  int64_t t = 0, p = 0;
  bool bad = false;
  for (int32_t j = threadIdx.x; j < bs; j += kAllocThreads) {
    const Growth g = growth(prefix, seq, j);
    if (!g.ok()) {
      bad = true;
      continue;
    }
    t += g.s - g.p;
    p += pages_spanned(g.s, shift) - pages_spanned(g.p, shift);
  }
  bad = __syncthreads_or(bad);
  int64_t tt, tp;
  block_scan2(t, p, tt, tp, sh);
  return {tt, tp, bad};
}

// The decision of an allocation: 0 = granted, else the PKV_ALLOC_* reason.
__device__ __forceinline__ int32_t alloc_verdict(const GrowthTotals& g, int64_t out_cap, int64_t free_size) {
  if (g.bad) return 3;                // PKV_ALLOC_BAD_LENGTHS
  if (g.tokens > out_cap) return 2;   // PKV_ALLOC_OUT_CAPACITY
  if (g.pages > free_size) return 1;  // PKV_ALLOC_NO_SPACE
  return 0;
}

// ---------------------------------------------------------------------------
// alloc_extend / alloc_decode: each request first fills the rest of its last,
// partly used page (the slots after last_loc), then takes whole pages from
// the ring front, request after request; a new page p holds the request's
// next logical tokens at slots p * page_size + offset.
//
// Every block scans the batch once into LDS (token and page offsets per
// request), then the grid strides over the batch's new tokens; each token
// finds its request by binary search in LDS.  The ring state is only read
// here; alloc_commit_kernel, stream-ordered after, moves it.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) alloc_extend_kernel(
    int32_t shift, int32_t bs, const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ last_loc, const int32_t* __restrict__ ring, int64_t cap,
    const int32_t* __restrict__ state, int32_t* __restrict__ out, int64_t out_cap) {
  extern __shared__ int32_t lds[];
  int32_t* tok_off = lds;           // [bs + 1]
  int32_t* pg_off = lds + bs + 1;   // [bs + 1]
  __shared__ int64_t sh[2 * (kAllocThreads / 64)];
  const int tid = threadIdx.x;

  int64_t carry_t = 0, carry_p = 0;
  bool bad = false;
  for (int32_t base = 0; base < bs; base += kAllocThreads) {
    const int32_t j = base + tid;
    int64_t nt = 0, np = 0;
    if (j < bs) {
      const Growth g = growth(prefix, seq, j);
      if (g.ok()) {
        nt = g.s - g.p;
        np = pages_spanned(g.s, shift) - pages_spanned(g.p, shift);
      } else {
        bad = true;
      }
    }
    int64_t tt, tp;
    block_scan2(nt, np, tt, tp, sh);
    // offsets are only used once the totals fit in out_cap <= INT32_MAX
    if (j < bs) {
      tok_off[j] = (int32_t)(carry_t + nt);
      pg_off[j] = (int32_t)(carry_p + np);
    }
    carry_t += tt;
    carry_p += tp;
  }
  bad = __syncthreads_or(bad);
  const int64_t head = state[0], size = state[1];
  if (alloc_verdict({carry_t, carry_p, bad}, out_cap, size) != 0) return;
  if (tid == 0) tok_off[bs] = (int32_t)carry_t;
  __syncthreads();

  const int32_t mask = (1 << shift) - 1;
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + tid; k < carry_t; k += (int64_t)gridDim.x * kAllocThreads) {
    int32_t lo = 0, hi = bs;  // tok_off[lo] <= k < tok_off[hi]
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (tok_off[mid] <= k) lo = mid;
      else hi = mid;
    }
    const Growth g = growth(prefix, seq, lo);
    const int64_t t = g.p + (k - tok_off[lo]);
    const int32_t held = pages_spanned(g.p, shift);
    const int64_t pidx = t >> shift;
    int64_t page;
    if (pidx < held) {
      page = (int64_t)last_loc[lo] >> shift;  // the partly used last page
    } else {
      page = ring[ring_index(head + pg_off[lo] + (pidx - held), cap)];
    }
    out[k] = (int32_t)((page << shift) + (t & mask));
  }
}

__global__ void __launch_bounds__(kAllocThreads) alloc_commit_kernel(int32_t shift, int32_t bs,
                                                                     const int32_t* __restrict__ prefix,
                                                                     const int32_t* __restrict__ seq, int64_t cap,
                                                                     int32_t* __restrict__ state, int64_t out_cap,
                                                                     int32_t* __restrict__ status) {
  __shared__ int64_t sh[2 * (kAllocThreads / 64)];
  const GrowthTotals g = growth_totals(prefix, seq, bs, shift, sh);
  if (threadIdx.x != 0) return;
  const int64_t head = state[0], size = state[1];
  const int32_t v = alloc_verdict(g, out_cap, size);
  if (v == 0) {
    state[0] = (int32_t)ring_index(head + g.pages, cap);
    state[1] = (int32_t)(size - g.pages);
  }
  *status = v;
}

// ---------------------------------------------------------------------------
// Page-aligned alloc: the first n_pages ring entries, each expanded to its
// page_size slots.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) alloc_pages_kernel(int32_t shift, int64_t n_pages,
                                                                    const int32_t* __restrict__ ring, int64_t cap,
                                                                    const int32_t* __restrict__ state,
                                                                    int32_t* __restrict__ out) {
  const int64_t head = state[0], size = state[1];
  if (n_pages > size) return;
  const int64_t n = n_pages << shift;
  const int32_t mask = (1 << shift) - 1;
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + threadIdx.x; k < n; k += (int64_t)gridDim.x * kAllocThreads)
    out[k] = (int32_t)(((int64_t)ring[ring_index(head + (k >> shift), cap)] << shift) + (k & mask));
}

__global__ void alloc_pages_commit_kernel(int64_t n_pages, int64_t cap, int32_t* __restrict__ state,
                                          int32_t* __restrict__ status) {
  if (threadIdx.x != 0) return;
  const int64_t head = state[0], size = state[1];
  if (n_pages > size) {
    *status = 1;  // PKV_ALLOC_NO_SPACE
    return;
  }
  state[0] = (int32_t)ring_index(head + n_pages, cap);
  state[1] = (int32_t)(size - n_pages);
  *status = 0;
}

// ---------------------------------------------------------------------------
// Free: the distinct pages of the freed slots, in increasing order, go to the
// back of the ring (the pages' unique(slots // page_size)).  A bitmap over the
// pages deduplicates and sorts at once: clear, mark, then one block walks
// the words in order and appends the set bits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + threadIdx.x; k < n; k += (int64_t)gridDim.x * kAllocThreads)
    p[k] = v;
}

__global__ void __launch_bounds__(kAllocThreads) free_mark_kernel(int32_t shift, const int32_t* __restrict__ slots,
                                                                  int64_t n, int64_t num_pages,
                                                                  uint32_t* __restrict__ bits) {
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * kAllocThreads) {
    const int32_t s = slots[k];
    if (s < 0) continue;
    const int64_t page = (int64_t)s >> shift;
    if (page >= num_pages) continue;  // the padding page and beyond never go back
    atomicOr(bits + (page >> 5), 1u << (page & 31));
  }
}

__global__ void __launch_bounds__(kCompactThreads) free_compact_kernel(const uint32_t* __restrict__ bits,
                                                                       int64_t words, int32_t* __restrict__ ring,
                                                                       int64_t cap, int32_t* __restrict__ state,
                                                                       int32_t* __restrict__ status) {
  constexpr int W = kCompactThreads / 64;
  __shared__ int64_t wsum[W];
  __shared__ int64_t total_sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  int64_t cnt = 0;
  for (int64_t k = tid; k < words; k += kCompactThreads) cnt += __popc(bits[k]);
  for (int d = 32; d > 0; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
  if (lane == 0) wsum[w] = cnt;
  __syncthreads();
  if (tid == 0) {
    int64_t t = 0;
    for (int k = 0; k < W; ++k) t += wsum[k];
    total_sh = t;
  }
  __syncthreads();
  const int64_t total = total_sh;
  const int64_t head = state[0], size = state[1];
  if (size + total > cap) {
    if (tid == 0) *status = 4;  // PKV_ALLOC_RING_FULL
    return;
  }
  int64_t at = head + size;  // ring position of the next appended page
  for (int64_t base = 0; base < words; base += kCompactThreads) {
    const int64_t k = base + tid;
    const uint32_t word = k < words ? bits[k] : 0u;
    const int32_t c = __popc(word);
    int32_t inc = c;
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t x = __shfl_up(inc, d, 64);
      if (lane >= d) inc += x;
    }
    __syncthreads();  // wsum is free again
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int64_t before = 0, chunk = 0;
    for (int q = 0; q < W; ++q) {
      if (q < w) before += wsum[q];
      chunk += wsum[q];
    }
    int64_t pos = at + before + inc - c;
    uint32_t rest = word;
    while (rest) {
      const int b = __ffs(rest) - 1;
      rest &= rest - 1;
      ring[ring_index(pos++, cap)] = (int32_t)((k << 5) + b);
    }
    at += chunk;
  }
  if (tid == 0) {
    state[1] = (int32_t)(size + total);
    *status = 0;
  }
}

// ---------------------------------------------------------------------------
// write_cache_indices: request i's row gets its prefix slots in columns
// [0, prefix_len) (when a prefix buffer is given) and its new slots in
// [prefix_len, seq_len), taken from out_cache_loc after the new tokens of
// the requests before it.  Block (i, c) writes columns [c, c + kRowChunk) of
// request i's row; a block whose columns hold new slots sums the earlier
// requests' new-token counts itself.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) write_rows_kernel(
    int32_t* __restrict__ table, int64_t rows, int64_t width, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq, const int32_t* __restrict__ out_loc,
    int64_t n_out, const int32_t* const* __restrict__ prefix_ptrs) {
  __shared__ int64_t red[kAllocThreads / 64];
  const int32_t i = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * kRowChunk;
  const int tid = threadIdx.x;
  const int64_t p = prefix[i], s = seq[i], r = rpi[i];
  if (p < 0 || s < p || s > width || r < 0 || r >= rows || c0 >= s) return;
  const int32_t* pre = prefix_ptrs ? prefix_ptrs[i] : nullptr;
  const bool has_new = c0 + kRowChunk > p;
  if (!has_new && !pre) return;
  int64_t pt = 0;
  if (has_new) {
    int64_t acc = 0;
    for (int32_t j = tid; j < i; j += kAllocThreads) {
      const int64_t pj = prefix[j], sj = seq[j];
      if (pj >= 0 && sj >= pj) acc += sj - pj;
    }
    for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    for (int q = 0; q < kAllocThreads / 64; ++q) pt += red[q];
  }
  int32_t* row = table + r * width;
  const int64_t end = min(c0 + kRowChunk, s);
  for (int64_t col = c0 + tid; col < end; col += kAllocThreads) {
    if (col < p) {
      if (pre) row[col] = pre[col];
    } else {
      const int64_t k = pt + col - p;
      if (k < n_out) row[col] = out_loc[k];
    }
  }
}

// Free list of pages first .. first + count - 1 (the pages' initial free list).
__global__ void __launch_bounds__(kAllocThreads) free_list_init_kernel(int32_t* __restrict__ ring, int32_t count,
                                                                       int32_t first, int32_t* __restrict__ state) {
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + threadIdx.x; k < count;
       k += (int64_t)gridDim.x * kAllocThreads)
    ring[k] = (int32_t)(first + k);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    state[0] = 0;
    state[1] = count;
  }
}

int grid_for(int64_t items) {
  const int64_t b = (items + kAllocThreads * 4 - 1) / (kAllocThreads * 4);
  return (int)(b < 1 ? 1 : (b > kAllocMaxBlocks ? kAllocMaxBlocks : b));
}

}  // namespace

hipError_t launch_alloc_extend(int32_t shift, int32_t bs, const int32_t* prefix, const int32_t* seq,
                               const int32_t* last_loc, int32_t* ring, int32_t cap, int32_t* state, int32_t* out,
                               int64_t out_cap, int32_t* status, hipStream_t s) {
  if (bs > 0) {
    const size_t lds = (size_t)(bs + 1) * 2 * sizeof(int32_t);
    hipLaunchKernelGGL(alloc_extend_kernel, dim3(grid_for(out_cap)), dim3(kAllocThreads), lds, s, shift, bs, prefix,
                       seq, last_loc, ring, (int64_t)cap, state, out, out_cap);
  }
  hipLaunchKernelGGL(alloc_commit_kernel, dim3(1), dim3(kAllocThreads), 0, s, shift, bs, prefix, seq, (int64_t)cap,
                     state, out_cap, status);
  return hipGetLastError();
}

hipError_t launch_alloc_pages(int32_t shift, int64_t n_pages, int32_t* ring, int32_t cap, int32_t* state,
                              int32_t* out, int32_t* status, hipStream_t s) {
  if (n_pages > 0)
    hipLaunchKernelGGL(alloc_pages_kernel, dim3(grid_for(n_pages << shift)), dim3(kAllocThreads), 0, s, shift,
                       n_pages, ring, (int64_t)cap, state, out);
  hipLaunchKernelGGL(alloc_pages_commit_kernel, dim3(1), dim3(64), 0, s, n_pages, (int64_t)cap, state, status);
  return hipGetLastError();
}

hipError_t launch_free(int32_t shift, const int32_t* slots, int64_t n, int32_t num_pages, int32_t* ring,
                       int32_t cap, int32_t* state, uint32_t* bits, int32_t* status, hipStream_t s) {
  const int64_t words = ((int64_t)num_pages + 31) / 32;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(words)), dim3(kAllocThreads), 0, s, bits, words, 0u);
  if (n > 0)
    hipLaunchKernelGGL(free_mark_kernel, dim3(grid_for(n)), dim3(kAllocThreads), 0, s, shift, slots, n,
                       (int64_t)num_pages, bits);
  hipLaunchKernelGGL(free_compact_kernel, dim3(1), dim3(kCompactThreads), 0, s, bits, words, ring, (int64_t)cap,
                     state, status);
  return hipGetLastError();
}

hipError_t launch_write_rows(int32_t* table, int64_t rows, int64_t width, const int32_t* rpi, const int32_t* prefix,
                             const int32_t* seq, const int32_t* out_loc, int64_t n_out,
                             const int32_t* const* prefix_ptrs, int32_t bs, int32_t max_seq_len, hipStream_t s) {
  if (bs == 0 || max_seq_len == 0) return hipSuccess;
  const unsigned chunks = (unsigned)(((int64_t)max_seq_len + kRowChunk - 1) / kRowChunk);
  hipLaunchKernelGGL(write_rows_kernel, dim3((unsigned)bs, chunks), dim3(kAllocThreads), 0, s, table, rows, width,
                     rpi, prefix, seq, out_loc, n_out, prefix_ptrs);
  return hipGetLastError();
}

hipError_t launch_free_list_init(int32_t* ring, int32_t first, int32_t count, int32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(free_list_init_kernel, dim3(grid_for(count)), dim3(kAllocThreads), 0, s, ring, count, first,
                     state);
  return hipGetLastError();
}

}  // namespace pkv
