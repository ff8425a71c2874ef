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
#include "pkv_alloc.h"

namespace pkv {

namespace {

constexpr int kAllocThreads = 256;
constexpr int kWideThreads = 1024;  // single-block kernels (commit, compact)
constexpr int kAllocMaxBlocks = 256;
constexpr int kRowChunk = 1024;  // new tokens per row-writing block

__device__ __forceinline__ int32_t pages_spanned(int64_t L, int32_t shift) {
  return L > 0 ? (int32_t)(((L - 1) >> shift) + 1) : 0;
}

// Request j grows from p to s tokens; decode batches (prefix == nullptr)
// grow by one token.
struct Growth {
  int64_t p, s;
  __device__ __forceinline__ bool ok() const { return p >= 0 && s >= p; }
  __device__ __forceinline__ int64_t tokens() const { return s - p; }
  __device__ __forceinline__ int64_t pages(int32_t shift) const {
    return pages_spanned(s, shift) - pages_spanned(p, shift);
  }
};

__device__ __forceinline__ int32_t decode_prefix(int32_t s) { return (int32_t)((uint32_t)s - 1u); }

__device__ __forceinline__ Growth growth(const int32_t* prefix, const int32_t* seq, int32_t j) {
  const int32_t s = seq[j];
  return {prefix ? prefix[j] : decode_prefix(s), s};
}

// x mod cap.  With a consistent state (head < cap, size <= cap) every
// position a call forms is below 2 cap, so a compare and a subtract do; the
// 64-bit remainder (a long instruction sequence on the GPU) is only the
// fallback that keeps a corrupt state in bounds.
__device__ __forceinline__ int64_t ring_index(int64_t x, int64_t cap) {
  if ((uint64_t)x < (uint64_t)cap) return x;
  if (x >= cap && (uint64_t)(x - cap) < (uint64_t)cap) return x - cap;
  const int64_t r = x % cap;
  return r < 0 ? r + cap : r;
}

// Exclusive prefix sums of a and b over a block of T threads; the block
// totals come back in ta, tb.  `sh` holds 2 * T / 64 entries.
template <int T>
__device__ __forceinline__ void block_scan2(int64_t& a, int64_t& b, int64_t& ta, int64_t& tb, int64_t* sh) {
  constexpr int W = T / 64;
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

template <int T>
__device__ GrowthTotals growth_totals(const int32_t* prefix, const int32_t* seq, int32_t bs, int32_t shift,
                                      int64_t* sh) {
  int64_t t = 0, p = 0;
  bool bad = false;
#pragma unroll 4
  for (int32_t j = threadIdx.x; j < bs; j += T) {
    const Growth g = growth(prefix, seq, j);
    if (g.ok()) {
      t += g.tokens();
      p += g.pages(shift);
    } else {
      bad = true;
    }
  }
  bad = __syncthreads_or(bad);
  int64_t tt, tp;
  block_scan2<T>(t, p, tt, tp, sh);
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
// Every block stages the batch's lengths in LDS with independent loads, each
// thread scans a contiguous run of requests, and one block scan turns the
// runs into per-request token and page offsets (in place).  The grid then
// strides over the batch's new tokens; each token finds its request by
// binary search in LDS.  The ring state is only read here;
// alloc_commit_kernel, stream-ordered after, moves it.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) alloc_extend_kernel(
    int32_t shift, int32_t bs, const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ last_loc, const int32_t* __restrict__ ring, int64_t cap,
    const int32_t* __restrict__ state, int32_t* __restrict__ out, int64_t out_cap) {
  extern __shared__ int32_t lds[];
  int32_t* tok = lds;          // [bs + 1]: seq_len, then the token offset
  int32_t* pg = lds + bs + 1;  // [bs + 1]: prefix_len, then the page offset
  __shared__ int64_t sh[2 * (kAllocThreads / 64)];
  const int tid = threadIdx.x;
  const int64_t head = state[0], size = state[1];

  {
    // all of a thread's loads are issued before the first is used
    constexpr int kMaxIpt = (kMaxAllocBatch + kAllocThreads - 1) / kAllocThreads;
    int32_t sv[kMaxIpt], pv[kMaxIpt];
#pragma unroll
    for (int i = 0; i < kMaxIpt; ++i) {
      const int32_t j = tid + i * kAllocThreads;
      sv[i] = j < bs ? seq[j] : 0;
      pv[i] = (j < bs && prefix) ? prefix[j] : 0;
    }
#pragma unroll
    for (int i = 0; i < kMaxIpt; ++i) {
      const int32_t j = tid + i * kAllocThreads;
      if (j < bs) {
        tok[j] = sv[i];
        pg[j] = prefix ? pv[i] : decode_prefix(sv[i]);
      }
    }
  }
  __syncthreads();
  const int32_t ipt = (bs + kAllocThreads - 1) / kAllocThreads;
  const int32_t j0 = min(tid * ipt, bs), j1 = min(j0 + ipt, bs);
  int64_t nt = 0, np = 0;
  bool bad = false;
  for (int32_t j = j0; j < j1; ++j) {
    const Growth g{pg[j], tok[j]};
    if (g.ok()) {
      nt += g.tokens();
      np += g.pages(shift);
    } else {
      bad = true;
    }
  }
  int64_t tt, tp;
  block_scan2<kAllocThreads>(nt, np, tt, tp, sh);
  bad = __syncthreads_or(bad);
  if (alloc_verdict({tt, tp, bad}, out_cap, size) != 0) return;
  // totals fit in out_cap <= INT32_MAX, so every offset fits in int32
  for (int32_t j = j0; j < j1; ++j) {
    const Growth g{pg[j], tok[j]};
    tok[j] = (int32_t)nt;
    pg[j] = (int32_t)np;
    nt += g.tokens();
    np += g.pages(shift);
  }
  if (tid == 0) tok[bs] = (int32_t)tt;
  __syncthreads();

  const int32_t mask = (1 << shift) - 1;
  for (int64_t k = (int64_t)blockIdx.x * kAllocThreads + tid; k < tt; k += (int64_t)gridDim.x * kAllocThreads) {
    int32_t lo = 0, hi = bs;  // tok[lo] <= k < tok[hi]
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (tok[mid] <= k) lo = mid;
      else hi = mid;
    }
    const Growth g = growth(prefix, seq, lo);
    const int64_t t = g.p + (k - tok[lo]);
    const int32_t held = pages_spanned(g.p, shift);
    const int64_t pidx = t >> shift;
    int64_t page;
    if (pidx < held) {
      page = (int64_t)last_loc[lo] >> shift;  // the partly used last page
    } else {
      page = ring[ring_index(head + pg[lo] + (pidx - held), cap)];
    }
    out[k] = (int32_t)((page << shift) + (t & mask));
  }
}

__global__ void __launch_bounds__(kWideThreads) alloc_commit_kernel(int32_t shift, int32_t bs,
                                                                    const int32_t* __restrict__ prefix,
                                                                    const int32_t* __restrict__ seq, int64_t cap,
                                                                    int32_t* __restrict__ state, int64_t out_cap,
                                                                    int32_t* __restrict__ status) {
  __shared__ int64_t sh[2 * (kWideThreads / 64)];
  const int64_t head = state[0], size = state[1];
  const GrowthTotals g = growth_totals<kWideThreads>(prefix, seq, bs, shift, sh);
  if (threadIdx.x != 0) return;
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

// Freed slots usually come a request's row at a time, so neighbouring lanes
// mostly hit the same page and the same bitmap word.  Lanes OR their bits
// over each run of equal words (a segmented scan across the wavefront) and
// only the run's last lane issues the atomic: one atomic per word per wave
// instead of one per slot.
__global__ void __launch_bounds__(kAllocThreads) free_mark_kernel(int32_t shift, const int32_t* __restrict__ slots,
                                                                  int64_t n, int64_t num_pages,
                                                                  uint32_t* __restrict__ bits) {
  const int lane = threadIdx.x & 63;
  for (int64_t base = (int64_t)blockIdx.x * kAllocThreads + (threadIdx.x & ~63); base < n;
       base += (int64_t)gridDim.x * kAllocThreads) {
    const int64_t k = base + lane;
    int64_t word = -1;
    uint32_t v = 0;
    if (k < n) {
      const int32_t s = slots[k];
      const int64_t page = (int64_t)s >> shift;
      if (s >= 0 && page < num_pages) {  // the padding page and beyond never go back
        word = page >> 5;
        v = 1u << (page & 31);
      }
    }
    // every lane takes part in both shuffles (a lane that skipped one would
    // hand its neighbour 0 instead of its word)
    const int64_t word_up = __shfl_up(word, 1, 64), word_dn = __shfl_down(word, 1, 64);
    int f = lane == 0 || word_up != word;  // a run starts here
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t vu = __shfl_up(v, d, 64);
      const int fu = __shfl_up(f, d, 64);
      if (lane >= d && !f) {
        v |= vu;
        f |= fu;
      }
    }
    const bool last = lane == 63 || word_dn != word;
    if (last && word >= 0) atomicOr(bits + word, v);
  }
}

// One block; thread t owns a contiguous run of words, so one block scan of
// the per-thread bit counts places every page, in increasing order.
__global__ void __launch_bounds__(kWideThreads) free_compact_kernel(const uint32_t* __restrict__ bits,
                                                                    int64_t words, int32_t* __restrict__ ring,
                                                                    int64_t cap, int32_t* __restrict__ state,
                                                                    int32_t* __restrict__ status) {
  __shared__ int64_t sh[2 * (kWideThreads / 64)];
  const int tid = threadIdx.x;
  const int64_t head = state[0], size = state[1];
  const int64_t wpt = (words + kWideThreads - 1) / kWideThreads;
  const int64_t w0 = min((int64_t)tid * wpt, words), w1 = min(w0 + wpt, words);
  int64_t cnt = 0, zero = 0;
  for (int64_t k = w0; k < w1; ++k) cnt += __popc(bits[k]);
  int64_t total, unused;
  block_scan2<kWideThreads>(cnt, zero, total, unused, sh);
  if (size + total > cap) {
    if (tid == 0) *status = 4;  // PKV_ALLOC_RING_FULL
    return;
  }
  int64_t pos = head + size + cnt;
  for (int64_t k = w0; k < w1; ++k) {
    uint32_t rest = bits[k];
    while (rest) {
      const int b = __ffs(rest) - 1;
      rest &= rest - 1;
      ring[ring_index(pos++, cap)] = (int32_t)((k << 5) + b);
    }
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
// the requests before it.
//
// New slots: block (g, y) takes requests 256 g .. 256 g + 255, scans their
// new-token counts in LDS, and writes their new tokens y * kRowChunk ..
// (+ gridDim.y * kRowChunk ...); each token finds its request by binary
// search.  The new tokens of earlier groups are summed by the block itself.
// A request with invalid lengths counts no tokens; one whose row is out of
// range or whose seq_len passes the row width writes none.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kAllocThreads) write_new_kernel(
    int32_t* __restrict__ table, int64_t rows, int64_t width, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq, const int32_t* __restrict__ out_loc,
    int64_t n_out, int32_t bs) {
  __shared__ int64_t off[kAllocThreads + 1];
  __shared__ int64_t sh[2 * (kAllocThreads / 64)];
  const int tid = threadIdx.x;
  const int32_t g0 = blockIdx.x * kAllocThreads;
  const int32_t n_in = min(kAllocThreads, bs - g0);
  int64_t e = 0, zero = 0;
  if (tid < n_in) {
    const int64_t p = prefix[g0 + tid], s = seq[g0 + tid];
    if (p >= 0 && s >= p) e = s - p;
  }
  int64_t tot, unused;
  block_scan2<kAllocThreads>(e, zero, tot, unused, sh);
  off[tid] = e;
  if (tid == 0) off[kAllocThreads] = tot;
  const int64_t k_begin = (int64_t)blockIdx.y * kRowChunk;
  if (k_begin >= tot) return;  // block-uniform
  int64_t acc = 0;
#pragma unroll 4
  for (int32_t j = tid; j < g0; j += kAllocThreads) {
    const int64_t p = prefix[j], s = seq[j];
    if (p >= 0 && s >= p) acc += s - p;
  }
  int64_t base;
  block_scan2<kAllocThreads>(acc, zero, base, unused, sh);  // also publishes off[]
  for (int64_t k0 = k_begin; k0 < tot; k0 += (int64_t)gridDim.y * kRowChunk) {
    const int64_t k1 = min(k0 + kRowChunk, tot);
    for (int64_t k = k0 + tid; k < k1; k += kAllocThreads) {
      int32_t lo = 0, hi = n_in;  // off[lo] <= k < off[hi]
      while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (off[mid] <= k) lo = mid;
        else hi = mid;
      }
      const int32_t j = g0 + lo;
      const int64_t p = prefix[j], s = seq[j], r = rpi[j];
      const int64_t q = base + k;
      if (s <= width && r >= 0 && r < rows && q < n_out) table[r * width + p + (k - off[lo])] = out_loc[q];
    }
  }
}

// Prefix slots: block (i, c) copies columns [c * kRowChunk, ...) of request
// i's prefix from its buffer.
__global__ void __launch_bounds__(kAllocThreads) write_prefix_kernel(int32_t* __restrict__ table, int64_t rows,
                                                                     int64_t width, const int32_t* __restrict__ rpi,
                                                                     const int32_t* __restrict__ prefix,
                                                                     const int32_t* __restrict__ seq,
                                                                     const int32_t* const* __restrict__ prefix_ptrs) {
  const int32_t i = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * kRowChunk;
  const int64_t p = prefix[i], s = seq[i], r = rpi[i];
  if (p < 0 || s < p || s > width || r < 0 || r >= rows || c0 >= p) return;
  const int32_t* pre = prefix_ptrs[i];
  if (!pre) return;
  int32_t* row = table + r * width;
  const int64_t end = min(c0 + kRowChunk, p);
  for (int64_t col = c0 + threadIdx.x; col < end; col += kAllocThreads) row[col] = pre[col];
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

// Blocks for a grid-stride loop over `items` at `per_thread` items a thread.
int grid_for(int64_t items, int per_thread = 4) {
  const int64_t b = (items + kAllocThreads * per_thread - 1) / (kAllocThreads * per_thread);
  return (int)(b < 1 ? 1 : (b > kAllocMaxBlocks ? kAllocMaxBlocks : b));
}

}  // namespace

hipError_t launch_alloc_extend(int32_t shift, int32_t bs, const int32_t* prefix, const int32_t* seq,
                               const int32_t* last_loc, int32_t* ring, int32_t cap, int32_t* state, int32_t* out,
                               int64_t out_cap, int32_t* status, hipStream_t s) {
  if (bs > 0) {
    const size_t lds = (size_t)(bs + 1) * 2 * sizeof(int32_t);
    // one new token per thread: the per-token chain (binary search, then
    // the request's lengths, then the ring entry) is latency, not bandwidth
    hipLaunchKernelGGL(alloc_extend_kernel, dim3(grid_for(out_cap, 1)), dim3(kAllocThreads), lds, s, shift, bs,
                       prefix, seq, last_loc, ring, (int64_t)cap, state, out, out_cap);
  }
  hipLaunchKernelGGL(alloc_commit_kernel, dim3(1), dim3(kWideThreads), 0, s, shift, bs, prefix, seq, (int64_t)cap,
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
  hipLaunchKernelGGL(free_compact_kernel, dim3(1), dim3(kWideThreads), 0, s, bits, words, ring, (int64_t)cap,
                     state, status);
  return hipGetLastError();
}

hipError_t launch_write_rows(int32_t* table, int64_t rows, int64_t width, const int32_t* rpi, const int32_t* prefix,
                             const int32_t* seq, const int32_t* out_loc, int64_t n_out,
                             const int32_t* const* prefix_ptrs, int32_t bs, int32_t max_seq_len, hipStream_t s) {
  if (bs == 0) return hipSuccess;
  if (prefix_ptrs && max_seq_len > 0) {
    const unsigned chunks = (unsigned)(((int64_t)max_seq_len + kRowChunk - 1) / kRowChunk);
    hipLaunchKernelGGL(write_prefix_kernel, dim3((unsigned)bs, chunks), dim3(kAllocThreads), 0, s, table, rows, width,
                       rpi, prefix, seq, prefix_ptrs);
  }
  if (n_out > 0) {
    const int64_t chunks = (n_out + kRowChunk - 1) / kRowChunk;
    const unsigned groups = (unsigned)((bs + kAllocThreads - 1) / kAllocThreads);
    hipLaunchKernelGGL(write_new_kernel, dim3(groups, (unsigned)(chunks < 4096 ? chunks : 4096)), dim3(kAllocThreads),
                       0, s, table, rows, width, rpi, prefix, seq, out_loc, n_out, bs);
  }
  return hipGetLastError();
}

hipError_t launch_free_list_init(int32_t* ring, int32_t first, int32_t count, int32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(free_list_init_kernel, dim3(grid_for(count)), dim3(kAllocThreads), 0, s, ring, count, first,
                     state);
  return hipGetLastError();
}

}  // namespace pkv
