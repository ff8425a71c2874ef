// Stream split for decode: the pieces shared by the MLA and the grouped-query
// decode kernels.
//
// What is computed: nothing of the attention itself -- this file lays the
// requests' key tiles (32 logical positions each) end to end, cuts the
// sequence into equal runs, one per workgroup (or group of workgroups), and
// resolves every tile to its slot ids through the request's table ([XPU]
// "From slots to a page table"; [BACKEND] init_forward_metadata).  A run
// may end inside a request; the pieces a request is cut into are merged
// exactly with log-sum-exp weights (the split/merge identity of the decode
// split-K, here with splits placed by the run boundaries).  Piece (run r,
// request i) has workspace id r + i: runs and requests are both in order,
// so (r, i) -> r + i is one-to-one over the pieces that exist.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "pkv_launch.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Planner: workgroup (i, c) resolves tiles kPlanTiles c .. of request i,
// one thread per key position, and writes their info words {request, tile,
// tiles of request, tile prefix, valid keys}; tokens past the request's end
// repeat its last key, whose weight is then exactly 0.  Every workgroup sums
// the tile counts itself (bs loads), so the planner is one launch with no
// serial pass; workgroup (i, 0) also writes the request's prefix, tile count
// and fallback flag, and (0, 0) the run length Bt and the tile total.
// ---------------------------------------------------------------------------
// Tiles per planner workgroup (256 threads: eight tiles at a time).  A
// workgroup's fixed cost (the O(bs) sums) and the empty workgroups past
// short requests' ends are what the planner spends its time on, so each
// takes several passes.
constexpr int kPlanTiles = 64;

__device__ __forceinline__ int32_t stream_tiles(int32_t L) { return L > 0 ? (L + kStreamT - 1) / kStreamT : 0; }

// With `skip` (cascade decode), request i's first skip[i] keys (a multiple
// of the tile) are left out: its tiles start at key skip[i].
__device__ __forceinline__ int32_t skip_tiles(const int32_t* skip, int32_t i, int32_t T) {
  return skip ? min(max(skip[i], 0) / kStreamT, T) : 0;
}

// Keys request k leaves to the prefix pass when the decode found the shared
// prefixes itself: its own shared keys, or for its group's reference member
// the most any other member shares (capped at the reference's length,
// rounded up to the tile).
__device__ __forceinline__ int32_t share_skip(const ShareArgs& a, const int32_t* kv_lens, int32_t k) {
  const int32_t s = a.s[k];
  if (s >= 0) return s;
  int32_t best = 0;
  const int32_t g0 = a.gs[k], g1 = a.ge[k];
  // eight members' entries are loaded at a time (a group spans at most 64
  // requests), unconditionally at clamped indices so that no branch on a
  // loaded value separates the loads; the reference's own entry is -1
  for (int32_t j0 = g0; j0 < g1; j0 += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.s[min(j0 + u, g1 - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u < g1 ? v[u] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) best = max(best, v[u]);
  }
  const int32_t L = max(kv_lens[k], 0);
  return min(best, (L + kStreamT - 1) / kStreamT * kStreamT);
}

// The prefix pass's work items for the group request k starts (0 when k
// starts no group, or the group shares nothing): slices of ms members times
// ch chunks.  *E_out: the prefix keys the group's reference reads.
__device__ __forceinline__ int32_t group_items(const ShareArgs& a, const int32_t* kv_lens, int32_t k, int32_t* E_out,
                                               int32_t* ref_out) {
  *E_out = 0;
  *ref_out = -1;
  if (a.gs[k] != k) return 0;
  const int32_t g1 = a.ge[k];
  if (g1 - k < 2) return 0;
  int32_t ref = -1, best = 0;
  for (int32_t j0 = k; j0 < g1; j0 += 8) {  // eight entries loaded at a time, as in share_skip
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.s[min(j0 + u, g1 - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u < g1 ? v[u] : 0;
    // (selects, not branches: a branch on a loaded value waits for it
    // before the next load is issued; best >= 0 absorbs the -1)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ref = v[u] < 0 ? j0 + u : ref;
      best = max(best, v[u]);
    }
  }
  if (ref < 0) return 0;
  const int32_t L = max(kv_lens[ref], 0);
  const int32_t E = min(L, min(best, (L + kStreamT - 1) / kStreamT * kStreamT));
  *E_out = E;
  *ref_out = ref;
  return E > 0 ? (g1 - k + a.ms - 1) / a.ms * a.ch : 0;
}

// tiles left out at the start of request k (T: its tiles)
__device__ __forceinline__ int32_t left_out(const int32_t* skip, const ShareArgs& a, const int32_t* kv_lens,
                                            int32_t k, int32_t T) {
  if (a.s) return min(share_skip(a, kv_lens, k) / kStreamT, T);
  return skip_tiles(skip, k, T);
}

template <int FMT>
__global__ void __launch_bounds__(256) stream_plan_kernel(DevMap m, int32_t bs, int32_t max_tiles, int32_t runs,
                                                       int32_t* __restrict__ header,
                                                       int32_t* __restrict__ prefix, int32_t* __restrict__ ntiles,
                                                       int32_t* __restrict__ fallback, int32_t* __restrict__ meta,
                                                       const int32_t* __restrict__ skip, StoreArgs app,
                                                       ShareArgs share) {
  __shared__ int32_t red[2][4];
  const int i = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x;
  if (i >= bs) {  // blocks past the batch carry the step's KV append
    if (c == 0) store_one_row(app, (int64_t)(i - bs) * kStoreRowsPerBlock + (tid >> 6), tid & 63);
    return;
  }
  const int32_t T_all = min(stream_tiles(m.kv_lens[i]), max_tiles);
  const bool lead = c == 0;
  if (!lead && c * kPlanTiles >= T_all) return;  // past the request's tiles (uniform per workgroup)
  // keys and tiles left out at the start
  const int32_t sk = share.s ? share_skip(share, m.kv_lens, i) : 0;
  const int32_t st = share.s ? min(sk / kStreamT, T_all) : skip_tiles(skip, i, T_all);
  const int32_t T = T_all - st;
  if (!lead && c * kPlanTiles >= T) return;
  if (lead && share.s) {
    // this request's skip, and the prefix pass's work if a shared group
    // starts here: slices of ms members times ch chunks of the group's
    // prefix keys [0, E) (chunks past the prefix's tiles hold no tiles;
    // their results are empty), listed after the work of every group that
    // starts earlier in the batch
    int32_t base = 0;
    for (int k = tid; k < i; k += 256) {
      int32_t e, r;
      base += group_items(share, m.kv_lens, k, &e, &r);
    }
    for (int o = 32; o > 0; o >>= 1) base += __shfl_xor(base, o, 64);
    if ((tid & 63) == 0) red[0][tid >> 6] = base;
    __syncthreads();
    base = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    __syncthreads();  // red is reused by the tile sums below
    int32_t E, ref;
    const int32_t cnt = group_items(share, m.kv_lens, i, &E, &ref);
    if (tid == 0) {
      share.skip[i] = sk;
      if (i == bs - 1) *share.count = base + cnt;
    }
    const int32_t tiles = (E + kStreamT - 1) / kStreamT;
    const int32_t tpc = (tiles + share.ch - 1) / share.ch;
    const ReqView rv = cnt > 0 ? request_view(m, ref) : ReqView{0, 0};
    for (int t = tid; t < cnt; t += 256) {
      const int32_t sl = t / share.ch, ck = t % share.ch;
      const int32_t i0 = i + sl * share.ms;
      PrefixItem it;
      it.i0 = i0;
      it.i1 = min(share.ge[i], i0 + share.ms);
      it.ref = ref;
      it.E = E;
      it.t0 = min(ck * tpc, tiles);
      it.t1 = min(ck * tpc + tpc, tiles);
      it.c = ck;
      it.limit = rv.limit;
      it.off_lo = (int32_t)(uint32_t)(uint64_t)rv.off;
      it.off_hi = (int32_t)(rv.off >> 32);
      it.pad0 = it.pad1 = 0;
      share.items[base + t] = it;
    }
  }
  int32_t tot = 0, pre = 0;
  for (int k = tid; k < bs; k += 256) {
    const int32_t Tk_all = min(stream_tiles(m.kv_lens[k]), max_tiles);
    const int32_t Tk = Tk_all - left_out(skip, share, m.kv_lens, k, Tk_all);
    tot += Tk;
    if (k < i) pre += Tk;
  }
  for (int o = 32; o > 0; o >>= 1) {
    tot += __shfl_xor(tot, o, 64);
    pre += __shfl_xor(pre, o, 64);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = tot;
    red[1][tid >> 6] = pre;
  }
  __syncthreads();
  tot = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  pre = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  // keys past max_kv_len (a caller error) are not read: the workspace holds
  // max_tiles tiles per request
  const int32_t L = min(max(m.kv_lens[i], 0), T_all * kStreamT);
  if (lead && tid == 0) {
    prefix[i] = pre;
    ntiles[i] = T;
    fallback[i] = 0;
    if (i == 0) {
      header[0] = max(1, (tot + runs - 1) / runs);
      header[1] = tot;
    }
  }
  // Thread tid takes key tid % 32 of tiles j0, j0 + 8, ...: every table
  // load of the workgroup is issued before the first store, so the loads
  // cost one latency instead of one per pass.
  const SlotMap<FMT> sm = make_slotmap<FMT>(m, i);
  const int j_end = min(T, (c + 1) * kPlanTiles);
  const int j0 = c * kPlanTiles + (tid >> 5);
  const int f = tid & 31;
  constexpr int kPasses = kPlanTiles / (256 / 32);
  int32_t key[kPasses], raw[kPasses];
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int32_t jt = st + j0 + u * (256 / 32);  // key tile
    key[u] = min(jt * kStreamT + f, L - 1);
    raw[u] = sm.raw(key[u]);
  }
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int j = j0 + u * (256 / 32);
    if (j < j_end) {
      int32_t* tile = meta + (int64_t)(pre + j) * kStreamMetaWords;
      const int32_t jt = st + j;
      tile[f] = sm.finish(raw[u], key[u], true);
      if (f < 8) {
        int32_t v = 0;
        if (f == 0) v = i;
        else if (f == 1) v = j;
        else if (f == 2) v = T;
        else if (f == 3) v = pre;
        else if (f == 4) v = min(kStreamT, L - jt * kStreamT);
        tile[32 + f] = v;
      }
    }
  }
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// [header | tile prefix[bs] | tiles[bs] | fallback flags[bs] | meta[bs * max tiles][40] |
//  pieces o[(runs + bs) * Hq * Dv] | pieces lse[(runs + bs) * Hq]]
size_t stream_ws_layout(int32_t bs, int32_t max_tiles, int32_t runs, int32_t Hq, int32_t Dv, void* base,
                        StreamWs* w) {
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* at = b ? b + off : nullptr;
    off += al256(bytes);
    return at;
  };
  char* hdr = take(256);
  char* pre = take((size_t)bs * 4);
  char* nt = take((size_t)bs * 4);
  char* fb = take((size_t)bs * 4);
  char* meta = take((size_t)bs * max_tiles * kStreamMetaWords * 4);
  const size_t pieces = (size_t)runs + bs;
  char* o = take(pieces * Hq * Dv * 4);
  char* l = take(pieces * Hq * 4);
  if (w) {
    w->header = reinterpret_cast<int32_t*>(hdr);
    w->prefix = reinterpret_cast<int32_t*>(pre);
    w->ntiles = reinterpret_cast<int32_t*>(nt);
    w->fallback = reinterpret_cast<int32_t*>(fb);
    w->meta = reinterpret_cast<int32_t*>(meta);
    w->o = reinterpret_cast<float*>(o);
    w->lse = reinterpret_cast<float*>(l);
  }
  return off;
}

hipError_t launch_stream_plan(const DevMap& m, int32_t bs, int32_t max_tiles, int32_t runs, const StreamWs& w,
                              hipStream_t s, const int32_t* skip, const StoreArgs* st, const ShareArgs* share) {
  StoreArgs a{};
  if (st) a = *st;
  ShareArgs sh{};
  if (share) sh = *share;
  const int64_t store_blocks = (a.n + kStoreRowsPerBlock - 1) / kStoreRowsPerBlock;
  const dim3 grid((unsigned)(bs + store_blocks), (unsigned)std::max(1, (max_tiles + kPlanTiles - 1) / kPlanTiles));
  if (m.fmt == MAP_TOKEN_TABLE)
    hipLaunchKernelGGL(stream_plan_kernel<SLOT_TABLE>, grid, dim3(256), 0, s, m, bs, max_tiles, runs, w.header,
                       w.prefix, w.ntiles, w.fallback, w.meta, skip, a, sh);
  else
    hipLaunchKernelGGL(stream_plan_kernel<SLOT_PAGES>, grid, dim3(256), 0, s, m, bs, max_tiles, runs, w.header,
                       w.prefix, w.ntiles, w.fallback, w.meta, skip, a, sh);
  return hipGetLastError();
}

// One workgroup per CU of the current device.  The count is cached per
// device in atomics: threads making their first call at once may each ask
// the runtime, and all store the same value.
int32_t device_cu_count() {
  static std::atomic<int32_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int32_t n = cached[dev].load(std::memory_order_acquire);
  if (n == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    n = c;
    cached[dev].store(n, std::memory_order_release);
  }
  return n;
}

}  // namespace pkv
