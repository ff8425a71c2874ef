// Paged decode attention for grouped-query heads: the split plans, the
// split-K partial kernels and the log-sum-exp merges.
//
// What is computed ([XPU] "From slots to a page table"; [BACKEND]
// init_forward_metadata with its per-request split count): one new query per
// request attends over its L keys; key t of request i lives at the slot the
// request's table resolves t to.  The keys are cut into pieces at *logical*
// positions; each piece produces a normalised partial output and its
// log-sum-exp, and the merge combines them exactly.  Piece boundaries depend
// only on logical positions (the request lengths), never on where pages
// live, so moving pages around cannot change a single bit of the output.
//
// bf16 pools (pool [slots][Hkv][D], token-major): stream split.  The stream
// planner (pkv_stream.hip) lays all requests' 32-key tiles end to end and
// cuts the sequence into equal runs; each run is streamed by hg workgroups
// (one per group of WAVES KV heads) on one XCD.  Wave w owns KV head g and
// its G = Hq / Hkv query heads:
//   S^T[16 tokens x 16 heads] = K_tile[16 x D] * Q^T[D x 16] on
//   v_mfma_f32_16x16x32_bf16 (tokens as M, so K rows load from HBM straight
//   into A-operand registers); softmax on the MFMA output registers; P
//   (16 heads x 32 tokens) is already the A operand of the PV product; V
//   goes through LDS and comes back transposed with ds_read_b64_tr_b16, four
//   tokens of one d column per lane per read.
// f32 pools: per-request splits of `chunk` logical positions listed by a
// one-block planner (live (request, split) items in request order; block b
// takes item b / hg and KV-head group b % hg), VALU dot products with 16
// lanes per token.
#include <math.h>

#include <algorithm>

#include "pkv_launch.h"

namespace pkv {

constexpr int kTile = 32;  // tokens per tile of the bf16 kernel

// ---------------------------------------------------------------------------
// split plan of the f32 path: live items in request order; an empty request
// still gets one item, which writes its zero output and -inf lse.  Each item
// carries what a split needs to start streaming at once (its request's table
// view and key range), so the split kernel's first dependent loads are the
// table entries.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) decode_plan_kernel(DevMap m, int32_t bs, int32_t chunk, int32_t max_splits,
                                                           WorkItem* __restrict__ items, int32_t* __restrict__ count) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0;
  for (int32_t base = 0; base < bs; base += 1024) {
    const int32_t i = base + tid;
    int32_t n = 0, L = 0;
    if (i < bs) {
      L = m.kv_lens[i];
      n = L > 0 ? min((L + chunk - 1) / chunk, max_splits) : 1;
    }
    int32_t x = n;  // inclusive wave scan
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int32_t w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int32_t y = __shfl_up(w, d, 64);
        if (lane >= d) w += y;
      }
      if (lane < 16) wsum[lane] = w;  // inclusive over waves
    }
    __syncthreads();
    const int32_t off = carry + (wave > 0 ? wsum[wave - 1] : 0) + x - n;
    if (n > 0) {
      const ReqView v = request_view(m, i);
      const int32_t ns = L > 0 ? n : 0;
      for (int32_t s = 0; s < n; ++s) {
        WorkItem w;
        w.i = i;
        w.s = s;
        w.ns = ns;
        w.t_end = min((s + 1) * chunk, L);
        w.limit = v.limit;
        w.off_lo = (int32_t)(v.off & 0xffffffff);
        w.off_hi = (int32_t)(v.off >> 32);
        w.pad = 0;
        items[off + s] = w;
      }
    }
    carry += wsum[15];
    __syncthreads();
  }
  if (tid == 0) *count = carry;
}

// ---------------------------------------------------------------------------
// bf16 tile helpers.  Per wavefront and 32-token tile: the tile's 32 slot
// ids sit in lanes 0..31 of one register and reach the lanes that need them
// by ds_bpermute; K rows go straight into MFMA A-operand registers, V rows
// into registers (decode_issue); decode_compute does the tile's math.
// ---------------------------------------------------------------------------
template <int D>
struct DecodeTile {
  static constexpr int NK = D / 32;        // MFMAs along d for S
  static constexpr int CPT = D / 8;        // 16-byte chunks per head slice
  static constexpr int TPI = 64 / CPT;     // tokens per V load instruction
  static constexpr int VIT = kTile / TPI;  // V load instructions per tile
  bf16x8 k[2][NK];
  u32x4 v[VIT];
};

template <int D>
__device__ __forceinline__ void decode_issue(DecodeTile<D>& T, int32_t tile_slot, int lane, const bf16* kb,
                                             const bf16* vb, int64_t row_elems) {
  constexpr int NK = DecodeTile<D>::NK, CPT = DecodeTile<D>::CPT, TPI = DecodeTile<D>::TPI;
  constexpr int VIT = DecodeTile<D>::VIT;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t slot = shfl_i(tile_slot, a * 16 + col);
    // MFMA kk takes d = kk*32 + grp*8 .. +8: the 4 lanes of a token read 64
    // contiguous bytes per instruction
    const bf16* kp = kb + slot * row_elems + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) T.k[a][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + kk * 32));
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int64_t slot = shfl_i(tile_slot, it * TPI + lane / CPT);
    T.v[it] = *reinterpret_cast<const u32x4*>(vb + slot * row_elems + (lane % CPT) * 8);
  }
}

template <int D>
__device__ __forceinline__ void decode_compute(const DecodeTile<D>& T, int t0, int t_end, int lane, const bf16x8* qb,
                                               float scale_log2, bf16* vt, f32x4* acc, float& m_run, float& l_run) {
  constexpr int NK = DecodeTile<D>::NK, CPT = DecodeTile<D>::CPT, TPI = DecodeTile<D>::TPI;
  constexpr int VIT = DecodeTile<D>::VIT;
  constexpr int NT = D / 16;
  constexpr int LDS = D + 8;
  const int grp = lane >> 4;
  // ---- S^T = K Q^T  (rows: tokens a*16 + 4*grp + rr; column: head lane & 15)
  f32x4 sacc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) sacc[a] = mfma16x16x32(T.k[a][kk], qb[kk], sacc[a]);
  }
  // ---- V tile to LDS; keys past the end hold 0 (P * NaN would poison the sum)
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int row = it * TPI + lane / CPT;
    const bool ok = t0 + row < t_end;
    u32x4 w = T.v[it];
    if (!ok) w = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(vt + row * LDS + (lane % CPT) * 8) = w;
  }
  // ---- online softmax (log2 domain)
  float sv[2][4];
  float mt = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = t0 + a * 16 + grp * 4 + rr;
      const float x = (t < t_end) ? sacc[a][rr] * scale_log2 : -INFINITY;
      sv[a][rr] = x;
      mt = fmaxf(mt, x);
    }
  mt = fmaxf(mt, shfl_xor(mt, 16));
  mt = fmaxf(mt, shfl_xor(mt, 32));
  const float m_new = fmaxf(m_run, mt);
  const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
  float psum = 0.f;
  bf16x8 pa;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float p = fast_exp2(sv[a][rr] - m_new);
      psum += p;
      pa[a * 4 + rr] = (bf16)p;
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  // rows of acc are heads 4*grp + rr; their alpha lives in lane 4*grp + rr
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float ar = shfl(alpha, grp * 4 + rr);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt][rr] *= ar;
  }
  __builtin_amdgcn_wave_barrier();
  // ---- O += P V.  B operand of lane (col, grp) = V[a*16 + 4*grp + rr][nt*16 + col]
  // for a = 0, 1 and rr = 0..3: two transposed LDS reads
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16x16x32(pa, lds_v_operand(vt, LDS, 0, nt * 16, lane), acc[nt]);
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// bf16 MFMA stream-split kernel.  The hg workgroups of a run are 8 blocks
// apart (block b: run (b / 8hg) * 8 + b % 8, KV-head group (b / 8) % hg);
// wave w owns KV head group * WAVES + w.  A wave streams its run
// tile after tile across request boundaries with NS register tile sets (NS - 1
// tiles in flight during a tile's math), so no split restarts its pipeline and
// every CU streams the same number of bytes.  Per tile the wave loads the
// planner's 40 words (slot ids in lanes 0..31, info in lanes 32..36), the K
// and V rows and the queries of the tile's request (the queries ride along
// with every tile so that no load is conditional).  A request finished inside
// the run is written directly; one cut by a run boundary leaves a piece
// (id run + request) for the merge.
// ---------------------------------------------------------------------------
// Minimum workgroups per CU the stream kernels are compiled for.  At D =
// 128 four waves with three tile sets need a whole SIMD's registers (VGPRs
// and AGPRs) each, so W = 4 is one workgroup per CU.  Narrower workgroups (KV
// head counts not divisible by 4) share a CU with their siblings, as the
// plan's run count assumes, but are still given a whole SIMD's registers
// per wave: asking for 4 / W workgroups would cap each wave at 256 or 128
// registers and spill the tile sets.
constexpr int stream_min_blocks(int waves, int ns) { return waves >= 4 ? (ns <= 2 ? 8 / waves : 4 / waves) : 1; }

template <int D>
struct StreamSet {
  DecodeTile<D> t;
  bf16x8 q[D / 32];
  // the planner's words for the tile: request, key tile within it, the
  // request's tile count and first tile in the stream, valid keys
  int i, jt, T, P, valid;
};

// One run of the stream, by workgroup `bid` (vt: this wave's V tile in LDS;
// prefix_skip: per request the keys a shared-prefix pass reads instead).
template <int D, int WAVES, int NS>
__device__ __forceinline__ void stream_run(
    int bid, bf16* vt, const bf16* k_pool, const bf16* v_pool, const bf16* __restrict__ q, int32_t Hq, int32_t Hkv,
    int32_t G, int32_t hg, const int32_t* __restrict__ header, const int32_t* __restrict__ meta, float scale_log2,
    bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    const int32_t* __restrict__ prefix_skip) {
  constexpr int NK = D / 32;
  constexpr int NT = D / 16;

  // the hg workgroups of a run sit on one XCD (dispatch goes round robin
  // over the 8 XCDs), so the halves of a slot's row meet in one L2
  const int run = (bid / (8 * hg)) * 8 + bid % 8;
  const int Bt = header[0], total = header[1];
  const int G0 = run * Bt;
  if (G0 >= total) return;
  const int n = min(Bt, total - G0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = ((bid / 8) % hg) * WAVES + wave;
  const int64_t row_elems = (int64_t)Hkv * D;
  const bf16* kb = k_pool + (int64_t)g * D;
  const bf16* vb = v_pool + (int64_t)g * D;
  const bool qok = col < G;

  auto meta_word = [&](int r) -> int32_t {
    return meta[(int64_t)(G0 + min(r, n - 1)) * kStreamMetaWords + min(lane, kStreamMetaWords - 1)];
  };
  // (the planner words are read out of mv here, so that mv is dead once
  // the tile is issued and its register can take the next word's load)
  auto issue = [&](StreamSet<D>& S, int32_t mv) {
    decode_issue<D>(S.t, mv, lane, kb, vb, row_elems);
    const int i = __builtin_amdgcn_readlane(mv, 32);
    S.i = i;
    S.jt = __builtin_amdgcn_readlane(mv, 33);
    S.T = __builtin_amdgcn_readlane(mv, 34);
    S.P = __builtin_amdgcn_readlane(mv, 35);
    S.valid = __builtin_amdgcn_readlane(mv, 36);
    // columns past G read the group's first query row: finite scores in
    // columns no output row reads (a column's softmax and its P*V column
    // use only that column).  Zeroing them instead is a select on the
    // loaded value, which makes the compiler wait for these loads, and
    // so for every load issued before them, at the loop's back edge.
    const bf16* qp = q + ((int64_t)i * Hq + g * G + (qok ? col : 0)) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) S.q[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 32));
  };

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto finish = [&](int i, int P, int T) {
    const int b0 = P / Bt, b1 = (P + T - 1) / Bt;
    // (a request part of whose keys the prefix pass reads is merged
    // afterwards: its result is a piece)
    const bool direct = b0 == b1 && prefix_skip[i] == 0;
    float l_tot = l_run + shfl_xor(l_run, 16);
    l_tot += shfl_xor(l_tot, 32);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hr = grp * 4 + rr;
      const float lt = shfl(l_tot, hr);
      const float mr = shfl(m_run, hr);
      if (hr < G) {
        const int h = g * G + hr;
        const float inv = 1.0f / lt;
        const float lse_nat = (mr + __log2f(lt)) * kLn2;
        if (direct) {
          const int64_t o = (int64_t)i * Hq + h;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) out[o * D + nt * 16 + col] = (bf16)(acc[nt][rr] * inv);
          if (lse && col == 0) lse[o] = lse_nat;
        } else {
          const int64_t o = ((int64_t)run + i) * Hq + h;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) ws_o[o * D + nt * 16 + col] = acc[nt][rr] * inv;
          if (col == 0) ws_lse[o] = lse_nat;
        }
      }
    }
  };

  auto step = [&](int r, StreamSet<D>& cur) {
    const int i = cur.i, jt = cur.jt, T = cur.T, P = cur.P, valid = cur.valid;
    if (r == 0 || jt == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    decode_compute<D>(cur.t, 0, valid, lane, cur.q, scale_log2, vt, acc, m_run, l_run);
    if (r == n - 1 || jt == T - 1) finish(i, P, T);
  };

  StreamSet<D> S[NS];
  if (n < NS) {  // a short run: its tiles at once
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) issue(S[k], meta_word(k));
#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
      if (k < n) step(k, S[k]);
    return;
  }
  // Tile r sits in set r % NS and is issued NS - 1 tiles ahead of its use.
  // The loop runs whole rounds of NS tiles with no exit between them, and is
  // entered only when there is a round to run: a round that could stop
  // after any tile, or a loop that could be skipped, gives the compiler
  // paths on which a tile's loads were never issued (or spills the sets
  // across the skip), and the wait counts, which must hold on every path,
  // then drain the loads in flight at every round.  The last n % NS tiles,
  // issued by the loop, are taken afterwards.  (Issues past the end re-read
  // the run's last tile; nothing uses them.)
  // A tile's meta word is loaded two tiles before the tile is issued, into
  // M[tile % NS]: loads complete in order, so waiting for a word loaded one
  // tile earlier would also wait for the tile issued before it (the one
  // about to be computed), and the next issue could not go out ahead of it.
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) issue(S[k], meta_word(k));
  int32_t M[NS];
  M[(NS - 1) % NS] = meta_word(NS - 1);
  M[0] = meta_word(NS);
  int r = 0;
  do {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int32_t mv_new = meta_word(r + j + NS + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(S[(j + NS - 1) % NS], M[(j + NS - 1) % NS]);
      M[(j + 1) % NS] = mv_new;
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      step(r + j, S[j]);
    }
    r += NS;
  } while (r + NS <= n);
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (r + j < n) step(r + j, S[j]);
}

// ---------------------------------------------------------------------------
// Cascade decode over shared prefixes ([XPU] introduction and [MINI]: the
// requests of a group reuse the same prefix pages; [BACKEND]: split-K with a
// log-sum-exp merge).  Request i of group g splits its keys at S_g, the
// group's shared prefix length rounded down to the 32-key tile: keys
// [0, min(L_i, S_g)) are the same slots for every member, [S_g, L_i) its
// own.  The shared part is read once per group and KV head and scored
// against every member's queries together; the own part goes through the
// stream kernel with the first S_g keys skipped; a final merge combines the
// prefix chunks and the suffix pieces.  The result is the same attention as
// paged_decode_attn, with every shared K/V row leaving HBM once per group.
// ---------------------------------------------------------------------------

// The cascade's plan.  Blocks [0, nb): skip[i] = S_g for a member of group g
// (groups are increasing, disjoint ranges of the batch), 0 for a request in
// no group.  Block nb + g: group g's prefix work items, listed after those
// of every earlier group: min(ceil(members / ms), slices) slices of ms
// members times `chunks` chunks of the prefix keys [0, E), E = min(S_g, the
// longest member's length), read through the longest member's table (the
// first on ties; every member's prefix keys are among its keys).  The
// chunks split the group's own prefix tiles evenly; a chunk past them holds
// no tiles and its results are empty.  The last group's block writes the
// item count (block 0 does when there are no groups).
__global__ void __launch_bounds__(256) cascade_plan_kernel(DevMap m, const int32_t* __restrict__ group_indptr,
                                                           const int32_t* __restrict__ prefix_len,
                                                           int32_t num_groups, int32_t bs, int32_t ms,
                                                           int32_t slices, int32_t chunks,
                                                           int32_t* __restrict__ skip,
                                                           PrefixItem* __restrict__ items,
                                                           int32_t* __restrict__ count) {
  __shared__ int32_t red[3][4];
  const int tid = threadIdx.x;
  const int nb = (bs + 255) / 256;
  if ((int)blockIdx.x < nb) {
    if (num_groups == 0 && blockIdx.x == 0 && tid == 0) *count = 0;
    const int i = blockIdx.x * 256 + tid;
    if (i >= bs) return;
    int lo = 0, hi = num_groups;  // last g with group_indptr[g] <= i, in [lo, hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (group_indptr[mid] <= i) lo = mid;
      else hi = mid;
    }
    int32_t v = 0;
    if (num_groups > 0 && group_indptr[lo] <= i && i < group_indptr[lo + 1])
      v = max(prefix_len[lo], 0) & ~(kTile - 1);
    skip[i] = v;
    return;
  }
  const int g = (int)blockIdx.x - nb;
  auto n_slices = [&](int k) {
    const int a = max(group_indptr[k], 0), b = min(group_indptr[k + 1], bs);
    return b > a ? min((b - a + ms - 1) / ms, slices) : 0;
  };
  const int ga = max(group_indptr[g], 0), gb = min(group_indptr[g + 1], bs);
  int base = 0;
  for (int k = tid; k < g; k += 256) base += n_slices(k);
  // the longest member, the first on ties: the largest (L, -k)
  int bl = -1, bk = bs;
  for (int k = ga + tid; k < gb; k += 256) {
    const int L = max(m.kv_lens[k], 0);
    if (L > bl) {
      bl = L;
      bk = k;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    base += __shfl_xor(base, o, 64);
    const int ol = __shfl_xor(bl, o, 64), ok = __shfl_xor(bk, o, 64);
    if (ol > bl || (ol == bl && ok < bk)) {
      bl = ol;
      bk = ok;
    }
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = base;
    red[1][tid >> 6] = bl;
    red[2][tid >> 6] = bk;
  }
  __syncthreads();
  base = (red[0][0] + red[0][1] + red[0][2] + red[0][3]) * chunks;
  bl = red[1][0];
  bk = red[2][0];
  for (int w = 1; w < 4; ++w)
    if (red[1][w] > bl || (red[1][w] == bl && red[2][w] < bk)) {
      bl = red[1][w];
      bk = red[2][w];
    }
  const int cnt = n_slices(g) * chunks;
  if (g == num_groups - 1 && tid == 0) *count = base + cnt;
  if (cnt == 0) return;  // no member (uniform per workgroup)
  const int32_t S = max(prefix_len[g], 0) & ~(kTile - 1);
  const int32_t E = min(S, bl);
  const int32_t tiles = (E + kTile - 1) / kTile;
  const int32_t tpc = (tiles + chunks - 1) / chunks;
  const ReqView rv = request_view(m, bk);
  for (int t = tid; t < cnt; t += 256) {
    const int32_t sl = t / chunks, ck = t % chunks;
    const int32_t i0 = ga + sl * ms;
    PrefixItem it;
    it.i0 = i0;
    it.i1 = min(gb, i0 + ms);
    it.ref = bk;
    it.E = E;
    it.t0 = min(ck * tpc, tiles);
    it.t1 = min(ck * tpc + tpc, tiles);
    it.c = ck;
    it.limit = rv.limit;
    it.off_lo = (int32_t)(uint32_t)(uint64_t)rv.off;
    it.off_hi = (int32_t)(rv.off >> 32);
    it.pad0 = it.pad1 = 0;
    items[base + t] = it;
  }
}

// One tile of the shared prefix against NB blocks of 16 query rows.  Like
// decode_compute, with a key limit per query row (lane column) instead of
// one per tile, the V tile staged in LDS once for all blocks, and rows that
// have seen no key yet kept at m = -inf without NaNs.
template <int D, int NB>
__device__ __forceinline__ void cascade_tile(const DecodeTile<D>& T, int t0, int v_end, const int (&lim)[NB],
                                             int lane, const bf16x8 (&qb)[NB][D / 32], float scale_log2, bf16* vt,
                                             f32x4 (&acc)[NB][D / 16], float (&m_run)[NB], float (&l_run)[NB]) {
  constexpr int NK = DecodeTile<D>::NK, CPT = DecodeTile<D>::CPT, TPI = DecodeTile<D>::TPI;
  constexpr int VIT = DecodeTile<D>::VIT;
  constexpr int NT = D / 16;
  constexpr int LDS = D + 8;
  const int grp = lane >> 4;
  f32x4 sacc[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc[b][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) sacc[b][a] = mfma16x16x32(T.k[a][kk], qb[b][kk], sacc[b][a]);
    }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int row = it * TPI + lane / CPT;
    u32x4 w = T.v[it];
    if (t0 + row >= v_end) w = u32x4{0u, 0u, 0u, 0u};  // keys past the prefix: P = 0 there, V must not be NaN
    *reinterpret_cast<u32x4*>(vt + row * LDS + (lane % CPT) * 8) = w;
  }
  bf16x8 pa[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float sv[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float x = (t0 + a * 16 + grp * 4 + rr < lim[b]) ? sacc[b][a][rr] * scale_log2 : -INFINITY;
        sv[a][rr] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run[b], mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing seen yet: every p and alpha is 0
    const float alpha = fast_exp2(m_run[b] - m_use);
    float psum = 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float p = fast_exp2(sv[a][rr] - m_use);
        psum += p;
        pa[b][a * 4 + rr] = (bf16)p;
      }
    l_run[b] = l_run[b] * alpha + psum;
    m_run[b] = m_new;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float ar = shfl(alpha, grp * 4 + rr);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[b][nt][rr] *= ar;
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bf16x8 vop = lds_v_operand(vt, LDS, 0, nt * 16, lane);
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b][nt] = mfma16x16x32(pa[b], vop, acc[b][nt]);
  }
  __builtin_amdgcn_wave_barrier();
}

constexpr int kShareChunks = 4;  // chunks of a group's prefix in the prefix pass
constexpr int kCascadeCols = 32;  // query rows (member x head) per wave: two MFMA column blocks

// One prefix work item of the cascade: members [i0, i1) (consecutive
// requests of one group, up to 32 / G of them so their rows fill two
// 16-row MFMA column blocks) against tiles [t_begin, t_end) of the prefix
// keys [0, E), read through the table of the group's reference member
// (view rv; its keys [0, E) every member shares up to its own limit).  Row
// limits: min(kv_len, lim_arr[member]).
// Every (member, head) row gets a partial result in chunk slot c, o = 0 /
// lse = -inf where the chunk holds none of the member's prefix keys.
template <int D, int W, int FMT>
__device__ __forceinline__ void cascade_prefix_work(const DevMap& m, const bf16* k_pool, const bf16* v_pool,
                                                    const bf16* __restrict__ q, int32_t bs, int32_t Hq,
                                                    int32_t Hkv, int32_t G, int i0, int i1, ReqView rv,
                                                    const int32_t* lim_arr, int E, int t_begin, int t_end, int c,
                                                    int ms, float scale_log2, float* __restrict__ ws_po,
                                                    float* __restrict__ ws_plse, bf16* vt, int bid) {
  constexpr int NK = D / 32;
  constexpr int NT = D / 16;
  constexpr int NB = kCascadeCols / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int h = ((bid / 8) % (Hkv / W)) * W + wave;  // KV head

  // Lane l < 32 resolves key 32 t + l (keys past E, and tiles past t_end,
  // read the padding slot).  As in the stream kernel, three tile sets in
  // fixed registers: while tile t is computed, tiles t + 1 and t + 2 are in
  // flight.  A tile's table entry is loaded (raw_word, the bare load of a
  // real entry) a tile before its rows are issued and checked (slot_of)
  // then, so no wait for it is also a wait for rows still in flight (loads
  // complete in order).  Every load is issued unconditionally; only the
  // compute stops at t_end.
  const SlotMap<FMT> sm = slotmap_from_view<FMT>(m, rv);
  const int64_t row_elems = (int64_t)Hkv * D;
  const bf16* kb = k_pool + (int64_t)h * D;
  const bf16* vb = v_pool + (int64_t)h * D;
  auto raw_word = [&](int t) -> int32_t { return sm.raw(min(t * kTile + (lane & 31), E - 1)); };
  auto slot_of = [&](int t, int32_t r) -> int32_t {
    const int key = t * kTile + (lane & 31);
    return sm.finish(r, min(key, E - 1), key < E);
  };

  // Start-up order: the first four tiles' table entries, the queries, the
  // row limits' loads; the first two tiles' rows go out as soon as their
  // entries are in, and only then are the limits formed (a select on a
  // loaded value waits for it, and so for every load issued before it).
  // Tile k's entry is held in R[(k - t_begin) % 3] from two tiles before
  // its rows are issued (the first two tiles' in a0, a1).
  const int32_t a0 = raw_word(t_begin), a1 = raw_word(t_begin + 1);
  int32_t R[3];
  R[2] = raw_word(t_begin + 2);
  R[0] = raw_word(t_begin + 3);
  // rows: column cc of block b is member i0 + cc / G, query head h G + cc %
  // G.  A column past the slice's rows reads member i0's query and limit
  // loads (finite values) and gets limit 0, so all its keys are masked and
  // nothing of it is written.
  bf16x8 qb[NB][NK];
  int l_kv[NB], l_cap[NB];
  bool okb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int cc = b * 16 + col;
    const int mm = i0 + cc / G;
    okb[b] = cc < ms * G && mm < i1;
    const int mr = okb[b] ? mm : i0;
    const bf16* qp = q + ((int64_t)mr * Hq + h * G + cc % G) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qb[b][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 32));
    l_kv[b] = m.kv_lens[mr];
    l_cap[b] = lim_arr[mr];
  }
  DecodeTile<D> T[3];
  __builtin_amdgcn_sched_barrier(0);
  decode_issue<D>(T[0], slot_of(t_begin, a0), lane, kb, vb, row_elems);
  decode_issue<D>(T[1], slot_of(t_begin + 1, a1), lane, kb, vb, row_elems);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  int lim[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) lim[b] = okb[b] ? min(l_kv[b], l_cap[b]) : 0;
  f32x4 acc[NB][NT];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[b][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
  }

  {
    // step t: tile t + 2's rows (its entry, r_use, was loaded two tiles
    // ago: waiting for it waits for no tile not yet computed), the entry of
    // tile t + 4 into the register tile t + 1's entry held, then tile t
    auto step = [&](int t, DecodeTile<D>& cur, DecodeTile<D>& nxt2, int32_t r_use, int32_t& r_load) {
      const int32_t rn = raw_word(t + 4);
      __builtin_amdgcn_sched_barrier(0);
      decode_issue<D>(nxt2, slot_of(t + 2, r_use), lane, kb, vb, row_elems);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      r_load = rn;
      if (t < t_end) cascade_tile<D, NB>(cur, t * kTile, E, lim, lane, qb, scale_log2, vt, acc, m_run, l_run);
    };
    for (int t = t_begin; t < t_end; t += 3) {
      step(t, T[0], T[2], R[2], R[1]);
      step(t + 1, T[1], T[0], R[0], R[2]);
      step(t + 2, T[2], T[1], R[1], R[0]);
    }
  }

  // ---- partial results: lane (col, grp) holds O[row 4 grp + rr][d 16 nt + col]
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float l_tot = l_run[b] + shfl_xor(l_run[b], 16);
    l_tot += shfl_xor(l_tot, 32);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hr = grp * 4 + rr;
      const float lt = shfl(l_tot, hr);
      const float mr = shfl(m_run[b], hr);
      const int cc = b * 16 + hr;
      const int mm = i0 + cc / G;
      if (cc < ms * G && mm < i1) {
        const int64_t o = ((int64_t)c * bs + mm) * Hq + h * G + cc % G;
        const bool any = lt > 0.f;
        const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ws_po[o * D + nt * 16 + col] = acc[b][nt][rr] * inv;
        if (col == 0) ws_plse[o] = any ? (mr + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  }
}

// The bf16 decode's main launch: workgroups [0, n_stream) stream the runs
// of every request's own keys; the rest take the shared-prefix work items
// listed by the planner (*count of them, at most cap): the prefixes
// paged_decode_attn found, or the caller's groups of the cascade decode;
// they stride over them.  One launch, so the prefix work starts on each CU
// as soon as its run is done, and a batch without shared prefixes pays no
// second launch.
template <int D, int WAVES, int NS, int FMT>
__global__ void __launch_bounds__(64 * WAVES, stream_min_blocks(WAVES, NS)) decode_share_kernel(
    const bf16* k_pool, const bf16* v_pool, const bf16* __restrict__ q, int32_t Hq, int32_t Hkv, int32_t G,
    int32_t hg, const int32_t* __restrict__ header, const int32_t* __restrict__ meta, float scale_log2,
    bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int32_t n_stream, DevMap m, int32_t bs, const PrefixItem* __restrict__ items, const int32_t* __restrict__ count,
    const int32_t* __restrict__ skip, int32_t ms, int32_t cap, float* __restrict__ ws_po,
    float* __restrict__ ws_plse) {
  __shared__ __attribute__((aligned(16))) bf16 vsm[WAVES][kTile * (D + 8)];
  bf16* vt = vsm[threadIdx.x >> 6];
  if ((int)blockIdx.x < n_stream) {
    stream_run<D, WAVES, NS>((int)blockIdx.x, vt, k_pool, v_pool, q, Hq, Hkv, G, hg, header, meta, scale_log2, out,
                             lse, ws_o, ws_lse, skip);
    return;
  }
  const int b = (int)blockIdx.x - n_stream;  // n_stream is a multiple of 8: b keeps the XCD of blockIdx
  const int works = ((int)gridDim.x - n_stream) / hg;
  // the first item is loaded beside the count (at an index clamped into
  // the list's capacity), not after it
  int w = (b / (8 * hg)) * 8 + b % 8;
  PrefixItem it = items[min(w, cap - 1)];
  const int n_items = *count;
  // (both loads stand here, issued together: the compiler would otherwise
  // move the item's load into the loop, after the wait for the count)
  asm volatile("" ::"s"(n_items), "s"(it.i0), "s"(it.i1), "s"(it.E), "s"(it.t0), "s"(it.t1), "s"(it.c),
               "s"(it.limit), "s"(it.off_lo), "s"(it.off_hi));
  while (w < n_items) {
    cascade_prefix_work<D, WAVES, FMT>(m, k_pool, v_pool, q, bs, Hq, Hkv, G, it.i0, it.i1, prefix_item_view(it), skip,
                                       it.E, it.t0, it.t1, it.c, ms, scale_log2, ws_po, ws_plse, vt, b);
    w += works;
    if (w < n_items) it = items[w];
  }
}

// ---------------------------------------------------------------------------
// Shared prefixes found by paged_decode_attn itself ([MINI] prefix caching
// and [XPU]: requests that share a prefix read the same pages; the pages
// give no interface for it, so a plain decode looks for it).  One wave per
// request.  Within each 64-request block of the batch, consecutive
// requests whose keys start at the same slot form a group; the group's
// reference is its longest member (the first on ties); every other member
// shares the keys before the first page (token-table maps: the first slot)
// where its table and the reference's differ.  Per request the kernel
// writes s: the shared keys rounded down to the 32-key tile, or the whole
// request rounded up to it when every key is shared, 0 when nothing is, -1
// for the reference; and the group's bounds.  The planner derives each
// request's skip from them and the prefix pass reads each shared tile once
// for the whole group.  Grouping changes which keys a piece holds, never
// the result beyond rounding: every key is still read exactly once per
// request, by the prefix pass or the stream kernel.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(64) share_detect_kernel(DevMap m, int32_t bs, int32_t* __restrict__ s_out,
                                                          int32_t* __restrict__ gs_out, int32_t* __restrict__ ge_out) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const int base = i & ~63;
  const int j = base + lane;
  const bool in = j < bs;
  const int32_t Lj = in ? max(m.kv_lens[j], 0) : 0;
  int32_t key = -1;
  if (in && Lj > 0) {
    const SlotMap<FMT> smj = make_slotmap<FMT>(m, j);
    key = smj(0, true);
    if (key == smj.pad) key = -1;  // dummies on the padding page are never grouped
  }
  const int32_t prev = __shfl_up(key, 1, 64);
  const bool opens = !in || lane == 0 || key < 0 || key != prev;
  const uint64_t starts = __builtin_amdgcn_ballot_w64(opens);
  const int li = i - base;
  const uint64_t upto = (li == 63) ? ~0ull : ((2ull << li) - 1);
  const int gs_l = 63 - __builtin_clzll(starts & upto);  // lane 0 always opens
  const uint64_t after = starts & ~upto;
  const int ge_l = after ? __builtin_ctzll(after) : 64;
  const int gs = base + gs_l, ge = min(base + ge_l, bs);
  // the reference: the longest member, the first on ties
  int64_t pk = (in && lane >= gs_l && lane < ge_l) ? (((int64_t)Lj << 8) | (63 - lane)) : -1;
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(pk, o, 64);
    pk = y > pk ? y : pk;
  }
  const int ref = base + 63 - (int)(pk & 255);
  int32_t s = 0;
  const int32_t key_i = __shfl(key, li, 64);
  if (ge - gs >= 2 && key_i >= 0) {
    if (i == ref) {
      s = -1;
    } else {
      const int32_t Li = __shfl(Lj, li, 64), Lr = __shfl(Lj, ref - base, 64);
      const int32_t n = min(Li, Lr);
      const int32_t gran = FMT == SLOT_PAGES ? (1 << m.page_shift) : 1;  // one probe per page
      const SlotMap<FMT> smi = make_slotmap<FMT>(m, i), smr = make_slotmap<FMT>(m, ref);
      const int32_t nk = (n + gran - 1) / gran;
      // 4 x 64 probes per pass, every table load of the pass issued before
      // the first comparison (a prefix of a few hundred pages then costs one
      // load latency, not one per 64 pages)
      constexpr int kProbeRounds = 4;
      int32_t c = n;
      for (int32_t kb = 0; kb < nk; kb += 64 * kProbeRounds) {
        int32_t ra[kProbeRounds], rb[kProbeRounds];
#pragma unroll
        for (int u = 0; u < kProbeRounds; ++u) {
          const int32_t t = min(kb + u * 64 + lane, nk - 1) * gran;
          ra[u] = smi.raw(t);
          rb[u] = smr.raw(t);
        }
        uint64_t mm = 0;
        int u_hit = 0;
#pragma unroll
        for (int u = kProbeRounds - 1; u >= 0; --u) {
          const int32_t k = kb + u * 64 + lane;
          const int32_t a = smi.finish(ra[u], min(k, nk - 1) * gran, true);
          const int32_t b = smr.finish(rb[u], min(k, nk - 1) * gran, true);
          const uint64_t mu = __builtin_amdgcn_ballot_w64(k < nk && (a != b || a == smi.pad));
          if (mu) {  // the lowest round with a mismatch wins
            mm = mu;
            u_hit = u;
          }
        }
        if (mm) {
          c = min(n, (kb + u_hit * 64 + (int32_t)__builtin_ctzll(mm)) * gran);
          break;
        }
      }
      s = c >= Li ? (Li + kTile - 1) / kTile * kTile : c / kTile * kTile;
    }
  }
  if (lane == 0) {
    s_out[i] = s;
    gs_out[i] = gs;
    ge_out[i] = ge;
  }
}

// Final merge of a decode with a shared-prefix pass: one wavefront per
// (request, head) over the suffix pieces (ids run + request, every one in
// the workspace) and, for a request whose skip is nonzero, the prefix
// chunks.  A request outside the prefix pass that one run finished was
// written by the stream kernel and is skipped here.
template <int D>
__global__ void __launch_bounds__(256) cascade_merge_kernel(int32_t bs, int32_t Hq, int32_t chunks,
                                                            const int32_t* __restrict__ header,
                                                            const int32_t* __restrict__ prefix,
                                                            const int32_t* __restrict__ ntiles,
                                                            const int32_t* __restrict__ skip,
                                                            const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_lse,
                                                            const float* __restrict__ ws_po,
                                                            const float* __restrict__ ws_plse,
                                                            bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)bs * Hq) return;
  const int i = (int)(idx / Hq), h = (int)(idx % Hq);
  // the request's words go out together (the skip word, used after the
  // divisions, was otherwise loaded in a second round trip)
  const int sk = skip[i];
  const int T = ntiles[i];
  const int Bt = header[0];
  const int P = prefix[i];
  asm volatile("" ::"v"(sk), "v"(T), "v"(P));
  const int b0 = P / Bt, b1 = T > 0 ? (P + T - 1) / Bt : b0 - 1;
  const int nc = sk > 0 ? chunks : 0;
  if (nc == 0 && b0 == b1) return;
  auto piece = [&](int k, const float*& o) -> float {  // k < pieces: suffix, else prefix chunk
    const int np = b1 - b0 + 1;
    if (k < np) {
      const int64_t row = ((int64_t)(b0 + k) + i) * Hq + h;
      o = ws_o + row * D;
      return ws_lse[row];
    }
    const int64_t row = ((int64_t)(k - np) * bs + i) * Hq + h;
    o = ws_po + row * D;
    return ws_plse[row];
  };
  const int n = (b1 - b0 + 1) + nc;
  // the first KB sources' lse and partial rows are all loaded at once (they
  // are independent); a request with more sources takes the rest in a loop
  constexpr int KB = 12;
  float lb[KB], ob[KB][E];
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    lb[k] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) ob[k][e] = 0.f;
    if (k < n) {
      const float* o;
      lb[k] = piece(k, o);
#pragma unroll
      for (int e = 0; e < E; ++e) ob[k][e] = o[lane * E + e];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KB; ++k) mx = fmaxf(mx, lb[k]);
  for (int k = KB; k < n; ++k) {
    const float* o;
    mx = fmaxf(mx, piece(k, o));
  }
  bf16* op = out + idx * D + lane * E;
  if (mx == -INFINITY) {  // no key at all
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = (bf16)0.0f;
    if (lse && lane == 0) lse[idx] = -INFINITY;
    return;
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float sum = 0.f;
  // sources without keys (lse = -inf) weigh 0 and their rows are finite
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const float wgt = lb[k] == -INFINITY ? 0.f : __expf(lb[k] - mx);
    sum += wgt;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, ob[k][e], acc[e]);
  }
  for (int k = KB; k < n; ++k) {
    const float* o;
    const float l = piece(k, o);
    if (l == -INFINITY) continue;
    const float wgt = __expf(l - mx);
    sum += wgt;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, o[lane * E + e], acc[e]);
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int e = 0; e < E; ++e) op[e] = (bf16)(acc[e] * inv);
  if (lse && lane == 0) lse[idx] = mx + __logf(sum);
}

// ---------------------------------------------------------------------------
// VALU split kernel (f32 pools).  16 lanes per token, 4 tokens in flight per
// wave; each lane group keeps its own online-softmax state, merged across
// groups at the end.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void load_vals(const T* p, float* v, int n);
template <> __device__ __forceinline__ void load_vals<float>(const float* p, float* v, int n) {
  for (int e = 0; e < n; e += 4) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p + e);
    v[e] = w[0]; v[e + 1] = w[1]; v[e + 2] = w[2]; v[e + 3] = w[3];
  }
}
template <> __device__ __forceinline__ void load_vals<bf16>(const bf16* p, float* v, int n) {
  for (int e = 0; e < n; e += 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + e);
    v[e] = bf16_lo(w.x); v[e + 1] = bf16_hi(w.x); v[e + 2] = bf16_lo(w.y); v[e + 3] = bf16_hi(w.y);
  }
}

template <typename T, int D, int GM, int WAVES, int FMT>
__global__ void __launch_bounds__(64 * WAVES) decode_valu_kernel(
    DevMap m, const T* __restrict__ k_pool, const T* __restrict__ v_pool, const T* __restrict__ q, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t hg, int32_t chunk, int32_t max_splits, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ item_count, float scale_log2, T* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int E = D / 16;
  const int w_item = blockIdx.x / hg;
  if (w_item >= *item_count) return;
  const WorkItem item = items[w_item];
  const int i = item.i;
  const int s = item.s;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = (blockIdx.x % hg) * WAVES + wave;
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int ns = item.ns;
  if (ns == 0) {
    for (int n = 0; n < G; ++n) {
      const int64_t h = (int64_t)i * Hq + g * G + n;
      for (int d = lane; d < D; d += 64) out[h * D + d] = from_f32<T>(0.0f);
      if (lse && lane == 0) lse[h] = -INFINITY;
    }
    return;
  }
  const int t_begin = s * chunk;
  const int t_end = item.t_end;
  const SlotMap<FMT> sm = slotmap_from_view<FMT>(m, item_view(item));

  float qv[GM][E];
#pragma unroll
  for (int n = 0; n < GM; ++n) {
    if (n < G) {
      load_vals<T>(q + ((int64_t)i * Hq + g * G + n) * D + c * E, qv[n], E);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) qv[n][e] = 0.f;
    }
  }
  float mr[GM], lr[GM], o[GM][E];
#pragma unroll
  for (int n = 0; n < GM; ++n) {
    mr[n] = -INFINITY;
    lr[n] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[n][e] = 0.f;
  }
  const int64_t row_elems = (int64_t)Hkv * D;
  for (int t = t_begin + grp; t < t_end; t += 4) {
    const int64_t slot = sm(t, true);
    float kv[E], vv[E];
    load_vals<T>(k_pool + slot * row_elems + (int64_t)g * D + c * E, kv, E);
    load_vals<T>(v_pool + slot * row_elems + (int64_t)g * D + c * E, vv, E);
#pragma unroll
    for (int n = 0; n < GM; ++n) {
      if (n >= G) break;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(qv[n][e], kv[e], d);
      d += shfl_xor(d, 1);
      d += shfl_xor(d, 2);
      d += shfl_xor(d, 4);
      d += shfl_xor(d, 8);
      const float x = d * scale_log2;
      const float mn = fmaxf(mr[n], x);
      const float al = fast_exp2(mr[n] - mn);
      const float p = fast_exp2(x - mn);
      lr[n] = lr[n] * al + p;
#pragma unroll
      for (int e = 0; e < E; ++e) o[n][e] = fmaf(p, vv[e], o[n][e] * al);
      mr[n] = mn;
    }
  }
  // merge the four lane groups (groups without tokens carry m = -inf, l = 0)
#pragma unroll
  for (int n = 0; n < GM; ++n) {
    if (n >= G) break;
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float m2 = shfl_xor(mr[n], x);
      const float l2 = shfl_xor(lr[n], x);
      const float mn = fmaxf(mr[n], m2);
      const float a1 = (mr[n] == -INFINITY) ? 0.f : fast_exp2(mr[n] - mn);
      const float a2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
      lr[n] = lr[n] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float o2 = shfl_xor(o[n][e], x);
        o[n][e] = o[n][e] * a1 + o2 * a2;
      }
      mr[n] = mn;
    }
    if (grp == 0) {
      const int64_t h = (int64_t)i * Hq + g * G + n;
      const float inv = 1.0f / lr[n];
      const float lse_nat = (mr[n] + __log2f(lr[n])) * kLn2;
      if (ns == 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) out[h * D + c * E + e] = from_f32<T>(o[n][e] * inv);
        if (lse && c == 0) lse[h] = lse_nat;
      } else {
        float* po = ws_o + (h * max_splits + s) * D + c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) po[e] = o[n][e] * inv;
        if (c == 0) ws_lse[h * max_splits + s] = lse_nat;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split partials: lse = log sum_s exp(lse_s) and
// o = sum_s exp(lse_s - lse) o_s.  One wavefront per (request, head);
// requests that used a single split were finished by the split kernel.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) decode_merge_kernel(const int32_t* __restrict__ kv_lens, int32_t bs,
                                                           int32_t Hq, int32_t Dv, int32_t chunk,
                                                           int32_t max_splits, const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_lse, T* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ float wsh[4][kMaxSplits];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  if (idx >= (int64_t)bs * Hq) return;
  const int i = (int)(idx / Hq);
  const int L = kv_lens[i];
  const int ns = L > 0 ? min((L + chunk - 1) / chunk, max_splits) : 0;
  if (ns <= 1) return;
  const float* pl = ws_lse + idx * max_splits;
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, pl[s]);
  for (int x = 32; x > 0; x >>= 1) mx = fmaxf(mx, shfl_xor(mx, x));
  float tot = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float w = __expf(pl[s] - mx);
    wsh[wave][s] = w;
    tot += w;
  }
  for (int x = 32; x > 0; x >>= 1) tot += shfl_xor(tot, x);
  __builtin_amdgcn_wave_barrier();
  const float inv = 1.0f / tot;
  const float* po = ws_o + idx * max_splits * Dv;
  // 8 partial rows in flight per lane before any is used
  for (int d = lane; d < Dv; d += 64) {
    float a = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (s0 + k < ns) ? po[(int64_t)(s0 + k) * Dv + d] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < ns) a = fmaf(wsh[wave][s0 + k], v[k], a);
    }
    out[idx * Dv + d] = from_f32<T>(a * inv);
  }
  if (lse && lane == 0) lse[idx] = mx + __logf(tot);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
enum DecodeKind : int32_t { DK_NONE = 0, DK_STREAM = 1, DK_VALU = 2, DK_MLA = 3 };
constexpr int kStreamSets = 3;  // register tile sets of the stream kernel

static int decode_kind(const PoolInfo& p, int32_t Hq) {
  if (p.kind == 1) return mla_decode_supported(p, Hq) ? DK_MLA : DK_NONE;
  if (p.head_dim_qk != p.head_dim_v || (p.head_dim_qk != 64 && p.head_dim_qk != 128)) return DK_NONE;
  if (Hq <= 0 || Hq % p.num_kv_heads != 0) return DK_NONE;
  const int G = Hq / p.num_kv_heads;
  if (p.dtype == 1 && G <= 16) return DK_STREAM;
  if (p.dtype == 0 && G <= 8) return DK_VALU;
  return DK_NONE;
}

bool decode_supported(const PoolInfo& p, int32_t num_q_heads) { return decode_kind(p, num_q_heads) != DK_NONE; }

DecodePlan plan_decode(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len) {
  DecodePlan plan;
  plan.kind = decode_kind(p, Hq);
  if (plan.kind == DK_MLA) return plan_mla_decode(p, bs, Hq, max_kv_len);
  if (plan.kind == DK_STREAM) {
    // runs: workgroups that fit on the device at once, over the KV-head groups
    const int Hkv = p.num_kv_heads;
    const int W = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0 ? 2 : 1);
    const int per_cu = (kStreamSets <= 2 ? 8 : 4) / W;
    plan.chunk = max_kv_len > 0 ? (max_kv_len + kStreamT - 1) / kStreamT : 0;  // tiles per request, at most
    plan.max_splits = std::max(8, device_cu_count() * per_cu / (Hkv / W) / 8 * 8);  // a multiple of 8
    return plan;
  }
  // Chunk of logical tokens per split: the largest power of two in
  // [64, 1024] that still leaves ~16 wavefronts per CU on average (the mean
  // length is taken as max_kv_len / 2), so long requests spread over the 256
  // CUs while the merge traffic stays a small fraction of the KV bytes.
  const double wave_tokens = (double)bs * p.num_kv_heads * 0.5 * (double)max_kv_len;
  int chunk = 64;
  for (int c = 1024; c >= 64; c >>= 1) {
    if (wave_tokens / c >= 4096.0) {
      chunk = c;
      break;
    }
  }
  int splits = max_kv_len > 0 ? (max_kv_len + chunk - 1) / chunk : 1;
  while (splits > kMaxSplits) {
    chunk *= 2;
    splits = (max_kv_len + chunk - 1) / chunk;
  }
  plan.chunk = chunk;
  plan.max_splits = splits < 1 ? 1 : splits;
  return plan;
}

// workspace: [item count | items[bs * max_splits] | partial o | partial lse]

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t decode_ws_layout(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t Hq, void* base,
                        DecodeWs* w) {
  size_t off = 0;
  char* b = static_cast<char*>(base);
  if (w) w->count = reinterpret_cast<int32_t*>(b + off);
  off += 256;
  if (w) w->items = reinterpret_cast<WorkItem*>(b + off);
  off += align256((size_t)bs * plan.max_splits * sizeof(WorkItem));
  if (plan.max_splits > 1) {
    const size_t rows = (size_t)bs * Hq * plan.max_splits;
    if (w) w->o = reinterpret_cast<float*>(b + off);
    off += align256(rows * p.head_dim_v * sizeof(float));
    if (w) w->lse = reinterpret_cast<float*>(b + off);
    off += align256(rows * sizeof(float));
  } else if (w) {
    w->o = nullptr;
    w->lse = nullptr;
  }
  return off;
}

// ---- shared prefixes found by the stream decode itself
struct ShareWs {
  int32_t* s;
  int32_t* gs;
  int32_t* ge;
  int32_t* skip;
  int32_t* count;
  PrefixItem* items;  // at most bs * kShareChunks (every slice holds a member)
  float* po;          // prefix partials [kShareChunks][bs][Hq][Dv]
  float* plse;        // [kShareChunks][bs][Hq]
  int32_t ms;
};

// [stream workspace | s, gs, ge, skip [bs] | items [bs][ipr] | prefix o | prefix lse]
static size_t stream_decode_ws_layout(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t Hq, void* base,
                                      StreamWs* sw, ShareWs* sh) {
  char* b = static_cast<char*>(base);
  size_t off = stream_ws_layout(bs, plan.chunk, plan.max_splits, Hq, p.head_dim_v, base, sw);
  auto take = [&](size_t bytes) {
    char* at = b ? b + off : nullptr;
    off += align256(bytes);
    return at;
  };
  const int G = Hq / p.num_kv_heads;
  const int32_t ms = std::max(1, kCascadeCols / G);
  char* a_s = take((size_t)bs * 4);
  char* a_gs = take((size_t)bs * 4);
  char* a_ge = take((size_t)bs * 4);
  char* a_skip = take((size_t)bs * 4);
  char* a_count = take(4);
  char* a_items = take((size_t)bs * kShareChunks * sizeof(PrefixItem));
  char* a_po = take((size_t)kShareChunks * bs * Hq * p.head_dim_v * 4);
  char* a_pl = take((size_t)kShareChunks * bs * Hq * 4);
  if (sh) {
    sh->s = reinterpret_cast<int32_t*>(a_s);
    sh->gs = reinterpret_cast<int32_t*>(a_gs);
    sh->ge = reinterpret_cast<int32_t*>(a_ge);
    sh->skip = reinterpret_cast<int32_t*>(a_skip);
    sh->count = reinterpret_cast<int32_t*>(a_count);
    sh->items = reinterpret_cast<PrefixItem*>(a_items);
    sh->po = reinterpret_cast<float*>(a_po);
    sh->plse = reinterpret_cast<float*>(a_pl);
    sh->ms = ms;
  }
  return off;
}

size_t decode_workspace_bytes(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t Hq) {
  if (plan.kind == DK_MLA)  // slices of rows reuse one workspace
    return stream_ws_layout(bs, plan.chunk, plan.max_splits, mla_slice_rows(Hq), p.head_dim_v, nullptr, nullptr);
  if (plan.kind == DK_STREAM) return stream_decode_ws_layout(p, plan, bs, Hq, nullptr, nullptr, nullptr);
  return decode_ws_layout(p, plan, bs, Hq, nullptr, nullptr);
}

template <int D, int W>
static void launch_valu(unsigned blocks, hipStream_t s, const DevMap& m, const PoolInfo& p, int32_t layer,
                        const void* q, int32_t Hq, int32_t G, int32_t hg, const DecodePlan& plan, const DecodeWs& w,
                        float sl2, void* out, float* lse) {
  auto kern = (m.fmt == MAP_TOKEN_TABLE) ? decode_valu_kernel<float, D, 8, W, SLOT_TABLE>
                                         : decode_valu_kernel<float, D, 8, W, SLOT_PAGES>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * W), 0, s, m, reinterpret_cast<const float*>(p.k_layer(layer)),
                     reinterpret_cast<const float*>(p.v_layer(layer)), static_cast<const float*>(q), Hq,
                     p.num_kv_heads, G, hg, plan.chunk, plan.max_splits, w.items, w.count, sl2,
                     static_cast<float*>(out), lse, w.o, w.lse);
}

// The prefix pass's inputs to decode_share_kernel: its work items (at
// most cap; cap 0 launches no prefix workgroups), each request's skip, the
// members per slice and the partial results' slots.
struct PrefixPass {
  const PrefixItem* items;
  const int32_t* count;
  const int32_t* skip;
  int32_t ms;
  int32_t cap;
  float* po;
  float* plse;
};

template <int D, int W, int FMT>
static void launch_share_main(int32_t runs, int32_t hg, hipStream_t s, const PoolInfo& p, int32_t layer,
                              const DevMap& m, const void* q, int32_t bs, int32_t Hq, int32_t G, const StreamWs& w,
                              const PrefixPass& pp, float sl2, void* out, float* lse) {
  // the prefix work: one work per CU covers the usual count
  const int64_t works = (std::min<int64_t>(pp.cap, device_cu_count()) + 7) / 8 * 8;
  const int32_t n_stream = runs * hg;
  hipLaunchKernelGGL((decode_share_kernel<D, W, kStreamSets, FMT>), dim3((unsigned)(n_stream + works * hg)),
                     dim3(64 * W), 0, s, reinterpret_cast<const bf16*>(p.k_layer(layer)),
                     reinterpret_cast<const bf16*>(p.v_layer(layer)), static_cast<const bf16*>(q), Hq, p.num_kv_heads,
                     G, hg, w.header, w.meta, sl2, static_cast<bf16*>(out), lse, w.o, w.lse, n_stream, m, bs, pp.items,
                     pp.count, pp.skip, pp.ms, pp.cap, pp.po, pp.plse);
}

// decode_share_kernel for the pool's head dim, the waves per workgroup W
// (one KV head each) and the map's slot form
static void launch_share_any(int32_t W, int32_t runs, int32_t hg, hipStream_t s, const PoolInfo& p, int32_t layer,
                             const DevMap& m, const void* q, int32_t bs, int32_t Hq, int32_t G, const StreamWs& w,
                             const PrefixPass& pp, float sl2, void* out, float* lse) {
  const bool tab = m.fmt == MAP_TOKEN_TABLE;
  auto go = [&](auto launch) { launch(runs, hg, s, p, layer, m, q, bs, Hq, G, w, pp, sl2, out, lse); };
  if (p.head_dim_qk == 128) {
    if (W == 4) tab ? go(launch_share_main<128, 4, SLOT_TABLE>) : go(launch_share_main<128, 4, SLOT_PAGES>);
    else if (W == 2) tab ? go(launch_share_main<128, 2, SLOT_TABLE>) : go(launch_share_main<128, 2, SLOT_PAGES>);
    else tab ? go(launch_share_main<128, 1, SLOT_TABLE>) : go(launch_share_main<128, 1, SLOT_PAGES>);
  } else {
    if (W == 4) tab ? go(launch_share_main<64, 4, SLOT_TABLE>) : go(launch_share_main<64, 4, SLOT_PAGES>);
    else if (W == 2) tab ? go(launch_share_main<64, 2, SLOT_TABLE>) : go(launch_share_main<64, 2, SLOT_PAGES>);
    else tab ? go(launch_share_main<64, 1, SLOT_TABLE>) : go(launch_share_main<64, 1, SLOT_PAGES>);
  }
}

// The bf16 decode: find shared prefixes (share_detect_kernel), plan the
// stream of every request's own tiles (the append, if any, rides in the
// planner launch), stream them and read each group's shared prefix once
// (decode_share_kernel), then merge pieces and prefix chunks.  Without
// shared prefixes the prefix pass finds no work and every request one run
// finishes is written by the stream kernel directly.
static hipError_t launch_stream_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m,
                                       int32_t bs, const DecodePlan& plan, float sl2, void* out, float* lse, void* ws,
                                       hipStream_t s, const StoreArgs* st) {
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int W = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0 ? 2 : 1);
  const int hg = Hkv / W;
  const int32_t runs = plan.max_splits;
  if (runs % 8 != 0) return hipErrorInvalidValue;  // the block -> (run, head group) map needs whole XCD rounds
  StreamWs w;
  ShareWs sh;
  stream_decode_ws_layout(p, plan, bs, Hq, ws, &w, &sh);
  if (m.fmt == MAP_TOKEN_TABLE)
    hipLaunchKernelGGL(share_detect_kernel<SLOT_TABLE>, dim3((unsigned)bs), dim3(64), 0, s, m, bs, sh.s, sh.gs, sh.ge);
  else
    hipLaunchKernelGGL(share_detect_kernel<SLOT_PAGES>, dim3((unsigned)bs), dim3(64), 0, s, m, bs, sh.s, sh.gs, sh.ge);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ShareArgs sa;
  sa.s = sh.s;
  sa.gs = sh.gs;
  sa.ge = sh.ge;
  sa.skip = sh.skip;
  sa.items = sh.items;
  sa.count = sh.count;
  sa.ms = sh.ms;
  sa.ch = kShareChunks;
  e = launch_stream_plan(m, bs, plan.chunk, runs, w, s, nullptr, st, &sa);
  if (e != hipSuccess) return e;
  const int D = p.head_dim_qk;
  const PrefixPass pp{sh.items, sh.count, sh.skip, sh.ms, bs * kShareChunks, sh.po, sh.plse};
  timer_before(s);
  launch_share_any(W, runs, hg, s, p, layer, m, q, bs, Hq, G, w, pp, sl2, out, lse);
  e = hipGetLastError();
  timer_after(s);
  if (e != hipSuccess) return e;
  const unsigned mblocks = (unsigned)(((int64_t)bs * Hq + 3) / 4);
  if (D == 128)
    hipLaunchKernelGGL(cascade_merge_kernel<128>, dim3(mblocks), dim3(256), 0, s, bs, Hq, kShareChunks, w.header,
                       w.prefix, w.ntiles, sh.skip, w.o, w.lse, sh.po, sh.plse, static_cast<bf16*>(out), lse);
  else
    hipLaunchKernelGGL(cascade_merge_kernel<64>, dim3(mblocks), dim3(256), 0, s, bs, Hq, kShareChunks, w.header,
                       w.prefix, w.ntiles, sh.skip, w.o, w.lse, sh.po, sh.plse, static_cast<bf16*>(out), lse);
  return hipGetLastError();
}

// ---- cascade decode host side
CascadePlan plan_cascade(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len, int32_t num_groups,
                         int32_t max_group_size, int32_t max_prefix_len) {
  CascadePlan cp;
  cp.dp = plan_decode(p, bs, Hq, max_kv_len);
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  cp.ms = std::max(1, kCascadeCols / G);
  cp.slices = (int32_t)std::max<int64_t>(1, ((int64_t)max_group_size + cp.ms - 1) / cp.ms);
  const int ptiles = std::max(1, (std::min(max_prefix_len, max_kv_len) + kTile - 1) / kTile);
  const int64_t items = std::max<int64_t>(1, (int64_t)num_groups * cp.slices * Hkv);
  // about four waves per CU over the prefix work
  const int chunks = (int)std::min<int64_t>(ptiles, std::max<int64_t>(1, (device_cu_count() * 4 + items - 1) / items));
  const int tpc = (ptiles + chunks - 1) / chunks;
  cp.chunks = (ptiles + tpc - 1) / tpc;
  cp.cap = std::max<int64_t>(1, (int64_t)num_groups * cp.slices * cp.chunks);
  return cp;
}

// [stream workspace | skip[bs] | count | items[cap] | prefix o[chunks][bs][Hq][D] | prefix lse[chunks][bs][Hq]]
size_t cascade_ws_layout(const PoolInfo& p, const CascadePlan& cp, int32_t bs, int32_t Hq, void* base,
                         CascadeWs* w) {
  char* b = static_cast<char*>(base);
  size_t off = stream_ws_layout(bs, cp.dp.chunk, cp.dp.max_splits, Hq, p.head_dim_v, base, w ? &w->stream : nullptr);
  auto take = [&](size_t bytes) {
    char* at = b ? b + off : nullptr;
    off += align256(bytes);
    return at;
  };
  char* skip = take((size_t)bs * 4);
  char* count = take(4);
  char* items = take((size_t)cp.cap * sizeof(PrefixItem));
  char* po = take((size_t)cp.chunks * bs * Hq * p.head_dim_v * 4);
  char* pl = take((size_t)cp.chunks * bs * Hq * 4);
  if (w) {
    w->skip = reinterpret_cast<int32_t*>(skip);
    w->count = reinterpret_cast<int32_t*>(count);
    w->items = reinterpret_cast<PrefixItem*>(items);
    w->po = reinterpret_cast<float*>(po);
    w->plse = reinterpret_cast<float*>(pl);
  }
  return off;
}

// The cascade: list each request's skip and the groups' prefix work
// (cascade_plan_kernel), plan the stream of every request's own tiles,
// stream them and read each group's prefix once (decode_share_kernel, as
// for the prefixes paged_decode_attn finds), then merge.
hipError_t launch_decode_cascade(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m,
                                 int32_t bs, const CascadePlan& cp, const int32_t* group_indptr,
                                 const int32_t* prefix_len, int32_t num_groups, float sm_scale, void* out, float* lse,
                                 void* ws, hipStream_t s) {
  if (bs == 0) return hipSuccess;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int W = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0 ? 2 : 1);
  const int hg = Hkv / W;
  const int32_t runs = cp.dp.max_splits;
  if (cp.dp.kind != DK_STREAM || runs % 8 != 0) return hipErrorInvalidValue;
  CascadeWs w;
  cascade_ws_layout(p, cp, bs, Hq, ws, &w);
  const int32_t nb = (bs + 255) / 256;
  hipLaunchKernelGGL(cascade_plan_kernel, dim3((unsigned)(nb + num_groups)), dim3(256), 0, s, m, group_indptr,
                     prefix_len, num_groups, bs, cp.ms, cp.slices, cp.chunks, w.skip, w.items, w.count);
  hipError_t e = launch_stream_plan(m, bs, cp.dp.chunk, runs, w.stream, s, w.skip);
  if (e != hipSuccess) return e;
  const float sl2 = sm_scale * kLog2e;
  if (cp.cap > INT32_MAX) return hipErrorInvalidValue;  // the API refuses such bounds first
  const PrefixPass pp{w.items, w.count, w.skip, cp.ms, num_groups > 0 ? (int32_t)cp.cap : 0, w.po, w.plse};
  timer_before(s);
  launch_share_any(W, runs, hg, s, p, layer, m, q, bs, Hq, G, w.stream, pp, sl2, out, lse);
  e = hipGetLastError();
  timer_after(s);
  if (e != hipSuccess) return e;
  const unsigned mblocks = (unsigned)(((int64_t)bs * Hq + 3) / 4);
  if (p.head_dim_qk == 128)
    hipLaunchKernelGGL(cascade_merge_kernel<128>, dim3(mblocks), dim3(256), 0, s, bs, Hq, cp.chunks, w.stream.header,
                       w.stream.prefix, w.stream.ntiles, w.skip, w.stream.o, w.stream.lse, w.po, w.plse,
                       static_cast<bf16*>(out), lse);
  else
    hipLaunchKernelGGL(cascade_merge_kernel<64>, dim3(mblocks), dim3(256), 0, s, bs, Hq, cp.chunks, w.stream.header,
                       w.stream.prefix, w.stream.ntiles, w.skip, w.stream.o, w.stream.lse, w.po, w.plse,
                       static_cast<bf16*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m, int32_t bs,
                         const DecodePlan& plan, float sm_scale, void* out, float* lse, void* ws, hipStream_t s,
                         const StoreArgs* st) {
  if (bs == 0) {  // nothing to attend: only the append, if any
    return st && st->n > 0 ? launch_store_args(*st, s) : hipSuccess;
  }
  if (plan.kind == DK_MLA)
    return launch_mla_decode(p, layer, q, Hq, m, bs, plan, sm_scale * kLog2e, out, lse, ws, s, st);
  if (plan.kind == DK_STREAM)
    return launch_stream_decode(p, layer, q, Hq, m, bs, plan, sm_scale * kLog2e, out, lse, ws, s, st);
  if (st && st->n > 0) {  // the fp32 path has no planner launch to carry it
    hipError_t e = launch_store_args(*st, s);
    if (e != hipSuccess) return e;
  }
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int W = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0 ? 2 : 1);
  const int hg = Hkv / W;
  DecodeWs w;
  decode_ws_layout(p, plan, bs, Hq, ws, &w);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, m, bs, plan.chunk, plan.max_splits, w.items,
                     w.count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((int64_t)bs * plan.max_splits * hg);
  const float sl2 = sm_scale * kLog2e;
  const int D = p.head_dim_qk;
  timer_before(s);
  if (D == 128) {
    if (W == 4) launch_valu<128, 4>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
    else if (W == 2) launch_valu<128, 2>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
    else launch_valu<128, 1>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
  } else {
    if (W == 4) launch_valu<64, 4>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
    else if (W == 2) launch_valu<64, 2>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
    else launch_valu<64, 1>(blocks, s, m, p, layer, q, Hq, G, hg, plan, w, sl2, out, lse);
  }
  e = hipGetLastError();
  timer_after(s);
  if (e != hipSuccess || plan.max_splits <= 1) return e;
  const unsigned mblocks = (unsigned)(((int64_t)bs * Hq + 3) / 4);
  if (p.dtype == 1)
    hipLaunchKernelGGL(decode_merge_kernel<bf16>, dim3(mblocks), dim3(256), 0, s, m.kv_lens, bs, Hq, p.head_dim_v,
                       plan.chunk, plan.max_splits, w.o, w.lse, static_cast<bf16*>(out), lse);
  else
    hipLaunchKernelGGL(decode_merge_kernel<float>, dim3(mblocks), dim3(256), 0, s, m.kv_lens, bs, Hq, p.head_dim_v,
                       plan.chunk, plan.max_splits, w.o, w.lse, static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace pkv
