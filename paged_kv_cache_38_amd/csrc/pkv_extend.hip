// Paged extend / prefill attention (bf16, MFMA).
//
// What is computed ([BACKEND] "例子": the new tokens of each request, counted
// by qo_indptr, attend over the request's kv_lens keys -- cached prefix plus
// this step's tokens -- read through the page table; [OMNI] "Attention
// execution": a causal segment Q[s:e] sees K[:e], a full segment sees every
// key).  Causal alignment is bottom-right: the j-th of n new queries sits at
// position L - n + j and sees keys 0 .. L - n + j.  An empty key set gives a
// zero output and lse = -inf ([XPU] "Approach 2" guard).  With a CONTIGUOUS
// map this is the ragged (varlen) variant over gathered K/V.
//
// Layout on gfx950: one workgroup per (query tile, query head, request); four
// wavefronts of 16 RB query rows each (RB 16-row blocks: 3 at D = 64, 2 at
// D = 128).  Key tiles of 64 tokens move HBM -> LDS through the table by
// global_load_lds (token-major rows, 16-byte chunks XOR-swizzled), S stages
// deep, so the next tiles' reads overlap this tile's MFMA work:
//   S^T[16 keys x 16 rows] = K_tile[16 x D] * Q^T[D x 16]   (v_mfma_f32_16x16x32_bf16)
// leaves each lane one query row (lane % 16) and 16 keys, so the row softmax
// needs only two cross-lane steps, and P is already the B operand of
//   O^T[D x 16 rows] += V^T[D x 32 keys] * P^T[32 keys x 16 rows]
// whose A operand comes from LDS with ds_read_b64_tr_b16.  Every K and V
// fragment read from LDS feeds the RB row blocks of the wave.
#include <math.h>

#include <type_traits>

#include "pkv_launch.h"

namespace pkv {

constexpr int kBN = 64;   // keys per tile
constexpr float kExtSlack = 8.0f;  // log2 headroom before a row's running max moves

// Rows: D = 64 takes three 16-row blocks per wave (192 query rows per
// workgroup, 216 VGPRs, two workgroups per CU), so every K and V fragment
// read from LDS feeds three MFMAs and a (request, head) pair re-streams its
// keys once per 192 queries; D = 128 takes two (128 rows, two per CU).
template <int D>
struct ExtendCfg {
  static constexpr int RB = D == 64 ? 3 : 2;  // 16-row blocks per wave
  static constexpr int OCC = 2;               // workgroups per CU the registers allow
  static constexpr int WR = 16 * RB;          // query rows per wave
  static constexpr int BM = 4 * WR;           // query rows per workgroup (four waves)
  static constexpr int NK = D / 32;          // k-steps of the score product
  static constexpr int NT = D / 16;          // 16-wide d tiles of O
  static constexpr int CPK = D / 8;          // 16-byte chunks per key row (one head)
  static constexpr int TILE = kBN * D * 2;   // bytes of one K (or V) tile
  static constexpr int NI = 2 * TILE / 1024 / 4;  // K+V DMA instructions per wave per tile
  static constexpr int S = D == 64 ? 3 : 2;  // LDS stages (tiles resident)
  // memory operations a wave may leave outstanding when tile kt must have
  // landed: the later tiles' DMAs and the newest table load
  static constexpr int WAIT = (S - 2) * NI + 1;
};

// Byte offset of 16-byte chunk c of key row t in an LDS tile: rows are
// D * 2 bytes apart and chunk c sits at c ^ (t & 7), so the eight rows a
// K-operand read touches at once, and the four rows of a transposed V read,
// fall in different banks.
template <int D>
__device__ __forceinline__ int ext_off(int t, int c) {
  return (t * (D / 8) + (c ^ (t & 7))) * 16;
}

// B operand of P*V from a swizzled tile: lane (n = l%16, j = l/16) receives
// V[r0 + 4j + r][c0 + n] (low half) and V[r0 + 16 + 4j + r][c0 + n] (high half).
template <int D>
__device__ __forceinline__ bf16x8 ext_v_operand(const char* tile, int r0, int c0, int lane) {
  const int x = lane & 15, j = lane >> 4;
  const int t = r0 + 4 * j + (x >> 2);
  const int c = c0 + 4 * (x & 3);
  const char* lo = tile + ext_off<D>(t, c >> 3) + (c & 7) * 2;
  const i16x4 a = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
  const i16x4 b = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * D * 2));
  const bf16x4 ba = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
  return bf16x8{ba[0], ba[1], ba[2], ba[3], bb[0], bb[1], bb[2], bb[3]};
}

// O^T += V^T P^T over a 16-key slice with v_mfma_f32_16x16x16_bf16: A = V^T
// (lane (x, j) holds V[4j + r][x], r = 0..3: the low half of the transposed
// read above), B = P^T (lane (row, j) holds P[row][4j + r]: the keys the
// score layout leaves in the lane).
__device__ __forceinline__ f32x4 mfma16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Softcap ([XPU] "Approach 2": the ragged call passes softcap; a score s
// becomes cap tanh(s / cap)).  Scores stay in the kernel's raw domain (the
// scale is applied inside exp2), so a raw score x turns into
// (cap / scale) tanh(x scale / cap) = b - 2 b / (exp2(a x) + 1) with
// a = 2 log2(e) scale / cap and b = cap / scale: one exp2 and one
// reciprocal per score, saturating to +-b at the extremes.
struct SoftCap {
  float a, b;
  __device__ __forceinline__ float operator()(float x) const {
    return b - 2.0f * b * __builtin_amdgcn_rcpf(fast_exp2(a * x) + 1.0f);
  }
};

template <int D, int FMT, bool SC>
__global__ void __launch_bounds__(256, ExtendCfg<D>::OCC) extend_kernel(DevMap m, const char* k_pool, const char* v_pool,
                                                     int64_t row_bytes, const bf16* __restrict__ q, int64_t total_q,
                                                     const int32_t* __restrict__ qo_indptr, int32_t Hq, int32_t n_req,
                                                     int32_t n_qtiles, int32_t G, int32_t causal_all,
                                                     const int32_t* __restrict__ causal_flags, SoftCap cap,
                                                     float scale_log2, bf16* __restrict__ out,
                                                     float* __restrict__ lse) {
  using C = ExtendCfg<D>;
  constexpr int NK = C::NK, NT = C::NT, CPK = C::CPK, NI = C::NI, S = C::S;
  constexpr int kRB = C::RB, kWR = C::WR, kBM = C::BM;
  __shared__ __attribute__((aligned(1024))) char kv_lds[S][2][C::TILE];
  __shared__ __attribute__((aligned(256))) int32_t tab_lds[4][S + 1][64];

  // blocks are dealt to the 8 XCDs round robin (block b on XCD b % 8).  The
  // (request, head) pairs are spread over the XCDs round robin too (pair p
  // on XCD p % 8), so every request's work is split evenly across them.
  // Non-causal calls run all query tiles of one pair back to back on one
  // XCD, sharing its L2, so each key/value tile leaves HBM once.  Causal
  // calls go by query tile, last tiles first: a later tile sees more keys,
  // so the longest blocks start first and the short ones fill the tail
  // (the tiles of one pair still share an XCD; a causal region is short).
  const int x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
  const int ppx = (int)(((int64_t)n_req * Hq + 7) / 8);  // pairs per XCD
  const bool qt_major = causal_all && !causal_flags;
  const int pair = x + 8 * (qt_major ? k % ppx : k / n_qtiles);
  const int qt = qt_major ? n_qtiles - 1 - k / ppx : k % n_qtiles;
  const int h = pair % Hq;
  const int i = pair / Hq;
  if (i >= n_req) return;
  // mixed causal/full segments ([OMNI] "Attention execution") carry one
  // flag per request
  const int causal = causal_flags ? (causal_flags[i] != 0) : causal_all;
  const int q0 = qo_indptr[i];
  // rows past total_q (a qo_indptr beyond the buffers) are never touched
  const int n = (q0 < 0 || q0 >= total_q) ? 0 : (int)min((int64_t)(qo_indptr[i + 1] - q0), total_q - q0);
  if (qt * kBM >= n) return;
  int L = m.kv_lens[i];
  if (FMT == SLOT_CONTIG && m.total_k <= 0) L = 0;  // nothing gathered: no row is readable
  if (L < 0) L = 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = h / G;
  // A block whose rows fit one wave runs key-split: every wave takes all of
  // its rows and its own 16-key slice (keys 16 w .. 16 w + 15) of each tile,
  // and the four partial softmax states are merged through LDS at the end.
  // Otherwise a short block would leave three waves with no rows, and its
  // tiles would wait on one wave's chain of dependent phases.
  const bool ks = n - qt * kBM <= kWR;
  const int rw = qt * kBM + (ks ? 0 : w * kWR);  // first query row (within the request) of this wave

  // keys any row of this block may see
  int kv_end = L;
  if (causal) kv_end = min(L, L - n + min(qt * kBM + kBM, n));
  if (kv_end < 0) kv_end = 0;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  // keys this wave's rows may see, and where the causal mask starts to bite
  const int w_end = causal ? max(0, min(L, L - n + min(rw + kWR, n))) : L;
  const int w_free = causal ? max(0, L - n + rw + 1) : L;  // keys visible to every row of the wave

  // Q^T operands: lane (row col of row block rb, group grp) holds
  // q[row][kk*32 + grp*8 .. +8]
  bf16x8 qb[kRB][NK];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    const bool ok = row < n;
    const bf16* qp = q + ((int64_t)(q0 + (ok ? row : 0)) * Hq + h) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + kk * 32);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      qb[rb][kk] = as_bf16x8(v);
    }
  }
  int row_end[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    row_end[rb] = causal ? min(L, L - n + row + 1) : L;
  }

  f32x4 acc[kRB][NT];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc_l[kRB];  // row sums (any column)
  float m_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    acc_l[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
  }

  if (ntiles > 0) {
    const SlotMap<FMT> sm = make_slotmap<FMT>(m, i);
    const char* kb = k_pool + (int64_t)g * D * 2;
    const char* vb = v_pool + (int64_t)g * D * 2;
    // table entries of a tile's 64 keys (keys past kv_end repeat the last
    // visible key, so every row read is a real, finite one)
    auto tab_dma = [&](int kt) {
      const int t = min(min(kt, ntiles - 1) * kBN + lane, kv_end - 1);
      dma4(sm.raw_ptr(t), lds_off(&tab_lds[w][kt % (S + 1)][0]));
    };
    // K and V rows of a tile; wave w moves chunk positions
    // [w * NI/2 * 64, (w + 1) * NI/2 * 64) of each.  A lane's key row within
    // the tile and its swizzled byte offset within the row are the same for
    // every tile, so they are computed once.
    int dt[NI / 2], dc[NI / 2];
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
      const unsigned pos = (unsigned)((w * (NI / 2) + j) * 64 + lane);
      dt[j] = (int)(pos / CPK);
      dc[j] = (int)(((pos % CPK) ^ (pos / CPK & 7)) * 16);
    }
    const uint32_t rbytes = (uint32_t)row_bytes;  // one token row (all heads) is far below 4 GiB
    auto kv_dma = [&](int kt) {
      const int32_t* tr = &tab_lds[w][kt % (S + 1)][0];
      const int k0 = min(kt, ntiles - 1) * kBN;
      char* kt_lds = kv_lds[kt % S][0];
      char* vt_lds = kv_lds[kt % S][1];
#pragma unroll
      for (int j = 0; j < NI / 2; ++j) {
        const int tt = min(k0 + dt[j], kv_end - 1);
        const uint32_t slot = (uint32_t)sm.finish(tr[dt[j]], tt, true);  // in [0, num_slots)
        const uint64_t off = (uint64_t)slot * rbytes + (uint32_t)dc[j];
        dma16(kb + off, lds_off(kt_lds + (w * (NI / 2) + j) * 1024));
        dma16(vb + off, lds_off(vt_lds + (w * (NI / 2) + j) * 1024));
      }
    };
    // prologue: queue = [tables 0 .. S-1 landed] tile 0 .. tile S-2, table S-1 ..
    for (int k = 0; k < S; ++k) tab_dma(k);
    // the tables and the queries have landed.  A wait the compiler sees:
    // otherwise it adds its own before the first score product, where it
    // would also drain the tile DMAs issued below
    __builtin_amdgcn_s_waitcnt(0);
    for (int k = 0; k < S - 1; ++k) kv_dma(k);

    // per-lane parts of the LDS addresses; the tile loop is unrolled by the
    // stage count so stage bases and subtile steps become immediates.
    // K operand (token a*16 + col, chunk kk*4 + grp): chunk bits above the
    // swizzle are kk / 2, so two bases (kk even / odd) cover every read.
    const int sk = col & 7;
    const int kbase0 = (col * CPK + (grp ^ sk)) * 16;
    const int kbase1 = (col * CPK + ((4 + grp) ^ sk)) * 16;
    // V operand (token b*32 + 4j + x/4, chunk 2 nt + (x&3)/2): four bases by
    // nt & 3, the rest immediates
    int vbase[4];
    {
      const int x = lane & 15, j = lane >> 4;
      const int t = 4 * j + (x >> 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) vbase[u] = (t * CPK + ((2 * u + ((x & 3) >> 1)) ^ (t & 7))) * 16 + (x & 1) * 8;
    }
    const char* lds0 = &kv_lds[0][0][0];
    const bf16x8 ones = bf16x8{(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};

    // ---- S^T = K Q^T of tile kt (stage st): four 16-key subtiles x kRB
    // 16-row blocks (softcapped, if asked)
    auto qk = [&](auto stage_c, f32x4 (&sacc)[4][kRB]) {
      constexpr int st = decltype(stage_c)::value;
      const char* ks = lds0 + (st * 2 + 0) * C::TILE;
#pragma unroll
      for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[a2][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const char* kb = ks + ((kk & 1) ? kbase1 : kbase0) + (kk >> 1) * 128;
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2) {
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + a2 * 16 * CPK * 16));
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) sacc[a2][rb] = mfma16x16x32(ka, qb[rb][kk], sacc[a2][rb]);
        }
      }
      if constexpr (SC) {
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sacc[a2][rb][rr] = cap(sacc[a2][rb][rr]);
      }
    };

    // ---- the softmax of tile kt's scores and O^T += V^T P^T (stage st)
    auto smpv = [&](int kt, auto stage_c, auto mask_c, f32x4 (&sacc)[4][kRB]) {
      constexpr int st = decltype(stage_c)::value;
      constexpr bool MASK = decltype(mask_c)::value;
      const char* vs = lds0 + (st * 2 + 1) * C::TILE;
      const int k0 = kt * kBN;

      // ---- online softmax (log2 domain); lane holds keys k0 + 16a + 4grp + rr
      // of row rb*16 + col.  The max is taken on raw scores (the scale is
      // positive), so each probability is one fma and one exp2.  O is kept
      // transposed (lane col = row, like the scores), so the per-row rescale
      // is a plain multiply in every lane: no cross-lane traffic.
      // Keys past a row's visible range get -inf in place (boundary tiles
      // only).  The row's reference m_run moves only when a score passes it
      // by more than kExtSlack (log2 units), so probabilities stay below
      // 2^kExtSlack and the accumulators are rescaled only on the (rare)
      // tiles where some row of the wave moves; any reference gives the same
      // normalised result.  A row's first visible key always moves it
      // (-inf + slack = -inf).  One branch covers all row blocks, so the
      // softmax of the row blocks stays one basic block.
      if (MASK) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int lim = row_end[rb] - k0 - grp * 4;  // key a2*16 + rr of this lane is visible below lim
#pragma unroll
          for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (a2 * 16 + rr >= lim) sacc[a2][rb][rr] = -INFINITY;
        }
      }
      // Common case first: each lane compares its own maximum with the
      // row's reference, and only when some lane of the wave passes it does
      // the wave take the cross-lane row maxima and rescale.
      float lane_max[kRB];
      bool lane_bump = false;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float mr = -INFINITY;
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) mr = fmaxf(mr, sacc[a2][rb][rr]);
        lane_max[rb] = mr;
        lane_bump |= mr * scale_log2 > m_run[rb] + kExtSlack;
      }
      if (__builtin_amdgcn_ballot_w64(lane_bump) != 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const float m_tile = max_xor16_32(lane_max[rb]) * scale_log2;
          const bool bump = m_tile > m_run[rb] + kExtSlack;  // the same in the row's four lanes
          const float alpha = bump ? fast_exp2(m_run[rb] - m_tile) : 1.0f;
          m_run[rb] = bump ? m_tile : m_run[rb];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rb][nt] *= alpha;
          acc_l[rb] *= alpha;
        }
      }
      bf16x8 pa[kRB][2];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // a row that has seen no key yet keeps m = -inf: use 0 so p = 0
        const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            pa[rb][a2 >> 1][(a2 & 1) * 4 + rr] = (bf16)fast_exp2(fmaf(sacc[a2][rb][rr], scale_log2, -mu));
      }

      // ---- O^T += V^T P^T over two 32-key halves (each V fragment serves
      // both row blocks); the row sums ride along as a row of ones in V^T
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const char* lo = vs + vbase[nt & 3] + (nt >> 2) * 128 + b2 * 32 * CPK * 16;
          const i16x4 va = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
          const i16x4 vc = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * CPK * 16));
          const bf16x4 ba = __builtin_bit_cast(bf16x4, va), bc = __builtin_bit_cast(bf16x4, vc);
          const bf16x8 vf = bf16x8{ba[0], ba[1], ba[2], ba[3], bc[0], bc[1], bc[2], bc[3]};
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb][nt] = mfma16x16x32(vf, pa[rb][b2], acc[rb][nt]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc_l[rb] = mfma16x16x32(ones, pa[rb][b2], acc_l[rb]);
      }
    };

    // ---- key-split form of the two above: this wave's 16-key slice of
    // the tile against all kRB row blocks.  The lane holds keys
    // k0 + 16 w + 4 grp + rr of row rb * 16 + col, which is also the B
    // operand of the 16-key P V^T product.
    auto qk_ks = [&](auto stage_c, f32x4 (&sacc)[kRB]) {
      constexpr int st = decltype(stage_c)::value;
      const char* ks_lds = lds0 + (st * 2 + 0) * C::TILE + w * 16 * CPK * 16;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 ka =
            as_bf16x8(*reinterpret_cast<const u32x4*>(ks_lds + ((kk & 1) ? kbase1 : kbase0) + (kk >> 1) * 128));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[rb] = mfma16x16x32(ka, qb[rb][kk], sacc[rb]);
      }
      if constexpr (SC) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sacc[rb][rr] = cap(sacc[rb][rr]);
      }
    };
    auto smpv_ks = [&](int kt, auto stage_c, auto mask_c, f32x4 (&sacc)[kRB]) {
      constexpr int st = decltype(stage_c)::value;
      constexpr bool MASK = decltype(mask_c)::value;
      const char* vs = lds0 + (st * 2 + 1) * C::TILE + w * 16 * CPK * 16;
      const int k0 = kt * kBN + w * 16;
      if (MASK) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int lim = row_end[rb] - k0 - grp * 4;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (rr >= lim) sacc[rb][rr] = -INFINITY;
        }
      }
      float lane_max[kRB];
      bool lane_bump = false;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float mr = fmaxf(fmaxf(sacc[rb][0], sacc[rb][1]), fmaxf(sacc[rb][2], sacc[rb][3]));
        lane_max[rb] = mr;
        lane_bump |= mr * scale_log2 > m_run[rb] + kExtSlack;
      }
      if (__builtin_amdgcn_ballot_w64(lane_bump) != 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const float m_tile = max_xor16_32(lane_max[rb]) * scale_log2;
          const bool bump = m_tile > m_run[rb] + kExtSlack;
          const float alpha = bump ? fast_exp2(m_run[rb] - m_tile) : 1.0f;
          m_run[rb] = bump ? m_tile : m_run[rb];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rb][nt] *= alpha;
          acc_l[rb] *= alpha;
        }
      }
      i16x4 pb[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
        bf16x4 p;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) p[rr] = (bf16)fast_exp2(fmaf(sacc[rb][rr], scale_log2, -mu));
        pb[rb] = __builtin_bit_cast(i16x4, p);
      }
      const i16x4 ones4 = __builtin_bit_cast(i16x4, bf16x4{(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const i16x4 va = lds_read_tr16(reinterpret_cast<const bf16*>(vs + vbase[nt & 3] + (nt >> 2) * 128));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[rb][nt] = mfma16x16x16(va, pb[rb], acc[rb][nt]);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) acc_l[rb] = mfma16x16x16(ones4, pb[rb], acc_l[rb]);
    };

    auto step = [&](int kt, auto stage_c, auto ks_c) {
      constexpr bool KS = decltype(ks_c)::value;
      tab_dma(kt + S);
      wait_vm<C::WAIT>();  // tile kt and table kt + S - 1 have landed
      __syncthreads();     // tile kt visible to all waves; every wave is past tile kt - 1
      kv_dma(kt + S - 1);  // into the stage tile kt - 1 used
      // a wave whose rows are all past n, or whose rows see none of this
      // tile's keys, only helps move the tiles; keys past what every row of
      // the wave sees need the per-element mask
      if (rw < n && kt * kBN < w_end) {
        if constexpr (KS) {
          f32x4 sacc[kRB];
          qk_ks(stage_c, sacc);
          if (kt * kBN + kBN <= w_free)
            smpv_ks(kt, stage_c, std::false_type{}, sacc);
          else
            smpv_ks(kt, stage_c, std::true_type{}, sacc);
        } else {
          f32x4 sacc[4][kRB];
          qk(stage_c, sacc);
          if (kt * kBN + kBN <= w_free)
            smpv(kt, stage_c, std::false_type{}, sacc);
          else
            smpv(kt, stage_c, std::true_type{}, sacc);
        }
      }
    };
    auto tiles = [&](auto ks_c) {
      for (int kt = 0; kt < ntiles; kt += S) {
        step(kt, std::integral_constant<int, 0>{}, ks_c);
        if (kt + 1 < ntiles) step(kt + 1, std::integral_constant<int, 1>{}, ks_c);
        if constexpr (S > 2) {
          if (kt + 2 < ntiles) step(kt + 2, std::integral_constant<int, 2 % S>{}, ks_c);
        }
        if constexpr (S > 3) {
          if (kt + 3 < ntiles) step(kt + 3, std::integral_constant<int, 3 % S>{}, ks_c);
        }
        static_assert(S <= 4, "the tile loop is unrolled for at most four stages");
      }
    };
    if (ks)
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    wait_vm<0>();  // no load may still target this block's LDS when it ends
  }

  if (ks) {
    // ---- merge the four waves' partial states of the block's rows: each
    // wave leaves its O rows (fp32), row references and row sums in the
    // tile buffers, then wave w finishes d columns [D / 4 w, D / 4 (w + 1))
    // of every row: O = sum_w exp2(m_w - m) O_w / sum_w exp2(m_w - m) l_w.
    static_assert(4 * kWR * D * 4 <= S * 2 * C::TILE, "partial rows fit the tile buffers");
    static_assert(2 * 4 * kWR * 4 <= (int)sizeof(tab_lds), "row statistics fit the table buffers");
    float* po = reinterpret_cast<float*>(&kv_lds[0][0][0]);  // [wave][row][d]
    float* pm = reinterpret_cast<float*>(&tab_lds[0][0][0]);  // [wave][row]
    float* pl = pm + 4 * kWR;
    __syncthreads();  // every wave is done with the tiles
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int r = rb * 16 + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(po + ((w * kWR + r) * D + nt * 16 + grp * 4)) = acc[rb][nt];
      if (grp == 0) {
        pm[w * kWR + r] = m_run[rb];
        pl[w * kWR + r] = acc_l[rb][0];
      }
    }
    __syncthreads();
    constexpr int DW = D / 4;  // d columns this wave finishes
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int r = rb * 16 + col;
      const int row = rw + r;
      float mw[4], m = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        mw[v] = pm[v * kWR + r];
        m = fmaxf(m, mw[v]);
      }
      float wt[4], lt = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        wt[v] = mw[v] == -INFINITY ? 0.f : fast_exp2(mw[v] - m);
        lt += wt[v] * pl[v * kWR + r];
      }
      const bool any = lt > 0.f;
      const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
      for (int d4 = 0; d4 < DW / 16; ++d4) {
        const int d0 = w * DW + d4 * 16 + grp * 4;
        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) o += wt[v] * *reinterpret_cast<const f32x4*>(po + ((v * kWR + r) * D + d0));
        if (row < n) {
          bf16x4 ov;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) ov[rr] = (bf16)(o[rr] * inv);
          *reinterpret_cast<bf16x4*>(out + ((int64_t)(q0 + row) * Hq + h) * D + d0) = ov;
        }
      }
      if (lse && w == 0 && grp == 0 && row < n)
        lse[(int64_t)(q0 + row) * Hq + h] = any ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    }
    return;
  }

  // ---- finalise: lane (row col of block rb, group grp) holds
  // O[row][16 nt + 4 grp + rr] and the row's sum in acc_l
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    if (row < n) {
      const int64_t o = ((int64_t)(q0 + row) * Hq + h);
      const float lt = acc_l[rb][0];
      const bool any = lt > 0.f;
      const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v[rr] = (bf16)(acc[rb][nt][rr] * inv);
        *reinterpret_cast<bf16x4*>(out + o * D + nt * 16 + grp * 4) = v;
      }
      if (lse && grp == 0) lse[o] = any ? (m_run[rb] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// The same extend with the two waves of each SIMD in opposite phases.
//
// A wave's work per 64-key tile t splits into a matrix phase, MM(t) = the
// P V^T of tile t - 1 and the K Q^T of tile t, and a softmax phase SM(t)
// (masks, row maxima, exponentials: vector ALU).  Eight waves share the
// tiles; waves w and w + 4 sit on the same SIMD.  Group A (waves 0..3) runs
// MM(t) while group B (waves 4..7) runs SM(t - 1), and then A runs SM(t)
// while B runs MM(t), with a workgroup barrier between the halves, so each
// SIMD has one wave on the matrix cores while the other is on the vector
// ALU.  The two waves of a SIMD take adjacent row ranges, so a short query
// block still pairs its waves.
// ---------------------------------------------------------------------------
template <int D>
struct PpCfg {
  static constexpr int RB = D == 64 ? 3 : 2;  // 16-row blocks per wave
  static constexpr int W = 8;                 // waves per workgroup
  static constexpr int WR = 16 * RB;          // query rows per wave
  static constexpr int BM = W * WR;           // query rows per workgroup
  static constexpr int NK = D / 32;
  static constexpr int NT = D / 16;
  static constexpr int CPK = D / 8;
  static constexpr int TILE = kBN * D * 2;
  static constexpr int NI = 2 * TILE / 1024 / W;  // K+V DMA instructions per wave per tile
  static constexpr int S = D == 64 ? 5 : 4;       // LDS stages
  static constexpr int R = S + 1;                 // table ring entries per wave (the prologue loads S at once)
  // Iteration t issues the table of tile t + S and then the rows of tile
  // t + S - 2.  Before its first barrier it needs tile t's rows and tile
  // t + S - 2's table; the memory operations a wave may leave outstanding
  // then are the smaller of those issued after either.
  static constexpr int WAIT_ROWS = (S - 3) * (NI + 1) + 1;
  static constexpr int WAIT_TAB = 2 * NI + 2;
  static constexpr int WAIT = WAIT_ROWS < WAIT_TAB ? WAIT_ROWS : WAIT_TAB;
  static constexpr int WAIT0 = (S - 3) * NI + 1;  // iteration 0: the prologue issued no tables between its tiles
};

template <int D, int FMT, bool SC>
__global__ void __launch_bounds__(512, 1) extend_pp_kernel(DevMap m, const char* k_pool, const char* v_pool,
                                                       int64_t row_bytes, const bf16* __restrict__ q, int64_t total_q,
                                                       const int32_t* __restrict__ qo_indptr, int32_t Hq,
                                                       int32_t n_req, int32_t n_qtiles, int32_t G, int32_t causal_all,
                                                       const int32_t* __restrict__ causal_flags, SoftCap cap,
                                                       float scale_log2, bf16* __restrict__ out,
                                                       float* __restrict__ lse) {
  using C = PpCfg<D>;
  constexpr int NK = C::NK, NT = C::NT, CPK = C::CPK, NI = C::NI, S = C::S, R = C::R;
  constexpr int kRB = C::RB, kWR = C::WR, kBM = C::BM;
  static_assert(C::WAIT0 <= C::WAIT && C::WAIT < 64, "wait counts");
  __shared__ __attribute__((aligned(1024))) char kv_lds[S][2][C::TILE];
  __shared__ __attribute__((aligned(256))) int32_t tab_lds[C::W][R][64];

  // block -> (pair, query tile) exactly as in extend_kernel
  const int x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
  const int ppx = (int)(((int64_t)n_req * Hq + 7) / 8);
  const bool qt_major = causal_all && !causal_flags;
  const int pair = x + 8 * (qt_major ? k % ppx : k / n_qtiles);
  const int qt = qt_major ? n_qtiles - 1 - k / ppx : k % n_qtiles;
  const int h = pair % Hq;
  const int i = pair / Hq;
  if (i >= n_req) return;
  const int causal = causal_flags ? (causal_flags[i] != 0) : causal_all;
  const int q0 = qo_indptr[i];
  const int n = (q0 < 0 || q0 >= total_q) ? 0 : (int)min((int64_t)(qo_indptr[i + 1] - q0), total_q - q0);
  if (qt * kBM >= n) return;
  int L = m.kv_lens[i];
  if (FMT == SLOT_CONTIG && m.total_k <= 0) L = 0;
  if (L < 0) L = 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = h / G;
  const int grp_w = w >> 2;  // 0: group A, 1: group B
  const int rw = qt * kBM + (2 * (w & 3) + grp_w) * kWR;  // the SIMD's two waves take adjacent rows

  int kv_end = L;
  if (causal) kv_end = min(L, L - n + min(qt * kBM + kBM, n));
  if (kv_end < 0) kv_end = 0;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const int w_end = causal ? max(0, min(L, L - n + min(rw + kWR, n))) : L;
  const int w_free = causal ? max(0, L - n + rw + 1) : L;
  // tiles this wave computes (0 when its rows are all past n)
  const int Tw = rw < n ? min(ntiles, (w_end + kBN - 1) / kBN) : 0;

  bf16x8 qb[kRB][NK];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    const bool ok = row < n;
    const bf16* qp = q + ((int64_t)(q0 + (ok ? row : 0)) * Hq + h) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + kk * 32);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      qb[rb][kk] = as_bf16x8(v);
    }
  }
  int row_end[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    row_end[rb] = causal ? min(L, L - n + row + 1) : L;
  }

  f32x4 acc[kRB][NT];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc_l[kRB];
  float m_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    acc_l[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
  }

  if (ntiles > 0) {
    const SlotMap<FMT> sm = make_slotmap<FMT>(m, i);
    const char* kb = k_pool + (int64_t)g * D * 2;
    const char* vb = v_pool + (int64_t)g * D * 2;
    auto tab_dma = [&](int kt) __attribute__((always_inline)) {
      const int t = min(min(kt, ntiles - 1) * kBN + lane, kv_end - 1);
      dma4(sm.raw_ptr(t), lds_off(&tab_lds[w][kt % R][0]));
    };
    int dt[NI / 2], dc[NI / 2];
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
      const unsigned pos = (unsigned)((w * (NI / 2) + j) * 64 + lane);
      dt[j] = (int)(pos / CPK);
      dc[j] = (int)(((pos % CPK) ^ (pos / CPK & 7)) * 16);
    }
    const uint32_t rbytes = (uint32_t)row_bytes;
    auto kv_dma = [&](int kt) __attribute__((always_inline)) {
      const int32_t* tr = &tab_lds[w][kt % R][0];
      const int k0 = min(kt, ntiles - 1) * kBN;
      char* kt_lds = kv_lds[kt % S][0];
      char* vt_lds = kv_lds[kt % S][1];
#pragma unroll
      for (int j = 0; j < NI / 2; ++j) {
        const int tt = min(k0 + dt[j], kv_end - 1);
        const uint32_t slot = (uint32_t)sm.finish(tr[dt[j]], tt, true);
        const uint64_t off = (uint64_t)slot * rbytes + (uint32_t)dc[j];
        dma16(kb + off, lds_off(kt_lds + (w * (NI / 2) + j) * 1024));
        dma16(vb + off, lds_off(vt_lds + (w * (NI / 2) + j) * 1024));
      }
    };
    // prologue: the tables of tiles 0 .. S - 1 and the queries land (a wait
    // the compiler sees), then the rows of tiles 0 .. S - 3
    for (int kk = 0; kk < S; ++kk) tab_dma(kk);
    __builtin_amdgcn_s_waitcnt(0);
    for (int kk = 0; kk < S - 2; ++kk) kv_dma(kk);

    const int sk = col & 7;
    const int kbase0 = (col * CPK + (grp ^ sk)) * 16;
    const int kbase1 = (col * CPK + ((4 + grp) ^ sk)) * 16;
    int vbase[4];
    {
      const int xx = lane & 15, j = lane >> 4;
      const int t = 4 * j + (xx >> 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) vbase[u] = (t * CPK + ((2 * u + ((xx & 3) >> 1)) ^ (t & 7))) * 16 + (xx & 1) * 8;
    }
    const char* lds0 = &kv_lds[0][0][0];
    const bf16x8 ones = bf16x8{(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};

    f32x4 sacc[4][kRB];    // scores of the tile whose softmax is next
    bf16x8 pa[kRB][2];     // probabilities of the tile whose P V^T is next

    // K Q^T of the tile in stage st
    auto qk = [&](auto stage_c) __attribute__((always_inline)) {
      constexpr int st = decltype(stage_c)::value;
      const char* ks = lds0 + (st * 2 + 0) * C::TILE;
#pragma unroll
      for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[a2][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const char* kp = ks + ((kk & 1) ? kbase1 : kbase0) + (kk >> 1) * 128;
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2) {
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + a2 * 16 * CPK * 16));
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) sacc[a2][rb] = mfma16x16x32(ka, qb[rb][kk], sacc[a2][rb]);
        }
      }
    };
    // O^T += V^T P^T of the tile in stage st (row sums as a row of ones)
    auto pv = [&](auto stage_c) __attribute__((always_inline)) {
      constexpr int st = decltype(stage_c)::value;
      const char* vs = lds0 + (st * 2 + 1) * C::TILE;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const char* lo = vs + vbase[nt & 3] + (nt >> 2) * 128 + b2 * 32 * CPK * 16;
          const i16x4 va = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
          const i16x4 vc = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * CPK * 16));
          const bf16x4 ba = __builtin_bit_cast(bf16x4, va), bc = __builtin_bit_cast(bf16x4, vc);
          const bf16x8 vf = bf16x8{ba[0], ba[1], ba[2], ba[3], bc[0], bc[1], bc[2], bc[3]};
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb][nt] = mfma16x16x32(vf, pa[rb][b2], acc[rb][nt]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc_l[rb] = mfma16x16x32(ones, pa[rb][b2], acc_l[rb]);
      }
    };
    // softmax of tile kt's scores into pa (softcap, masks, reference moves
    // and rescales exactly as in extend_kernel)
    auto smx = [&](int kt, auto mask_c) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      const int k0 = kt * kBN;
      if constexpr (SC) {
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sacc[a2][rb][rr] = cap(sacc[a2][rb][rr]);
      }
      if (MASK) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int lim = row_end[rb] - k0 - grp * 4;
#pragma unroll
          for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (a2 * 16 + rr >= lim) sacc[a2][rb][rr] = -INFINITY;
        }
      }
      float lane_max[kRB];
      bool lane_bump = false;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float mr = -INFINITY;
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) mr = fmaxf(mr, sacc[a2][rb][rr]);
        lane_max[rb] = mr;
        lane_bump |= mr * scale_log2 > m_run[rb] + kExtSlack;
      }
      if (__builtin_amdgcn_ballot_w64(lane_bump) != 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const float m_tile = max_xor16_32(lane_max[rb]) * scale_log2;
          const bool bump = m_tile > m_run[rb] + kExtSlack;
          const float alpha = bump ? fast_exp2(m_run[rb] - m_tile) : 1.0f;
          m_run[rb] = bump ? m_tile : m_run[rb];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rb][nt] *= alpha;
          acc_l[rb] *= alpha;
        }
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            pa[rb][a2 >> 1][(a2 & 1) * 4 + rr] = (bf16)fast_exp2(fmaf(sacc[a2][rb][rr], scale_log2, -mu));
      }
    };
    auto SM = [&](int kt) __attribute__((always_inline)) {
      if (kt >= 0 && kt < Tw) {
        if (kt * kBN + kBN <= w_free) smx(kt, std::false_type{});
        else smx(kt, std::true_type{});
      }
    };
    // MM(t): P V^T of tile t - 1 (stage SP), K Q^T of tile t (stage SK)
    auto MM = [&](int t, auto sk_c, auto sp_c) __attribute__((always_inline)) {
      if (t >= 1 && t - 1 < Tw) pv(sp_c);
      if (t < Tw) qk(sk_c);
    };
    // iteration t (stage j = t % S): slot 2t then slot 2t + 1
    auto iter = [&](int t, auto j_c) __attribute__((always_inline)) {
      constexpr int j = decltype(j_c)::value;
      tab_dma(t + S);
      if (t == 0) wait_vm<C::WAIT0>();
      else wait_vm<C::WAIT>();
      __syncthreads();     // tile t in LDS; every wave past slot 2t - 1
      kv_dma(t + S - 2);   // into the stage of tile t - 2 (last read in slot 2t - 1)
      if (grp_w == 0) MM(t, std::integral_constant<int, j>{}, std::integral_constant<int, (j + S - 1) % S>{});
      else SM(t - 1);
      __syncthreads();
      if (grp_w == 0) SM(t);
      else MM(t, std::integral_constant<int, j>{}, std::integral_constant<int, (j + S - 1) % S>{});
    };
    static_assert(S == 4 || S == 5, "the iteration loop is unrolled for four or five stages");
    for (int tb = 0; tb <= ntiles; tb += S) {
      iter(tb, std::integral_constant<int, 0>{});
      if (tb + 1 <= ntiles) iter(tb + 1, std::integral_constant<int, 1>{});
      if (tb + 2 <= ntiles) iter(tb + 2, std::integral_constant<int, 2>{});
      if (tb + 3 <= ntiles) iter(tb + 3, std::integral_constant<int, 3>{});
      if constexpr (S > 4) {
        if (tb + 4 <= ntiles) iter(tb + 4, std::integral_constant<int, 4 % S>{});
      }
    }
    wait_vm<0>();  // no load may still target this block's LDS when it ends
  }

#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw + rb * 16 + col;
    if (row < n) {
      const int64_t o = ((int64_t)(q0 + row) * Hq + h);
      const float lt = acc_l[rb][0];
      const bool any = lt > 0.f;
      const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v[rr] = (bf16)(acc[rb][nt][rr] * inv);
        *reinterpret_cast<bf16x4*>(out + o * D + nt * 16 + grp * 4) = v;
      }
      if (lse && grp == 0) lse[o] = any ? (m_run[rb] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 pools: the same attention on the vector ALUs, in fp32 throughout.  One
// wavefront per (request, query head, four query rows): lane group r = lane
// / 16 holds row r, and lane c = lane % 16 holds elements [c E, c E + E) of
// the row's query, of every key and value it reads and of its output (E = D
// / 16).  The four rows read the same keys, four at a time (loads first,
// then the dot products, reduced over the 16 lanes of a row), with an online
// softmax per row.  Keys past a row's visible range get a zero weight;
// every row read is a real key of the request (past the wave's last visible
// key, reads repeat that key), so no NaN of an unused slot enters a sum.
// ---------------------------------------------------------------------------
template <int D, int FMT, bool SC>
__global__ void __launch_bounds__(256) extend_f32_kernel(DevMap m, const float* k_pool, const float* v_pool,
                                                         int64_t row_elems, const float* __restrict__ q,
                                                         int64_t total_q, const int32_t* __restrict__ qo_indptr,
                                                         int32_t Hq, int32_t n_req, int32_t n_qtiles, int32_t G,
                                                         int32_t causal_all, const int32_t* __restrict__ causal_flags,
                                                         SoftCap cap, float scale_log2, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  constexpr int E = D / 16;
  constexpr int UK = 4;  // keys per step
  const int qt = (int)(blockIdx.x % n_qtiles);
  const int rest = (int)(blockIdx.x / n_qtiles);
  const int h = rest % Hq, i = rest / Hq;
  if (i >= n_req) return;
  const int causal = causal_flags ? (causal_flags[i] != 0) : causal_all;
  const int q0 = qo_indptr[i];
  const int n = (q0 < 0 || q0 >= total_q) ? 0 : (int)min((int64_t)(qo_indptr[i + 1] - q0), total_q - q0);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane >> 4, c = lane & 15;
  const int wrow = qt * 16 + w * 4;  // first row of this wave
  if (wrow >= n) return;             // uniform per wave
  int L = m.kv_lens[i];
  if (FMT == SLOT_CONTIG && m.total_k <= 0) L = 0;
  if (L < 0) L = 0;
  const int row = wrow + r;
  const bool ok = row < n;
  const int row_end = ok ? (causal ? max(0, min(L, L - n + row + 1)) : L) : 0;
  int wave_end = row_end;
  for (int o = 16; o <= 32; o <<= 1) wave_end = max(wave_end, __shfl_xor(wave_end, o, 64));
  float qv[E];
  {
    const float* qp = q + ((int64_t)(q0 + (ok ? row : 0)) * Hq + h) * D + c * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(qp + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) qv[e + k] = ok ? v[k] : 0.f;
    }
  }
  const SlotMap<FMT> sm = make_slotmap<FMT>(m, i);
  const int g = h / G;
  const float* kb = k_pool + (int64_t)g * D + c * E;
  const float* vb = v_pool + (int64_t)g * D + c * E;
  float m_run = -INFINITY, l_run = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int t0 = 0; t0 < wave_end; t0 += UK) {
    float kv[UK][E], vv[UK][E];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int64_t slot = sm(min(t0 + u, wave_end - 1), true);
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(kb + slot * row_elems + e);
        const f32x4 b = *reinterpret_cast<const f32x4*>(vb + slot * row_elems + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kv[u][e + k] = a[k];
          vv[u][e + k] = b[k];
        }
      }
    }
    float x[UK];
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(qv[e], kv[u][e], d);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) d += __shfl_xor(d, off, 64);
      if constexpr (SC) d = cap(d);
      x[u] = (t0 + u < row_end) ? d * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[u]);
    }
    // a row that has seen no key yet keeps m = -inf: use 0 so every weight is 0
    const float mu = mx == -INFINITY ? 0.f : mx;
    const float corr = fast_exp2(m_run - mu);
    l_run *= corr;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const float p = fast_exp2(x[u] - mu);
      l_run += p;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(p, vv[u][e], o[e]);
    }
    m_run = mx;
  }
  if (ok) {
    const int64_t idx = (int64_t)(q0 + row) * Hq + h;
    const bool any = l_run > 0.f;
    const float inv = any ? 1.0f / l_run : 0.f;
    float* op = out + idx * D + c * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      f32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = o[e + k] * inv;
      *reinterpret_cast<f32x4*>(op + e) = v;
    }
    if (lse && c == 0) lse[idx] = any ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool extend_supported(const PoolInfo& p, int32_t num_q_heads) {
  return p.kind == 0 && (p.dtype == 1 || p.dtype == 0) && p.head_dim_qk == p.head_dim_v &&
         (p.head_dim_qk == 64 || p.head_dim_qk == 128) && num_q_heads % p.num_kv_heads == 0;
}

template <int D, int FMT>
static void launch_ext_f32(hipStream_t s, const DevMap& m, const char* kp, const char* vp, int64_t row_elems,
                           const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t max_q_len, int32_t bs,
                           int32_t G, int32_t causal, const int32_t* flags, float softcap, float sm_scale, void* out,
                           float* lse) {
  const int32_t qtiles = (max_q_len + 15) / 16;  // 16 rows per workgroup (four waves of four)
  const dim3 grid((unsigned)((int64_t)bs * Hq * qtiles));
  const float sl2 = sm_scale * kLog2e;
  const float* k = reinterpret_cast<const float*>(kp);
  const float* v = reinterpret_cast<const float*>(vp);
  if (softcap > 0.0f) {
    const SoftCap cap{2.0f * kLog2e * sm_scale / softcap, softcap / sm_scale};
    hipLaunchKernelGGL((extend_f32_kernel<D, FMT, true>), grid, dim3(256), 0, s, m, k, v, row_elems,
                       static_cast<const float*>(q), tq, qo, Hq, bs, qtiles, G, causal, flags, cap, sl2,
                       static_cast<float*>(out), lse);
  } else {
    hipLaunchKernelGGL((extend_f32_kernel<D, FMT, false>), grid, dim3(256), 0, s, m, k, v, row_elems,
                       static_cast<const float*>(q), tq, qo, Hq, bs, qtiles, G, causal, flags, SoftCap{0.f, 0.f}, sl2,
                       static_cast<float*>(out), lse);
  }
}

template <int D>
static void launch_ext_f32_fmt(hipStream_t s, const DevMap& m, const char* kp, const char* vp, int64_t row_elems,
                               const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t max_q_len, int32_t bs,
                               int32_t G, int32_t causal, const int32_t* flags, float softcap, float sm_scale,
                               void* out, float* lse) {
  if (m.fmt == MAP_TOKEN_TABLE)
    launch_ext_f32<D, SLOT_TABLE>(s, m, kp, vp, row_elems, q, tq, qo, Hq, max_q_len, bs, G, causal, flags, softcap,
                                  sm_scale, out, lse);
  else if (m.fmt == MAP_CONTIGUOUS)
    launch_ext_f32<D, SLOT_CONTIG>(s, m, kp, vp, row_elems, q, tq, qo, Hq, max_q_len, bs, G, causal, flags, softcap,
                                   sm_scale, out, lse);
  else
    launch_ext_f32<D, SLOT_PAGES>(s, m, kp, vp, row_elems, q, tq, qo, Hq, max_q_len, bs, G, causal, flags, softcap,
                                  sm_scale, out, lse);
}

template <int D, int FMT>
static void launch_ext(dim3 grid, hipStream_t s, const DevMap& m, const char* kp, const char* vp, int64_t row_bytes,
                       const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t G, int32_t causal,
                       const int32_t* flags, float softcap, float sm_scale, void* out, float* lse, bool pp) {
  const int32_t qtiles = (int32_t)grid.y;
  const int32_t nreq = (int32_t)grid.z;
  const int64_t pairs = (int64_t)nreq * Hq;
  const dim3 g1((unsigned)(8 * ((pairs + 7) / 8) * qtiles));
  const float sl2 = sm_scale * kLog2e;
  // pp: the phase-alternating kernel (see launch_extend)
  if (pp) {
    const SoftCap cap{2.0f * kLog2e * sm_scale / softcap, softcap / sm_scale};
    hipLaunchKernelGGL((extend_pp_kernel<D, FMT, true>), g1, dim3(512), 0, s, m, kp, vp, row_bytes,
                       static_cast<const bf16*>(q), tq, qo, Hq, nreq, qtiles, G, causal, flags, cap, sl2,
                       static_cast<bf16*>(out), lse);
  } else if (softcap > 0.0f) {
    const SoftCap cap{2.0f * kLog2e * sm_scale / softcap, softcap / sm_scale};
    hipLaunchKernelGGL((extend_kernel<D, FMT, true>), g1, dim3(256), 0, s, m, kp, vp, row_bytes,
                       static_cast<const bf16*>(q), tq, qo, Hq, nreq, qtiles, G, causal, flags, cap, sl2,
                       static_cast<bf16*>(out), lse);
  } else {
    hipLaunchKernelGGL((extend_kernel<D, FMT, false>), g1, dim3(256), 0, s, m, kp, vp, row_bytes,
                       static_cast<const bf16*>(q), tq, qo, Hq, nreq, qtiles, G, causal, flags, SoftCap{0.f, 0.f},
                       sl2, static_cast<bf16*>(out), lse);
  }
}

template <int D>
static void launch_ext_fmt(dim3 grid, hipStream_t s, const DevMap& m, const char* kp, const char* vp,
                           int64_t row_bytes, const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t G,
                           int32_t causal, const int32_t* flags, float softcap, float sm_scale, void* out,
                           float* lse, bool pp) {
  if (m.fmt == MAP_TOKEN_TABLE)
    launch_ext<D, SLOT_TABLE>(grid, s, m, kp, vp, row_bytes, q, tq, qo, Hq, G, causal, flags, softcap, sm_scale, out,
                              lse, pp);
  else if (m.fmt == MAP_CONTIGUOUS)
    launch_ext<D, SLOT_CONTIG>(grid, s, m, kp, vp, row_bytes, q, tq, qo, Hq, G, causal, flags, softcap, sm_scale, out,
                               lse, pp);
  else
    launch_ext<D, SLOT_PAGES>(grid, s, m, kp, vp, row_bytes, q, tq, qo, Hq, G, causal, flags, softcap, sm_scale, out,
                              lse, pp);
}

hipError_t launch_extend(const PoolInfo& p, int32_t layer, const void* q, int64_t total_q, const int32_t* qo_indptr,
                         int32_t Hq, int32_t max_q_len, const DevMap& m, int32_t bs, int32_t max_kv_len,
                         int32_t causal, const int32_t* causal_flags, float softcap, float sm_scale, void* out,
                         float* lse, hipStream_t s) {
  (void)max_kv_len;
  if (bs == 0 || max_q_len == 0) return hipSuccess;
  // contiguous (ragged) maps read the caller's gathered K/V, paged maps the pool
  const char* kp = reinterpret_cast<const char*>(m.fmt == MAP_CONTIGUOUS ? m.contig_k : p.k_layer(layer));
  const char* vp = reinterpret_cast<const char*>(m.fmt == MAP_CONTIGUOUS ? m.contig_v : p.v_layer(layer));
  const int G = Hq / p.num_kv_heads;
  if (p.dtype == 0) {  // fp32 pool: the vector-ALU kernel
    const int64_t row_elems = (int64_t)p.num_kv_heads * p.head_dim_qk;
    timer_before(s);
    if (p.head_dim_qk == 128)
      launch_ext_f32_fmt<128>(s, m, kp, vp, row_elems, q, total_q, qo_indptr, Hq, max_q_len, bs, G, causal,
                              causal_flags, softcap, sm_scale, out, lse);
    else
      launch_ext_f32_fmt<64>(s, m, kp, vp, row_elems, q, total_q, qo_indptr, Hq, max_q_len, bs, G, causal,
                             causal_flags, softcap, sm_scale, out, lse);
    hipError_t e = hipGetLastError();
    timer_after(s);
    return e;
  }
  // (query tiles, -, requests); the launcher flattens it XCD-aware
  // The phase-alternating kernel (extend_pp_kernel) pays where the softmax
  // phase is heavy (a softcap adds an exp2 and a reciprocal per score) and
  // the query blocks fill its larger workgroups (at least one on average):
  // measured, softcapped mixed spans 0.40 -> 0.375 ms; uncapped mixed spans
  // 0.31 -> 0.33 and the encoder-decoder extend 0.17 -> 0.32 ms (short
  // blocks leave a CU with one mostly empty workgroup).
  const int pp_bm = p.head_dim_qk == 128 ? PpCfg<128>::BM : PpCfg<64>::BM;
  const bool pp = softcap > 0.0f && total_q >= (int64_t)bs * pp_bm;
  const int bm = pp ? pp_bm : (p.head_dim_qk == 128 ? ExtendCfg<128>::BM : ExtendCfg<64>::BM);
  const dim3 grid(1, (unsigned)((max_q_len + bm - 1) / bm), (unsigned)bs);
  const int64_t row_bytes = (int64_t)p.num_kv_heads * p.head_dim_qk * 2;  // one token row, all KV heads
  if (row_bytes > (int64_t)UINT32_MAX) return hipErrorInvalidValue;  // the kernel's row offsets are 32-bit
  timer_before(s);
  if (p.head_dim_qk == 128)
    launch_ext_fmt<128>(grid, s, m, kp, vp, row_bytes, q, total_q, qo_indptr, Hq, G, causal, causal_flags, softcap,
                        sm_scale, out, lse, pp);
  else
    launch_ext_fmt<64>(grid, s, m, kp, vp, row_bytes, q, total_q, qo_indptr, Hq, G, causal, causal_flags, softcap,
                       sm_scale, out, lse, pp);
  hipError_t e = hipGetLastError();
  timer_after(s);
  return e;
}

}  // namespace pkv
