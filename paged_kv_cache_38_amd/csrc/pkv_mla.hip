// MLA (latent) paged decode.
//
// What is computed: the decode of [XPU] "From slots to a page table" and
// [BACKEND] init_forward_metadata over a latent pool -- one cached row per
// token of head_dim_qk = 576 values (512 latent + 64 rope, [BACKEND] "页表构建":
// kv_lora_rank / qk_rope_head_dim), shared by every query head.  Keys are the
// whole row; values are its first 512 entries.  The result is softmax
// attention over each request's keys in logical order; splitting is an
// implementation detail merged back exactly with log-sum-exp weights.
//
// Design for gfx950 (one workgroup per CU, all query heads of a request in
// one workgroup, so every latent row leaves HBM exactly once):
//
//  * Work split.  The requests' 32-token tiles are laid end to end and the
//    grid (one workgroup per CU) takes equal contiguous runs of them, so every
//    CU streams the same number of bytes whatever the length mix.  A run may
//    end inside a request and the next run continue it: such pieces are
//    partial results, merged afterwards.  A planner kernel resolves every tile
//    to its 32 slot ids (through any table format) before the main kernel
//    starts, so the main kernel never touches a table.
//  * Streaming.  Tiles move HBM -> LDS with global_load_lds_dwordx4 (no
//    staging registers), four tiles deep: while tile r is computed, tiles
//    r+1 .. r+3 are in flight (about 100 KiB per CU).  The tile layout in LDS is row-major with a
//    16-byte-chunk XOR swizzle (chunk c of token t sits at c ^ (t & 7)), so
//    both the K-operand reads and the transposed V-operand reads are free of
//    bank conflicts.  These loads are issued from inline assembly and waited
//    on explicitly, because the compiler would otherwise drain the whole
//    queue before every LDS read.
//  * Math.  Wave w computes S^T = K Q^T for its 32 heads (queries held in
//    registers) and the softmax for them; P goes through LDS; then every wave
//    computes O += P V for all heads over its own slice of the 512 value
//    columns (accumulators in AGPRs).  The softmax reference is the maximum
//    of a piece's first tile and then stays fixed, so the accumulators are
//    never rescaled (any reference gives the same normalised result); should
//    a later score exceed it by more than 2^64 (P could overflow), the
//    request is recomputed exactly by a fallback in the merge pass.
#include <math.h>

#include <algorithm>

#include "pkv_launch.h"

namespace pkv {

constexpr int kMlaQK = 576;
constexpr int kMlaV = 512;
constexpr int kMlaT = kStreamT;                   // tokens per tile
constexpr int kMlaRowChunks = kMlaQK / 8;         // 72 sixteen-byte chunks per row
constexpr int kMlaRowBytes = kMlaQK * 2;          // 1152
constexpr int kMlaTileBytes = kMlaT * kMlaRowBytes;  // 36864
constexpr int kMlaMetaWords = kStreamMetaWords;   // per tile: 32 slot ids + 8 info words
constexpr int kMlaBufs = 4;                       // LDS tile buffers: three tiles in flight during compute
constexpr int kMlaMetaRing = 8;                   // per-wave ring of per-tile slot ids / info
constexpr float kMlaHeadroom = 64.0f;             // log2 units a score may exceed the reference by

// Launch shape per workgroup of HPB heads (16, 32 or 64): W waves; wave w
// computes scores for HB blocks of 16 heads and output columns
// [w * CW, (w + 1) * CW) of all HPB heads.  A wave then holds 72 VGPRs of
// queries and 128 accumulators.  More than 64 heads take sibling workgroups
// (one per 64 heads) that stream the same tiles on the same XCD, the second
// read served by its L2.
template <int HPB>
struct MlaCfg {
  static constexpr int W = HPB / 16;
  static constexpr int HB = 1;
  static constexpr int NHB = HPB / 16;
  static constexpr int CW = kMlaV / W;
  static constexpr int NCB = CW / 16;
  static constexpr int NI = (kMlaTileBytes / 1024) / W;  // tile DMA instructions per wave
};

// The P*V accumulators live in AGPRs for the whole kernel: outside the MFMAs
// they are only read (through this), never redefined in a branch, which would
// make the compiler copy all of them on every tile.
__device__ __forceinline__ float acc_get(float a) {
  float v;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// byte offset of chunk c of token t inside a swizzled tile
__device__ __forceinline__ int mla_chunk_off(int t, int c) { return (t * kMlaRowChunks + (c ^ (t & 7))) * 16; }

// B operand of P*V (16x16x32 MFMA) from a swizzled tile: lane (n = l%16,
// j = l/16) receives V[4j + r][c0 + n] (r = 0..3) and V[16 + 4j + r][c0 + n].
__device__ __forceinline__ bf16x8 mla_v_operand(const char* tile, int c0, int lane) {
  const int x = lane & 15, j = lane >> 4;
  const int t = 4 * j + (x >> 2);
  const int c = c0 + 4 * (x & 3);
  const char* lo = tile + mla_chunk_off(t, c >> 3) + (c & 7) * 2;
  const i16x4 a = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
  const i16x4 b = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * kMlaRowBytes));
  const bf16x4 ba = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
  return bf16x8{ba[0], ba[1], ba[2], ba[3], bb[0], bb[1], bb[2], bb[3]};
}

// O += P V for one tile over a wave's NCB column blocks and NHB head
// blocks; P fragments of all heads and four column blocks of V at a time
// in registers.  Column block cb = 4 m + u of the whole row: the
// transposed read of lane (x, j) starts at token t = 4 j + x / 4, chunk
// 8 (cb / 4) + ((2 u + (x & 3) / 2) ^ (t & 7)): four per-lane bases (u) plus
// compile-time offsets.  ZERO starts the accumulators from zero.
template <int NHB, int NCB, bool ZERO>
__device__ __forceinline__ void mla_pv(f32x4 (&acc)[NHB][NCB], const char* tile, const bf16x8* p_lds, int w,
                                       int lane) {
  const int x = lane & 15, jg = lane >> 4;
  const int t = 4 * jg + (x >> 2);
  const char* vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    vb[u] = tile + (t * kMlaRowChunks + ((2 * u + ((x & 3) >> 1)) ^ (t & 7))) * 16 + (x & 1) * 8 +
            (w * NCB / 4) * 128;
  bf16x8 pf[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) pf[hb] = p_lds[hb * 64 + lane];
#pragma unroll
  for (int cg = 0; cg < NCB; cg += 4) {
    bf16x8 vf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const char* lo = vb[u] + (cg / 4) * 128;
      const i16x4 va = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
      const i16x4 vc = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * kMlaRowBytes));
      const bf16x4 ba = __builtin_bit_cast(bf16x4, va), bc = __builtin_bit_cast(bf16x4, vc);
      vf[u] = bf16x8{ba[0], ba[1], ba[2], ba[3], bc[0], bc[1], bc[2], bc[3]};
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[hb][cg + u] = mfma16x16x32(pf[hb], vf[u], ZERO ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[hb][cg + u]);
  }
}

// ---------------------------------------------------------------------------
// Main kernel.
// ---------------------------------------------------------------------------
template <int HPB>
__global__ void __launch_bounds__(64 * MlaCfg<HPB>::W, 1) mla_decode_kernel(
    const char* kpool, const bf16* __restrict__ q, int32_t HQ, int32_t sibs, const int32_t* __restrict__ header,
    const int32_t* __restrict__ meta, float scale_log2, bf16* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int32_t* __restrict__ fallback) {
  using C = MlaCfg<HPB>;
  constexpr int W = C::W, HB = C::HB, NHB = C::NHB, CW = C::CW, NCB = C::NCB, NI = C::NI;
  constexpr int NK = kMlaQK / 32;  // 18 k-steps of the score product

  __shared__ __attribute__((aligned(1024))) char tiles[kMlaBufs][kMlaTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 p_lds[NHB * 64];
  __shared__ __attribute__((aligned(256))) int32_t meta_lds[W][kMlaMetaRing][64];
  __shared__ __attribute__((aligned(16))) float l_lds[HPB];
  __shared__ __attribute__((aligned(16))) float m_lds[HPB];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // run and sibling: siblings sit 8 workgroups apart, on the same XCD
  const int run = sibs == 1 ? (int)blockIdx.x : (int)(blockIdx.x / 16 * 8 + blockIdx.x % 8);
  const int h0 = sibs == 1 ? 0 : (int)(blockIdx.x / 8 % 2) * HPB;
  const int Bt = header[0], total = header[1];
  const int G0 = run * Bt;
  if (G0 >= total) return;
  const int n = min(Bt, total - G0);

  // ---- loaders (every wave issues the same number of each, in the same order)
  auto meta_dma = [&](int r) {
    const int g = G0 + min(r, n - 1);
    dma4(meta + (int64_t)g * kMlaMetaWords + min(lane, kMlaMetaWords - 1), lds_off(&meta_lds[w][r & (kMlaMetaRing - 1)][0]));
  };
  auto tile_dma = [&](int r) {
    const int32_t* ms = &meta_lds[w][r & (kMlaMetaRing - 1)][0];
    char* buf = tiles[r % kMlaBufs];
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recompute the per-lane positions every tile instead of holding them
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int pos = (w * NI + j) * 64 + ln;  // 16-byte chunk position in the tile
      const int t = pos / kMlaRowChunks;
      const int c = (pos - t * kMlaRowChunks) ^ (t & 7);
      const int64_t slot = ms[t];
      dma16(kpool + slot * kMlaRowBytes + c * 16, lds_off(buf + (w * NI + j) * 1024));
    }
  };

  f32x4 acc[NHB][NCB];
#pragma unroll
  for (int a = 0; a < NHB; ++a)
#pragma unroll
    for (int b = 0; b < NCB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 qf[HB][NK];
  float m_ref[HB], l_part[HB];

  // Per iteration r a wave issues meta(r + 6) then tile(r + 3); tile(r) is
  // then followed in the queue by meta(r + 4), tile(r + 1), meta(r + 5),
  // tile(r + 2), meta(r + 6): 2 NI + 3 operations.  The prologue builds that
  // state for r = 0.
  constexpr int kWait = 2 * NI + 3 < 63 ? 2 * NI + 3 : 63;
  meta_dma(0);
  meta_dma(1);
  meta_dma(2);
  wait_vm<0>();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    meta_dma(k + 3);
    tile_dma(k);
  }

  for (int r = 0; r < n; ++r) {
    meta_dma(r + 6);
    wait_vm<kWait>();   // tile(r) (and every meta before it) has landed
    __syncthreads();    // tile r visible to all waves; every wave is past P*V of tile r - 1
    tile_dma(r + 3);    // into the buffer tile r - 1 used

    const int32_t* info = &meta_lds[w][r & (kMlaMetaRing - 1)][32];
    const int i = __builtin_amdgcn_readfirstlane(info[0]);
    const int jt = __builtin_amdgcn_readfirstlane(info[1]);
    const int T = __builtin_amdgcn_readfirstlane(info[2]);
    const int P = __builtin_amdgcn_readfirstlane(info[3]);
    const int valid = __builtin_amdgcn_readfirstlane(info[4]);
    const bool seg_begin = (r == 0) || (jt == 0);
    const bool seg_end = (r == n - 1) || (jt == T - 1);
    const char* tile = tiles[r % kMlaBufs];

    if (seg_begin) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = h0 + (w * HB + hb) * 16 + col;
        const bf16* qp = q + ((int64_t)i * HQ + h) * kMlaQK + grp * 8;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) qf[hb][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 32));
        l_part[hb] = 0.f;
      }
    }

    // ---- S^T = K Q^T for this wave's heads.  Chunk 4kk + grp of token t
    // sits at 8 (kk / 2) + ((4 (kk & 1) + grp) ^ (t & 7)): two per-lane bases
    // (even / odd kk) plus compile-time offsets.
    f32x4 sacc[2][HB];
    {
      const int t = col;  // token 16a + col; (t & 7) is the same for a = 0, 1
      const char* kb_even = tile + (t * kMlaRowChunks + (grp ^ (t & 7))) * 16;
      const char* kb_odd = tile + (t * kMlaRowChunks + ((4 + grp) ^ (t & 7))) * 16;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[a][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K fragments stream through a window of KD k-steps (2 fragments each);
      // a sched barrier per step keeps the compiler from hoisting all 36
      // reads (which would need 144 more VGPRs)
      constexpr int KD = 5;
      bf16x8 kf[KD][2];
      auto kload = [&](int kk, bf16x8* dst) {
        const char* kb = (kk & 1) ? kb_odd : kb_even;
#pragma unroll
        for (int a = 0; a < 2; ++a)
          dst[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + a * 16 * kMlaRowBytes + (kk >> 1) * 128));
      };
#pragma unroll
      for (int kk = 0; kk < KD - 1; ++kk) kload(kk, kf[kk]);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (kk + KD - 1 < NK) kload(kk + KD - 1, kf[(kk + KD - 1) % KD]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) sacc[a][hb] = mfma16x16x32(kf[kk % KD][a], qf[hb][kk], sacc[a][hb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- softmax (log2 domain) for head 16 * (w * HB + hb) + col; this lane
    // holds tokens 16a + 4 grp + rr.  The reference maximum is the first
    // tile's maximum and stays fixed for the piece, so the accumulators are
    // never rescaled; a later score more than kMlaHeadroom above it (P could
    // overflow) sends the request to the exact fallback in the merge pass.
    bool over = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float x[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = 16 * a + 4 * grp + rr;
          x[a][rr] = t < valid ? sacc[a][hb][rr] * scale_log2 : -INFINITY;
        }
      if (seg_begin) {
        float mt = -INFINITY;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) mt = fmaxf(mt, x[a][rr]);
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        m_ref[hb] = mt;
      }
      bf16x8 pa;
      float ps = 0.f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          over |= x[a][rr] > m_ref[hb] + kMlaHeadroom;
          const float p = fast_exp2(x[a][rr] - m_ref[hb]);
          ps += p;
          pa[a * 4 + rr] = (bf16)p;
        }
      l_part[hb] += ps;
      p_lds[(w * HB + hb) * 64 + lane] = pa;
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) fallback[i] = 1;
    __syncthreads();  // P of every wave is in LDS

    // ---- O += P V over this wave's columns, all heads (the first tile of a
    // piece starts the accumulators from zero inside the MFMA)
    if (seg_begin)
      mla_pv<NHB, NCB, true>(acc, tile, p_lds, w, lane);
    else
      mla_pv<NHB, NCB, false>(acc, tile, p_lds, w, lane);

    if (seg_end) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float lt = l_part[hb] + shfl_xor(l_part[hb], 16);
        lt += shfl_xor(lt, 32);
        if (grp == 0) {
          l_lds[(w * HB + hb) * 16 + col] = lt;
          m_lds[(w * HB + hb) * 16 + col] = m_ref[hb];
        }
      }
      __syncthreads();
      const int b0 = P / Bt, b1 = (P + T - 1) / Bt;
      const bool direct = b0 == b1;
      // per-lane bases computed here (not hoisted out of the tile loop), then
      // compile-time offsets: head 16 hb + 4 grp + rr, column w CW + 16 cb + col
      int g4 = 4 * grp;
      asm volatile("" : "+v"(g4));
      const int64_t row0 = (direct ? (int64_t)i * HQ : ((int64_t)run + i) * HQ) + h0 + g4;
      bf16* ob = out + row0 * kMlaV + w * CW + col;
      float* wb = ws_o + row0 * kMlaV + w * CW + col;
      float* lb = (direct ? lse : ws_lse) + (lse || !direct ? row0 : 0);
      const bool write_lse = (lse || !direct) && w == 0 && col == 0;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&l_lds[hb * 16 + g4]);
        const f32x4 mv = *reinterpret_cast<const f32x4*>(&m_lds[hb * 16 + g4]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hoff = hb * 16 + rr;
          const float inv = 1.0f / lv[rr];
          if (direct) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) ob[hoff * kMlaV + cb * 16] = (bf16)(acc_get(acc[hb][cb][rr]) * inv);
          } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) wb[hoff * kMlaV + cb * 16] = acc_get(acc[hb][cb][rr]) * inv;
          }
          if (write_lse) lb[hoff] = (mv[rr] + __log2f(lv[rr])) * kLn2;
        }
      }
      // no zeroing here: the next segment's first tile rescales every head
      // by exp2(-inf) = 0 (the accumulators are finite), and redefining the
      // accumulators in this branch would cost a full copy per tile
    }
  }
  wait_vm<0>();  // no load may still target this workgroup's LDS when it ends
}

// ---------------------------------------------------------------------------
// Exact fallback for one (request, head): plain online softmax over the
// request's keys, one key at a time (lane l holds query values 9l .. 9l+8 and
// value columns 8l .. 8l+7).  Only requests whose scores outran the fixed
// softmax reference by more than the headroom come here.
// ---------------------------------------------------------------------------
__device__ void mla_exact_one(const char* kpool, const bf16* q_row, const int32_t* meta, int P, int L, float scale_log2,
                              int lane, bf16* op, float* lse_out) {
  float qv[9];
#pragma unroll
  for (int e = 0; e < 9; ++e) qv[e] = (float)q_row[lane * 9 + e];
  float m = -INFINITY, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < L; ++t) {
    const int64_t slot = meta[(int64_t)(P + t / kMlaT) * kMlaMetaWords + t % kMlaT];
    const bf16* row = reinterpret_cast<const bf16*>(kpool + slot * kMlaRowBytes);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 9; ++e) d += qv[e] * (float)row[lane * 9 + e];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += shfl_xor(d, off);
    const float sc = d * scale_log2;
    const float mn = fmaxf(m, sc);
    const float corr = fast_exp2(m - mn), p = fast_exp2(sc - mn);
    l = l * corr + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * corr + p * (float)row[lane * 8 + e];
    m = mn;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) op[e] = (bf16)(o[e] / l);
  if (lse_out && lane == 0) *lse_out = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Merge: one wavefront per (request, head).  Requests finished inside one run
// were written directly; empty requests get zeros and lse = -inf; flagged
// requests are recomputed exactly; the rest combine their pieces (ids
// run + request) with log-sum-exp weights.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mla_merge_kernel(int32_t bs, int32_t Hq, const int32_t* __restrict__ header,
                                                        const int32_t* __restrict__ prefix,
                                                        const int32_t* __restrict__ ntiles,
                                                        const int32_t* __restrict__ fallback,
                                                        const float* __restrict__ ws_o,
                                                        const float* __restrict__ ws_lse, const char* kpool,
                                                        const bf16* __restrict__ q, const int32_t* __restrict__ meta,
                                                        const int32_t* __restrict__ kv_lens, float scale_log2,
                                                        bf16* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)bs * Hq) return;
  const int i = (int)(idx / Hq), h = (int)(idx % Hq);
  bf16* op = out + idx * kMlaV + lane * 8;
  const int T = ntiles[i];
  if (T == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e] = (bf16)0.0f;
    if (lse && lane == 0) lse[idx] = -INFINITY;
    return;
  }
  const int P = prefix[i];
  if (fallback[i]) {
    const int L = min(kv_lens[i], T * kMlaT);
    mla_exact_one(kpool, q + idx * kMlaQK, meta, P, L, scale_log2, lane, op, lse ? lse + idx : nullptr);
    return;
  }
  const int Bt = header[0];
  const int b0 = P / Bt, b1 = (P + T - 1) / Bt;
  if (b0 == b1) return;
  float mx = -INFINITY;
  for (int b = b0; b <= b1; ++b) mx = fmaxf(mx, ws_lse[((int64_t)b + i) * Hq + h]);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  for (int b = b0; b <= b1; ++b) {
    const int64_t row = ((int64_t)b + i) * Hq + h;
    const float wgt = __expf(ws_lse[row] - mx);
    const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + row * kMlaV + lane * 8);
    const f32x4 x0 = src[0], x1 = src[1];
    sum += wgt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] += wgt * x0[e];
      o[4 + e] += wgt * x1[e];
    }
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int e = 0; e < 8; ++e) op[e] = (bf16)(o[e] * inv);
  if (lse && lane == 0) lse[idx] = mx + __logf(sum);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool mla_decode_supported(const PoolInfo& p, int32_t Hq) {
  return p.kind == 1 && p.dtype == 1 && p.num_kv_heads == 1 && p.head_dim_qk == kMlaQK && p.head_dim_v == kMlaV &&
         (Hq == 16 || Hq == 32 || Hq == 64 || Hq == 128);
}

DecodePlan plan_mla_decode(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len) {
  (void)p;
  (void)bs;
  DecodePlan plan;
  plan.kind = 3;
  plan.chunk = max_kv_len > 0 ? (max_kv_len + kMlaT - 1) / kMlaT : 0;  // tiles per request, at most
  // runs of tiles: one workgroup per CU, two sibling workgroups per run
  // above 64 heads (an even split of the CUs)
  plan.max_splits = Hq > 64 ? std::max(8, device_cu_count() / 2 / 8 * 8) : device_cu_count();
  return plan;
}

template <int HPB>
static void launch_mla_main(int32_t runs, int32_t Hq, hipStream_t s, const char* kp, const void* q, const StreamWs& w,
                            float sl2, void* out, float* lse) {
  const int sibs = Hq / HPB;
  hipLaunchKernelGGL((mla_decode_kernel<HPB>), dim3(runs * sibs), dim3(64 * MlaCfg<HPB>::W), 0, s, kp,
                     static_cast<const bf16*>(q), Hq, sibs, w.header, w.meta, sl2, static_cast<bf16*>(out), lse,
                     w.o, w.lse, w.fallback);
}

hipError_t launch_mla_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m, int32_t bs,
                             const DecodePlan& plan, float sl2, void* out, float* lse, void* ws, hipStream_t s) {
  StreamWs w;
  stream_ws_layout(bs, plan.chunk, plan.max_splits, Hq, kMlaV, ws, &w);
  const int32_t runs = plan.max_splits;
  hipError_t e = launch_stream_plan(m, bs, plan.chunk, runs, w, s);
  if (e != hipSuccess) return e;
  const char* kp = p.k_layer(layer);
  timer_before(s);
  if (Hq >= 64) launch_mla_main<64>(runs, Hq, s, kp, q, w, sl2, out, lse);
  else if (Hq == 32) launch_mla_main<32>(runs, Hq, s, kp, q, w, sl2, out, lse);
  else launch_mla_main<16>(runs, Hq, s, kp, q, w, sl2, out, lse);
  e = hipGetLastError();
  timer_after(s);
  if (e != hipSuccess) return e;
  const unsigned mblocks = (unsigned)(((int64_t)bs * Hq + 3) / 4);
  hipLaunchKernelGGL(mla_merge_kernel, dim3(mblocks), dim3(256), 0, s, bs, Hq, w.header, w.prefix, w.ntiles,
                     w.fallback, w.o, w.lse, kp, static_cast<const bf16*>(q), w.meta, m.kv_lens, sl2,
                     static_cast<bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace pkv
