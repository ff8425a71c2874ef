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
// Design for gfx950 (one workgroup per CU holding every query head of the
// request, so every latent row leaves HBM exactly once):
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
//  * Math.  Each wave owns 32 query heads (16 when there are fewer than 128)
//    end to end: S^T = K Q^T with the queries in registers, the softmax, and
//    O += P V over all 512 value columns with the accumulators in AGPRs, P
//    going straight from the score registers into the MFMA A operand.  The
//    scores come in two halves of 16 tokens with their results in VGPRs.
//    Every K and V fragment read from LDS feeds two MFMAs (two 16-head
//    blocks), and one barrier per tile is the only synchronisation.  The
//    softmax reference is the maximum over the first half of a piece's first
//    tile and then stays fixed, so the accumulators are never rescaled (any
//    reference gives the same normalised result); should a later score
//    exceed it by more than 2^64 (P could overflow), the request is
//    recomputed exactly by a fallback in the merge pass.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "pkv_launch.h"

namespace pkv {

constexpr int kMlaQK = 576;
constexpr int kMlaV = 512;
constexpr int kMlaT = kStreamT;                   // tokens per tile
constexpr int kMlaRowBytes = kMlaQK * 2;          // 1152
constexpr int kMlaTileBytes = kMlaT * kMlaRowBytes;  // 36864
// LDS tile layout: the main part holds chunks 0..63 of every row (1024 B
// per row, values 0..511: all of V and most of K), the tail part chunks
// 64..71 (the 64 rope values) of every row, 128 B per row, in the order the
// waves move them.  In both, chunk c of row t sits at position c ^ (t & 7)
// of its row (c counted from the part's first chunk).
constexpr int kMlaMainBytes = 1024;
constexpr int kMlaTailOff = kMlaT * kMlaMainBytes;  // 32768
constexpr int kMlaMetaWords = kStreamMetaWords;   // per tile: 32 slot ids + 8 info words
constexpr int kMlaBufs = 4;                       // LDS tile buffers: three tiles in flight during compute
constexpr int kMlaMetaRing = 8;                   // per-wave ring of per-tile slot ids / info
constexpr int kMlaSlice = 128;                    // rows (heads x drafts) of one main-kernel launch
constexpr int kMlaMaxRows = 1024;                 // rows of one call, in slices of kMlaSlice
constexpr float kMlaHeadroom = 64.0f;             // log2 units a score may exceed the reference by

// Launch shape: W waves per workgroup, HB blocks of 16 query heads per wave
// (Hq = 16 HB W).  A wave owns its heads end to end: queries in registers
// (72 VGPRs per 16 heads), scores, softmax and the P*V accumulators of all
// 512 value columns (128 AGPRs per 16 heads), so P never leaves the wave.
// With HB = 2 every K and V fragment read from LDS feeds two MFMAs.
template <int HB, int W>
struct MlaShape {
  static constexpr int RPW = kMlaT / W;      // tile rows moved per wave
  static constexpr int NI = RPW + RPW / 8;   // tile DMA instructions per wave (a row each, a tail per 8 rows)
  static_assert(RPW * W == kMlaT && RPW % 8 == 0, "rows split evenly over the waves, tails in groups of eight");
};

// The P*V accumulators live in AGPRs for the whole kernel: outside the MFMAs
// they are only read (through this), never redefined in a branch, which would
// make the compiler copy all of them on every tile.
__device__ __forceinline__ float acc_get(float a) {
  float v;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// One MFMA of the score product, issued from inline assembly so that its
// result lands in VGPRs.  Left to the compiler, every MFMA of this kernel
// takes the AGPR-result form: the score accumulators would then claim AGPRs
// beside the 256 P*V accumulators, and the compiler would shuttle
// accumulators between the register files on every tile.  Opaque to the
// compiler, the asm carries the wait states the hardware needs after a
// half's last MFMA: the 19 that cover a VALU read of a 16-pass result.  Its
// operands come from LDS reads and global loads, never from a VALU write
// just before it (which would need two more wait states; a test checks the
// built code for that).  FIRST starts the accumulator from zero.
__device__ __forceinline__ void mfma_score(f32x4& c, const bf16x8& a, const bf16x8& b, bool first, bool tail) {
  if (first)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  else if (tail)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// V operand reads of column group m (column blocks 4 m .. 4 m + 3) for
// O += P V.  The B operand of column block cb = 4 m + u comes from two
// transposed reads: lane (x, j) starts at token t = 4 j + x / 4, chunk
// 8 m + ((2 u + (x & 3) / 2) ^ (t & 7)), so four per-lane bases (u) plus
// compile-time offsets cover every read; lane (x, j) then holds
// V[4j + r][16 cb + x] and V[16 + 4j + r][16 cb + x] (r = 0..3), the token
// order of the P fragment the score layout leaves in the lane.
__device__ __forceinline__ void mla_v_group(const char* tile, int lane, int m, bf16x8 (&vf)[4]) {
  const int x = lane & 15, jg = lane >> 4;
  const int t = 4 * jg + (x >> 2);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const char* lo = tile + t * kMlaMainBytes + ((2 * u + ((x & 3) >> 1)) ^ (t & 7)) * 16 + (x & 1) * 8 + m * 128;
    const i16x4 va = lds_read_tr16(reinterpret_cast<const bf16*>(lo));
    const i16x4 vc = lds_read_tr16(reinterpret_cast<const bf16*>(lo + 16 * kMlaMainBytes));
    const bf16x4 ba = __builtin_bit_cast(bf16x4, va), bc = __builtin_bit_cast(bf16x4, vc);
    vf[u] = bf16x8{ba[0], ba[1], ba[2], ba[3], bc[0], bc[1], bc[2], bc[3]};
  }
}

// O += P V for one tile over all 32 column blocks of the wave's HB head
// blocks.  ZERO starts the accumulators from zero inside the MFMA.
template <int HB, bool ZERO>
__device__ __forceinline__ void mla_pv(f32x4 (&acc)[HB][kMlaV / 16], const char* tile, const bf16x8 (&pa)[HB],
                                       int lane) {
  // groups of four column blocks, the next group's reads in flight while
  // this group's MFMAs run
  bf16x8 vf[2][4];
  mla_v_group(tile, lane, 0, vf[0]);
#pragma unroll
  for (int m = 0; m < kMlaV / 64; ++m) {
    if (m + 1 < kMlaV / 64) mla_v_group(tile, lane, m + 1, vf[(m + 1) & 1]);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[hb][4 * m + u] = mfma16x16x32(pa[hb], vf[m & 1][u], ZERO ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[hb][4 * m + u]);
    __builtin_amdgcn_sched_barrier(0);  // keep later groups' reads from being hoisted (VGPRs)
  }
}

// ---------------------------------------------------------------------------
// Main kernel: one workgroup per run (one per CU).
// ---------------------------------------------------------------------------
// VERIFY (target verification, [BACKEND] init_forward_metadata's
// target-verify branch): every request carries n_draft query tokens whose
// heads are folded into the head dimension (row = draft * hq_base + head,
// HQ = n_draft * hq_base rows), and the keys include the drafts.  Draft j
// sits at position L - n_draft + j and sees keys 0 .. L - n_draft + j
// (bottom-right, as in extend), so the tiles holding the last n_draft - 1
// keys take a per-row mask.
template <int HB, int W, bool VERIFY>
__global__ void __launch_bounds__(64 * W, 1) mla_decode_kernel(
    const char* kpool, const bf16* __restrict__ q, int32_t HQ, const int32_t* __restrict__ header,
    const int32_t* __restrict__ meta, float scale_log2, bf16* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int32_t* __restrict__ fallback,
    const int32_t* __restrict__ kv_lens, int32_t n_draft, int32_t hq_base, int32_t row_stride, int32_t row_off) {
  constexpr int NI = MlaShape<HB, W>::NI, RPW = MlaShape<HB, W>::RPW;
  constexpr int NK = kMlaQK / 32;  // 18 k-steps of the score product
  constexpr int NC = kMlaV / 16;   // 32 column blocks of the output

  __shared__ __attribute__((aligned(1024))) char tiles[kMlaBufs][kMlaTileBytes];
  __shared__ __attribute__((aligned(256))) int32_t meta_lds[W][kMlaMetaRing][64];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int run = (int)blockIdx.x;
  const int Bt = header[0], total = header[1];
  const int G0 = run * Bt;
  if (G0 >= total) return;
  const int n = min(Bt, total - G0);
  const int hw = w * HB * 16;  // first head of this wave

  // ---- loaders (every wave issues the same number of each, in the same order)
  auto tile_slots = [&](int r) -> int32_t {  // lane l: slot of row l % 32 of tile r
    return meta_lds[w][r & (kMlaMetaRing - 1)][lane & 31];
  };
  auto meta_dma = [&](int r) {
    const int g = G0 + min(r, n - 1);
    dma4(meta + (int64_t)g * kMlaMetaWords + min(lane, kMlaMetaWords - 1), lds_off(&meta_lds[w][r & (kMlaMetaRing - 1)][0]));
  };
  // Wave w moves rows w, w + W, ... of a tile: per row one 64-lane DMA of
  // chunks 0..63 into the main part, from the row's address in SGPRs (slot
  // id via v_readlane), lane l fetching chunk l ^ (row & 7); and per eight
  // rows one 64-lane DMA of their chunks 64..71 into the tail part (lane l:
  // row l / 8 of the group, its slot read from the ring by tail_slots).
  // Part p of 3 issues rows [p RPW / 3, (p + 1) RPW / 3) of the wave and,
  // with the last part, the tail DMAs: the main loop spreads a tile's DMAs
  // over its phases.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  struct TailSlots {
    int32_t s[RPW / 8];
  };
  auto tail_slots = [&](int r) {
    TailSlots ts;
#pragma unroll
    for (int g8 = 0; g8 < RPW / 8; ++g8)
      ts.s[g8] = meta_lds[w][r & (kMlaMetaRing - 1)][(g8 * 8 + (lane >> 3)) * W + wu];
    return ts;
  };
  auto tile_dma = [&](int r, int32_t vslot, TailSlots ts, auto part_c) {
    constexpr int p = decltype(part_c)::value;
    char* buf = tiles[r % kMlaBufs];
    // pinned here: without it the slot reads and address arithmetic of every
    // part get hoisted to the top of the tile, where they wait for the LDS
    // read of the slots before the first score step can start
    asm volatile("" : "+v"(vslot));
#pragma unroll
    for (int k = p * RPW / 3; k < (p + 1) * RPW / 3; ++k) {
      const int t = k * W + wu;
      const int32_t slot = __builtin_amdgcn_readlane(vslot, t);
      const char* row = kpool + (int64_t)slot * kMlaRowBytes;
      dma16_s(row, ((uint32_t)lane ^ (uint32_t)(t & 7)) << 4, lds_off(buf + t * kMlaMainBytes));
    }
    if constexpr (p == 2) {
#pragma unroll
      for (int g8 = 0; g8 < RPW / 8; ++g8) asm volatile("" : "+v"(ts.s[g8]));
#pragma unroll
      for (int g8 = 0; g8 < RPW / 8; ++g8) {
        const int k = g8 * 8 + (lane >> 3);
        const int t = k * W + wu;
        const char* src = kpool + (int64_t)ts.s[g8] * kMlaRowBytes + (64 + ((lane & 7) ^ (t & 7))) * 16;
        dma16(src, lds_off(buf + kMlaTailOff + (wu * RPW + g8 * 8) * 128));
      }
    }
  };

  f32x4 acc[HB][NC];
#pragma unroll
  for (int a = 0; a < HB; ++a)
#pragma unroll
    for (int b = 0; b < NC; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 qf[HB][NK];
  float m_ref[HB], l_part[HB];
  float s_over[HB];  // raw score above which P could overflow (kMlaHeadroom past the reference)
  // VERIFY: the request's first key that the first draft cannot see (a
  // row's draft index is worked out in the tiles that need it)
  int k_zone = 0;

  // Per iteration r a wave issues meta(r + 6) then tile(r + 3); tile(r) is
  // then followed in the queue by meta(r + 4), tile(r + 1), meta(r + 5),
  // tile(r + 2), meta(r + 6): 2 NI + 3 operations.  The prologue builds that
  // state for r = 0.  (Above 63 the counter's maximum waits for more.)
  constexpr int kWait = 2 * NI + 3 < 63 ? 2 * NI + 3 : 63;
  meta_dma(0);
  meta_dma(1);
  meta_dma(2);
  wait_vm<0>();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    meta_dma(k + 3);
    const int32_t vs = tile_slots(k);
    const TailSlots ts = tail_slots(k);
    tile_dma(k, vs, ts, std::integral_constant<int, 0>{});
    tile_dma(k, vs, ts, std::integral_constant<int, 1>{});
    tile_dma(k, vs, ts, std::integral_constant<int, 2>{});
  }
  // the info words of a tile (request, tile of the request, tiles of the
  // request, first tile of the request, valid keys) are loaded into SGPRs
  // one tile ahead, so their LDS latency never sits at the top of a tile
  auto tile_info = [&](int r, int k) { return __builtin_amdgcn_readlane(meta_lds[w][r & (kMlaMetaRing - 1)][32 + min(lane, 4)], k); };
  int i = tile_info(0, 0), jt = tile_info(0, 1), T = tile_info(0, 2), P = tile_info(0, 3), valid = tile_info(0, 4);

  for (int r = 0; r < n; ++r) {
    meta_dma(r + 6);
    wait_vm<kWait>();   // tile(r) (and every meta before it) has landed
    __syncthreads();    // tile r visible to all waves; every wave is past tile r - 1
    // tile r + 3 goes into the buffer tile r - 1 used, in three parts; its
    // slot ids are read here and used a few score steps later
    const int32_t vs_next = tile_slots(r + 3);
    const TailSlots ts_next = tail_slots(r + 3);
    const int32_t info_next = meta_lds[w][(r + 1) & (kMlaMetaRing - 1)][32 + min(lane, 4)];
    const bool seg_begin = (r == 0) || (jt == 0);
    const bool seg_end = (r == n - 1) || (jt == T - 1);
    const char* tile = tiles[r % kMlaBufs];

    if (seg_begin) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = hw + hb * 16 + col;
        const bf16* qp = q + ((int64_t)i * row_stride + row_off + h) * kMlaQK + grp * 8;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) qf[hb][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 32));
        l_part[hb] = 0.f;
      }
      if constexpr (VERIFY) k_zone = kv_lens[i] - n_draft + 1;
      // Wait for the queries here, once per piece.  Left pending across the
      // branch, they would make the compiler wait on the memory counter in
      // the score loop of every tile, where the tile DMAs (invisible to it)
      // also count: that drains the whole tile ring each tile.
      __builtin_amdgcn_s_waitcnt(0);
    }

    // ---- S^T = K Q^T and the softmax (log2 domain), in two halves of 16
    // tokens (a = 0, 1), so that one half's scores take 8 VGPRs.  Chunk
    // 4kk + grp (kk < 16) of token t sits at 8 (kk / 2) + ((4 (kk & 1) + grp)
    // ^ (t & 7)) of its main row: two per-lane bases (even / odd kk) plus
    // compile-time offsets.  kk = 16, 17 read the tail part, whose row of
    // token 16a + col is ((16a + col) % W) RPW + (16a + col) / W.
    const char* kb_even = tile + col * kMlaMainBytes + (grp ^ (col & 7)) * 16;
    const char* kb_odd = tile + col * kMlaMainBytes + ((4 + grp) ^ (col & 7)) * 16;
    auto kload = [&](int a, int kk) -> bf16x8 {
      if (kk < 16) {
        const char* kb = (kk & 1) ? kb_odd : kb_even;
        return as_bf16x8(*reinterpret_cast<const u32x4*>(kb + a * 16 * kMlaMainBytes + (kk >> 1) * 128));
      }
      const int ta = 16 * a + col;
      const char* tb = tile + kMlaTailOff + ((ta % W) * RPW + ta / W) * 128 + ((4 * (kk & 1) + grp) ^ (ta & 7)) * 16;
      return as_bf16x8(*reinterpret_cast<const u32x4*>(tb));
    };
    // This lane holds tokens 16a + 4 grp + rr of head hw + 16 hb + col,
    // which is also the token order of P as the A operand of P*V.  The
    // reference maximum is taken over the first half of a piece's first tile
    // and stays fixed for the piece, so the accumulators are never rescaled
    // (any reference gives the same normalised result); a later score more
    // than kMlaHeadroom above it (P could overflow) sends the request to the
    // exact fallback in the merge pass.  Keys past the request's end (its
    // last tile only) get -inf in place; VERIFY: so do keys past each draft's
    // position, in the tiles that reach past the first draft's.  The scale
    // is positive (checked at the boundary): maxima and the overflow test
    // work on raw scores, each probability is one fma + exp2.
    // One stream of 2 x 18 k-steps, the first half's then the second's, the
    // K fragments KD - 1 steps ahead of their MFMAs across the half
    // boundary, so the first half's softmax runs with the second half's
    // first reads in flight.
    constexpr int KD = 5;  // K fragments: four k-steps (eight MFMAs) ahead
    bf16x8 kf[KD];
    f32x4 sh[2][HB];
    bool over = false;
    bf16x8 pa[HB];
    float ps[HB];
#pragma unroll
    for (int g = 0; g < KD - 1; ++g) kf[g] = kload(g / NK, g % NK);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int g = a * NK + kk;
        if (a == 0 && kk == 4) tile_dma(r + 3, vs_next, ts_next, std::integral_constant<int, 0>{});
        // the read of a later step goes out between this step's first and
        // second MFMA (the wave stalls at an MFMA until the previous one has
        // issued, so a read placed after both would leave later)
        mfma_score(sh[a][0], kf[g % KD], qf[0][kk], kk == 0, HB == 1 && kk == NK - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (g + KD - 1 < 2 * NK) kf[(g + KD - 1) % KD] = kload((g + KD - 1) / NK, (g + KD - 1) % NK);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 1; hb < HB; ++hb)
          mfma_score(sh[a][hb], kf[g % KD], qf[hb][kk], kk == 0, hb == HB - 1 && kk == NK - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (a == 0) tile_dma(r + 3, vs_next, ts_next, std::integral_constant<int, 1>{});
      if constexpr (VERIFY) {
        if (valid < kMlaT || jt * kMlaT + kMlaT > k_zone) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            int c = col;
            asm volatile("" : "+v"(c));  // recomputed here, not held across the loop (registers)
            const int jrow = (row_off + hw + hb * 16 + c) / hq_base;  // this row's draft
            const int lim = min(valid, k_zone + jrow - jt * kMlaT);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (16 * a + 4 * grp + rr >= lim) sh[a][hb][rr] = -INFINITY;
          }
        }
      } else if (valid < kMlaT) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (16 * a + 4 * grp + rr >= valid) sh[a][hb][rr] = -INFINITY;
      }
      // (written out here rather than as a lambda over sh[a]: passing the
      // array by reference kept it out of registers)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float mx = fmaxf(fmaxf(sh[a][hb][0], sh[a][hb][1]), fmaxf(sh[a][hb][2], sh[a][hb][3]));
        if (a == 0 && seg_begin) {
          m_ref[hb] = max_xor16_32(mx) * scale_log2;
          // VERIFY: a draft that sees none of the piece's first tile sees
          // none of the piece (keys only grow), and one that sees none of
          // its first half sees none of the tile: any finite reference
          // gives P = 0
          if constexpr (VERIFY) m_ref[hb] = m_ref[hb] == -INFINITY ? 0.f : m_ref[hb];
          s_over[hb] = (m_ref[hb] + kMlaHeadroom) / scale_log2;
        }
        over |= mx > s_over[hb];
        float sum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = fast_exp2(fmaf(sh[a][hb][rr], scale_log2, -m_ref[hb]));
          sum += p;
          pa[hb][a * 4 + rr] = (bf16)p;
        }
        ps[hb] = a == 0 ? sum : ps[hb] + sum;
      }
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) l_part[hb] += ps[hb];
    if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) fallback[i] = 1;
    tile_dma(r + 3, vs_next, ts_next, std::integral_constant<int, 2>{});

    // ---- O += P V over all columns of this wave's heads (the first tile of
    // a piece starts the accumulators from zero inside the MFMA)
    if (seg_begin)
      mla_pv<HB, true>(acc, tile, pa, lane);
    else
      mla_pv<HB, false>(acc, tile, pa, lane);

    if (seg_end) {
      const int b0 = P / Bt, b1 = (P + T - 1) / Bt;
      const bool direct = b0 == b1;
      // outputs: row row_off + h of request i; pieces: this launch's HQ rows
      const int64_t row0 = (direct ? (int64_t)i * row_stride + row_off : ((int64_t)run + i) * HQ) + hw;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float lt = l_part[hb] + shfl_xor(l_part[hb], 16);
        lt += shfl_xor(lt, 32);  // row sum of head hw + 16 hb + col, in every lane of that column
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          // output rows of the accumulators are heads 16 hb + 4 grp + rr
          const int hr = 4 * grp + rr;
          const float lr = shfl(lt, hr);
          const float mr = shfl(m_ref[hb], hr);
          // (VERIFY: a piece none of whose keys a draft sees gives o = 0
          // and lse = -inf, which the merge weighs by zero)
          const bool any = !VERIFY || lr > 0.f;
          const float inv = any ? 1.0f / lr : 0.f;
          const int64_t row = row0 + hb * 16 + hr;
          if (direct) {
            bf16* ob = out + row * kMlaV + col;
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) ob[cb * 16] = (bf16)(acc_get(acc[hb][cb][rr]) * inv);
            if (lse && col == 0) lse[row] = any ? (mr + __log2f(lr)) * kLn2 : -INFINITY;
          } else {
            float* wb = ws_o + row * kMlaV + col;
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) wb[cb * 16] = acc_get(acc[hb][cb][rr]) * inv;
            if (col == 0) ws_lse[row] = any ? (mr + __log2f(lr)) * kLn2 : -INFINITY;
          }
        }
      }
      // no zeroing here: the next piece's first tile starts the
      // accumulators from zero inside the MFMA
    }
    i = __builtin_amdgcn_readlane(info_next, 0);
    jt = __builtin_amdgcn_readlane(info_next, 1);
    T = __builtin_amdgcn_readlane(info_next, 2);
    P = __builtin_amdgcn_readlane(info_next, 3);
    valid = __builtin_amdgcn_readlane(info_next, 4);
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
                                                        bf16* __restrict__ out, float* __restrict__ lse,
                                                        int32_t n_draft, int32_t hq_base, int32_t row_stride,
                                                        int32_t row_off) {
  const int lane = threadIdx.x & 63;
  const int64_t pid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (request, row of this launch)
  if (pid >= (int64_t)bs * Hq) return;
  const int i = (int)(pid / Hq), h = (int)(pid % Hq);
  const int64_t idx = (int64_t)i * row_stride + row_off + h;  // output row
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
    // keys this row sees (all of them for decode, where n_draft = 1 and
    // h < hq_base)
    const int L = min(min(kv_lens[i], T * kMlaT), kv_lens[i] - n_draft + 1 + (row_off + h) / hq_base);
    if (L <= 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) op[e] = (bf16)0.0f;
      if (lse && lane == 0) lse[idx] = -INFINITY;
      return;
    }
    mla_exact_one(kpool, q + idx * kMlaQK, meta, P, L, scale_log2, lane, op, lse ? lse + idx : nullptr);
    return;
  }
  const int Bt = header[0];
  const int b0 = P / Bt, b1 = (P + T - 1) / Bt;
  if (b0 == b1) return;
  // the first KB pieces' lse and rows are loaded at once (they are
  // independent); a request cut into more pieces takes the rest in a loop
  constexpr int KB = 4;
  float lb[KB];
  f32x4 xb[KB][2];
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    lb[k] = -INFINITY;
    xb[k][0] = xb[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (b0 + k <= b1) {
      const int64_t row = ((int64_t)(b0 + k) + i) * Hq + h;
      lb[k] = ws_lse[row];
      const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + row * kMlaV + lane * 8);
      xb[k][0] = src[0];
      xb[k][1] = src[1];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KB; ++k) mx = fmaxf(mx, lb[k]);
  for (int b = b0 + KB; b <= b1; ++b) mx = fmaxf(mx, ws_lse[((int64_t)b + i) * Hq + h]);
  if (mx == -INFINITY) {  // a draft that sees no key at all (kv_lens below n_draft)
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e] = (bf16)0.0f;
    if (lse && lane == 0) lse[idx] = -INFINITY;
    return;
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  // (pieces past the request, and pieces a draft sees no key of, weigh 0;
  // their rows are finite)
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const float wgt = lb[k] == -INFINITY ? 0.f : __expf(lb[k] - mx);
    sum += wgt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] += wgt * xb[k][0][e];
      o[4 + e] += wgt * xb[k][1][e];
    }
  }
  for (int b = b0 + KB; b <= b1; ++b) {
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
         (Hq == 16 || Hq == 32 || Hq == 64 || (Hq % kMlaSlice == 0 && Hq <= kMlaMaxRows));
}

int32_t mla_slice_rows(int32_t Hq) { return Hq < kMlaSlice ? Hq : kMlaSlice; }

DecodePlan plan_mla_decode(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len) {
  (void)p;
  (void)bs;
  (void)Hq;
  DecodePlan plan;
  plan.kind = 3;
  plan.chunk = max_kv_len > 0 ? (max_kv_len + kMlaT - 1) / kMlaT : 0;  // tiles per request, at most
  plan.max_splits = device_cu_count();  // runs of tiles: one workgroup per CU, all heads in it
  return plan;
}

template <int HB, int W>
static void launch_mla_main(int32_t runs, int32_t hs, hipStream_t s, const char* kp, const void* q,
                            const StreamWs& w, float sl2, void* out, float* lse, const int32_t* kv_lens,
                            int32_t n_draft, int32_t hq_base, int32_t rows, int32_t off) {
  if (n_draft > 1)
    hipLaunchKernelGGL((mla_decode_kernel<HB, W, true>), dim3(runs), dim3(64 * W), 0, s, kp,
                       static_cast<const bf16*>(q), hs, w.header, w.meta, sl2, static_cast<bf16*>(out), lse, w.o,
                       w.lse, w.fallback, kv_lens, n_draft, hq_base, rows, off);
  else
    hipLaunchKernelGGL((mla_decode_kernel<HB, W, false>), dim3(runs), dim3(64 * W), 0, s, kp,
                       static_cast<const bf16*>(q), hs, w.header, w.meta, sl2, static_cast<bf16*>(out), lse, w.o,
                       w.lse, w.fallback, kv_lens, 1, hq_base, rows, off);
}

hipError_t launch_mla_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m, int32_t bs,
                             const DecodePlan& plan, float sl2, void* out, float* lse, void* ws, hipStream_t s,
                             const StoreArgs* st) {
  return launch_mla_verify(p, layer, q, Hq, 1, m, bs, plan, sl2, out, lse, ws, s, st);
}

// More than kMlaSlice rows (many heads, or heads times drafts) run as
// consecutive slices of kMlaSlice rows: one plan, then the main kernel and the
// merge per slice, each reading and writing its rows of the full row list and
// reusing the one workspace in stream order.  A request that one slice sends
// to the exact fallback keeps the flag for the later slices, which is exact
// too.
hipError_t launch_mla_verify(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, int32_t n_draft,
                             const DevMap& m, int32_t bs, const DecodePlan& plan, float sl2, void* out, float* lse,
                             void* ws, hipStream_t s, const StoreArgs* st) {
  const int32_t hs = mla_slice_rows(Hq);
  StreamWs w;
  stream_ws_layout(bs, plan.chunk, plan.max_splits, hs, kMlaV, ws, &w);
  const int32_t runs = plan.max_splits;
  hipError_t e = launch_stream_plan(m, bs, plan.chunk, runs, w, s, nullptr, st);
  if (e != hipSuccess) return e;
  const char* kp = p.k_layer(layer);
  const int32_t hq_base = Hq / n_draft;
  const unsigned mblocks = (unsigned)(((int64_t)bs * hs + 3) / 4);
  for (int32_t off = 0; off < Hq; off += hs) {
    timer_before(s);
    if (hs == 128) launch_mla_main<2, 4>(runs, hs, s, kp, q, w, sl2, out, lse, m.kv_lens, n_draft, hq_base, Hq, off);
    else if (hs == 64) launch_mla_main<1, 4>(runs, hs, s, kp, q, w, sl2, out, lse, m.kv_lens, n_draft, hq_base, Hq, off);
    else if (hs == 32) launch_mla_main<1, 2>(runs, hs, s, kp, q, w, sl2, out, lse, m.kv_lens, n_draft, hq_base, Hq, off);
    else launch_mla_main<1, 1>(runs, hs, s, kp, q, w, sl2, out, lse, m.kv_lens, n_draft, hq_base, Hq, off);
    e = hipGetLastError();
    timer_after(s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(mblocks), dim3(256), 0, s, bs, hs, w.header, w.prefix, w.ntiles,
                       w.fallback, w.o, w.lse, kp, static_cast<const bf16*>(q), w.meta, m.kv_lens, sl2,
                       static_cast<bf16*>(out), lse, n_draft, hq_base, Hq, off);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
