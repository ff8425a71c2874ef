// MLA (latent) paged decode: the split-K partial kernel.
//
// What is computed: the decode of [XPU] "From slots to a page table" and
// [BACKEND] init_forward_metadata over a latent pool -- one cached row per
// token of head_dim_qk = 576 values (512 latent + 64 rope, [BACKEND] "页表构建":
// kv_lora_rank / qk_rope_head_dim), shared by every query head.  Keys are the
// whole row; values are its first 512 entries.  Splitting, planning and the
// log-sum-exp merge are those of the grouped-query decode (pkv_decode.hip).
//
// Layout on gfx950: one block per (item, group of up to 64 query heads);
// each wavefront owns 16 heads.  A 32-token tile of latent rows (36 KiB) is
// gathered into LDS once per block (double buffered) and shared by all
// wavefronts:
//   S^T[16 tokens x 16 heads] = K_tile[16 x 576] * Q^T[576 x 16]   (18 MFMAs per 16 tokens)
//   O[16 heads x 512]        += P[16 x 32] * V_tile[32 x 512]     (32 MFMAs, B from ds_read_b64_tr_b16)
// The latent rows are read from HBM exactly once per block; every head
// reuses them from LDS (the 128-head reuse is what makes this a dense
// contraction rather than a streaming dot product).
#include <math.h>

#include "pkv_launch.h"

namespace pkv {

constexpr int kMlaQK = 576;
constexpr int kMlaV = 512;
constexpr int kMlaTile = 32;
constexpr int kMlaLds = kMlaQK + 8;                 // LDS row stride (elements)
constexpr int kMlaChunks = kMlaTile * kMlaQK / 8;   // 16-byte chunks per tile
constexpr int kMlaCpt = kMlaQK / 8;                 // chunks per token row

template <int W>
struct MlaRegs {
  static constexpr int IT = (kMlaChunks + 64 * W - 1) / (64 * W);
  u32x4 v[IT];
};

template <int W, int FMT>
__device__ __forceinline__ void mla_load(MlaRegs<W>& R, const SlotMap<FMT>& sm, int t0, int t_end, const bf16* kp) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < MlaRegs<W>::IT; ++it) {
    const int c = min(it * 64 * W + tid, kMlaChunks - 1);
    const int tok = c / kMlaCpt, cc = c % kMlaCpt;
    const int t = t0 + tok;
    const int64_t slot = sm(t, t < t_end);
    R.v[it] = *reinterpret_cast<const u32x4*>(kp + slot * kMlaQK + cc * 8);
  }
}

template <int W>
__device__ __forceinline__ void mla_store(const MlaRegs<W>& R, int t0, int t_end, bf16* ks) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < MlaRegs<W>::IT; ++it) {
    const int c = it * 64 * W + tid;
    if (c < kMlaChunks) {
      const int tok = c / kMlaCpt, cc = c % kMlaCpt;
      u32x4 w = R.v[it];
      if (t0 + tok >= t_end) w = u32x4{0u, 0u, 0u, 0u};  // masked keys hold 0
      *reinterpret_cast<u32x4*>(ks + tok * kMlaLds + cc * 8) = w;
    }
  }
}

template <int W, int FMT>
__global__ void __launch_bounds__(64 * W, 1) mla_decode_kernel(
    DevMap m, const bf16* k_pool, const bf16* __restrict__ q, int32_t Hq, int32_t hg, int32_t chunk,
    int32_t max_splits, const WorkItem* __restrict__ items, const int32_t* __restrict__ item_count, float scale_log2,
    bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int NK = kMlaQK / 32;  // 18
  constexpr int NT = kMlaV / 16;   // 32
  __shared__ __attribute__((aligned(16))) bf16 ksm[2][kMlaTile * kMlaLds];

  const int w_item = blockIdx.x / hg;
  if (w_item >= *item_count) return;
  const WorkItem item = items[w_item];
  const int i = item.i, s = item.s, ns = item.ns;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int h0 = ((blockIdx.x % hg) * W + wave) * 16;  // this wave's 16 heads

  if (ns == 0) {  // empty key set: zero output, lse = -inf
    for (int n = 0; n < 16; ++n) {
      const int64_t h = (int64_t)i * Hq + h0 + n;
      for (int d = lane; d < kMlaV; d += 64) out[h * kMlaV + d] = (bf16)0.0f;
      if (lse && lane == 0) lse[h] = -INFINITY;
    }
    return;
  }
  const int t_begin = s * chunk;
  const int t_end = item.t_end;
  const SlotMap<FMT> sm = slotmap_from_view<FMT>(m, item_view(item));

  // Q^T operand: lane (head col, group grp) holds q[h0 + col][kk*32 + grp*8 .. +8]
  bf16x8 qb[NK];
  {
    const bf16* qp = q + ((int64_t)i * Hq + h0 + col) * kMlaQK + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qb[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 32));
  }
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (t_end - t_begin + kMlaTile - 1) / kMlaTile;
  MlaRegs<W> R;
  mla_load<W, FMT>(R, sm, t_begin, t_end, k_pool);
  mla_store<W>(R, t_begin, t_end, ksm[0]);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int t0 = t_begin + kt * kMlaTile;
    // next tile in flight during this tile's math (unconditional: past the
    // end it reads the padding row, which stays in cache)
    mla_load<W, FMT>(R, sm, t0 + kMlaTile, t_end, k_pool);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const bf16* ks = ksm[kt & 1];
    // ---- S^T = K Q^T
    f32x4 sacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 ka =
            as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (a * 16 + col) * kMlaLds + kk * 32 + grp * 8));
        sacc[a] = mfma16x16x32(ka, qb[kk], sacc[a]);
      }
    }
    // ---- online softmax (log2 domain); lane holds tokens a*16 + 4*grp + rr of head col
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
    const float alpha = fast_exp2(m_run - m_new);
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
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float ar = shfl(alpha, grp * 4 + rr);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][rr] *= ar;
    }
    // ---- O += P V, V = the first 512 columns of the latent rows
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16x16x32(pa, lds_v_operand(ks, kMlaLds, 0, nt * 16, lane), acc[nt]);
    if (kt + 1 < ntiles) mla_store<W>(R, t0 + kMlaTile, t_end, ksm[(kt + 1) & 1]);
    __syncthreads();
  }

  // ---- finalise: heads h0 + 4*grp + rr
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int hr = grp * 4 + rr;
    const float lt = shfl(l_tot, hr);
    const float mr = shfl(m_run, hr);
    const int64_t h = (int64_t)i * Hq + h0 + hr;
    const float inv = 1.0f / lt;
    const float lse_nat = (mr + __log2f(lt)) * kLn2;
    if (ns == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) out[h * kMlaV + nt * 16 + col] = (bf16)(acc[nt][rr] * inv);
      if (lse && col == 0) lse[h] = lse_nat;
    } else {
      float* po = ws_o + (h * max_splits + s) * kMlaV;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) po[nt * 16 + col] = acc[nt][rr] * inv;
      if (col == 0) ws_lse[h * max_splits + s] = lse_nat;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool mla_decode_supported(const PoolInfo& p, int32_t Hq) {
  return p.kind == 1 && p.dtype == 1 && p.num_kv_heads == 1 && p.head_dim_qk == kMlaQK && p.head_dim_v == kMlaV &&
         Hq > 0 && Hq % 16 == 0;
}

// Wavefronts per block: 4 (64 heads).  A wave holds its 16 heads' queries
// (72 VGPRs) and 16 x 512 fp32 accumulators (128), which only fits at one
// wave per SIMD, so a block of 4 fills a CU; larger head counts take
// several blocks per item.
static int mla_waves(int32_t Hq) {
  const int groups = Hq / 16;
  return groups % 4 == 0 ? 4 : (groups % 2 == 0 ? 2 : 1);
}

DecodePlan plan_mla_decode(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len) {
  (void)p;
  DecodePlan plan;
  plan.kind = 3;
  // Each split re-reads nothing but writes a 2 KiB partial row per head, so
  // splits are long: the largest power of two in [256, 4096] that still
  // gives ~2 blocks per CU on average (mean length taken as max_kv_len / 2).
  const int hg = (Hq / 16) / mla_waves(Hq);
  const double tokens = (double)bs * hg * 0.5 * (double)max_kv_len;
  int chunk = 256;
  for (int c = 4096; c >= 256; c >>= 1) {
    if (tokens / c >= 512.0) {
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

template <int W, int FMT>
static void launch_mla(unsigned blocks, hipStream_t s, const DevMap& m, const bf16* kp, const void* q, int32_t Hq,
                       int32_t hg, const DecodePlan& plan, const DecodeWs& w, float sl2, void* out, float* lse) {
  hipLaunchKernelGGL((mla_decode_kernel<W, FMT>), dim3(blocks), dim3(64 * W), 0, s, m, kp,
                     static_cast<const bf16*>(q), Hq, hg, plan.chunk, plan.max_splits, w.items, w.count, sl2,
                     static_cast<bf16*>(out), lse, w.o, w.lse);
}

template <int W>
static void launch_mla_fmt(unsigned blocks, hipStream_t s, const DevMap& m, const bf16* kp, const void* q,
                           int32_t Hq, int32_t hg, const DecodePlan& plan, const DecodeWs& w, float sl2, void* out,
                           float* lse) {
  if (m.fmt == MAP_TOKEN_TABLE)
    launch_mla<W, SLOT_TABLE>(blocks, s, m, kp, q, Hq, hg, plan, w, sl2, out, lse);
  else
    launch_mla<W, SLOT_PAGES>(blocks, s, m, kp, q, Hq, hg, plan, w, sl2, out, lse);
}

void launch_mla_split(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m, int32_t bs,
                      const DecodePlan& plan, const DecodeWs& w, float sl2, void* out, float* lse, hipStream_t s) {
  const int W = mla_waves(Hq);
  const int hg = (Hq / 16) / W;
  const unsigned blocks = (unsigned)((int64_t)bs * plan.max_splits * hg);
  const bf16* kp = reinterpret_cast<const bf16*>(p.k_layer(layer));
  if (W == 4) launch_mla_fmt<4>(blocks, s, m, kp, q, Hq, hg, plan, w, sl2, out, lse);
  else if (W == 2) launch_mla_fmt<2>(blocks, s, m, kp, q, Hq, hg, plan, w, sl2, out, lse);
  else launch_mla_fmt<1>(blocks, s, m, kp, q, Hq, hg, plan, w, sl2, out, lse);
}

}  // namespace pkv
