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
// Layout on gfx950: one block per (64-query tile, query head, request); four
// wavefronts of 16 query rows each.  Key tiles of 64 tokens are gathered
// through the table into LDS (token-major, 16-byte padded rows), double
// buffered so the next tile's HBM reads overlap this tile's MFMA work:
//   S^T[16 keys x 16 rows] = K_tile[16 x D] * Q^T[D x 16]   (v_mfma_f32_16x16x32_bf16)
// leaves each lane one query row (lane % 16) and 16 keys, so the row softmax
// needs only two cross-lane steps, and P is already the A operand of
//   O[16 rows x D] += P[16 x 32 keys] * V[32 keys x D]
// whose B operand comes from LDS with ds_read_b64_tr_b16.
#include <math.h>

#include "pkv_launch.h"

namespace pkv {

constexpr int kBM = 64;  // query rows per block
constexpr int kBN = 64;  // keys per tile

template <int D>
struct ExtendCfg {
  static constexpr int LDS = D + 8;          // LDS row stride (elements)
  static constexpr int NK = D / 32;          // MFMAs along d for S
  static constexpr int NT = D / 16;          // 16-wide d tiles of O
  static constexpr int CPK = D / 8;          // 16-byte chunks per key row (one head)
  static constexpr int KPI = 256 / CPK;      // keys per block-wide load instruction
  static constexpr int LIT = kBN / KPI;      // load instructions per tile per tensor
};

template <int D>
struct ExtendRegs {
  u32x4 k[ExtendCfg<D>::LIT];
  u32x4 v[ExtendCfg<D>::LIT];
};

// global -> registers for key tile starting at k0 (keys past kv_end read the
// padding row and are zeroed when written to LDS)
template <int D, int FMT>
__device__ __forceinline__ void extend_load(ExtendRegs<D>& R, const SlotMap<FMT>& sm, int k0, int kv_end,
                                            const bf16* kb, const bf16* vb, int64_t row_elems) {
  using C = ExtendCfg<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < C::LIT; ++it) {
    const int t = k0 + it * C::KPI + tid / C::CPK;
    const int64_t slot = sm(t, t < kv_end);
    const int64_t off = slot * row_elems + (tid % C::CPK) * 8;
    R.k[it] = *reinterpret_cast<const u32x4*>(kb + off);
    R.v[it] = *reinterpret_cast<const u32x4*>(vb + off);
  }
}

template <int D>
__device__ __forceinline__ void extend_store_lds(const ExtendRegs<D>& R, int k0, int kv_end, bf16* ks, bf16* vs) {
  using C = ExtendCfg<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < C::LIT; ++it) {
    const int row = it * C::KPI + tid / C::CPK;
    const bool ok = k0 + row < kv_end;
    u32x4 kw = R.k[it], vw = R.v[it];
    if (!ok) {
      kw = u32x4{0u, 0u, 0u, 0u};
      vw = u32x4{0u, 0u, 0u, 0u};  // masked keys must hold 0 (P * NaN would poison the sum)
    }
    const int o = row * C::LDS + (tid % C::CPK) * 8;
    *reinterpret_cast<u32x4*>(ks + o) = kw;
    *reinterpret_cast<u32x4*>(vs + o) = vw;
  }
}

template <int D, int FMT>
__global__ void __launch_bounds__(256, 2) extend_kernel(DevMap m, const bf16* k_pool, const bf16* v_pool,
                                                        int64_t row_elems, const bf16* __restrict__ q,
                                                        int64_t total_q, const int32_t* __restrict__ qo_indptr,
                                                        int32_t Hq,
                                                        int32_t G, int32_t causal, float scale_log2,
                                                        bf16* __restrict__ out, float* __restrict__ lse) {
  using C = ExtendCfg<D>;
  constexpr int LDS = C::LDS, NK = C::NK, NT = C::NT;
  __shared__ __attribute__((aligned(16))) bf16 ksm[2][kBN * LDS];
  __shared__ __attribute__((aligned(16))) bf16 vsm[2][kBN * LDS];

  const int qt = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const int q0 = qo_indptr[i];
  // rows past total_q (a qo_indptr beyond the buffers) are never touched
  const int n = (q0 < 0 || q0 >= total_q) ? 0 : (int)min((int64_t)(qo_indptr[i + 1] - q0), total_q - q0);
  if (qt * kBM >= n) return;
  int L = m.kv_lens[i];
  if (FMT == SLOT_CONTIG && m.total_k <= 0) L = 0;  // nothing gathered: no row is readable
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = h / G;
  const int r0 = qt * kBM + wave * 16;  // first query row (within the request) of this wave

  // keys any row of this tile may see
  int kv_end = L;
  if (causal) kv_end = min(L, L - n + min(qt * kBM + kBM, n));
  if (kv_end < 0) kv_end = 0;

  // Q^T operand: lane (row col, group grp) holds q[row][kk*32 + grp*8 .. +8]
  bf16x8 qb[NK];
  {
    const int row = r0 + col;
    const bool ok = row < n;
    const bf16* qp = q + ((int64_t)(q0 + (ok ? row : 0)) * Hq + h) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + kk * 32);
      if (!ok) w = u32x4{0u, 0u, 0u, 0u};
      qb[kk] = as_bf16x8(w);
    }
  }
  // last key (exclusive) this lane's row may see
  const int my_row = r0 + col;
  const int row_end = causal ? min(L, L - n + my_row + 1) : L;

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (kv_end + kBN - 1) / kBN;
  if (ntiles > 0) {
    const SlotMap<FMT> sm = make_slotmap<FMT>(m, i);
    const bf16* kb = k_pool + (int64_t)g * D;
    const bf16* vb = v_pool + (int64_t)g * D;
    ExtendRegs<D> R;
    extend_load<D, FMT>(R, sm, 0, kv_end, kb, vb, row_elems);
    extend_store_lds<D>(R, 0, kv_end, ksm[0], vsm[0]);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
      const int k0 = kt * kBN;
      // next tile's rows in flight during this tile's math (unconditional:
      // past the last tile it reads the padding row, which stays in cache)
      extend_load<D, FMT>(R, sm, k0 + kBN, kv_end, kb, vb, row_elems);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const bf16* ks = ksm[kt & 1];
      const bf16* vs = vsm[kt & 1];
      // ---- S^T: 4 subtiles of 16 keys
      f32x4 sacc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (a * 16 + col) * LDS + kk * 32 + grp * 8));
          sacc[a] = mfma16x16x32(ka, qb[kk], sacc[a]);
        }
      }
      // ---- online softmax for row my_row over keys k0 + a*16 + 4*grp + rr
      float sv[4][4];
      float mt = -INFINITY;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = k0 + a * 16 + grp * 4 + rr;
          const float x = (t < row_end) ? sacc[a][rr] * scale_log2 : -INFINITY;
          sv[a][rr] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      // a row that has seen no key yet keeps m = -inf; its p and alpha are 0
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
      bf16x8 pa[2];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = fast_exp2(sv[a][rr] - m_use);
          psum += p;
          pa[a >> 1][(a & 1) * 4 + rr] = (bf16)p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float ar = shfl(alpha, grp * 4 + rr);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][rr] *= ar;
      }
      // ---- O += P V over two 32-key halves
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = mfma16x16x32(pa[b], lds_v_operand(vs, LDS, b * 32, nt * 16, lane), acc[nt]);
      // ---- next tile into the other buffer
      if (kt + 1 < ntiles) extend_store_lds<D>(R, k0 + kBN, kv_end, ksm[(kt + 1) & 1], vsm[(kt + 1) & 1]);
      __syncthreads();
    }
  }

  // ---- finalise rows 4*grp + rr of this wave
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int rl = grp * 4 + rr;
    const float lt = shfl(l_tot, rl);
    const float mr = shfl(m_run, rl);
    const int row = r0 + rl;
    if (row < n) {
      const int64_t o = ((int64_t)(q0 + row) * Hq + h);
      const bool any = lt > 0.f;
      const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) out[o * D + nt * 16 + col] = (bf16)(acc[nt][rr] * inv);
      if (lse && col == 0) lse[o] = any ? (mr + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool extend_supported(const PoolInfo& p, int32_t num_q_heads) {
  return p.kind == 0 && p.dtype == 1 && p.head_dim_qk == p.head_dim_v &&
         (p.head_dim_qk == 64 || p.head_dim_qk == 128) && num_q_heads % p.num_kv_heads == 0;
}

template <int D, int FMT>
static void launch_ext(dim3 grid, hipStream_t s, const DevMap& m, const bf16* kp, const bf16* vp, int64_t row_elems,
                       const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t G, int32_t causal, float sl2,
                       void* out, float* lse) {
  hipLaunchKernelGGL((extend_kernel<D, FMT>), grid, dim3(256), 0, s, m, kp, vp, row_elems,
                     static_cast<const bf16*>(q), tq, qo, Hq, G, causal, sl2, static_cast<bf16*>(out), lse);
}

template <int D>
static void launch_ext_fmt(dim3 grid, hipStream_t s, const DevMap& m, const bf16* kp, const bf16* vp,
                           int64_t row_elems, const void* q, int64_t tq, const int32_t* qo, int32_t Hq, int32_t G,
                           int32_t causal, float sl2, void* out, float* lse) {
  if (m.fmt == MAP_TOKEN_TABLE)
    launch_ext<D, SLOT_TABLE>(grid, s, m, kp, vp, row_elems, q, tq, qo, Hq, G, causal, sl2, out, lse);
  else if (m.fmt == MAP_CONTIGUOUS)
    launch_ext<D, SLOT_CONTIG>(grid, s, m, kp, vp, row_elems, q, tq, qo, Hq, G, causal, sl2, out, lse);
  else
    launch_ext<D, SLOT_PAGES>(grid, s, m, kp, vp, row_elems, q, tq, qo, Hq, G, causal, sl2, out, lse);
}

hipError_t launch_extend(const PoolInfo& p, int32_t layer, const void* q, int64_t total_q, const int32_t* qo_indptr,
                         int32_t Hq,
                         int32_t max_q_len, const DevMap& m, int32_t bs, int32_t max_kv_len, int32_t causal,
                         float sm_scale, void* out, float* lse, hipStream_t s) {
  (void)max_kv_len;
  if (bs == 0 || max_q_len == 0) return hipSuccess;
  // contiguous (ragged) maps read the caller's gathered K/V, paged maps the pool
  const bf16* kp = reinterpret_cast<const bf16*>(m.fmt == MAP_CONTIGUOUS ? m.contig_k : p.k_layer(layer));
  const bf16* vp = reinterpret_cast<const bf16*>(m.fmt == MAP_CONTIGUOUS ? m.contig_v : p.v_layer(layer));
  const int G = Hq / p.num_kv_heads;
  const dim3 grid((unsigned)((max_q_len + kBM - 1) / kBM), (unsigned)Hq, (unsigned)bs);
  const int64_t row_elems = (int64_t)p.num_kv_heads * p.head_dim_qk;
  const float sl2 = sm_scale * kLog2e;
  timer_before(s);
  if (p.head_dim_qk == 128)
    launch_ext_fmt<128>(grid, s, m, kp, vp, row_elems, q, total_q, qo_indptr, Hq, G, causal, sl2, out, lse);
  else
    launch_ext_fmt<64>(grid, s, m, kp, vp, row_elems, q, total_q, qo_indptr, Hq, G, causal, sl2, out, lse);
  hipError_t e = hipGetLastError();
  timer_after(s);
  return e;
}

}  // namespace pkv
