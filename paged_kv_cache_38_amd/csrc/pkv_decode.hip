// Paged decode attention for grouped-query heads: split-K partial kernels and
// the log-sum-exp merge.
//
// What is computed ([XPU] "From slots to a page table"; [BACKEND]
// init_forward_metadata with its per-request split count): one new query per
// request attends over its L keys; key t of request i lives at the slot the
// request's table resolves t to.  The keys are cut into chunks of `chunk`
// *logical* positions; each chunk (split) produces a normalised partial
// output and its log-sum-exp, and the merge combines them exactly.  Split
// boundaries depend only on logical positions, never on where pages live, so
// moving pages around cannot change a single bit of the output.
//
// Layout on gfx950 (pool: [slots][Hkv][D], token-major):
//   block   = WAVES wavefronts of one (split, request); wave w owns KV head
//             g = blockIdx.z * WAVES + w and its G = Hq / Hkv query heads.
//   bf16:   S^T[16 tokens x 16 heads] = K_tile[16 x D] * Q^T[D x 16] with
//           v_mfma_f32_16x16x32_bf16 (tokens as M so that K loads straight
//           from HBM into the A operand: lane (t = l%16, j = l/16) reads D/4
//           contiguous elements of token t's head slice); the softmax runs on
//           the MFMA output registers; P (16 heads x 32 tokens) is already in
//           the A-operand layout of the PV product; V goes through LDS so each
//           lane can pick the 8 tokens of one d column the B operand needs.
//   f32 (and bf16 without MFMA): VALU dot products, 16 lanes per token.
#include <math.h>

#include "pkv_launch.h"

namespace pkv {

constexpr int kTile = 32;  // tokens per inner iteration of the MFMA kernel

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel
// ---------------------------------------------------------------------------
template <int D, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) decode_mfma_kernel(
    DevMap m, const bf16* __restrict__ k_pool, const bf16* __restrict__ v_pool, const bf16* __restrict__ q,
    int32_t Hq, int32_t Hkv, int32_t G, int32_t chunk, int32_t max_splits, float scale_log2,
    bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int NK = D / 32;         // MFMAs along d for S
  constexpr int DJ = D / 4;          // contiguous K elements per lane group
  constexpr int NT = D / 16;         // 16-wide d tiles of the PV product
  constexpr int CPT = D / 8;         // 16-byte chunks per V head slice
  constexpr int TPI = 64 / CPT;      // tokens per V load instruction
  constexpr int VIT = kTile / TPI;   // V load instructions per tile
  constexpr int LDS = D + 8;         // LDS row stride in elements (+16 B pad)
  __shared__ bf16 vsm[WAVES][kTile * LDS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int i = blockIdx.y;
  const int g = blockIdx.z * WAVES + wave;
  const int col = lane & 15;  // head column of S / d column of PV
  const int grp = lane >> 4;  // lane group 0..3
  const int L = m.kv_lens[i];

  if (L <= 0) {  // empty key set: zero output, lse = -inf ([XPU] "Approach 2" guard)
    if (s == 0) {
      for (int n = 0; n < G; ++n) {
        const int64_t h = (int64_t)i * Hq + g * G + n;
        for (int d = lane; d < D; d += 64) out[h * D + d] = (bf16)0.0f;
        if (lse && lane == 0) lse[h] = -INFINITY;
      }
    }
    return;
  }
  // keys past max_splits * chunk (a length above the caller's max_kv_len) are ignored
  const int ns = min((L + chunk - 1) / chunk, max_splits);
  if (s >= ns) return;
  const int t_begin = s * chunk;
  const int t_end = min(t_begin + chunk, L);
  const Resolver r = make_resolver(m, i);

  // Q^T operand: lane (n = col, j = grp) holds q[head n][j*DJ + kk*8 .. +8]
  bf16x8 qb[NK];
  {
    const bool ok = col < G;
    const bf16* qp = q + ((int64_t)i * Hq + g * G + (ok ? col : 0)) * D + grp * DJ;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + kk * 8);
      if (!ok) w = u32x4{0u, 0u, 0u, 0u};
      qb[kk] = as_bf16x8(w);
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t row_elems = (int64_t)Hkv * D;
  const bf16* kb = k_pool + (int64_t)g * D;
  const bf16* vb = v_pool + (int64_t)g * D;
  bf16* vt = vsm[wave];

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    // ---- global loads: K straight into A-operand registers, V into registers
    bf16x8 ka[2][NK];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int t = t0 + a * 16 + col;
      const int64_t slot = (t < t_end) ? r.slot(t) : r.pad_slot;
      const bf16* kp = kb + slot * row_elems + grp * DJ;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) ka[a][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + kk * 8));
    }
    u32x4 vr[VIT];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int t = t0 + it * TPI + lane / CPT;
      if (t < t_end) {
        const int64_t slot = r.slot(t);
        vr[it] = *reinterpret_cast<const u32x4*>(vb + slot * row_elems + (lane % CPT) * 8);
      } else {
        vr[it] = u32x4{0u, 0u, 0u, 0u};  // masked keys must hold 0 (P * NaN would poison the sum)
      }
    }
    // ---- S^T = K Q^T
    f32x4 sacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) sacc[a] = mfma16x16x32(ka[a][kk], qb[kk], sacc[a]);
    }
    // ---- V tile to LDS (row-major [token][d])
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int row = it * TPI + lane / CPT;
      *reinterpret_cast<u32x4*>(vt + row * LDS + (lane % CPT) * 8) = vr[it];
    }
    // ---- online softmax; lane holds tokens a*16 + 4*grp + rr of head col
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
    // ---- O += P V: B operand = 8 tokens (a*16 + 4*grp + rr) of d column nt*16 + col
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bf16x8 vbop;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) vbop[a * 4 + rr] = vt[(a * 16 + grp * 4 + rr) * LDS + nt * 16 + col];
      acc[nt] = mfma16x16x32(pa, vbop, acc[nt]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- finalise: per-head sums over the four lane groups
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int hr = grp * 4 + rr;
    const float lt = shfl(l_tot, hr);
    const float mr = shfl(m_run, hr);
    if (hr < G) {
      const int64_t h = (int64_t)i * Hq + g * G + hr;
      const float inv = 1.0f / lt;
      const float lse_nat = (mr + __log2f(lt)) * kLn2;
      if (ns == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) out[h * D + nt * 16 + col] = (bf16)(acc[nt][rr] * inv);
        if (lse && col == 0) lse[h] = lse_nat;
      } else {
        float* po = ws_o + (h * max_splits + s) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) po[nt * 16 + col] = acc[nt][rr] * inv;
        if (col == 0) ws_lse[h * max_splits + s] = lse_nat;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// VALU split kernel (f32 pools; also serves bf16 when asked for explicitly).
// 16 lanes per token, 4 tokens in flight per wave; each lane group keeps its
// own online-softmax state, merged across groups at the end.
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

template <typename T, int D, int GM, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) decode_valu_kernel(
    DevMap m, const T* __restrict__ k_pool, const T* __restrict__ v_pool, const T* __restrict__ q, int32_t Hq,
    int32_t Hkv, int32_t G, int32_t chunk, int32_t max_splits, float scale_log2, T* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int E = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int i = blockIdx.y;
  const int g = blockIdx.z * WAVES + wave;
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int L = m.kv_lens[i];
  if (L <= 0) {
    if (s == 0) {
      for (int n = 0; n < G; ++n) {
        const int64_t h = (int64_t)i * Hq + g * G + n;
        for (int d = lane; d < D; d += 64) out[h * D + d] = from_f32<T>(0.0f);
        if (lse && lane == 0) lse[h] = -INFINITY;
      }
    }
    return;
  }
  // keys past max_splits * chunk (a length above the caller's max_kv_len) are ignored
  const int ns = min((L + chunk - 1) / chunk, max_splits);
  if (s >= ns) return;
  const int t_begin = s * chunk;
  const int t_end = min(t_begin + chunk, L);
  const Resolver r = make_resolver(m, i);

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
    const int64_t slot = r.slot(t);
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
constexpr int kMaxSplits = 1024;

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
  for (int d = lane; d < Dv; d += 64) {
    float a = 0.f;
    for (int s = 0; s < ns; ++s) a = fmaf(wsh[wave][s], po[(int64_t)s * Dv + d], a);
    out[idx * Dv + d] = from_f32<T>(a * inv);
  }
  if (lse && lane == 0) lse[idx] = mx + __logf(tot);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
enum DecodeKind : int32_t { DK_NONE = 0, DK_MFMA = 1, DK_VALU = 2, DK_MLA = 3 };

bool mla_decode_supported(const PoolInfo& p, int32_t num_q_heads);
hipError_t launch_mla_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t num_q_heads, const DevMap& m,
                             int32_t bs, const DecodePlan& plan, float sm_scale, void* out, float* lse, void* ws,
                             hipStream_t s);
DecodePlan plan_mla_decode(const PoolInfo& p, int32_t bs, int32_t num_q_heads, int32_t max_kv_len);

static int decode_kind(const PoolInfo& p, int32_t Hq) {
  if (p.kind == 1) return mla_decode_supported(p, Hq) ? DK_MLA : DK_NONE;
  if (p.head_dim_qk != p.head_dim_v || (p.head_dim_qk != 64 && p.head_dim_qk != 128)) return DK_NONE;
  if (Hq <= 0 || Hq % p.num_kv_heads != 0) return DK_NONE;
  const int G = Hq / p.num_kv_heads;
  if (p.dtype == 1 && G <= 16) return DK_MFMA;
  if (p.dtype == 0 && G <= 8) return DK_VALU;
  return DK_NONE;
}

bool decode_supported(const PoolInfo& p, int32_t num_q_heads) { return decode_kind(p, num_q_heads) != DK_NONE; }

DecodePlan plan_decode(const PoolInfo& p, int32_t bs, int32_t Hq, int32_t max_kv_len) {
  DecodePlan plan;
  plan.kind = decode_kind(p, Hq);
  if (plan.kind == DK_MLA) return plan_mla_decode(p, bs, Hq, max_kv_len);
  // Chunk of logical tokens per split: the largest power of two in
  // [64, 2048] that still leaves ~16 wavefronts per CU on average (the mean
  // length is taken as max_kv_len / 2), so long requests spread over the
  // 256 CUs while the merge traffic stays a small fraction of the KV bytes.
  const double waves_per_token = (double)bs * p.num_kv_heads * 0.5 * (double)max_kv_len;
  int chunk = 64;
  for (int c = 2048; c >= 64; c >>= 1) {
    if (waves_per_token / c >= 4096.0) { chunk = c; break; }
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

size_t decode_workspace_bytes(const PoolInfo& p, const DecodePlan& plan, int32_t bs, int32_t Hq) {
  if (plan.max_splits <= 1) return 0;
  const size_t rows = (size_t)bs * Hq * plan.max_splits;
  const size_t o_bytes = (rows * p.head_dim_v * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * sizeof(float);
}

template <int D, int W>
static void launch_mfma(dim3 grid, hipStream_t s, const DevMap& m, const PoolInfo& p, int32_t layer, const void* q,
                        int32_t Hq, int32_t G, const DecodePlan& plan, float sl2, void* out, float* lse, float* wo,
                        float* wl) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, W>), grid, dim3(64 * W), 0, s, m,
                     reinterpret_cast<const bf16*>(p.k_layer(layer)), reinterpret_cast<const bf16*>(p.v_layer(layer)),
                     static_cast<const bf16*>(q), Hq, p.num_kv_heads, G, plan.chunk, plan.max_splits, sl2,
                     static_cast<bf16*>(out), lse, wo, wl);
}

template <typename T, int D, int W>
static void launch_valu(dim3 grid, hipStream_t s, const DevMap& m, const PoolInfo& p, int32_t layer, const void* q,
                        int32_t Hq, int32_t G, const DecodePlan& plan, float sl2, void* out, float* lse, float* wo,
                        float* wl) {
  hipLaunchKernelGGL((decode_valu_kernel<T, D, 8, W>), grid, dim3(64 * W), 0, s, m,
                     reinterpret_cast<const T*>(p.k_layer(layer)), reinterpret_cast<const T*>(p.v_layer(layer)),
                     static_cast<const T*>(q), Hq, p.num_kv_heads, G, plan.chunk, plan.max_splits, sl2,
                     static_cast<T*>(out), lse, wo, wl);
}

hipError_t launch_decode(const PoolInfo& p, int32_t layer, const void* q, int32_t Hq, const DevMap& m, int32_t bs,
                         const DecodePlan& plan, float sm_scale, void* out, float* lse, void* ws, hipStream_t s) {
  if (bs == 0) return hipSuccess;
  if (plan.kind == DK_MLA) return launch_mla_decode(p, layer, q, Hq, m, bs, plan, sm_scale, out, lse, ws, s);
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int W = (Hkv % 4 == 0) ? 4 : (Hkv % 2 == 0 ? 2 : 1);
  const dim3 grid((unsigned)plan.max_splits, (unsigned)bs, (unsigned)(Hkv / W));
  const float sl2 = sm_scale * kLog2e;
  float* wo = nullptr;
  float* wl = nullptr;
  if (plan.max_splits > 1) {
    const size_t rows = (size_t)bs * Hq * plan.max_splits;
    wo = static_cast<float*>(ws);
    wl = reinterpret_cast<float*>(static_cast<char*>(ws) + (rows * p.head_dim_v * sizeof(float) + 255) / 256 * 256);
  }
  const int D = p.head_dim_qk;
  timer_before(s);
  if (plan.kind == DK_MFMA) {
    if (D == 128) {
      if (W == 4) launch_mfma<128, 4>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else if (W == 2) launch_mfma<128, 2>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else launch_mfma<128, 1>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
    } else {
      if (W == 4) launch_mfma<64, 4>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else if (W == 2) launch_mfma<64, 2>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else launch_mfma<64, 1>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
    }
  } else {
    if (D == 128) {
      if (W == 4) launch_valu<float, 128, 4>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else if (W == 2) launch_valu<float, 128, 2>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else launch_valu<float, 128, 1>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
    } else {
      if (W == 4) launch_valu<float, 64, 4>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else if (W == 2) launch_valu<float, 64, 2>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
      else launch_valu<float, 64, 1>(grid, s, m, p, layer, q, Hq, G, plan, sl2, out, lse, wo, wl);
    }
  }
  hipError_t e = hipGetLastError();
  timer_after(s);
  if (e != hipSuccess || plan.max_splits <= 1) return e;
  const unsigned mblocks = (unsigned)(((int64_t)bs * Hq + 3) / 4);
  if (p.dtype == 1)
    hipLaunchKernelGGL(decode_merge_kernel<bf16>, dim3(mblocks), dim3(256), 0, s, m.kv_lens, bs, Hq, p.head_dim_v,
                       plan.chunk, plan.max_splits, wo, wl, static_cast<bf16*>(out), lse);
  else
    hipLaunchKernelGGL(decode_merge_kernel<float>, dim3(mblocks), dim3(256), 0, s, m.kv_lens, bs, Hq, p.head_dim_v,
                       plan.chunk, plan.max_splits, wo, wl, static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace pkv
