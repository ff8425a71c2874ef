// Device-side building blocks shared by the paged KV-cache kernels (gfx950).
//
// Sources, cited by short name:
//   [XPU]     "Enabling Encoder-Decoder Models on Intel XPU in SGLang: A KV-Cache Story"
//   [OMNI]    "Scheduler-Managed Paged KV Cache" (vLLM-Omni design documents)
//   [MINI]    "The KV pool, the page table and the token pool" (mini-sglang from Scratch)
//   [BACKEND] "AttentionBackend" (SGLang FlashInfer-MLA / FlashMLA backend notes)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum MapFmt : int32_t { MAP_TOKEN_TABLE = 0, MAP_CSR = 1, MAP_BLOCK_TABLE = 2, MAP_CONTIGUOUS = 3 };

// How a request's logical token t reaches its slot in the per-token pool view
// (the [XPU] "From slots to a page table" formula for page-granular tables,
// a direct read of the token-granular req_to_token row otherwise).
struct DevMap {
  int32_t fmt;
  int32_t page_shift;  // log2(page_size)
  const int32_t* kv_lens;
  // token table
  const int32_t* req_to_token;
  int64_t table_width;  // columns == row stride (row-major)
  int64_t table_rows;
  const int32_t* req_pool_indices;
  const int32_t* kv_start;  // may be null (all zero)
  // CSR
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int64_t kv_indices_len;
  // padded block table
  const int32_t* block_table;
  int64_t block_stride;
  // contiguous (gathered) K/V
  const int32_t* cu_seqlens_k;
  int64_t total_k;
  const void* contig_k;
  const void* contig_v;
  // pool bounds: any resolved slot outside [0, num_slots) reads pad_slot
  int64_t num_slots;
  int64_t pad_slot;
};

// Per-request resolver, built once per workgroup and kept in registers.
// Every index read from a table is range-checked: an out-of-range entry is
// read as the padding slot (memory-safe; the result for that request is
// then unspecified).
struct Resolver {
  const int32_t* base;  // token-table row (+kv_start) or page list
  int64_t limit;        // readable entries at base
  int64_t off;          // contiguous: first row of this request
  int64_t num_slots, pad_slot;
  int32_t fmt, shift, mask;

  __device__ __forceinline__ int64_t slot(int32_t t) const {
    int64_t s;
    if (fmt == MAP_CONTIGUOUS) {
      s = off + t;
    } else if (fmt == MAP_TOKEN_TABLE) {
      s = (t < limit) ? (int64_t)base[t] : pad_slot;
    } else {
      int32_t pi = t >> shift;
      int64_t page = (pi < limit) ? (int64_t)base[pi] : -1;
      s = (page < 0) ? pad_slot : ((page << shift) + (t & mask));
    }
    return ((uint64_t)s < (uint64_t)num_slots) ? s : pad_slot;
  }
};

__device__ __forceinline__ Resolver make_resolver(const DevMap& m, int32_t i) {
  Resolver r;
  r.fmt = m.fmt;
  r.shift = m.page_shift;
  r.mask = (1 << m.page_shift) - 1;
  r.num_slots = m.num_slots;
  r.pad_slot = m.pad_slot;
  r.off = 0;
  r.base = nullptr;
  r.limit = 0;
  if (m.fmt == MAP_TOKEN_TABLE) {
    int64_t row = m.req_pool_indices[i];
    int64_t start = m.kv_start ? (int64_t)m.kv_start[i] : 0;
    if (row >= 0 && row < m.table_rows && start >= 0 && start <= m.table_width) {
      r.base = m.req_to_token + row * m.table_width + start;
      r.limit = m.table_width - start;
    }
  } else if (m.fmt == MAP_CSR) {
    int64_t a = m.kv_indptr[i], b = m.kv_indptr[i + 1];
    if (a >= 0 && b >= a && b <= m.kv_indices_len) {
      r.base = m.kv_indices + a;
      r.limit = b - a;
    }
  } else if (m.fmt == MAP_BLOCK_TABLE) {
    r.base = m.block_table + (int64_t)i * m.block_stride;
    r.limit = m.block_stride;
  } else {
    r.off = m.cu_seqlens_k[i];
    r.num_slots = m.total_k;
    r.pad_slot = 0;
  }
  return r;
}

// Branch-free per-request slot lookup, specialised on the table family so the
// hot loops carry no format switch and every lookup is one unconditional
// load (out-of-range indices are clamped to a readable address and the
// result replaced by the padding slot).  Slots fit in 32 bits (the host
// rejects pools of 2^31 slots or more).
enum SlotFmt : int { SLOT_TABLE = 0, SLOT_PAGES = 1, SLOT_CONTIG = 2 };

template <int FMT>
struct SlotMap {
  const int32_t* base;  // never null: points at readable memory even when limit == 0
  int32_t limit;        // readable entries at base (tokens or pages)
  int32_t shift, mask;
  int32_t num_slots, pad;
  int32_t off;          // contiguous: first row of the request

  // slot of logical token t; `valid` false gives the padding slot
  __device__ __forceinline__ int32_t operator()(int32_t t, bool valid) const { return finish(raw(t), t, valid); }

  // Two halves of a lookup, so a loop can issue the table load early and
  // use it a tile later: raw() is the bare load (index clamped to a
  // readable entry), finish() the checks, with no memory access.
  // address raw(t) reads (any readable word for a contiguous map)
  __device__ __forceinline__ const int32_t* raw_ptr(int32_t t) const {
    if constexpr (FMT == SLOT_CONTIG) {
      return base;
    } else if constexpr (FMT == SLOT_TABLE) {
      return base + min(max(t, 0), max(limit - 1, 0));
    } else {
      return base + min(max(t >> shift, 0), max(limit - 1, 0));
    }
  }
  __device__ __forceinline__ int32_t raw(int32_t t) const {
    if constexpr (FMT == SLOT_CONTIG) {
      return 0;
    } else if constexpr (FMT == SLOT_TABLE) {
      return base[min(max(t, 0), max(limit - 1, 0))];
    } else {
      return base[min(max(t >> shift, 0), max(limit - 1, 0))];
    }
  }
  // (the tests use & rather than &&: every operand is cheap and side-effect
  // free, and a short-circuit would let the compiler move a table load
  // issued early into a branch of its own, with a wait for it there)
  __device__ __forceinline__ int32_t finish(int32_t r, int32_t t, bool valid) const {
    if constexpr (FMT == SLOT_CONTIG) {
      const int32_t s = off + t;
      return (valid && (uint32_t)s < (uint32_t)num_slots) ? s : pad;
    } else if constexpr (FMT == SLOT_TABLE) {
      const bool ok = valid & (t < limit);
      const int32_t s = ok ? r : pad;
      return ((uint32_t)s < (uint32_t)num_slots) ? s : pad;
    } else {
      const bool ok = valid & ((t >> shift) < limit) & (r >= 0);
      const int32_t s = ok ? ((r << shift) | (t & mask)) : pad;
      return ((uint32_t)s < (uint32_t)num_slots) ? s : pad;
    }
  }
};

// Where request i's table entries start (element offset into req_to_token,
// kv_indices or block_table) and how many are readable; limit 0 marks a
// malformed row/pointer, read as all padding.  Contiguous maps: the first
// gathered row.
struct ReqView {
  int64_t off;
  int32_t limit;
};

__device__ __forceinline__ ReqView request_view(const DevMap& m, int32_t i) {
  ReqView v{0, 0};
  if (m.fmt == MAP_TOKEN_TABLE) {
    const int64_t row = m.req_pool_indices[i];
    const int64_t start = m.kv_start ? (int64_t)m.kv_start[i] : 0;
    if (row >= 0 && row < m.table_rows && start >= 0 && start < m.table_width) {
      v.off = row * m.table_width + start;
      v.limit = (int32_t)(m.table_width - start);
    }
  } else if (m.fmt == MAP_CSR) {
    const int64_t a = m.kv_indptr[i], b = m.kv_indptr[i + 1];
    if (a >= 0 && b > a && b <= m.kv_indices_len) {
      v.off = a;
      v.limit = (int32_t)(b - a);
    }
  } else if (m.fmt == MAP_BLOCK_TABLE) {
    if (m.block_stride > 0) {
      v.off = (int64_t)i * m.block_stride;
      v.limit = (int32_t)m.block_stride;
    }
  } else {
    v.off = m.cu_seqlens_k[i];
    v.limit = 1;
  }
  return v;
}

template <int FMT>
__device__ __forceinline__ SlotMap<FMT> slotmap_from_view(const DevMap& m, ReqView v) {
  SlotMap<FMT> r;
  r.shift = m.page_shift;
  r.mask = (1 << m.page_shift) - 1;
  r.num_slots = (int32_t)m.num_slots;
  r.pad = (int32_t)m.pad_slot;
  r.off = 0;
  r.base = m.kv_lens;  // readable fallback
  r.limit = 0;
  if constexpr (FMT == SLOT_CONTIG) {
    r.off = (int32_t)v.off;
    r.num_slots = (int32_t)m.total_k;
    r.pad = 0;
  } else if (v.limit > 0) {
    const int32_t* tab = (FMT == SLOT_TABLE) ? m.req_to_token : (m.fmt == MAP_CSR ? m.kv_indices : m.block_table);
    r.base = tab + v.off;
    r.limit = v.limit;
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ SlotMap<FMT> make_slotmap(const DevMap& m, int32_t i) {
  return slotmap_from_view<FMT>(m, request_view(m, i));
}

// ---------------------------------------------------------------------------
// small numeric helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// xor-shuffle across the wavefront (ds_bpermute)
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }
// max over lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 lane-swap
// instructions (VALU, no LDS traffic)
__device__ __forceinline__ float max_xor16_32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
// integer lane gather (ds_bpermute): value of lane `src` (0..63)
__device__ __forceinline__ int32_t shfl_i(int32_t v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

__device__ __forceinline__ int32_t wave_lane() { return (int32_t)__lane_id(); }

// MFMA 16x16x32 bf16 -> f32 (gfx950).  Lane l supplies A[l%16][8*(l/16) .. +8]
// and B[8*(l/16) .. +8][l%16]; it receives D[4*(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the address of 4 consecutive 16-bit values (call
// them M[j][0..3]); lane i receives M[i/4 + 4r][i%4] for r = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// B operand of P*V for a 16x16x32 MFMA from a row-major [token][d] LDS tile
// (row stride `lds` elements): lane (n = l%16, j = l/16) receives
// V[r0 + 4j + r][c0 + n] for r = 0..3 (low half) and V[r0 + 16 + 4j + r][c0 + n]
// (high half); lane x of each 16-lane group points at row r0 + 4j + x/4,
// columns c0 + 4*(x%4) .. +4.
__device__ __forceinline__ bf16x8 lds_v_operand(const bf16* tile, int lds, int r0, int c0, int lane) {
  const int x = lane & 15, j = lane >> 4;
  const bf16* base = tile + (r0 + j * 4 + (x >> 2)) * lds + c0 + 4 * (x & 3);
  const i16x4 lo = lds_read_tr16(base);
  const i16x4 hi = lds_read_tr16(base + 16 * lds);
  const bf16x4 blo = __builtin_bit_cast(bf16x4, lo), bhi = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
}

// ---------------------------------------------------------------------------
// HBM -> LDS loads (global_load_lds_*) issued from inline assembly.  The
// compiler does not see them, so it never drains the whole memory queue for
// them; every user waits on them explicitly with wait_vm<N>() (N = memory
// operations issued after the one needed, counting every vector memory
// operation of the wave).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  // the LDS aperture is 4 GiB aligned: the low 32 bits of a flat LDS address
  // are the LDS byte offset
  return (uint32_t)(uintptr_t)p;
}
// one 16-byte chunk per lane, global -> LDS at m0 + 16 * lane
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// one 16-byte chunk per lane from base + off (base uniform, in SGPRs),
// global -> LDS at m0 + 16 * lane
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// one dword per lane, global -> LDS at m0 + 4 * lane
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

}  // namespace pkv
