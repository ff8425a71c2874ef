// Host-side launch interface of the slot allocator and row writing
// (pkv_alloc.hip), called by the C ABI (pkv_api.hip).  Internal to the
// library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int32_t kMaxAllocBatch = 8000;  // requests per alloc_extend call (LDS offsets)

hipError_t launch_free_list_init(int32_t* ring, int32_t first, int32_t count, int32_t* state, hipStream_t s);
hipError_t launch_alloc_pages(int32_t shift, int64_t n_pages, int32_t* ring, int32_t cap, int32_t* state,
                              int32_t* out, int32_t* status, hipStream_t s);
hipError_t launch_alloc_extend(int32_t shift, int32_t bs, const int32_t* prefix, const int32_t* seq,
                               const int32_t* last_loc, int32_t* ring, int32_t cap, int32_t* state, int32_t* out,
                               int64_t out_cap, int32_t* status, hipStream_t s);
hipError_t launch_free(int32_t shift, const int32_t* slots, int64_t n, int32_t num_pages, int32_t* ring,
                       int32_t cap, int32_t* state, uint32_t* bits, int32_t* status, hipStream_t s);
hipError_t launch_write_rows(int32_t* table, int64_t rows, int64_t width, const int32_t* rpi, const int32_t* prefix,
                             const int32_t* seq, const int32_t* out_loc, int64_t n_out,
                             const int32_t* const* prefix_ptrs, int32_t bs, int32_t max_seq_len, hipStream_t s);

}  // namespace pkv
