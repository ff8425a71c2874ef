// Host-side launch interface of the encoder-embedding block cache
// (pkv_enc.hip), called by the C ABI (pkv_api.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_enc_write(char* buffer, int32_t num_blocks, int32_t block_size, int64_t row_units, const char* src,
                            int32_t n, const int32_t* block_ids, hipStream_t s);
hipError_t launch_enc_merge(const char* buffer, int32_t num_blocks, int32_t block_size, int64_t row_units,
                            const int32_t* block_ids, int32_t max_blocks, const int64_t* positions, char* hidden,
                            int64_t num_tokens, int32_t* fill_count, hipStream_t s);
hipError_t launch_enc_check(const int32_t* fill_count, const int32_t* scheduled, int64_t num_tokens,
                            long long* counts_dev, hipStream_t s);

}  // namespace pkv
