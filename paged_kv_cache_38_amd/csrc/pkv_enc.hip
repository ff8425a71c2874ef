// Encoder-embedding block cache (the AWS Neuron on-device encoder cache
// notes: "Buffer Layout", "Write Path", "Read Path", "Merge Inside Compiled
// Graph").  One preallocated buffer [num_blocks][block_size][row] holds the
// encoder's post-merger embeddings, one item per block, the last block a
// scratch block for padding writes.  The encoder's output blocks are
// scattered into the buffer by block id; a prefill gathers blocks by id and
// puts each token's row at its position in the batch's hidden states (an
// int64 position map; anything outside [0, num_tokens) is a don't-care token
// and writes nothing); a fill count per hidden row feeds the fail-loud check
// that every scheduled position was filled.
//
// All of it is row copies: HBM-bound, with a fat row (40 KiB at the notes'
// Qwen3-VL geometry, fat_dim 20480 bf16) moved by one 256-thread workgroup
// as 16-byte vectors, four in flight per thread.
#include "pkv_enc.h"

namespace pkv {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kEncThreads = 256;

__device__ __forceinline__ void copy_row(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t units) {
  int64_t k = threadIdx.x;
  for (; k + 3 * kEncThreads < units; k += 4 * kEncThreads) {
    const u32x4 a = src[k], b = src[k + kEncThreads], c = src[k + 2 * kEncThreads], d = src[k + 3 * kEncThreads];
    dst[k] = a;
    dst[k + kEncThreads] = b;
    dst[k + 2 * kEncThreads] = c;
    dst[k + 3 * kEncThreads] = d;
  }
  for (; k < units; k += kEncThreads) dst[k] = src[k];
}

// Write path: workgroup r copies row r % block_size of source block
// r / block_size to its block id (ids outside the buffer are dropped).
__global__ void __launch_bounds__(kEncThreads) enc_write_kernel(u32x4* __restrict__ buffer, int32_t num_blocks,
                                                                int32_t block_size, int64_t row_units,
                                                                const u32x4* __restrict__ src,
                                                                const int32_t* __restrict__ block_ids) {
  const int64_t r = blockIdx.x;
  const int64_t k = r / block_size, t = r % block_size;
  const int32_t b = block_ids[k];
  if (b < 0 || b >= num_blocks) return;
  copy_row(buffer + ((int64_t)b * block_size + t) * row_units, src + r * row_units, row_units);
}

// Read path: workgroup r takes token t = r % block_size of gathered block
// j = r / block_size and copies it to hidden row positions[j][t] when that
// row is real.
__global__ void __launch_bounds__(kEncThreads) enc_merge_kernel(const u32x4* __restrict__ buffer, int32_t num_blocks,
                                                                int32_t block_size, int64_t row_units,
                                                                const int32_t* __restrict__ block_ids,
                                                                const int64_t* __restrict__ positions,
                                                                u32x4* __restrict__ hidden, int64_t num_tokens,
                                                                int32_t* __restrict__ fill_count) {
  const int64_t r = blockIdx.x;
  const int64_t j = r / block_size, t = r % block_size;
  const int64_t p = positions[r];
  const int32_t b = block_ids[j];
  if (p < 0 || p >= num_tokens || b < 0 || b >= num_blocks) return;  // sentinel, or a block outside the buffer
  if (fill_count && threadIdx.x == 0) atomicAdd(fill_count + p, 1);
  copy_row(hidden + p * row_units, buffer + ((int64_t)b * block_size + t) * row_units, row_units);
}

// Fail-loud check: counts[0] = scheduled rows never filled, counts[1] = rows
// filled more than once.  One workgroup.
__global__ void __launch_bounds__(1024) enc_check_kernel(const int32_t* __restrict__ fill_count,
                                                         const int32_t* __restrict__ scheduled, int64_t num_tokens,
                                                         long long* __restrict__ counts) {
  __shared__ long long red[2][16];
  long long missing = 0, doubled = 0;
  for (int64_t k = threadIdx.x; k < num_tokens; k += 1024) {
    const int32_t c = fill_count[k];
    const bool sched = scheduled ? scheduled[k] != 0 : true;
    missing += (sched && c == 0) ? 1 : 0;
    doubled += c > 1 ? 1 : 0;
  }
  for (int o = 32; o > 0; o >>= 1) {
    missing += __shfl_xor(missing, o, 64);
    doubled += __shfl_xor(doubled, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = missing;
    red[1][threadIdx.x >> 6] = doubled;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long a = 0, d = 0;
    for (int w = 0; w < 16; ++w) {
      a += red[0][w];
      d += red[1][w];
    }
    counts[0] = a;
    counts[1] = d;
  }
}

}  // namespace

hipError_t launch_enc_write(char* buffer, int32_t num_blocks, int32_t block_size, int64_t row_units, const char* src,
                            int32_t n, const int32_t* block_ids, hipStream_t s) {
  const int64_t rows = (int64_t)n * block_size;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(enc_write_kernel, dim3((unsigned)rows), dim3(kEncThreads), 0, s,
                     reinterpret_cast<u32x4*>(buffer), num_blocks, block_size, row_units,
                     reinterpret_cast<const u32x4*>(src), block_ids);
  return hipGetLastError();
}

hipError_t launch_enc_merge(const char* buffer, int32_t num_blocks, int32_t block_size, int64_t row_units,
                            const int32_t* block_ids, int32_t max_blocks, const int64_t* positions, char* hidden,
                            int64_t num_tokens, int32_t* fill_count, hipStream_t s) {
  const int64_t rows = (int64_t)max_blocks * block_size;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(enc_merge_kernel, dim3((unsigned)rows), dim3(kEncThreads), 0, s,
                     reinterpret_cast<const u32x4*>(buffer), num_blocks, block_size, row_units, block_ids, positions,
                     reinterpret_cast<u32x4*>(hidden), num_tokens, fill_count);
  return hipGetLastError();
}

hipError_t launch_enc_check(const int32_t* fill_count, const int32_t* scheduled, int64_t num_tokens,
                            long long* counts_dev, hipStream_t s) {
  hipLaunchKernelGGL(enc_check_kernel, dim3(1), dim3(1024), 0, s, fill_count, scheduled, num_tokens, counts_dev);
  return hipGetLastError();
}

}  // namespace pkv
