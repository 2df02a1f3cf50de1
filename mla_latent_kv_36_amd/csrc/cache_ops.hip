// Paged latent cache: append, gather (debug) and block-table validation.
//
// Only the latent c and the decoupled rotary key k^R of a token are cached
// ("Attention, Part 2: MQA, GQA and MLA", section "The MLA equations"), as one
// row [c | k^R] per token.  Rows live in fixed-size pages of a pool; a block
// table maps a sequence's logical page index to a page of the pool.  Row j of
// sequence b sits in page block_table[b, j / block_size] at slot
// j % block_size.  Every kernel here is pure data movement: bit-exact copies.
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

template <typename U>
__device__ __forceinline__ void copy_row(uint8_t* dst, const uint8_t* src, int row_bytes) {
  const int n = row_bytes / (int)sizeof(U);
  for (int k = threadIdx.x; k < n; k += blockDim.x)
    reinterpret_cast<U*>(dst)[k] = reinterpret_cast<const U*>(src)[k];
}

// One workgroup per new row (b, i).
template <typename U>
__global__ __launch_bounds__(64) void append_kernel(uint8_t* __restrict__ pool, int num_blocks,
                                                   const int32_t* __restrict__ table,
                                                   int max_blocks,
                                                   const int32_t* __restrict__ seq_lens,
                                                   const uint8_t* __restrict__ new_rows,
                                                   int T_new, int block_size, int row_bytes) {
  const int b = blockIdx.x / T_new;
  const int i = blockIdx.x - b * T_new;
  const int pos = seq_lens[b] + i;
  if (pos < 0) return;
  const int page = pos / block_size;
  if (page >= max_blocks) return;
  const int blk = table[(size_t)b * max_blocks + page];
  if (blk < 0 || blk >= num_blocks) return;
  uint8_t* dst = pool + ((size_t)blk * block_size + (pos - page * block_size)) * row_bytes;
  copy_row<U>(dst, new_rows + (size_t)blockIdx.x * row_bytes, row_bytes);
}

// One workgroup per (row j, sequence b).
template <typename U>
__global__ __launch_bounds__(64) void gather_kernel(const uint8_t* __restrict__ pool,
                                                   int num_blocks,
                                                   const int32_t* __restrict__ table,
                                                   int max_blocks,
                                                   const int32_t* __restrict__ seq_lens,
                                                   int cap, int block_size, int row_bytes,
                                                   uint8_t* __restrict__ dense) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int n = min(seq_lens[b], cap);
  if (j >= n) return;
  const int page = j / block_size;
  const int blk = clamp_block(table[(size_t)b * max_blocks + page], num_blocks);
  copy_row<U>(dense + ((size_t)b * cap + j) * row_bytes,
              pool + ((size_t)blk * block_size + (j - page * block_size)) * row_bytes, row_bytes);
}

__global__ void clear_flag_kernel(int32_t* flag) { *flag = 0; }

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ table, int B,
                                                      int max_blocks,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int block_size, int num_blocks,
                                                      int32_t* flag) {
  const int b = blockIdx.y;
  if (b >= B) return;
  const int n = seq_lens[b];
  const long long need = n > 0 ? ((long long)n + block_size - 1) / block_size : 0;
  if (need > max_blocks && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(flag, 2);
  const int lim = (int)(need < max_blocks ? need : max_blocks);
  for (int pg = blockIdx.x * blockDim.x + threadIdx.x; pg < lim; pg += gridDim.x * blockDim.x) {
    const int id = table[(size_t)b * max_blocks + pg];
    if (id < 0 || id >= num_blocks) atomicOr(flag, 1);
  }
}

}  // namespace

hipError_t launch_append(void* pool, int num_blocks, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, const void* new_rows, int B, int T_new,
                         int block_size, int row_bytes, hipStream_t stream) {
  if (B <= 0 || T_new <= 0) return hipSuccess;
  const dim3 grid((unsigned)(B * T_new));
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(append_kernel<uint4>, grid, dim3(64), 0, stream, (uint8_t*)pool,
                       num_blocks, block_table, max_blocks, seq_lens, (const uint8_t*)new_rows,
                       T_new, block_size, row_bytes);
  else
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(64), 0, stream, (uint8_t*)pool,
                       num_blocks, block_table, max_blocks, seq_lens, (const uint8_t*)new_rows,
                       T_new, block_size, row_bytes);
  return hipGetLastError();
}

hipError_t launch_gather(const void* pool, int num_blocks, const int32_t* block_table,
                         int max_blocks, const int32_t* seq_lens, int B, int cap,
                         int block_size, int row_bytes, void* dense, hipStream_t stream) {
  if (B <= 0 || cap <= 0) return hipSuccess;
  const dim3 grid((unsigned)cap, (unsigned)B);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(gather_kernel<uint4>, grid, dim3(64), 0, stream, (const uint8_t*)pool,
                       num_blocks, block_table, max_blocks, seq_lens, cap, block_size, row_bytes,
                       (uint8_t*)dense);
  else
    hipLaunchKernelGGL(gather_kernel<uint16_t>, grid, dim3(64), 0, stream, (const uint8_t*)pool,
                       num_blocks, block_table, max_blocks, seq_lens, cap, block_size, row_bytes,
                       (uint8_t*)dense);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* block_table, int B, int max_blocks,
                           const int32_t* seq_lens, int block_size, int num_blocks,
                           int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, stream, err_flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || B <= 0) return e;
  const unsigned gx = (unsigned)((max_blocks + 255) / 256);
  hipLaunchKernelGGL(validate_kernel, dim3(gx > 0 ? gx : 1, (unsigned)B), dim3(256), 0, stream,
                     block_table, B, max_blocks, seq_lens, block_size, num_blocks, err_flag);
  return hipGetLastError();
}

}  // namespace mla
