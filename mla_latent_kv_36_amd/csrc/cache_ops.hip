// Paged latent cache: append, gather (debug) and block-table validation; and a
// streaming read of device memory (the achievable HBM read rate, a
// measurement helper).
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

namespace {

// Streaming read of n 16-byte chunks: thread t of T reads chunks t, t + T,
// ... eight at a time as non-temporal loads and XORs them together; a
// workgroup's XOR reaches the sink through the wave's lane swaps, LDS and
// four atomic XORs.
constexpr int SR_GRID = 256;  // workgroups: one per compute unit of the chip
constexpr int SR_NT = 256;

__global__ __launch_bounds__(SR_NT) void stream_read_kernel(const u32x4* __restrict__ x, size_t n,
                                                            uint32_t* __restrict__ sink) {
  const size_t T = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * T < n; i += 8 * T) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(&x[i + k * T]);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; i < n; i += T) acc ^= __builtin_nontemporal_load(&x[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] ^= (uint32_t)__shfl_xor((int)acc[c], off);
  __shared__ u32x4 red[SR_NT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x < 4) {
    uint32_t r = 0u;
#pragma unroll
    for (int w = 0; w < SR_NT / 64; ++w) r ^= red[w][threadIdx.x];
    atomicXor(&sink[threadIdx.x], r);
  }
}

// The same read through direct-to-LDS copies: workgroup i streams the 1 KiB
// pieces [P i / G, P (i+1) / G) of the buffer's P whole pieces, wave w taking
// every fourth; each wave keeps SR_RING copies in flight through its own ring
// of SR_RING 1 KiB slots, and XORs a slot's 16 bytes per lane once it has
// landed, before the slot takes the next copy.  Workgroup 0 reads the tail
// under 1 KiB with plain loads.
constexpr int SR_RING = 8;

template <int N>
__device__ __forceinline__ void sr_wait(int ahead) {
  // this wave's copies have landed except the `ahead` most recent (< N)
  if (ahead >= N - 1) wait_vmcnt<N - 1>();
  else if (ahead == 6) wait_vmcnt<6>();
  else if (ahead == 5) wait_vmcnt<5>();
  else if (ahead == 4) wait_vmcnt<4>();
  else if (ahead == 3) wait_vmcnt<3>();
  else if (ahead == 2) wait_vmcnt<2>();
  else if (ahead == 1) wait_vmcnt<1>();
  else wait_vmcnt<0>();
}

__global__ __launch_bounds__(SR_NT) void stream_read_lds_kernel(const uint8_t* __restrict__ x,
                                                                size_t bytes,
                                                                uint32_t* __restrict__ sink) {
  __shared__ __align__(16) uint8_t ring[SR_NT / 64][SR_RING][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const size_t P = bytes >> 10;
  const size_t p0 = P * blockIdx.x / gridDim.x, p1 = P * (blockIdx.x + 1) / gridDim.x;
  // this wave's pieces: p0 + wave + 4k, k < n
  const long long n = p1 > p0 + wave ? (long long)((p1 - p0 - wave + 3) / 4) : 0;
  const uint32_t base = (uint32_t)(uintptr_t)&ring[wave][0][0];
  auto issue = [&](long long k) {
    copy16_to_lds(x + ((p0 + wave + 4 * k) << 10), (uint32_t)lane * 16,
                  base + (uint32_t)(k % SR_RING) * 1024);
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long long k = 0; k < SR_RING && k < n; ++k) issue(k);
  for (long long k = 0; k < n; ++k) {
    sr_wait<SR_RING>((int)min((long long)SR_RING - 1, n - 1 - k));
    acc ^= *reinterpret_cast<const u32x4*>(&ring[wave][k % SR_RING][16 * lane]);
    // the read has completed before the slot takes its next copy
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (3 << 14));  // lgkmcnt(0)
    if (k + SR_RING < n) issue(k + SR_RING);
  }
  if (blockIdx.x == 0) {
    const size_t t0 = P << 6, tn = bytes >> 4;  // 16-byte chunks of the tail
    const u32x4* xc = reinterpret_cast<const u32x4*>(x);
    for (size_t c = t0 + threadIdx.x; c < tn; c += SR_NT) acc ^= xc[c];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] ^= (uint32_t)__shfl_xor((int)acc[c], off);
  __shared__ u32x4 red[SR_NT / 64];
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x < 4) {
    uint32_t r = 0u;
#pragma unroll
    for (int w = 0; w < SR_NT / 64; ++w) r ^= red[w][threadIdx.x];
    atomicXor(&sink[threadIdx.x], r);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, bool lds,
                              hipStream_t stream) {
  if (lds)
    hipLaunchKernelGGL(stream_read_lds_kernel, dim3(SR_GRID), dim3(SR_NT), 0, stream,
                       static_cast<const uint8_t*>(src), bytes, static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL(stream_read_kernel, dim3(SR_GRID), dim3(SR_NT), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
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
