// Split-KV latent-attention decode for any shape and element type (fp32 or
// bf16): the path for shapes the MFMA kernel does not cover (for example fp32
// caches or latent widths other than 512).  It is a plain flash-decoding loop:
// one workgroup = one query row (b, t, h) x one split, 256 rows of the cache
// per step, fp32 throughout.
//
// Per step: each thread scores one cached row against the absorbed query held
// in LDS (content and rotary terms in one dot product, "Attention, Part 2: MQA,
// GQA and MLA", section "Why position needs its own key"), the block takes the
// step maximum, rescales its running sum and accumulator, and accumulates the
// weighted latents (the first d_c columns of each row, "How DeepSeek Rewrote
// the Transformer", section "Absorbed projections", point 3).
#include "common.h"
#include "launch.h"
#include "merge.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int MAX_DC_PER_THREAD = 8;  // d_c <= 2048

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.0f;
  for (int i = 0; i < NT / 64; ++i) r += red[i];
  return r;
}

template <typename E>
__global__ __launch_bounds__(NT) void decode_generic_kernel(const DecodeParams p) {
  extern __shared__ float smem[];
  const int W = p.d_c + p.d_r;
  float* sq = smem;          // [W] query
  float* sp = smem + W;      // [NT] probabilities of the current step
  float* red = sp + NT;      // [NT / 64]

  const int tid = threadIdx.x;
  const int TH = p.T * p.H;
  const int row = blockIdx.x;  // (b, t, h) flattened
  const int s = blockIdx.y;
  const int b = row / TH;
  const int rr = row - b * TH;
  const int t = rr / p.H;
  const int bs = p.block_size;
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  const int j0 = s * p.chunk_rows;
  const int j1 = min(j0 + p.chunk_rows, n_valid);
  const bool direct = (p.num_splits == 1);
  float* dst = direct ? p.o_lat + (size_t)row * p.d_c
                      : static_cast<float*>(p.part_o) +
                            (((size_t)b * p.num_splits + s) * TH + rr) * p.d_c;

  if (j0 >= j1) {
    if (direct) {
      for (int d = tid; d < p.d_c; d += NT) dst[d] = 0.0f;
      if (tid == 0 && p.lse != nullptr) p.lse[row] = -INFINITY;
    }
    return;
  }

  const E* q = static_cast<const E*>(p.q_abs) + (size_t)row * W;
  for (int k = tid; k < W; k += NT) sq[k] = Elem<E>::load(q, k);
  __syncthreads();

  const E* pool = static_cast<const E*>(p.pool);
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  auto row_ptr = [&](int j) {
    const int blk = clamp_block(table[j / bs], p.num_blocks);
    return pool + ((size_t)blk * bs + (j % bs)) * W;
  };

  float acc[MAX_DC_PER_THREAD];
#pragma unroll
  for (int i = 0; i < MAX_DC_PER_THREAD; ++i) acc[i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  for (int jb = j0; jb < j1; jb += NT) {
    const int j = jb + tid;
    float sc = -INFINITY;
    if (j < j1) {
      const E* r = row_ptr(j);
      float dot = 0.0f;
      for (int k = 0; k < W; ++k) dot += sq[k] * Elem<E>::load(r, k);
      sc = dot * p.scale_log2;
    }
    const float m_new = fmaxf(m_run, block_max(sc, red));
    const float alpha = exp2f(m_run - m_new);  // 0 on the first step
    const float e = (j < j1) ? exp2f(sc - m_new) : 0.0f;
    sp[tid] = e;
    l_run = l_run * alpha + block_sum(e, red);  // block_sum synchronises sp too
    m_run = m_new;
    const int n = min(NT, j1 - jb);
#pragma unroll
    for (int i = 0; i < MAX_DC_PER_THREAD; ++i) {
      const int d = tid + i * NT;
      if (d < p.d_c) {
        float a = acc[i] * alpha;
        for (int jj = 0; jj < n; ++jj) a += sp[jj] * Elem<E>::load(row_ptr(jb + jj), d);
        acc[i] = a;
      }
    }
    __syncthreads();
  }

  const float inv = 1.0f / l_run;
#pragma unroll
  for (int i = 0; i < MAX_DC_PER_THREAD; ++i) {
    const int d = tid + i * NT;
    if (d < p.d_c) dst[d] = acc[i] * inv;
  }
  if (tid == 0) {
    const float v = (m_run + log2f(l_run)) * kLn2;
    if (direct) {
      if (p.lse != nullptr) p.lse[row] = v;
    } else {
      p.part_lse[((size_t)b * p.num_splits + s) * TH + rr] = v;
    }
  }
}

// One wave per query row, CMB_ROWS rows per workgroup (merge_row).
constexpr int CMB_ROWS = 4;

template <typename PT>
__global__ __launch_bounds__(64 * CMB_ROWS) void combine_kernel(const DecodeParams p) {
  const long long nrows = (long long)p.B * p.T * p.H;
  const long long row = (long long)blockIdx.x * CMB_ROWS + (threadIdx.x >> 6);
  if (row >= nrows) return;
  merge_row<PT>(p, row, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeParams& p, int dtype, hipStream_t stream) {
  const long long rows = (long long)p.B * p.T * p.H;
  if (rows <= 0) return hipSuccess;
  const size_t shmem = (size_t)(p.d_c + p.d_r + NT + NT / 64) * sizeof(float);
  const dim3 grid((unsigned)rows, (unsigned)p.num_splits);
  if (dtype == 0)
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(NT), shmem, stream, p);
  else
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, dim3(NT), shmem, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.T * p.H;
  if (rows <= 0) return hipSuccess;
  const long long blocks = (rows + CMB_ROWS - 1) / CMB_ROWS;
  // bf16 partials come from the MFMA kernel only, whose d_c is 512
  if (p.part_bf16 && p.d_c != 512) return hipErrorInvalidValue;
  if (p.part_bf16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((unsigned)blocks), dim3(64 * CMB_ROWS), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)blocks), dim3(64 * CMB_ROWS), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace mla
