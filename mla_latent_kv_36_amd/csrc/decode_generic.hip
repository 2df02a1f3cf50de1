// Split-KV latent-attention decode for any shape and element type (fp32 or
// bf16): the path for shapes the MFMA kernel does not cover (for example fp32
// caches or latent widths other than 512).  A flash-decoding loop, fp32
// throughout: one workgroup = GH heads of one new token (b, t) x one split,
// GR cached rows per step, so that each cached row is read once for GH heads
// instead of once per head.
//
// Per step:
//  * scores: wave w takes rows w, w + 4, ... of the step; its lanes split the
//    row's columns (coalesced loads), each loaded element feeds the GH dot
//    products against the absorbed queries held in LDS (content and rotary
//    terms in one dot product, "Attention, Part 2: MQA, GQA and MLA", section
//    "Why position needs its own key");
//  * softmax: thread (head, row) takes one score; each head's GR scores sit in
//    one half-wave, which forms the step maximum and sum; a head's running
//    maximum and sum live in LDS;
//  * values: thread d accumulates latent column d of every head from the
//    weighted rows (the first d_c columns of each row, "How DeepSeek Rewrote
//    the Transformer", section "Absorbed projections", point 3), each loaded
//    element feeding GH accumulators.
#include "common.h"
#include "launch.h"
#include "merge.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int MAX_DC_PER_THREAD = 8;  // d_c <= 2048
constexpr int GH = kGenericHeads;     // heads per workgroup
constexpr int GR = NT / GH;           // cached rows per step (32: a half-wave per head)

template <typename E>
__global__ __launch_bounds__(NT) void decode_generic_kernel(const DecodeParams p) {
  extern __shared__ float smem[];
  const int W = p.d_c + p.d_r;
  float* sq = smem;              // [GH][W] queries
  float* sp = sq + GH * W;       // [GH][GR] scores, then probabilities, of the step
  float* sal = sp + GH * GR;     // [GH] rescale factor of the step
  float* sm_m = sal + GH;        // [GH] running maximum (log2 domain)
  float* sm_l = sm_m + GH;       // [GH] running sum

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int TH = p.T * p.H;
  const int gpt = (p.H + GH - 1) / GH;  // head groups per new token
  const int bt = blockIdx.x / gpt;
  const int h0 = (blockIdx.x - bt * gpt) * GH;
  const int b = bt / p.T, t = bt - b * p.T;
  const int nh = min(GH, p.H - h0);     // heads of this group
  const int s = blockIdx.y;
  const int bs = p.block_size;
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  const int j0 = s * p.chunk_rows;
  const int j1 = min(j0 + p.chunk_rows, n_valid);
  const bool direct = (p.num_splits == 1);
  auto dst_of = [&](int hh) {
    const size_t rr = (size_t)t * p.H + h0 + hh;
    return direct ? p.o_lat + ((size_t)b * TH + rr) * p.d_c
                  : static_cast<float*>(p.part_o) + (((size_t)b * p.num_splits + s) * TH + rr) * p.d_c;
  };

  if (j0 >= j1) {
    if (direct) {
      for (int i = tid; i < nh * p.d_c; i += NT) dst_of(i / p.d_c)[i % p.d_c] = 0.0f;
      if (tid < nh && p.lse != nullptr) p.lse[(size_t)b * TH + (size_t)t * p.H + h0 + tid] = -INFINITY;
    }
    return;
  }

  const E* qb = static_cast<const E*>(p.q_abs) + ((size_t)b * TH + (size_t)t * p.H + h0) * W;
  for (int i = tid; i < GH * W; i += NT) {
    const int hh = i / W;  // heads past the group's last take its last one (not stored)
    sq[i] = Elem<E>::load(qb + (size_t)min(hh, nh - 1) * W, i - hh * W);
  }
  if (tid < GH) {
    sm_m[tid] = -INFINITY;
    sm_l[tid] = 0.0f;
  }
  __syncthreads();

  const E* pool = static_cast<const E*>(p.pool);
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  auto row_ptr = [&](int j) {
    const int blk = clamp_block(table[j / bs], p.num_blocks);
    return pool + ((size_t)blk * bs + (j % bs)) * W;
  };

  float acc[GH][MAX_DC_PER_THREAD];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh)
#pragma unroll
    for (int i = 0; i < MAX_DC_PER_THREAD; ++i) acc[hh][i] = 0.0f;

  for (int jb = j0; jb < j1; jb += GR) {
    const int n = min(GR, j1 - jb);
    // scores of the step's rows for every head of the group
    for (int r = wave; r < GR; r += NT / 64) {
      float dot[GH];
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) dot[hh] = 0.0f;
      if (r < n) {
        const E* row = row_ptr(jb + r);
        for (int k = lane; k < W; k += 64) {
          const float x = Elem<E>::load(row, k);
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) dot[hh] += sq[hh * W + k] * x;
        }
      }
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        float v = dot[hh];
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0) sp[hh * GR + r] = r < n ? v * p.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: thread (hh, r), the GR scores of a head in one half-wave
    {
      const int hh = tid / GR, r = tid - hh * GR;
      const float v = sp[hh * GR + r];
      float mx = v;
      for (int o = GR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_old = sm_m[hh];
      const float m_new = fmaxf(m_old, mx);  // finite: every step holds a row
      const float e = exp2f(v - m_new);      // 0 for rows past the range
      float sum = e;
      for (int o = GR / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      sp[hh * GR + r] = e;
      __syncthreads();  // every thread has read sm_m before it changes
      if (r == 0) {
        const float alpha = exp2f(m_old - m_new);  // 0 on the first step
        sal[hh] = alpha;
        sm_l[hh] = sm_l[hh] * alpha + sum;
        sm_m[hh] = m_new;
      }
    }
    __syncthreads();
    // values: latent column d of every head from the weighted rows
#pragma unroll
    for (int i = 0; i < MAX_DC_PER_THREAD; ++i) {
      const int d = tid + i * NT;
      if (d < p.d_c) {
        float a[GH];
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) a[hh] = acc[hh][i] * sal[hh];
        for (int jj = 0; jj < n; ++jj) {
          const float x = Elem<E>::load(row_ptr(jb + jj), d);
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) a[hh] += sp[hh * GR + jj] * x;
        }
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) acc[hh][i] = a[hh];
      }
    }
    __syncthreads();  // sp and sal are rewritten by the next step
  }

#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    if (hh >= nh) break;
    const float inv = 1.0f / sm_l[hh];
    float* dst = dst_of(hh);
#pragma unroll
    for (int i = 0; i < MAX_DC_PER_THREAD; ++i) {
      const int d = tid + i * NT;
      if (d < p.d_c) dst[d] = acc[hh][i] * inv;
    }
  }
  if (tid < nh) {
    const float v = (sm_m[tid] + log2f(sm_l[tid])) * kLn2;
    const size_t rr = (size_t)t * p.H + h0 + tid;
    if (direct) {
      if (p.lse != nullptr) p.lse[(size_t)b * TH + rr] = v;
    } else {
      p.part_lse[((size_t)b * p.num_splits + s) * TH + rr] = v;
    }
  }
}

// For launches too small to fill the chip with head groups: one workgroup per
// query row (b, t, h) x split, NT cached rows per step -- each thread scores
// one row against the query held in LDS, the block takes the step maximum and
// sum, and each thread accumulates latent columns of the weighted rows.
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
__global__ __launch_bounds__(NT) void decode_generic_head_kernel(const DecodeParams p) {
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
  const long long groups = (long long)p.B * p.T * ((p.H + GH - 1) / GH);
  if (groups <= 0) return hipSuccess;
  if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
  if (groups * p.num_splits < 128) {
    // too few head groups to fill half the chip: a workgroup per query row
    const long long rows = (long long)p.B * p.T * p.H;
    const size_t shmem = (size_t)(p.d_c + p.d_r + NT + NT / 64) * sizeof(float);
    const dim3 grid((unsigned)rows, (unsigned)p.num_splits);
    if (dtype == 0)
      hipLaunchKernelGGL(decode_generic_head_kernel<float>, grid, dim3(NT), shmem, stream, p);
    else
      hipLaunchKernelGGL(decode_generic_head_kernel<uint16_t>, grid, dim3(NT), shmem, stream, p);
    return hipGetLastError();
  }
  const size_t shmem = (size_t)(GH * (p.d_c + p.d_r) + GH * GR + 3 * GH) * sizeof(float);
  const dim3 grid((unsigned)groups, (unsigned)p.num_splits);
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
