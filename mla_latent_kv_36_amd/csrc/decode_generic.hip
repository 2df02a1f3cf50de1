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
                      : p.part_o + (((size_t)b * p.num_splits + s) * TH + rr) * p.d_c;

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

// Log-sum-exp merge of the splits of one query row: with M = max_s lse_s and
// w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s
// ("Attention, Part 2: MQA, GQA and MLA": the partial results of disjoint row
// ranges combine exactly through their log-sum-exp).  Only splits that hold
// rows of this query are read (the same row arithmetic as the split
// kernels), in split order, so the result is deterministic.  One wave per
// query row; each lane owns 4 consecutive latent columns per 256-column block.
// The merge streams the partials once, so the loads of a row are issued
// together, as many as fit, rather than one split at a time.
constexpr int CMB_ROWS = 4;   // query rows (waves) per workgroup

__global__ __launch_bounds__(64 * CMB_ROWS) void combine_kernel(const DecodeParams p) {
  const int TH = p.T * p.H;
  const long long nrows = (long long)p.B * TH;
  const long long row = (long long)blockIdx.x * CMB_ROWS + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const int b = (int)(row / TH);
  const int rr = (int)(row - (long long)b * TH);
  const int t = rr / p.H;
  // this sequence's splits: the first one's partial index, their count and
  // the cache rows per split (a balanced plan: from the table the decode
  // kernel wrote; the plain plan: the same for every sequence)
  int P0, S, chunk;
  if (p.plan != nullptr) {
    const int4 e = *reinterpret_cast<const int4*>(p.plan + 4 * (size_t)b);
    P0 = __builtin_amdgcn_readfirstlane(e.x);
    S = __builtin_amdgcn_readfirstlane(e.y);
    chunk = __builtin_amdgcn_readfirstlane(e.z) * 32;
    if (S == 0) {  // no visible row in the sequence: o = 0, lse = -inf
      float* out = p.o_lat + (size_t)row * p.d_c;
      for (int d = lane; d < p.d_c; d += 64) out[d] = 0.0f;
      if (lane == 0 && p.lse != nullptr) p.lse[row] = -INFINITY;
      return;
    }
  } else {
    P0 = b * p.num_splits;
    S = p.num_splits;
    chunk = p.chunk_rows;
  }
  if (S <= 8 && p.d_c == 512) {
    // The common shape in one memory round trip: the sequence length, every
    // split's log-sum-exp (lane s) and every split's partial row (8 columns
    // per lane) are read before any of them is used.  Splits that hold no row
    // of this query were never written; they are left out by selection, not
    // by a zero weight, since their memory may hold anything.
    const float* lse_b = p.part_lse + (size_t)P0 * TH + rr;
    const float* po_b = p.part_o + ((size_t)P0 * TH + rr) * 512 + 4 * lane;
    const size_t sstride = (size_t)TH * 512;
    const int len = p.seq_lens[b];
    const float lse_l = lse_b[(size_t)min(lane, S - 1) * TH];
    f32x4 v0[8], v1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float* src = po_b + (size_t)min(k, S - 1) * sstride;
      v0[k] = *reinterpret_cast<const f32x4*>(src);
      v1[k] = *reinterpret_cast<const f32x4*>(src + 256);
    }
    // every value above is consumed here, so all 18 loads are issued before
    // the first wait (the compiler would otherwise interleave waits and loads)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(len), "v"(lse_l));
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" ::"v"(v0[k]), "v"(v1[k]));
    const int n_valid = visible_rows(len, p.T, t, p.causal, p.cap);
    const int ns = __builtin_amdgcn_readfirstlane(min(S, (n_valid + chunk - 1) / chunk));
    // no branches from here on: a branch would let the compiler move the
    // loads above behind it, one dependent round trip at a time
    float M = lane < ns ? lse_l : -INFINITY;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float e = lane < ns ? exp2f((lse_l - M) * kLog2e) : 0.0f;
    float den = e;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = __shfl(e, k);
      const f32x4 t0 = a0 + w * v0[k], t1 = a1 + w * v1[k];
      a0 = k < ns ? t0 : a0;
      a1 = k < ns ? t1 : a1;
    }
    // no visible row (ns == 0): o = 0, lse = -inf
    const float inv = ns > 0 ? 1.0f / den : 0.0f;
    // streaming stores: o_lat is read by the next kernel (no L2 lines left
    // dirty for the end-of-launch write-back)
    float* out = p.o_lat + (size_t)row * 512 + 4 * lane;
    __builtin_nontemporal_store(a0 * inv, reinterpret_cast<f32x4*>(out));
    __builtin_nontemporal_store(a1 * inv, reinterpret_cast<f32x4*>(out + 256));
    if (lane == 0 && p.lse != nullptr) p.lse[row] = ns > 0 ? M + logf(den) : -INFINITY;
    return;
  }
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  // one row per wave: the split count is the same in every lane
  const int ns = __builtin_amdgcn_readfirstlane(min(S, (n_valid + chunk - 1) / chunk));
  float* out = p.o_lat + (size_t)row * p.d_c;
  const float* lse_b = p.part_lse + (size_t)P0 * TH + rr;
  const float* po_b = p.part_o + ((size_t)P0 * TH + rr) * p.d_c;
  const size_t sstride = (size_t)TH * p.d_c;  // floats between splits of one row

  if (ns <= 0) {
    for (int d = lane; d < p.d_c; d += 64) out[d] = 0.0f;
    if (lane == 0 && p.lse != nullptr) p.lse[row] = -INFINITY;
    return;
  }
  // split s's log-sum-exp is read by lane s % 64 (all loads of a pass in
  // flight at once), then reduced across the wave in a fixed order
  float M = -INFINITY;
  for (int c = 0; c < ns; c += 64)
    if (c + lane < ns) M = fmaxf(M, lse_b[(size_t)(c + lane) * TH]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.0f;
  for (int c = 0; c < ns; c += 64)
    if (c + lane < ns) den += exp2f((lse_b[(size_t)(c + lane) * TH] - M) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  const float inv = 1.0f / den;

  if ((p.d_c & 511) == 0) {
    // 512 columns per pass, 8 per lane; the loads of up to 8 splits (16 x 16 B
    // per lane) are all issued before the first is used, so that enough bytes
    // are in flight to stream the partials at memory speed
    for (int d0 = 0; d0 < p.d_c; d0 += 512) {
      const int da = d0 + 4 * lane;
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < ns; s0 += 8) {
        // splits past the last one re-read the last one with weight 0, so
        // that every load is unconditional
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = exp2f((lse_b[(size_t)min(s0 + k, ns - 1) * TH] - M) * kLog2e);
          w[k] = s0 + k < ns ? e : 0.0f;
        }
        f32x4 v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float* src = po_b + (size_t)min(s0 + k, ns - 1) * sstride + da;
          v0[k] = *reinterpret_cast<const f32x4*>(src);
          v1[k] = *reinterpret_cast<const f32x4*>(src + 256);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          a0 += w[k] * v0[k];
          a1 += w[k] * v1[k];
        }
      }
      *reinterpret_cast<f32x4*>(out + da) = a0 * inv;
      *reinterpret_cast<f32x4*>(out + da + 256) = a1 * inv;
    }
  } else if ((p.d_c & 3) == 0) {
    for (int d = 4 * lane; d < p.d_c; d += 256) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      int s = 0;
      for (; s + 4 <= ns; s += 4) {  // four splits' loads in flight at a time
        f32x4 v[4];
        float w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = *reinterpret_cast<const f32x4*>(po_b + (size_t)(s + k) * sstride + d);
          w[k] = exp2f((lse_b[(size_t)(s + k) * TH] - M) * kLog2e);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) a += w[k] * v[k];
      }
      for (; s < ns; ++s) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(po_b + (size_t)s * sstride + d);
        a += exp2f((lse_b[(size_t)s * TH] - M) * kLog2e) * v;
      }
      *reinterpret_cast<f32x4*>(out + d) = a * inv;
    }
  } else {
    for (int d = lane; d < p.d_c; d += 64) {
      float a = 0.0f;
      for (int s = 0; s < ns; ++s)
        a += exp2f((lse_b[(size_t)s * TH] - M) * kLog2e) * po_b[(size_t)s * sstride + d];
      out[d] = a * inv;
    }
  }
  if (lane == 0 && p.lse != nullptr) p.lse[row] = M + logf(den);
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
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(64 * CMB_ROWS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
