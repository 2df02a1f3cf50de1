// The producer step of the latent cache on CDNA4 (gfx950): each new token's
// cached row [c | k^R] is made from its hidden vector h and written straight
// into the paged cache.
//
//   c   = W^DKV h                       ("Multi-head latent attention (MLA)",
//                                         section 2: the down-projection is
//                                         the only thing cached)
//   k^R = RoPE(W^KR h, position)        (same page, section 3: the decoupled
//                                         key has its own projection and is
//                                         rotated directly; the latent never is)
//
// "Attention, Part 2: MQA, GQA and MLA", section "The MLA equations" and its
// inference code compute exactly these two for the cache.  RoPE turns each
// consecutive pair (x[2i], x[2i+1]) by position * base^(-2i/d_rope) (the
// rotation of one pair by m*theta in section "Why position needs its own
// key"; the angle rule and the base are RoFormer's, which the pages cite
// without restating).
//
// Two kernels:
//   * kv_proj_mfma_kernel: [M tokens x d] . [d x (d_c + d_r)] on
//     v_mfma_f32_16x16x32_bf16.  M is small (a decode step's new tokens), so
//     the work is the weight stream; the k dimension is split over
//     workgroups (fp32 partial sums in a workspace) so that enough compute
//     units stream it.  Each workgroup stages a 64-token and a 64-column
//     tile of hidden vectors and weights over its k range (at most 512) in
//     LDS, all of it requested at once, and runs 4 waves of 16 tokens x 64
//     columns.
//   * kv_rope_append_kernel: sums the partials in split order (deterministic),
//     rotates the k^R pairs, rounds to the cache type and writes the row into
//     its page slot.  The rotation angle is formed and reduced to [-pi, pi]
//     in double precision: at positions near 10^5 an fp32 product
//     position*theta is off by ~0.01 rad.
// fp32 caches and shapes outside the MFMA kernel take kv_proj_generic_kernel
// (one thread per output, no k split) and the same second kernel.
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int PJ_TM = 64;     // tokens per workgroup tile
constexpr int PJ_TN = 64;     // output columns per workgroup tile
constexpr int PJ_KMAX = 512;  // k per workgroup at most (one staged 1 KiB row)

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// part[z, m, n] = sum over this split's k of hidden[m, k] * Wcat[n, k], with
// Wcat = [W^DKV ; W^KR] (rows n < d_c from W^DKV, the rest from W^KR).
// A split covers at most 512 k: the workgroup's 64 hidden rows and 64 weight
// rows over its k range are all requested at once, as direct-to-LDS copies
// of 1 KiB (one staged row each), so that the workgroup pays one memory
// latency; the MFMAs then run from LDS.  16-byte chunk c of staged row r sits
// at position c ^ (r & 15), so that the 16 rows an MFMA operand reads at one
// k fall in distinct banks.  Rows past M or N are clamped (their sums are not
// stored) and k past d within a row re-reads the last chunk (k-steps past the
// split are not multiplied).
__global__ __launch_bounds__(256) void kv_proj_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, float* __restrict__ part, int M, int d, int d_c,
    int d_r, int steps_per_split, int xcds) {
  __shared__ __align__(16) uint8_t st[(PJ_TM + PJ_TN) * 1024];  // hidden rows, then weight rows
  const int N = d_c + d_r;
  // Workgroup i runs on XCD i % xcds (queried on the host), and each XCD has
  // its own L2.  Tiles are
  // numbered column tile fastest, then token tile, then k split, and XCD x
  // takes a contiguous block of them: the hidden-vector slice of a (token
  // tile, split) and the weight slice of a (column tile, split) then come
  // from memory once per XCD and from its L2 for the other tiles that read
  // them.  Ids past the last full set of xcds keep the plain order.
  const int ntn = (N + PJ_TN - 1) / PJ_TN;
  const int ntm = (M + PJ_TM - 1) / PJ_TM;
  const int total = (int)gridDim.x;
  const int full = total - total % xcds;
  const int i = blockIdx.x;
  const int t = i < full ? (i % xcds) * (full / xcds) + i / xcds : i;
  const int n0 = (t % ntn) * PJ_TN;
  const int m0 = ((t / ntn) % ntm) * PJ_TM;
  const int z = t / (ntn * ntm);
  const int nk = d / 32;
  const int s_begin = z * steps_per_split;
  const int steps = min(steps_per_split, nk - s_begin);  // k-steps of 32 (<= 16)
  const int k0 = 32 * s_begin;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches

  // staged row q < 64: hidden row m0 + q; q >= 64: weight row n0 + q - 64
  const uint32_t st_base = (uint32_t)(uintptr_t)st;
#pragma unroll
  for (int j = 0; j < (PJ_TM + PJ_TN) / 4; ++j) {
    const int q = wave + 4 * j;
    const int r = q & 63;
    const uint16_t* src;
    if (q < PJ_TM) {
      src = hidden + (size_t)min(m0 + r, M - 1) * d;
    } else {
      const int n = min(n0 + r, N - 1);
      src = n < d_c ? w_dkv + (size_t)n * d : w_kr + (size_t)(n - d_c) * d;
    }
    const int c = lane ^ (r & 15);
    copy16_to_lds(reinterpret_cast<const uint8_t*>(src), 2u * (uint32_t)min(k0 + 8 * c, d - 8),
                  st_base + q * 1024);
  }
  wait_vmcnt<0>();
  lds_barrier();

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // wave w: tokens 16w + (l & 15) (A), columns 16j + (l & 15) (B), k
  // 32s + 8(l >> 4) .. +7, i.e. chunk 4s + (l >> 4)
  const int i16 = lane & 15, g = lane >> 4;
  const uint8_t* arow = st + (16 * wave + i16) * 1024;
  auto step = [&](int s) __attribute__((always_inline)) {
    const int pos = ((4 * s + g) ^ i16) * 16;  // every operand row here has (row & 15) == i16
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + pos);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b =
          *reinterpret_cast<const bf16x8*>(st + (PJ_TM + 16 * j + i16) * 1024 + pos);
      acc[j] = mfma16(a, b, acc[j]);
    }
  };
  // a full split as straight-line code with its operands read three steps
  // ahead, so that LDS latency is hidden under the MFMAs of earlier steps
  if (steps == PJ_KMAX / 32) {
    constexpr int AH = 3;
    bf16x8 fa[AH], fb[AH][4];
    auto read = [&](int s, int k) __attribute__((always_inline)) {
      const int pos = ((4 * s + g) ^ i16) * 16;
      fa[k] = *reinterpret_cast<const bf16x8*>(arow + pos);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[k][j] = *reinterpret_cast<const bf16x8*>(st + (PJ_TM + 16 * j + i16) * 1024 + pos);
    };
#pragma unroll
    for (int s = 0; s < AH; ++s) read(s, s);
#pragma unroll
    for (int s = 0; s < PJ_KMAX / 32; ++s) {
      const int k = s % AH;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma16(fa[k], fb[k][j], acc[j]);
      if (s + AH < PJ_KMAX / 32) read(s + AH, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int s = 0; s < steps; ++s) step(s);
  }
  // D: lane l holds column 16j + (l & 15), tokens 16w + 4(l >> 4) + i
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + i16;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * wave + 4 * g + i;
      if (m < M) part[((size_t)z * M + m) * N + n] = acc[j][i];
    }
  }
}

// Any element type and shape: one thread per (token, output column), the
// whole dot product in fp32; the result goes to partial slot 0.
template <typename E>
__global__ __launch_bounds__(256) void kv_proj_generic_kernel(
    const E* __restrict__ hidden, const E* __restrict__ w_dkv, const E* __restrict__ w_kr,
    float* __restrict__ part, int M, int d, int d_c, int d_r) {
  const int N = d_c + d_r;
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (m >= M || n >= N) return;
  const E* h = hidden + (size_t)m * d;
  const E* w = n < d_c ? w_dkv + (size_t)n * d : w_kr + (size_t)(n - d_c) * d;
  float s = 0.0f;
  for (int k = 0; k < d; ++k) s += Elem<E>::load(h, k) * Elem<E>::load(w, k);
  part[(size_t)m * N + n] = s;
}

// (cos, sin) of the angle of pair q of a d_r-wide rotary vector at position
// pos.  The angle pos * theta is formed and reduced to [-pi, pi] in double
// precision (exact enough at any int32 position); the reduced angle then
// goes through the fp32 sine and cosine, accurate to a few ulp there.
__device__ __forceinline__ void rope_angle(int pos, int q, int d_r, double log2_base,
                                           float& c, float& s) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double theta = exp2(-(2.0 * q / d_r) * log2_base);
  const double a = (double)pos * theta;
  const double r = a - kTwoPi * rint(a * (1.0 / kTwoPi));
  sincosf((float)r, &s, &c);
}

// One workgroup per token m = b * T_new + i; thread t owns the column pairs
// p = t and p = t + blockDim.x (2p, 2p + 1 < N <= 4 * blockDim.x).  The
// partial sums of the first 16 splits are requested first, then the page is
// looked up through the scalar cache (uniform indexes: its waits leave the
// vector loads in flight), so the round trips overlap.
template <typename E>
__global__ __launch_bounds__(1024) void kv_rope_append_kernel(
    const float* __restrict__ part, int ksplit, int M, int d_c, int d_r, void* pool,
    int num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ seq_lens, int T_new, int block_size, double log2_base) {
  typedef const int32_t __attribute__((address_space(4)))* cptr;
  const int N = d_c + d_r;
  const int m = blockIdx.x;
  if (m >= M) return;
  const int b = m / T_new;
  const int i = m - b * T_new;
  // partial sums in split order, the first 16 splits' loads issued together
  // (unconditional, on clamped indices; splits past the last are left out by
  // selection), further splits 16 at a time
  float2 v[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pc = min((int)threadIdx.x + u * (int)blockDim.x, N / 2 - 1);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[u][k] = *reinterpret_cast<const float2*>(
          part + ((size_t)min(k, ksplit - 1) * M + m) * N + 2 * pc);
  }
  const int pos = ((cptr)seq_lens)[b] + i;
  const int page = pos / block_size;
  const bool in_table = pos >= 0 && page < max_blocks;
  const int blk = in_table ? ((cptr)block_table)[(size_t)b * max_blocks + page] : -1;
  float v0[2] = {0.0f, 0.0f}, v1[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = threadIdx.x + u * blockDim.x;
    if (2 * p >= N) continue;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v0[u] = k < ksplit ? v0[u] + v[u][k].x : v0[u];
      v1[u] = k < ksplit ? v1[u] + v[u][k].y : v1[u];
    }
    for (int z0 = 16; z0 < ksplit; z0 += 16) {
      float2 w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        w[k] = *reinterpret_cast<const float2*>(
            part + ((size_t)min(z0 + k, ksplit - 1) * M + m) * N + 2 * p);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v0[u] = z0 + k < ksplit ? v0[u] + w[k].x : v0[u];
        v1[u] = z0 + k < ksplit ? v1[u] + w[k].y : v1[u];
      }
    }
  }
  if (blk < 0 || blk >= num_blocks) return;  // position or page id out of range
  E* row = static_cast<E*>(pool) + ((size_t)blk * block_size + pos % block_size) * N;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = threadIdx.x + u * blockDim.x;
    if (2 * p >= N) continue;
    float r0 = v0[u], r1 = v1[u];
    if (2 * p >= d_c) {
      float c, s;
      rope_angle(pos, p - d_c / 2, d_r, log2_base, c, s);
      r0 = v0[u] * c - v1[u] * s;
      r1 = v0[u] * s + v1[u] * c;
    }
    Elem<E>::store(row, 2 * p, r0);
    Elem<E>::store(row, 2 * p + 1, r1);
  }
}

// In place: x[m, h, 2q .. 2q+1] turned by positions[m] * base^(-2q/d_r).
template <typename E>
__global__ __launch_bounds__(256) void rope_kernel(E* __restrict__ x,
                                                   const int32_t* __restrict__ positions,
                                                   int M, int heads, int d_r, double log2_base) {
  const int m = blockIdx.x;
  if (m >= M) return;
  const int pos = positions[m];
  const int pairs = heads * (d_r / 2);
  for (int t = threadIdx.x; t < pairs; t += blockDim.x) {
    const int h = t / (d_r / 2);
    const int q = t - h * (d_r / 2);
    E* v = x + ((size_t)m * heads + h) * d_r;
    float c, s;
    rope_angle(pos, q, d_r, log2_base, c, s);
    const float a = Elem<E>::load(v, 2 * q), bb = Elem<E>::load(v, 2 * q + 1);
    Elem<E>::store(v, 2 * q, a * c - bb * s);
    Elem<E>::store(v, 2 * q + 1, a * s + bb * c);
  }
}

}  // namespace

bool kv_proj_mfma_supported(int dtype, int d_model) {
  return dtype == 1 && d_model > 0 && d_model % 32 == 0;
}

int kv_produce_ksplit(int dtype, int M, int d_model, int d_c, int d_r, int cus) {
  if (!kv_proj_mfma_supported(dtype, d_model) || M <= 0) return 1;
  const int N = d_c + d_r;
  const long long tiles = (long long)((N + PJ_TN - 1) / PJ_TN) * ((M + PJ_TM - 1) / PJ_TM);
  const int nk = d_model / 32;
  // as many splits as keep the grid within one workgroup per compute unit,
  // but at least enough for 512 k (16 k-steps) per split
  long long ks = cus / tiles;
  const long long ks_min = (nk + PJ_KMAX / 32 - 1) / (PJ_KMAX / 32);
  if (ks < ks_min) ks = ks_min;
  if (ks > nk) ks = nk;
  const int per = (int)((nk + ks - 1) / ks);
  return (nk + per - 1) / per;
}

hipError_t launch_kv_produce(int dtype, const void* hidden, int d_model, const void* w_dkv,
                             const void* w_kr, float rope_base, float* part, int ksplit,
                             void* pool, int num_blocks, const int32_t* block_table,
                             int max_blocks, const int32_t* seq_lens, int B, int T_new,
                             int block_size, int d_c, int d_r, int xcds, hipStream_t stream) {
  const int M = B * T_new;
  const int N = d_c + d_r;
  if (M <= 0) return hipSuccess;
  if (kv_proj_mfma_supported(dtype, d_model)) {
    const int nk = d_model / 32;
    const int per = (nk + ksplit - 1) / ksplit;
    if (ksplit < 1 || per > PJ_KMAX / 32) return hipErrorInvalidValue;  // at most 512 k a split
    const long long tiles =
        (long long)((N + PJ_TN - 1) / PJ_TN) * ((M + PJ_TM - 1) / PJ_TM) * ksplit;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_proj_mfma_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_dkv),
                       static_cast<const uint16_t*>(w_kr), part, M, d_model, d_c, d_r, per,
                       xcds < 1 ? 1 : xcds);
  } else {
    if (ksplit != 1) return hipErrorInvalidValue;
    const dim3 grid((N + 255) / 256, M);
    if (dtype == 0)
      hipLaunchKernelGGL(kv_proj_generic_kernel<float>, grid, dim3(256), 0, stream,
                         static_cast<const float*>(hidden), static_cast<const float*>(w_dkv),
                         static_cast<const float*>(w_kr), part, M, d_model, d_c, d_r);
    else
      hipLaunchKernelGGL(kv_proj_generic_kernel<uint16_t>, grid, dim3(256), 0, stream,
                         static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_dkv),
                         static_cast<const uint16_t*>(w_kr), part, M, d_model, d_c, d_r);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const double log2_base = log2((double)rope_base);
  // one thread per column pair (up to 1024 threads, then a loop)
  const int threads = min(1024, (N / 2 + 63) / 64 * 64);
  if (dtype == 0)
    hipLaunchKernelGGL(kv_rope_append_kernel<float>, dim3(M), dim3(threads), 0, stream, part,
                       ksplit, M, d_c, d_r, pool, num_blocks, block_table, max_blocks, seq_lens,
                       T_new, block_size, log2_base);
  else
    hipLaunchKernelGGL(kv_rope_append_kernel<uint16_t>, dim3(M), dim3(threads), 0, stream, part,
                       ksplit, M, d_c, d_r, pool, num_blocks, block_table, max_blocks, seq_lens,
                       T_new, block_size, log2_base);
  return hipGetLastError();
}

hipError_t launch_rope(int dtype, void* x, const int32_t* positions, int M, int heads, int d_r,
                       float rope_base, hipStream_t stream) {
  if (M <= 0 || heads <= 0 || d_r <= 0) return hipSuccess;
  const double log2_base = log2((double)rope_base);
  if (dtype == 0)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(M), dim3(256), 0, stream,
                       static_cast<float*>(x), positions, M, heads, d_r, log2_base);
  else
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(M), dim3(256), 0, stream,
                       static_cast<uint16_t*>(x), positions, M, heads, d_r, log2_base);
  return hipGetLastError();
}

}  // namespace mla
