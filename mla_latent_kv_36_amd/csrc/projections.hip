// The two per-head projections around latent attention.
//
// absorb_q: q_abs[m, h, :d_c] = q_nope[m, h, :] . W^UK[h] (W^UK[h] is d_nope x
//   d_c), q_abs[m, h, d_c:] = q_rope[m, h, :]  -- the query side of absorption
//   ("Attention, Part 2: MQA, GQA and MLA", section "The trick that makes it
//   fast": the new query is multiplied once by W_uk(h)^T).
// out_proj: out[m, h, v] = sum_c W^UV[h, v, c] o_lat[m, h, c]  -- the value side,
//   applied once per head after the latent-space sum (same section).
//
// Both are small batched GEMMs whose weights dominate the bytes at decode
// batch sizes; each workgroup streams one head's weight slice once and reuses
// it across a block of query rows held in LDS.  fp32 accumulation.
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int ABS_NT = 256;  // columns of d_c per workgroup
constexpr int ABS_MT = 16;   // query rows per workgroup

template <typename E>
__global__ __launch_bounds__(ABS_NT) void absorb_q_kernel(const E* __restrict__ q_nope,
                                                         const E* __restrict__ q_rope,
                                                         const E* __restrict__ w_uk,
                                                         E* __restrict__ q_abs, int M, int H,
                                                         int d_n, int d_c, int d_r) {
  extern __shared__ float sq[];  // [ABS_MT][d_n]
  const int h = blockIdx.x;
  const int c = blockIdx.y * ABS_NT + threadIdx.x;
  const int m0 = blockIdx.z * ABS_MT;
  const int mt = min(ABS_MT, M - m0);
  const int W = d_c + d_r;

  for (int i = threadIdx.x; i < ABS_MT * d_n; i += ABS_NT) {
    const int mi = i / d_n, d = i - mi * d_n;
    sq[i] = (mi < mt) ? Elem<E>::load(q_nope, ((size_t)(m0 + mi) * H + h) * d_n + d) : 0.0f;
  }
  __syncthreads();

  if (c < d_c) {
    float acc[ABS_MT];
#pragma unroll
    for (int i = 0; i < ABS_MT; ++i) acc[i] = 0.0f;
    const E* wcol = w_uk + (size_t)h * d_n * d_c + c;
    for (int d = 0; d < d_n; ++d) {
      const float w = Elem<E>::load(wcol, (size_t)d * d_c);
#pragma unroll
      for (int i = 0; i < ABS_MT; ++i) acc[i] += sq[i * d_n + d] * w;
    }
#pragma unroll
    for (int i = 0; i < ABS_MT; ++i)
      if (i < mt) Elem<E>::store(q_abs, ((size_t)(m0 + i) * H + h) * W + c, acc[i]);
  }
  if (blockIdx.y == 0) {  // the rotary part is carried over unchanged
    for (int i = threadIdx.x; i < mt * d_r; i += ABS_NT) {
      const int mi = i / d_r, r = i - mi * d_r;
      q_abs[((size_t)(m0 + mi) * H + h) * W + d_c + r] =
          q_rope[((size_t)(m0 + mi) * H + h) * d_r + r];
    }
  }
}

constexpr int OP_T = 16;   // output tile: 16 rows x 16 value columns
constexpr int OP_K = 64;   // latent columns per LDS step

template <typename E>
__global__ __launch_bounds__(256) void out_proj_kernel(const float* __restrict__ o_lat,
                                                      const E* __restrict__ w_uv,
                                                      E* __restrict__ out, int M, int H,
                                                      int d_c, int d_v) {
  __shared__ float so[OP_T][OP_K + 1];
  __shared__ float sw[OP_T][OP_K + 1];
  const int h = blockIdx.x;
  const int v0 = blockIdx.y * OP_T;
  const int m0 = blockIdx.z * OP_T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc = 0.0f;
  for (int c0 = 0; c0 < d_c; c0 += OP_K) {
    for (int i = threadIdx.x; i < OP_T * OP_K; i += 256) {
      const int r = i / OP_K, k = i - r * OP_K;
      const int c = c0 + k;
      so[r][k] = (m0 + r < M && c < d_c) ? o_lat[((size_t)(m0 + r) * H + h) * d_c + c] : 0.0f;
      sw[r][k] = (v0 + r < d_v && c < d_c)
                     ? Elem<E>::load(w_uv, ((size_t)h * d_v + v0 + r) * d_c + c)
                     : 0.0f;
    }
    __syncthreads();
#pragma unroll 16
    for (int k = 0; k < OP_K; ++k) acc += so[ty][k] * sw[tx][k];
    __syncthreads();
  }
  const int m = m0 + ty, v = v0 + tx;
  if (m < M && v < d_v) Elem<E>::store(out, ((size_t)m * H + h) * d_v + v, acc);
}

}  // namespace

hipError_t launch_absorb_q(int dtype, const void* q_nope, const void* q_rope, const void* w_uk,
                           void* q_abs, int M, int H, int d_n, int d_c, int d_r,
                           hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(H, (d_c + ABS_NT - 1) / ABS_NT, (M + ABS_MT - 1) / ABS_MT);
  const size_t shmem = (size_t)ABS_MT * d_n * sizeof(float);
  if (dtype == 0)
    hipLaunchKernelGGL(absorb_q_kernel<float>, grid, dim3(ABS_NT), shmem, stream,
                       (const float*)q_nope, (const float*)q_rope, (const float*)w_uk,
                       (float*)q_abs, M, H, d_n, d_c, d_r);
  else
    hipLaunchKernelGGL(absorb_q_kernel<uint16_t>, grid, dim3(ABS_NT), shmem, stream,
                       (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk,
                       (uint16_t*)q_abs, M, H, d_n, d_c, d_r);
  return hipGetLastError();
}

hipError_t launch_out_proj(int dtype, const float* o_lat, const void* w_uv, void* out, int M,
                           int H, int d_c, int d_v, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(H, (d_v + OP_T - 1) / OP_T, (M + OP_T - 1) / OP_T);
  if (dtype == 0)
    hipLaunchKernelGGL(out_proj_kernel<float>, grid, dim3(256), 0, stream, o_lat,
                       (const float*)w_uv, (float*)out, M, H, d_c, d_v);
  else
    hipLaunchKernelGGL(out_proj_kernel<uint16_t>, grid, dim3(256), 0, stream, o_lat,
                       (const uint16_t*)w_uv, (uint16_t*)out, M, H, d_c, d_v);
  return hipGetLastError();
}

}  // namespace mla
