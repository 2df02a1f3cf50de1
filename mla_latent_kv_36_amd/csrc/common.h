// Internal helpers shared by the libmla kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(uint16_t)))) uint16_t u16x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 storage is handled as raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Element access for the two storage types the library supports.
template <typename E> struct Elem;
template <> struct Elem<float> {
  using storage = float;
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  using storage = uint16_t;
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Reductions across lane l and lane l ^ 32 (or l ^ 16) on the VALU with the
// gfx950 lane-swap instructions: each lane gets back {x[l], x[l ^ 32]} (resp.
// {x[l], x[l ^ 16]}), so a symmetric operation of the pair is the reduction.
// Maximum of two floats as one v_max_f32.  fmaxf on values that arrive as
// bit patterns (the lane swaps below) makes the compiler quieten possible
// signalling NaNs first (two extra instructions); the reductions here only
// see scores, -inf or quiet NaN, for which the plain instruction is exact.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows a query of new token t may attend to, capped by the host-side bound.
__device__ __forceinline__ int visible_rows(int seq_len, int T, int t, int causal,
                                            int cap) {
  int n = causal ? seq_len - T + t + 1 : seq_len;
  n = n < cap ? n : cap;
  return n > 0 ? n : 0;
}

__device__ __forceinline__ int clamp_block(int id, int num_blocks) {
  return id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
}

}  // namespace mla
