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

// Makes a uniform value live in a scalar register at this point (no code).
__device__ __forceinline__ void pin_sgpr(int x) { asm volatile("" ::"s"(x)); }

// Workgroup barrier for LDS traffic only.  __syncthreads() is a release/acquire
// fence plus s_barrier, and the release makes the wave wait for every vector
// memory operation in flight -- including the direct-to-LDS copies of units
// still ahead, which would drain the copy pipeline at every barrier.  Here
// each wave waits only for its own LDS reads and writes (lgkmcnt(0)); copies
// are waited for explicitly (vmcnt) before the barrier that publishes them.
// The signal fences keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte direct-to-LDS copy per lane: lane l reads gbase + voff (its own
// offset) and writes LDS byte lds + 16*l.  Written as assembly so that the
// compiler does not track it: its own tracking treats every later LDS read as
// possibly overlapping a copy in flight and would wait for all copies
// (vmcnt(0)) before the first one, draining the pipeline.  Completion is
// instead waited for explicitly with wait_vmcnt before the barrier that hands
// the slot to the readers.  The copy has no result register; its address
// operands are read at issue.  On gfx9 a copy that reads M0 needs one wait
// state after M0 is written (the s_nop).
// gbase and lds are the same in every lane; they are moved to scalar
// registers explicitly so that the constraints hold whatever the compiler
// concludes about their uniformity.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* gbase, uint32_t voff,
                                              uint32_t lds) {
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint8_t* gs = (const uint8_t*)(uintptr_t)(((uint64_t)ghi << 32) | glo);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(gs)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N), expcnt and lgkmcnt unconstrained.  gfx9 encoding:
  // vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
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
