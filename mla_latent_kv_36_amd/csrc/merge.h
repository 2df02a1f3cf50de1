// Log-sum-exp merge of split partials: one query row per wave (not part of
// the C ABI).
#pragma once

#include "common.h"
#include "launch.h"

namespace mla {

// Log-sum-exp merge of the splits of one query row: with M = max_s lse_s and
// w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s
// ("Attention, Part 2: MQA, GQA and MLA": the partial results of disjoint row
// ranges combine exactly through their log-sum-exp).  Only splits that hold
// rows of this query are read (the same row arithmetic as the split
// kernels), in split order, so the result is deterministic.  One wave per
// query row.  The merge streams the partials once, so the loads of a row are
// issued together, as many as fit, rather than one split at a time.
// Partials are fp32 (PT = float) or bf16 (PT = uint16_t, d_c = 512 only).
// 8 of a partial row's 512 columns per lane: fp32 partials, columns 4l .. 4l+3
// and 256 + 4l .. +3 (two 16-byte loads); bf16 partials, columns 8l .. 8l+7
// (one 16-byte load).  Raw loads first (`raw`), converted after every load of
// the row is in flight (`lo`, `hi`: the lane's first and last 4 columns).
//
// kDev: the partials were stored by other workgroups of the running launch
// with device-scope stores, and are read with device-scope loads (which do not
// take stale lines from this XCD's L2); bf16 partials only.
template <bool kDev>
__device__ __forceinline__ float ld_lse(const float* p) {
  if constexpr (kDev) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

template <typename PT> struct Part8;
template <> struct Part8<float> {
  struct Raw { f32x4 a, b; };
  template <bool kDev = false>
  __device__ __forceinline__ static Raw load(const float* row, int lane) {
    static_assert(!kDev, "device-scope merges read bf16 partials");
    return {*reinterpret_cast<const f32x4*>(row + 4 * lane),
            *reinterpret_cast<const f32x4*>(row + 256 + 4 * lane)};
  }
  __device__ __forceinline__ static void hold(const Raw& r) { asm volatile("" ::"v"(r.a), "v"(r.b)); }
  __device__ __forceinline__ static f32x4 lo(const Raw& r) { return r.a; }
  __device__ __forceinline__ static f32x4 hi(const Raw& r) { return r.b; }
  __device__ __forceinline__ static float* col_lo(float* out, int lane) { return out + 4 * lane; }
  __device__ __forceinline__ static float* col_hi(float* out, int lane) { return out + 256 + 4 * lane; }
};
template <> struct Part8<uint16_t> {
  using Raw = u16x8;
  template <bool kDev = false>
  __device__ __forceinline__ static Raw load(const uint16_t* row, int lane) {
    if constexpr (kDev) {
      // two 8-byte device-scope loads (atomic loads are at most 8 bytes)
      const uint64_t* w = reinterpret_cast<const uint64_t*>(row + 8 * lane);
      typedef __attribute__((__vector_size__(2 * sizeof(uint64_t)))) uint64_t u64x2;
      const u64x2 v = {__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
      return __builtin_bit_cast(u16x8, v);
    } else {
      return *reinterpret_cast<const u16x8*>(row + 8 * lane);
    }
  }
  __device__ __forceinline__ static void hold(const Raw& r) { asm volatile("" ::"v"(r)); }
  __device__ __forceinline__ static f32x4 lo(const Raw& r) {
    return {bf16_to_f32(r[0]), bf16_to_f32(r[1]), bf16_to_f32(r[2]), bf16_to_f32(r[3])};
  }
  __device__ __forceinline__ static f32x4 hi(const Raw& r) {
    return {bf16_to_f32(r[4]), bf16_to_f32(r[5]), bf16_to_f32(r[6]), bf16_to_f32(r[7])};
  }
  __device__ __forceinline__ static float* col_lo(float* out, int lane) { return out + 8 * lane; }
  __device__ __forceinline__ static float* col_hi(float* out, int lane) { return out + 8 * lane + 4; }
};

// ---- bf16 partials of 512 columns (the MFMA kernel's) ----
// The merge of one query row (o_lat row b * T*H + rr, token t) from the S
// partials P0 .. P0+S-1 of its sequence, which cover `chunk` cache rows each,
// by one wave: lane l takes columns 8l .. 8l+7.  Splits that hold no row of
// this query were never written; they are left out by selection, not by a
// zero weight, since their memory may hold anything.
//
// Up to 8 splits, in one memory round trip: row8_issue requests the sequence
// length, every split's log-sum-exp (lane s) and every split's 8 columns
// (splits past S - 1 re-read the last one); row8_finish merges them.  A
// caller may issue several rows before the first finish, so that all of
// their loads are in flight together.
struct Row8Loads {
  int len;
  float lse_l;
  u16x8 v[8];
};
template <bool kDev>
__device__ __forceinline__ void row8_issue(const DecodeParams& p, int b, int rr, int lane, int P0,
                                           int S, Row8Loads& L) {
  const int TH = p.T * p.H;
  const uint16_t* po_b = static_cast<const uint16_t*>(p.part_o) + ((size_t)P0 * TH + rr) * 512;
  const size_t sstride = (size_t)TH * 512;
  L.len = p.seq_lens[b];
  L.lse_l = ld_lse<kDev>(p.part_lse + (size_t)P0 * TH + rr + (size_t)min(lane, S - 1) * TH);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    L.v[k] = Part8<uint16_t>::template load<kDev>(po_b + (size_t)min(k, S - 1) * sstride, lane);
}
// every loaded value is used here, so that the loads stay ahead of the first
// wait (the compiler would otherwise interleave waits and loads)
__device__ __forceinline__ void row8_hold(const Row8Loads& L) {
  asm volatile("" ::"v"(L.len), "v"(L.lse_l));
#pragma unroll
  for (int k = 0; k < 8; ++k) Part8<uint16_t>::hold(L.v[k]);
}
// the lane's merged columns (lo: 8l .. 8l+3, hi: 8l+4 .. 8l+7) and the row's
// log-sum-exp; no visible row gives o = 0, lse = -inf
__device__ __forceinline__ void row8_finish(const DecodeParams& p, const Row8Loads& L, int t,
                                           int lane, int S, int chunk, f32x4& lo, f32x4& hi,
                                           float& lse) {
  using P8 = Part8<uint16_t>;
  const int n_valid = visible_rows(L.len, p.T, t, p.causal, p.cap);
  const int ns = __builtin_amdgcn_readfirstlane(min(S, (n_valid + chunk - 1) / chunk));
  // no branches from here on: a branch would let the compiler move the loads
  // behind it, one dependent round trip at a time
  float M = lane < ns ? L.lse_l : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float e = lane < ns ? exp2f((L.lse_l - M) * kLog2e) : 0.0f;
  float den = e;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float w = __shfl(e, k);
    const f32x4 t0 = a0 + w * P8::lo(L.v[k]), t1 = a1 + w * P8::hi(L.v[k]);
    a0 = k < ns ? t0 : a0;
    a1 = k < ns ? t1 : a1;
  }
  const float inv = ns > 0 ? 1.0f / den : 0.0f;
  lo = a0 * inv;
  hi = a1 * inv;
  lse = ns > 0 ? M + logf(den) : -INFINITY;
}

// Any number of splits: the log-sum-exps are read by lane s % 64 (all loads of
// a pass in flight at once) and reduced across the wave in a fixed order; with
// at most 64 splits each lane keeps its split's weight, and the weights are
// taken from the lanes rather than read again; the partials are read 8 splits
// at a time, all 8 loads issued before the first is used.
template <bool kDev>
__device__ __forceinline__ void row_merge512(const DecodeParams& p, int b, int rr, int t,
                                             int lane, int P0, int S, int chunk, f32x4& lo,
                                             f32x4& hi, float& lse) {
  using P8 = Part8<uint16_t>;
  const int TH = p.T * p.H;
  const float* lse_b = p.part_lse + (size_t)P0 * TH + rr;
  const uint16_t* po_b = static_cast<const uint16_t*>(p.part_o) + ((size_t)P0 * TH + rr) * 512;
  const size_t sstride = (size_t)TH * 512;
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  const int ns = __builtin_amdgcn_readfirstlane(min(S, (n_valid + chunk - 1) / chunk));
  if (ns <= 0) {
    lo = hi = f32x4{0.f, 0.f, 0.f, 0.f};
    lse = -INFINITY;
    return;
  }
  float M = -INFINITY;
  float lse_l = -INFINITY;  // lane's split (ns <= 64)
  for (int c = 0; c < ns; c += 64)
    if (c + lane < ns) {
      lse_l = ld_lse<kDev>(lse_b + (size_t)(c + lane) * TH);
      M = fmaxf(M, lse_l);
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.0f;
  const float e_l = lane < ns ? exp2f((lse_l - M) * kLog2e) : 0.0f;
  if (ns <= 64) {
    den = e_l;
  } else {
    for (int c = 0; c < ns; c += 64)
      if (c + lane < ns) den += exp2f((ld_lse<kDev>(lse_b + (size_t)(c + lane) * TH) - M) * kLog2e);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  const float inv = 1.0f / den;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += 8) {
    // splits past the last one re-read the last one with weight 0, so that
    // every load is unconditional
    float w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float e = ns <= 64
          ? __shfl(e_l, min(s0 + k, ns - 1))
          : exp2f((ld_lse<kDev>(lse_b + (size_t)min(s0 + k, ns - 1) * TH) - M) * kLog2e);
      w[k] = s0 + k < ns ? e : 0.0f;
    }
    typename P8::Raw v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = P8::template load<kDev>(po_b + (size_t)min(s0 + k, ns - 1) * sstride, lane);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a0 += w[k] * P8::lo(v[k]);
      a1 += w[k] * P8::hi(v[k]);
    }
  }
  lo = a0 * inv;
  hi = a1 * inv;
  lse = M + logf(den);
}

// Merges query row `row` (sequence b = row / (T H)) from the S partials
// P0 .. P0+S-1 of its sequence, which cover `chunk` cache rows each, with one
// wave, into o_lat (and lse); lane is the lane index.
template <typename PT, bool kDev = false>
__device__ void merge_row_splits(const DecodeParams& p, long long row, int lane, int P0, int S,
                                 int chunk) {
  using P8 = Part8<PT>;
  const int TH = p.T * p.H;
  const int b = (int)(row / TH);
  const int rr = (int)(row - (long long)b * TH);
  const int t = rr / p.H;
  const PT* part = static_cast<const PT*>(p.part_o);
  const float* lse_b = p.part_lse + (size_t)P0 * TH + rr;
  if constexpr (sizeof(PT) == 2) {
    // bf16 partials come from the MFMA kernel, whose d_c is 512
    f32x4 lo, hi;
    float lse;
    if (S <= 8) {
      Row8Loads L;
      row8_issue<kDev>(p, b, rr, lane, P0, S, L);
      __builtin_amdgcn_sched_barrier(0);
      row8_hold(L);
      row8_finish(p, L, t, lane, S, chunk, lo, hi, lse);
    } else {
      row_merge512<kDev>(p, b, rr, t, lane, P0, S, chunk, lo, hi, lse);
    }
    // streaming stores: o_lat is read by the next kernel (no L2 lines left
    // dirty for the end-of-launch write-back)
    float* out = p.o_lat + (size_t)row * 512;
    __builtin_nontemporal_store(lo, reinterpret_cast<f32x4*>(out + 8 * lane));
    __builtin_nontemporal_store(hi, reinterpret_cast<f32x4*>(out + 8 * lane + 4));
    if (lane == 0 && p.lse != nullptr) p.lse[row] = lse;
    return;
  }
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  // one row per wave: the split count is the same in every lane
  const int ns = __builtin_amdgcn_readfirstlane(min(S, (n_valid + chunk - 1) / chunk));
  float* out = p.o_lat + (size_t)row * p.d_c;
  const PT* po_b = part + ((size_t)P0 * TH + rr) * p.d_c;
  const size_t sstride = (size_t)TH * p.d_c;  // elements between splits of one row

  if (ns <= 0) {
    for (int d = lane; d < p.d_c; d += 64) out[d] = 0.0f;
    if (lane == 0 && p.lse != nullptr) p.lse[row] = -INFINITY;
    return;
  }
  // split s's log-sum-exp is read by lane s % 64 (all loads of a pass in
  // flight at once), then reduced across the wave in a fixed order; with at
  // most 64 splits each lane keeps its split's weight, and the weights below
  // are taken from the lanes rather than read again
  float M = -INFINITY;
  float lse_l = -INFINITY;  // lane's split (ns <= 64)
  for (int c = 0; c < ns; c += 64)
    if (c + lane < ns) {
      lse_l = ld_lse<kDev>(lse_b + (size_t)(c + lane) * TH);
      M = fmaxf(M, lse_l);
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.0f;
  const float e_l = lane < ns ? exp2f((lse_l - M) * kLog2e) : 0.0f;
  if (ns <= 64) {
    den = e_l;
  } else {
    for (int c = 0; c < ns; c += 64)
      if (c + lane < ns) den += exp2f((ld_lse<kDev>(lse_b + (size_t)(c + lane) * TH) - M) * kLog2e);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  const float inv = 1.0f / den;

  if ((p.d_c & 511) == 0) {
    // 512 columns per pass, 8 per lane; the loads of up to 8 splits are all
    // issued before the first is used, so that enough bytes are in flight to
    // stream the partials at memory speed
    for (int d0 = 0; d0 < p.d_c; d0 += 512) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < ns; s0 += 8) {
        // splits past the last one re-read the last one with weight 0, so
        // that every load is unconditional
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = ns <= 64
              ? __shfl(e_l, min(s0 + k, ns - 1))
              : exp2f((ld_lse<kDev>(lse_b + (size_t)min(s0 + k, ns - 1) * TH) - M) * kLog2e);
          w[k] = s0 + k < ns ? e : 0.0f;
        }
        typename P8::Raw v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          v[k] = P8::template load<kDev>(po_b + (size_t)min(s0 + k, ns - 1) * sstride + d0, lane);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          a0 += w[k] * P8::lo(v[k]);
          a1 += w[k] * P8::hi(v[k]);
        }
      }
      *reinterpret_cast<f32x4*>(P8::col_lo(out + d0, lane)) = a0 * inv;
      *reinterpret_cast<f32x4*>(P8::col_hi(out + d0, lane)) = a1 * inv;
    }
  } else if constexpr (sizeof(PT) == 4 && !kDev) {
    const float* pf = reinterpret_cast<const float*>(po_b);
    if ((p.d_c & 3) == 0) {
      for (int d = 4 * lane; d < p.d_c; d += 256) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        int s = 0;
        for (; s + 4 <= ns; s += 4) {  // four splits' loads in flight at a time
          f32x4 v[4];
          float w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[k] = *reinterpret_cast<const f32x4*>(pf + (size_t)(s + k) * sstride + d);
            w[k] = exp2f((lse_b[(size_t)(s + k) * TH] - M) * kLog2e);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) a += w[k] * v[k];
        }
        for (; s < ns; ++s) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(pf + (size_t)s * sstride + d);
          a += exp2f((lse_b[(size_t)s * TH] - M) * kLog2e) * v;
        }
        *reinterpret_cast<f32x4*>(out + d) = a * inv;
      }
    } else {
      for (int d = lane; d < p.d_c; d += 64) {
        float a = 0.0f;
        for (int s = 0; s < ns; ++s)
          a += exp2f((lse_b[(size_t)s * TH] - M) * kLog2e) * pf[(size_t)s * sstride + d];
        out[d] = a * inv;
      }
    }
  }
  if (lane == 0 && p.lse != nullptr) p.lse[row] = M + logf(den);
}


// Merges query row `row` with one wave, the sequence's splits taken from the
// plan: a balanced plan's per-sequence table (written by the decode kernel),
// or the plain plan's split count and length.
template <typename PT>
__device__ void merge_row(const DecodeParams& p, long long row, int lane) {
  const int b = (int)(row / (p.T * p.H));
  if (p.plan != nullptr) {
    const int4 e = *reinterpret_cast<const int4*>(p.plan + 4 * (size_t)b);
    const int S = __builtin_amdgcn_readfirstlane(e.y);
    if (S == 0) {  // no visible row in the sequence: o = 0, lse = -inf
      float* out = p.o_lat + (size_t)row * p.d_c;
      for (int d = lane; d < p.d_c; d += 64) out[d] = 0.0f;
      if (lane == 0 && p.lse != nullptr) p.lse[row] = -INFINITY;
      return;
    }
    merge_row_splits<PT>(p, row, lane, __builtin_amdgcn_readfirstlane(e.x), S,
                         __builtin_amdgcn_readfirstlane(e.z) * 32);
  } else {
    merge_row_splits<PT>(p, row, lane, b * p.num_splits, p.num_splits, p.chunk_rows);
  }
}

}  // namespace mla
