// Split-KV latent-attention decode for the DeepSeek shape on CDNA4 (gfx950).
//
// One workgroup = 64 query rows (64 heads of one new token) x one contiguous
// range of 64-token cache pages of one sequence.  The range is processed in
// 32-token units (half pages, 36 KiB contiguous in HBM) through a software
// pipeline in which three things overlap in every step j:
//   * copies: unit j+3 is copied into LDS with 128-bit direct-to-LDS loads;
//   * scores: unit j+1 is scored, S^T = K . Q^T on MFMA over all 576 columns --
//     the content term (first 512) and the rotary term (last 64) are one dot
//     product ("Attention, Part 2: MQA, GQA and MLA", the absorbed path adds the
//     two terms before scaling) -- followed by the online softmax in the log2
//     domain, which writes P (bf16) for the unit;
//   * values: O += P . V for unit j, V being the first 512 columns of the SAME
//     LDS rows ("How DeepSeek Rewrote the Transformer", section "Absorbed
//     projections", point 3), with O in registers for the whole range.
// One workgroup barrier per step hands P of unit j+1 and the LDS slots over.
// The range's result is written normalised with its log-sum-exp, as the final
// output (one split) or as a partial for the log-sum-exp merge.
//
// Waves (8, two per SIMD) have fixed roles and separate loops that meet at the
// same barriers:
//   score waves 0..3: wave w owns query rows 16w..16w+15 outright: their
//     absorbed queries sit in registers (72 VGPRs, the B operand of
//     v_mfma_f32_16x16x32_bf16), the wave scores all 32 tokens of a unit and
//     runs the softmax of its rows with no other wave involved;
//   value waves 4..7: wave 4+v owns latent columns 128v..128v+127 of O for all
//     64 rows (128 VGPRs, v_mfma_f32_32x32x16_bf16), issues the copies, and
//     reads V with the transposing LDS read (ds_read_b64_tr_b16), 4 tokens x
//     16 columns per 16-lane group.
// A row's reference maximum is only raised when a unit's maximum exceeds it by
// more than 2^8, so the accumulator rescale is skipped on almost every unit;
// probabilities then stay below 2^8, which bf16 and the fp32 sums carry with
// unchanged relative precision.
//
// LDS: a ring of 4 latent slots (32 rows x 1 KiB: the c part of a unit), 3
// rotary slots (32 rows x 128 B: the k^R part), P double-buffered by unit
// parity, and the per-row rescale factors.  16-byte chunk c of latent row t
// sits at chunk position c ^ (t & 15) of its row, and of rotary row t at
// c ^ ((t >> 1) & 7).  With these placements the 128-bit score reads (16 rows
// at one chunk) are free of bank conflicts, and so are the transposing reads
// provided the 4 rows of each 16-lane group lie 4 tokens apart: the values
// MFMA therefore walks each 16-token k-step in the order
// token(lhi, e) = 4*(e & 3) + 2*lhi + (e >> 2) for k-slot 8*lhi + e, and P is
// written in that order (the sum over tokens does not depend on it).  Layouts
// were chosen by measuring SQ_LDS_BANK_CONFLICT on gfx950.
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DC = 512;
constexpr int DR = 64;
constexpr int W = DC + DR;
constexpr int BS = 64;                      // tokens per page
constexpr int UNIT = 32;                    // tokens per pipeline step
constexpr int ROWS = 64;                    // query rows per workgroup
constexpr int NT = 512;                     // threads per workgroup
constexpr int ROW_BYTES = W * 2;            // 1152
constexpr int TILE_BYTES = BS * ROW_BYTES;  // 73728 per page in HBM
constexpr int LAT_SLOTS = 4;
constexpr int ROT_SLOTS = 3;
constexpr int P_LD = 40;                    // bf16 per row of a P tile (32 + pad)
constexpr int QSTEPS = W / 32;              // 18 k-steps of 32 columns
constexpr int COPIES = 9;                   // direct-to-LDS copies per value wave per unit
constexpr float kRescaleSlack = 8.0f;       // log2 units

struct __align__(16) Smem {
  uint8_t lat[LAT_SLOTS][UNIT * 1024];
  uint8_t rot[ROT_SLOTS][UNIT * 128];
  uint16_t p[2][ROWS * P_LD];  // [unit parity]
  float alpha[2][ROWS];
  float lrow[ROWS];
  float mrow[ROWS];
  int flag[2][4];  // [unit parity][score wave]: some row of the wave raised its max
};

__device__ __forceinline__ int lat_sw(int t) { return t & 15; }
__device__ __forceinline__ int rot_sw(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

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
__device__ __forceinline__ void copy16_to_lds(const uint8_t* gbase, uint32_t voff,
                                              uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(gbase)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N), expcnt and lgkmcnt unconstrained.  gfx9 encoding:
  // vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(const DecodeParams p) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave index as a scalar: the role branches below are uniform (scalar)
  // branches, so a wave never steps through the other role's barriers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  const int G = (p.T * p.H) / ROWS;
  const int S = p.num_splits;
  int idx = blockIdx.x;
  const int g = idx % G;
  idx /= G;
  const int s = idx % S;
  const int b = idx / S;

  const int TH = p.T * p.H;
  const int rb = g * ROWS;  // first query row (t*H + h) of the group
  const int t = rb / p.H;
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  const int pages = (n_valid + BS - 1) / BS;
  const int p0 = s * p.chunk_pages;
  const int p1 = min(p0 + p.chunk_pages, pages);
  const bool direct = (S == 1);

  if (p0 >= p1) {
    if (direct) {  // no visible row: o = 0, lse = -inf
      float* dst = p.o_lat + ((size_t)b * TH + rb) * DC;
      for (int i = tid; i < ROWS * DC; i += NT) dst[i] = 0.0f;
      if (p.lse != nullptr && tid < ROWS) p.lse[(size_t)b * TH + rb + tid] = -INFINITY;
    }
    return;
  }
  // units of this range: 32-token halves of pages p0.., up to the last visible token
  const int tok0 = p0 * BS;
  const int U = min(2 * (p1 - p0), (n_valid - tok0 + UNIT - 1) / UNIT);
  auto unit_valid = [&](int u) { return min(UNIT, n_valid - tok0 - u * UNIT); };

  if (wave < 4) {
    // =============================== score waves ===============================
    const int r16 = lane & 15;  // row within the wave's 16, and token within a 16-token tile
    const int g4 = lane >> 4;   // 8-column group of a k-step; 4-token group of an output
    const int srow = 16 * wave + r16;

    bf16x8 qf[QSTEPS];  // B operand: Q[srow][32kk + 8*g4 .. +7]
    {
      const uint16_t* q = static_cast<const uint16_t*>(p.q_abs) +
                          ((size_t)b * TH + rb + srow) * W + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < QSTEPS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(q + 32 * kk);
    }
    // A operand: K[token r16 (+16 ti)][32kk + 8*g4 .. +7]: latent chunk
    // c = 4kk + g4, stored at position c ^ lat_sw(r16); rotary chunk
    // c = 4(kk-16) + g4 at position c ^ rot_sw(r16).
    const int tsw = lat_sw(r16);
    int loff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) loff[j] = r16 * 1024 + (((4 * j + g4) ^ tsw) << 4);
    int roff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) roff[j] = r16 * 128 + (((4 * j + g4) ^ rot_sw(r16)) << 4);

    float m_run = -INFINITY;  // reference max (log2 units) of row srow
    float l_run = 0.0f;       // running sum in that reference

    auto score_softmax = [&](int u) {
      const uint8_t* lat = sm.lat[u & 3];
      const uint8_t* rot = sm.rot[u % 3];
      f32x4 acc[2];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ti][i] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {  // content term: latent chunks 0..63
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
          const bf16x8 k = *reinterpret_cast<const bf16x8*>(
              lat + loff[kk & 3] + ti * 16 * 1024 + ((4 * kk & ~15) << 4));
          acc[ti] = mfma16(k, qf[kk], acc[ti]);
        }
      }
#pragma unroll
      for (int kk = 16; kk < QSTEPS; ++kk) {  // rotary term
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
          const bf16x8 k =
              *reinterpret_cast<const bf16x8*>(rot + roff[kk - 16] + ti * 16 * 128);
          acc[ti] = mfma16(k, qf[kk], acc[ti]);
        }
      }
      // lane holds row srow, tokens 16ti + 4*g4 + i of the unit
      const int valid = unit_valid(u);
      float mx = -INFINITY;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = 16 * ti + 4 * g4 + i;
          const float v = (tk < valid) ? acc[ti][i] * p.scale_log2 : -INFINITY;
          acc[ti][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = xor32_max(xor16_max(mx));
      const bool raise = mx > m_run + kRescaleSlack;  // always on the first unit
      const float m_new = raise ? mx : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      float sum = 0.0f;
      // token 16ti + 4*g4 + i goes to k-slot 16ti + 4i + g4 (see the LDS notes)
      uint16_t* prow = sm.p[u & 1] + srow * P_LD + g4;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(acc[ti][i] - m_new);
          sum += e;
          prow[16 * ti + 4 * i] = f32_to_bf16(e);
        }
      }
      sum = xor32_sum(xor16_sum(sum));
      l_run = l_run * alpha + sum;
      if (lane < 16) sm.alpha[u & 1][srow] = alpha;
      const bool any_raise = __any(raise);
      if (lane == 0) sm.flag[u & 1][wave] = any_raise ? 1 : 0;
    };

    // prologue: unit 0 (copies issued by the value waves)
    lds_barrier();                         // B0: unit 0 landed
    if (unit_valid(0) < UNIT) lds_barrier();
    score_softmax(0);
    lds_barrier();                         // E
    if (U > 1 && unit_valid(1) < UNIT) lds_barrier();
    for (int j = 0; j < U; ++j) {
      if (j + 1 < U) score_softmax(j + 1);
      lds_barrier();                       // E
      if (j + 2 < U && unit_valid(j + 2) < UNIT) lds_barrier();
    }

    if (lane < 16) {
      sm.lrow[srow] = l_run;
      sm.mrow[srow] = m_run;
    }
    lds_barrier();                         // F
    if (tid < ROWS) {
      const float v = (sm.mrow[tid] + log2f(sm.lrow[tid])) * kLn2;
      if (direct) {
        if (p.lse != nullptr) p.lse[(size_t)b * TH + rb + tid] = v;
      } else {
        p.part_lse[((size_t)b * S + s) * TH + rb + tid] = v;
      }
    }
  } else {
    // =============================== value waves ===============================
    const int v = wave - 4;
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    // Page ids are read through the constant address space: the index is
    // uniform, so this is a scalar load (lgkmcnt), and the wait for it does not
    // drain the copies in flight (vmcnt).
    const int32_t __attribute__((address_space(4)))* ctable =
        (const int32_t __attribute__((address_space(4)))*)table;
    const uint8_t* pool = static_cast<const uint8_t*>(p.pool);

    // Copies: value wave v fills latent rows t = v + 4i (i < 8) and the rotary
    // rows 8v..8v+7 of a unit; lane l fetches the chunk that belongs at LDS
    // chunk position l of its row (latent) or slot l of its 8-row block (rotary).
    int cl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cl[i] = (lane ^ lat_sw(v + 4 * i)) << 4;
    const int rt_row = 8 * v + (lane >> 3);
    const int cr = rt_row * ROW_BYTES + 1024 + (((lane & 7) ^ rot_sw(rt_row)) << 4);
    // Page-table entry of unit u (clamped to the range's last unit, so the
    // read stays inside the range's pages).  Inside the loop it is read one
    // step ahead, before the barrier whose wait covers the scalar load, and
    // range-checked only where the copies use it.
    auto page_raw = [&](int u) { return ctable[(tok0 + min(u, U - 1) * UNIT) / BS]; };
    const uint32_t lat_base = (uint32_t)(uintptr_t)&sm.lat[0][0];
    const uint32_t rot_base = (uint32_t)(uintptr_t)&sm.rot[0][0];
    auto issue = [&](int u, int raw) {
      const int blk = clamp_block(raw, p.num_blocks);
      const uint8_t* src =
          pool + (size_t)blk * TILE_BYTES + ((tok0 + u * UNIT) % BS) * ROW_BYTES;
      const uint32_t lat = lat_base + (u & 3) * (UNIT * 1024);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = v + 4 * i;
        copy16_to_lds(src + row * ROW_BYTES, (uint32_t)cl[i & 3], lat + row * 1024);
      }
      copy16_to_lds(src, (uint32_t)cr, rot_base + (u % 3) * (UNIT * 128) + v * 1024);
    };
    // Rows past the visible length of a partial unit are zeroed once it has
    // landed: stale contents (possibly NaN) must not reach P.V.
    auto zero_tail = [&](int u) {
      const int valid = unit_valid(u);
      const u32x4 z = {0u, 0u, 0u, 0u};
      u32x4* dl = reinterpret_cast<u32x4*>(sm.lat[u & 3]);
      for (int q = valid * 64 + tid - 256; q < UNIT * 64; q += 256) dl[q] = z;
      u32x4* dr = reinterpret_cast<u32x4*>(sm.rot[u % 3]);
      for (int q = valid * 8 + tid - 256; q < UNIT * 8; q += 256) dr[q] = z;
    };

    // Transposing-read offsets of this lane: in 16-lane group gq, lane i points
    // at token 4*(i >> 2) + 2*lhi + sel (+ 16*ks), columns 128v + 32dt + 16*gq
    // + 4*(i & 3); result lane i holds column .. + i for the 4 tokens.
    const int i16 = lane & 15;
    const int gq = (lane >> 4) & 1;
    int voff[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int sel = 0; sel < 2; ++sel) {
        const int tk = 4 * (i16 >> 2) + 2 * lhi + sel;  // + 16*ks (multiple of 16)
        const int col = 128 * v + 32 * dt + 16 * gq + 4 * (i16 & 3);
        const int chunk = col >> 3;
        voff[dt][sel] = tk * 1024 + ((chunk ^ lat_sw(tk)) << 4) + ((col & 4) << 1);
      }
    const int poff = l32 * P_LD + 8 * lhi;  // bf16 elements

    f32x16 o[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rt][dt][r] = 0.0f;

    // prologue: copies of units 0..2, wait for unit 0, then unit 1
    issue(0, page_raw(0));
    if (U > 1) issue(1, page_raw(1));
    if (U > 2) issue(2, page_raw(2));
    int raw_next = page_raw(3);
    if (U > 2) wait_vmcnt<2 * COPIES>(); else if (U > 1) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
    lds_barrier();                         // B0
    if (unit_valid(0) < UNIT) {
      zero_tail(0);
      lds_barrier();
    }
    if (U > 1) {
      if (U > 2) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
    }
    lds_barrier();                         // E
    if (U > 1 && unit_valid(1) < UNIT) {
      zero_tail(1);
      lds_barrier();
    }

    for (int j = 0; j < U; ++j) {
      const bool ahead = j + 3 < U;
      if (ahead) issue(j + 3, raw_next);
      const uint8_t* lat = sm.lat[j & 3];
      const uint16_t* pp = sm.p[j & 1];
      const int4 fl = *reinterpret_cast<const int4*>(sm.flag[j & 1]);
      if (fl.x | fl.y | fl.z | fl.w) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 al =
                *reinterpret_cast<const float4*>(&sm.alpha[j & 1][32 * rt + 8 * r4 + 4 * lhi]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              o[rt][dt][4 * r4 + 0] *= al.x;
              o[rt][dt][4 * r4 + 1] *= al.y;
              o[rt][dt][4 * r4 + 2] *= al.z;
              o[rt][dt][4 * r4 + 3] *= al.w;
            }
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf0 = *reinterpret_cast<const bf16x8*>(pp + poff + 16 * ks);
        const bf16x8 pf1 = *reinterpret_cast<const bf16x8*>(pp + 32 * P_LD + poff + 16 * ks);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 v0 = lds_tr16(lat + voff[dt][0] + 16 * ks * 1024);
          const s16x4 v1 = lds_tr16(lat + voff[dt][1] + 16 * ks * 1024);
          const short vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
          o[0][dt] = mfma32(pf0, vf, o[0][dt]);
          o[1][dt] = mfma32(pf1, vf, o[1][dt]);
        }
      }
      raw_next = page_raw(j + 4);
      if (j + 2 < U) {
        if (ahead) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
      }
      lds_barrier();                       // E
      if (j + 2 < U && unit_valid(j + 2) < UNIT) {
        zero_tail(j + 2);
        lds_barrier();
      }
    }

    lds_barrier();                         // F
    float* dst = direct ? p.o_lat + ((size_t)b * TH + rb) * DC
                        : p.part_o + (((size_t)b * S + s) * TH + rb) * DC;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + 8 * (r >> 2) + 4 * lhi + (r & 3);
        const float inv = 1.0f / sm.lrow[row];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          dst[(size_t)row * DC + 128 * v + 32 * dt + l32] = o[rt][dt][r] * inv;
      }
    }
  }
}

}  // namespace

bool decode_mfma_supported(int dtype, int d_c, int d_r, int block_size, int T, int H) {
  return dtype == 1 && d_c == DC && d_r == DR && block_size == BS && ((T * H) % ROWS) == 0;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  const int G = (p.T * p.H) / ROWS;
  const long long grid = (long long)p.B * p.num_splits * G;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
