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
#include <type_traits>

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
constexpr int QSTEPS = W / 32;              // 18 k-steps of 32 columns (score MFMA)
constexpr int COPIES = 18;                  // direct-to-LDS copies per copy wave per unit
constexpr float kRescaleSlack = 8.0f;       // log2 units

constexpr int S_LD = 36;                    // floats per row of the score tile (32 + pad)
constexpr int A_SPLIT = 9;                  // score k-steps of unit j+2 run between M(j) and E(j)

struct __align__(16) Smem {
  uint8_t lat[LAT_SLOTS][UNIT * 1024];
  uint8_t rot[ROT_SLOTS][UNIT * 128];
  float s[ROWS * S_LD];        // raw scores of one unit, [row][token]
  uint16_t p[ROWS * P_LD];     // probabilities of one unit (bf16), [row][k-slot]
  float alpha[ROWS];           // per-row rescale factor of that unit
  float lrow[ROWS];
  int flag[2];                 // [copy wave]: some row of its 32 raised its max
};

__device__ __forceinline__ int lat_sw(int t) { return t & 15; }
__device__ __forceinline__ int rot_sw(int t) { return (t >> 1) & 7; }

// Token (within a 16-token k-step of P.V) held at P k-slot m, 0 <= m < 16.
// The value waves' transposing reads take the 4 tokens of a slot quad 4
// apart (which keeps those reads free of bank conflicts), so slot 8h + e
// holds token 4(e & 3) + 2h + (e >> 2).
__device__ __forceinline__ int tok_of(int m) {
  return 4 * (m & 3) + 2 * (m >> 3) + ((m >> 2) & 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(uint16_t)))) uint16_t u16x8;

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
  // Workgroup i is dispatched to XCD i % 8, and each XCD has its own L2.  XCD
  // x gets a contiguous block of (sequence, split) pairs, and all G 64-row
  // groups of each: the pages of a pair and the absorbed queries of a
  // sequence then come from HBM once per XCD and from L2 for the other
  // workgroups that read them.  Ids past the last full set of 8G keep the
  // plain order.
  constexpr int XCDS = 8;
  const int i = blockIdx.x;
  const int full = (int)gridDim.x - (int)gridDim.x % (XCDS * G);
  int g, pair;
  if (i < full) {
    const int r = i / XCDS;
    g = r % G;
    pair = (i % XCDS) * (full / G / XCDS) + r / G;
  } else {
    g = i % G;
    pair = i / G;
  }
  const int s = pair % S;
  const int b = pair / S;

  const int TH = p.T * p.H;
  const int rb = g * ROWS;  // first query row (t*H + h) of the group
  const int t = rb / p.H;
  const int n_valid = visible_rows(p.seq_lens[b], p.T, t, p.causal, p.cap);
  // this range: cache rows tok0 .. tok_end-1 (tok0 is a multiple of UNIT)
  const int tok0 = s * p.chunk_rows;
  const int tok_end = min(tok0 + p.chunk_rows, n_valid);
  const bool direct = (S == 1);

  if (tok0 >= tok_end) {
    if (direct) {  // no visible row: o = 0, lse = -inf
      float* dst = p.o_lat + ((size_t)b * TH + rb) * DC;
      for (int i = tid; i < ROWS * DC; i += NT) dst[i] = 0.0f;
      if (p.lse != nullptr && tid < ROWS) p.lse[(size_t)b * TH + rb + tid] = -INFINITY;
    }
    return;
  }
  // its 32-row units; only the last unit of the sequence can be partial
  const int U = (tok_end - tok0 + UNIT - 1) / UNIT;
  auto unit_valid = [&](int u) { return min(UNIT, tok_end - tok0 - u * UNIT); };

  // Two barriers per unit.  Barrier schedule, the same for every wave: B0,
  // then M(j) and E(j) for j = -1 .. U-1, then F.
  //   E(j-1) .. M(j): score waves finish the scores of unit j+1 and store them
  //     raw (fp32) in sm.s; value waves read P(j) and V(j) into registers and
  //     start O += P(j) V(j); copy waves issue the copies of unit j+3 and
  //     wait for unit j+2.
  //   M(j) .. E(j): copy waves turn sm.s into P(j+1) (softmax, 32 rows each),
  //     on the same SIMDs where the score waves start on unit j+2, so that
  //     VALU and MFMA work overlap there; value waves finish O += P(j) V(j).
  // Each of sm.s, sm.p and sm.alpha is written in one phase and read in the
  // other, so one buffer of each suffices.
  if (wave < 2) {
    // =============================== score waves ===============================
    // Wave w owns query rows 32w .. 32w+31 as two 16-row tiles rt.  S^T = K . Q^T
    // on v_mfma_f32_16x16x32_bf16 over all 576 columns, for two 16-token tiles
    // ti: A = 16 tokens x 32 columns of K (lane l: token l & 15, columns
    // 8(l >> 4) .. +7), B = the same columns of Q^T for one row tile, held in
    // registers for the whole range (2 x 18 k-steps, 144 VGPRs).  Each K
    // fragment feeds both row tiles; the four (rt, ti) accumulators are four
    // independent MFMA chains.  A lane's results are query row 32w + 16rt +
    // (l & 15), tokens 16ti + 4(l >> 4) .. +3: one 16-byte store each.
    const int n16 = lane & 15;
    const int g4 = lane >> 4;
    bf16x8 qf[2][QSTEPS];  // Q[32w + 16rt + n16][32kk + 8*g4 .. +7]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint16_t* q = static_cast<const uint16_t*>(p.q_abs) +
                          ((size_t)b * TH + rb + 32 * wave + 16 * rt + n16) * W + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < QSTEPS; ++kk)
        qf[rt][kk] = *reinterpret_cast<const bf16x8*>(q + 32 * kk);
    }
    // K fragment offsets: latent chunk c = 4kk + g4 of token n16 sits at chunk
    // position c ^ lat_sw(n16) (only the low 4 bits of c take part), rotary
    // chunk c = 4(kk - 16) + g4 at c ^ rot_sw(n16); token tile ti adds 16 KiB
    // (latent) or 2 KiB (rotary).
    int loff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) loff[j] = n16 * 1024 + (((4 * j + g4) ^ lat_sw(n16)) << 4);
    int roff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) roff[j] = n16 * 128 + (((4 * j + g4) ^ rot_sw(n16)) << 4);

    f32x4 acc[2][2];  // [rt][ti], carried from the first k-steps to the rest
    auto kfrag = [&](int u, int kk, int ti) {
      const uint8_t* a = kk < 16 ? sm.lat[u & 3] + loff[kk & 3] + ti * 16 * 1024 + ((kk >> 2) << 8)
                                 : sm.rot[u % 3] + roff[kk - 16] + ti * 16 * 128;
      return *reinterpret_cast<const bf16x8*>(a);
    };
    // k-steps [KB, KE) of unit u, fragments read KDEPTH k-steps ahead
    auto steps = [&](int u, auto kb_tag, auto ke_tag) {
      constexpr int KB = decltype(kb_tag)::value, KE = decltype(ke_tag)::value;
      constexpr int KDEPTH = 4;
      bf16x8 kf[KDEPTH][2];
#pragma unroll
      for (int kk = KB; kk < KB + KDEPTH && kk < KE; ++kk) {
        kf[kk % KDEPTH][0] = kfrag(u, kk, 0);
        kf[kk % KDEPTH][1] = kfrag(u, kk, 1);
      }
#pragma unroll
      for (int kk = KB; kk < KE; ++kk) {
        const bf16x8 k0 = kf[kk % KDEPTH][0];
        const bf16x8 k1 = kf[kk % KDEPTH][1];
        if (kk + KDEPTH < KE) {
          kf[kk % KDEPTH][0] = kfrag(u, kk + KDEPTH, 0);
          kf[kk % KDEPTH][1] = kfrag(u, kk + KDEPTH, 1);
        }
        acc[0][0] = mfma16(k0, qf[0][kk], acc[0][0]);
        acc[1][0] = mfma16(k0, qf[1][kk], acc[1][0]);
        acc[0][1] = mfma16(k1, qf[0][kk], acc[0][1]);
        acc[1][1] = mfma16(k1, qf[1][kk], acc[1][1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using K0 = std::integral_constant<int, 0>;
    using KA = std::integral_constant<int, A_SPLIT>;
    using KN = std::integral_constant<int, QSTEPS>;
    auto first_steps = [&](int u) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rt][ti][i] = 0.0f;
      steps(u, K0{}, KA{});
    };
    auto finish_and_store = [&](int u) {
      steps(u, KA{}, KN{});
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          *reinterpret_cast<f32x4*>(&sm.s[(32 * wave + 16 * rt + n16) * S_LD + 16 * ti + 4 * g4]) =
              acc[rt][ti];
    };

    lds_barrier();                         // B0: unit 0 landed
    first_steps(0);
    for (int j = -1; j < U; ++j) {
      if (j + 1 < U) finish_and_store(j + 1);
      lds_barrier();                       // M(j)
      if (j + 2 < U) first_steps(j + 2);
      lds_barrier();                       // E(j)
    }
    lds_barrier();                         // F
  } else if (wave >= 4 && wave < 6) {
    // ============================ copy / softmax waves ===========================
    // Copy wave c fills latent rows t = c + 2i (i < 16) and the rotary rows
    // 16c .. 16c+15 of a unit: 18 direct-to-LDS copies of 1 KiB.  Lane l
    // fetches the chunk that belongs at LDS chunk position l of its row
    // (latent), or at slot l & 7 of row 8q + (l >> 3) (rotary).  It also runs
    // the softmax of query rows 32c .. 32c+31.
    const int c = wave - 4;
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    // Page ids are read through the constant address space: the index is
    // uniform, so this is a scalar load (lgkmcnt), and the wait for it does not
    // drain the copies in flight (vmcnt).
    const int32_t __attribute__((address_space(4)))* ctable =
        (const int32_t __attribute__((address_space(4)))*)table;
    const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
    int cl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cl[i] = (lane ^ lat_sw(c + 2 * i)) << 4;
    int cr[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 8 * (2 * c + e) + (lane >> 3);
      cr[e] = row * ROW_BYTES + 1024 + (((lane & 7) ^ rot_sw(row)) << 4);
    }
    // Page-table entry of unit u (clamped to the range's last unit, so the
    // read stays inside the range's pages); read one step ahead in the loop.
    auto page_raw = [&](int u) { return ctable[(tok0 + min(u, U - 1) * UNIT) / BS]; };
    const uint32_t lat_base = (uint32_t)(uintptr_t)&sm.lat[0][0];
    const uint32_t rot_base = (uint32_t)(uintptr_t)&sm.rot[0][0];
    auto issue = [&](int u, int raw) {
      const int blk = clamp_block(raw, p.num_blocks);
      const uint8_t* src = pool + (size_t)blk * TILE_BYTES + ((tok0 + u * UNIT) % BS) * ROW_BYTES;
      const uint32_t lat = lat_base + (u & 3) * (UNIT * 1024);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = c + 2 * i;
        copy16_to_lds(src + row * ROW_BYTES, (uint32_t)cl[i & 7], lat + row * 1024);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
        copy16_to_lds(src, (uint32_t)cr[e],
                      rot_base + (u % 3) * (UNIT * 128) + (2 * c + e) * 1024);
    };
    // Rows past the visible length of the range's last unit are zeroed once
    // it has landed and before V is read from it: stale contents (possibly
    // NaN) must not reach P.V.  The score waves may read those rows
    // meanwhile; their scores are masked out.
    auto zero_tail = [&](int u) {
      const int valid = unit_valid(u);
      if (valid >= UNIT) return;
      const int zt = lane + 64 * c;
      const u32x4 z = {0u, 0u, 0u, 0u};
      u32x4* dl = reinterpret_cast<u32x4*>(sm.lat[u & 3]);
      for (int q = valid * 64 + zt; q < UNIT * 64; q += 128) dl[q] = z;
      u32x4* dr = reinterpret_cast<u32x4*>(sm.rot[u % 3]);
      for (int q = valid * 8 + zt; q < UNIT * 8; q += 128) dr[q] = z;
    };

    // softmax lanes: query row 32c + (l & 31), P k-slots 8h + e (+16ks),
    // h = l >> 5, e < 8, ks < 2: 16 scores per lane, the other 16 of the row
    // in lane l ^ 32
    const int srow = 32 * c + l32;
    float m_run = -INFINITY;  // reference max (log2 units) of row srow
    float l_run = 0.0f;       // running sum in that reference
    const float c_log2 = p.scale_log2;
    auto softmax = [&](int u) {
      // Scale and subtract stay separate operations, so the maximal score
      // gives exactly exp2(0) = 1.
#pragma clang fp contract(off)
      float x[2][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // slot 8h + e of k-step ks holds token 16ks + tok_of(8h + e): token
        // pairs 16ks + 2h + 4q, +1 give slots e = q and e = q + 4
        const float* srd = &sm.s[srow * S_LD + 16 * ks + 2 * lhi];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float2 pr = *reinterpret_cast<const float2*>(srd + 4 * q);
          x[ks][q] = pr.x * c_log2;
          x[ks][q + 4] = pr.y * c_log2;
        }
      }
      const int valid = unit_valid(u);
      if (valid < UNIT) {  // only the range's last unit can be partial
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (16 * ks + tok_of(8 * lhi + e) >= valid) x[ks][e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[ks][e]);
      mx = xor32_max(mx);
      const bool raise = mx > m_run + kRescaleSlack;  // always on the first unit
      const float m_new = raise ? mx : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      float sum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ex = __builtin_amdgcn_exp2f(x[ks][e] - m_new);
          sum += ex;
          pb[e] = f32_to_bf16(ex);
        }
        *reinterpret_cast<u16x8*>(&sm.p[srow * P_LD + 16 * ks + 8 * lhi]) = pb;
      }
      sum = xor32_sum(sum);
      l_run = l_run * alpha + sum;
      if (lhi == 0) sm.alpha[srow] = alpha;
      const bool any_raise = __any(raise);
      if (lane == 0) sm.flag[c] = any_raise ? 1 : 0;
    };

    issue(0, page_raw(0));
    if (U > 1) issue(1, page_raw(1));
    if (U > 2) issue(2, page_raw(2));
    int raw_next = page_raw(3);
    if (U > 2) wait_vmcnt<2 * COPIES>(); else if (U > 1) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
    lds_barrier();                         // B0: unit 0 landed
    zero_tail(0);
    for (int j = -1; j < U; ++j) {
      if (j >= 0 && j + 3 < U) {
        issue(j + 3, raw_next);
        raw_next = page_raw(j + 4);
      }
      if (j + 2 < U) {  // unit j+2 landed: only unit j+3 may still be in flight
        if (j + 3 < U) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
      }
      lds_barrier();                       // M(j)
      if (j + 1 < U) softmax(j + 1);
      if (j + 2 < U) zero_tail(j + 2);
      lds_barrier();                       // E(j)
    }
    if (lhi == 0) {
      sm.lrow[srow] = l_run;
      const float lse = (m_run + log2f(l_run)) * kLn2;
      if (direct) {
        if (p.lse != nullptr) p.lse[(size_t)b * TH + rb + srow] = lse;
      } else {
        p.part_lse[((size_t)b * S + s) * TH + rb + srow] = lse;
      }
    }
    lds_barrier();                         // F
  } else {
    // =============================== value waves ===============================
    // Value wave v owns latent columns 128v .. 128v+127 of O for all 64 rows.
    const int v = (wave & 1) + 2 * (wave >> 2);
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
        const int tkv = 4 * (i16 >> 2) + 2 * lhi + sel;  // + 16*ks (multiple of 16)
        const int col = 128 * v + 32 * dt + 16 * gq + 4 * (i16 & 3);
        const int chunk = col >> 3;
        voff[dt][sel] = tkv * 1024 + ((chunk ^ lat_sw(tkv)) << 4) + ((col & 4) << 1);
      }
    const int poff = l32 * P_LD + 8 * lhi;  // bf16 elements

    f32x16 o[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rt][dt][r] = 0.0f;

    bf16x8 pf[2][2], vf[2][4];
    // P(j), the rescale flags and V(j) into registers, rescale O if a row of
    // unit j raised its reference max, and the MFMAs of k-step 0.
    auto pv_first = [&](int j) {
      const uint8_t* lat = sm.lat[j & 3];
      const int2 fl = *reinterpret_cast<const int2*>(sm.flag);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pf[ks][0] = *reinterpret_cast<const bf16x8*>(sm.p + poff + 16 * ks);
        pf[ks][1] = *reinterpret_cast<const bf16x8*>(sm.p + 32 * P_LD + poff + 16 * ks);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 v0 = lds_tr16(lat + voff[dt][0] + 16 * ks * 1024);
          const s16x4 v1 = lds_tr16(lat + voff[dt][1] + 16 * ks * 1024);
          const short vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          vf[ks][dt] = __builtin_bit_cast(bf16x8, vv);
        }
      }
      if (fl.x | fl.y) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[32 * rt + 8 * r4 + 4 * lhi]);
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
      for (int dt = 0; dt < 4; ++dt) {
        o[0][dt] = mfma32(pf[0][0], vf[0][dt], o[0][dt]);
        o[1][dt] = mfma32(pf[0][1], vf[0][dt], o[1][dt]);
      }
    };
    auto pv_second = [&]() {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        o[0][dt] = mfma32(pf[1][0], vf[1][dt], o[0][dt]);
        o[1][dt] = mfma32(pf[1][1], vf[1][dt], o[1][dt]);
      }
    };

    lds_barrier();                         // B0
    for (int j = -1; j < U; ++j) {
      if (j >= 0) pv_first(j);
      lds_barrier();                       // M(j)
      if (j >= 0) pv_second();
      lds_barrier();                       // E(j)
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
