// Split-KV latent-attention decode for the DeepSeek shape on CDNA4 (gfx950).
//
// One workgroup = 64 query rows (64 heads of one new token) x one contiguous
// range of cache rows of one sequence.  The range is processed in 32-token
// units (half pages, 36 KiB contiguous in HBM) through a software pipeline
// with one workgroup barrier per step; in step j:
//   * copies: unit j+4 is issued into LDS with 128-bit direct-to-LDS loads
//     (latent columns only) and unit j+3 is waited for;
//   * scores: unit j+2 is scored, S^T = K . Q^T on MFMA over all 576 columns
//     -- the content term (first 512) and the rotary term (last 64) are one
//     dot product ("Attention, Part 2: MQA, GQA and MLA", the absorbed path
//     adds the two terms before scaling); the raw scores go to LDS;
//   * softmax: unit j+1, online, in the log2 domain, writing P (bf16) and the
//     rows' rescale factors;
//   * values: O += P . V for unit j, V being the first 512 columns of the SAME
//     LDS rows ("How DeepSeek Rewrote the Transformer", section "Absorbed
//     projections", point 3), with O in registers for the whole range.
// The range's result is written normalised with its log-sum-exp, as the final
// output (one split) or as a partial for the log-sum-exp merge.
//
// Waves (8; wave w and wave w + 4 share a SIMD) have fixed roles and separate
// loops that meet at the same barriers:
//   score waves 0, 1: wave w holds the absorbed queries of rows 32w..32w+31 in
//     registers (144 VGPRs, the B operand of v_mfma_f32_16x16x32_bf16), reads
//     K fragments from LDS, and reads the unit's rotary key columns straight
//     from memory into registers one unit ahead;
//   copy waves 4, 5 (on the score waves' SIMDs): the softmax of rows 32..47
//     and 48..63, then the copies;
//   value waves 2, 3, 6, 7: wave v owns latent columns 128v..128v+127 of O for
//     all 64 rows (128 VGPRs, v_mfma_f32_32x32x16_bf16) and reads V with the
//     transposing LDS read (ds_read_b64_tr_b16); waves 2 and 3 also run the
//     softmax of rows 0..15 and 16..31, before their P.V.
// Each SIMD thus carries MFMAs (score or P.V) and the VALU work of one 16-row
// softmax: with one wave's VALU work slowed by another's MFMAs on the same
// SIMD, the four SIMDs then take about the same time per unit.
// A row's reference maximum is only raised when a unit's maximum exceeds it by
// more than 2^8, so the accumulator rescale is skipped on almost every unit;
// probabilities then stay below 2^8, which bf16 and the fp32 sums carry with
// unchanged relative precision.
//
// LDS: a ring of 4 latent slots (32 rows x 1 KiB: the c part of a unit), raw
// scores and P double-buffered by unit parity, and the per-row rescale
// factors.  16-byte chunk c of latent row t sits at chunk position c ^ (t & 15)
// of its row.  With this placement the 128-bit score reads (16 rows at one
// chunk) are free of bank conflicts, and so are the transposing reads provided
// the 4 rows of each 16-lane group lie 4 tokens apart: the values MFMA
// therefore walks each 16-token k-step in the order
// token(lhi, e) = 4*(e & 3) + 2*lhi + (e >> 2) for k-slot 8*lhi + e, and P is
// written in that order (the sum over tokens does not depend on it).  Layouts
// were chosen by measuring SQ_LDS_BANK_CONFLICT on gfx950.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "merge.h"

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
constexpr int P_LD = 40;                    // bf16 per row of a P tile (32 + pad)
constexpr int S_LD = 36;                    // floats per row of a score tile (32 + pad)
constexpr int QSTEPS = W / 32;              // 18 k-steps of 32 columns (score MFMA)
constexpr int LSTEPS = DC / 32;             // 16 of them over the latent columns
constexpr int COPIES = 16;                  // direct-to-LDS copies per copy wave per unit
constexpr float kRescaleSlack = 8.0f;       // log2 units

struct __align__(16) Smem {
  uint8_t lat[LAT_SLOTS][UNIT * 1024];  // latent columns of 4 units (32 rows x 1 KiB)
  float s[2][ROWS * S_LD];     // raw scores by unit parity, [row][token]
  uint16_t p[2][ROWS * P_LD];  // probabilities (bf16) by unit parity, [row][k-slot]
  float alpha[2][ROWS];        // per-row rescale factor, by unit parity
  float lrow[ROWS];            // 1 / (row sum), after the last unit
  int flag[2][4];              // [unit parity][row group]: some row of its 16 raised its max
  int item[8];                 // this workgroup's work item under a balanced plan
};

__device__ __forceinline__ int lat_sw(int t) { return t & 15; }

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

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}


// Online softmax of one 16-row group of a unit, in the log2 domain: raw
// scores sm.s -> probabilities sm.p (bf16, in the k-slot order of P.V), the
// rows' rescale factors and the group's rescale flag.  Lane l takes row
// 16 grp + (l & 15) and P k-slots 8 g8 .. +7 (g8 = l >> 4: k-step g8 >> 1,
// half g8 & 1); the other 24 scores of the row are in lanes l ^ 16, l ^ 32,
// l ^ 48.  m_run is the row's reference maximum; l_lane is this lane's share
// of the row sum in that reference (the four shares are added once, after
// the last unit).
//
// The reference is raised only when a score exceeds it by more than the
// slack, so on almost every unit no score does, and neither the row maximum
// nor any exchange between lanes is needed: the test is one wave-wide vote.
__device__ __forceinline__ void softmax_unit(Smem& sm, int u, int valid, int grp, int lane,
                                             float c_log2, float& m_run, float& l_lane) {
  // Scale and subtract stay separate operations, so the maximal score gives
  // exactly exp2(0) = 1.
#pragma clang fp contract(off)
  const int i16 = lane & 15;
  const int g8 = lane >> 4;
  const int srow = 16 * grp + i16;
  // k-slot 8h + e of k-step ks holds token 16ks + tok_of(8h + e): token pairs
  // 16ks + 2h + 4q, +1 give slots e = q and e = q + 4
  const float* srd = &sm.s[u & 1][srow * S_LD + 16 * (g8 >> 1) + 2 * (g8 & 1)];
  float x[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float2 pr = *reinterpret_cast<const float2*>(srd + 4 * q);
    x[q] = pr.x * c_log2;
    x[q + 4] = pr.y * c_log2;
  }
  if (valid < UNIT) {  // only the range's last unit can be partial
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (16 * (g8 >> 1) + tok_of(8 * (g8 & 1) + e) >= valid) x[e] = -INFINITY;
  }
  // some score of this lane above the reference by more than the slack
  // (always on the first unit, whose reference is -inf)
  const float lim = m_run + kRescaleSlack;
  const bool over = ((x[0] > lim) | (x[1] > lim)) | ((x[2] > lim) | (x[3] > lim)) |
                    ((x[4] > lim) | (x[5] > lim)) | ((x[6] > lim) | (x[7] > lim));
  int raised = 0;
  float alpha = 1.0f;
  if (__any(over)) {
    // the rows' maxima; a row whose maximum passes the slack takes it as its
    // new reference, and its sum and output are scaled by alpha
    float mx = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])),
                    vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
    mx = xor32_max(xor16_max(mx));
    const bool raise = mx > lim;
    const float m_new = raise ? mx : m_run;
    alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    l_lane = l_lane * alpha;
    raised = __any(raise) ? 1 : 0;
  }
  float ex[8];
  u16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ex[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
    pb[e] = f32_to_bf16(ex[e]);
  }
  *reinterpret_cast<u16x8*>(&sm.p[u & 1][srow * P_LD + 8 * g8]) = pb;
  l_lane += ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
  // the value waves read the factors of all 64 rows when any group's flag is
  // set, so every group writes its rows' factors (1 where nothing rose)
  if (g8 == 0) sm.alpha[u & 1][srow] = alpha;
  if (lane == 0) sm.flag[u & 1][grp] = raised;
}

// After the last unit: the rows' sums (the four lanes' shares added), the
// reciprocals of those for the normalisation, and the rows' log-sum-exp
// (natural log) to the output or to the split's partial (kDev: with a
// device-scope store, for a merge in the same launch).
template <bool kDev>
__device__ __forceinline__ void softmax_finish(Smem& sm, const DecodeParams& p, int grp, int lane,
                                               float m_run, float l_lane, bool direct, int b,
                                               int pidx, int TH, int rb, int rows_here) {
  const float l_run = xor32_sum(xor16_sum(l_lane));
  if ((lane >> 4) != 0) return;
  const int srow = 16 * grp + (lane & 15);
  sm.lrow[srow] = 1.0f / l_run;
  const float lse = (m_run + log2f(l_run)) * kLn2;
  if (srow >= rows_here) return;  // past the token's last head: not stored
  if (direct) {
    if (p.lse != nullptr) p.lse[(size_t)b * TH + rb + srow] = lse;
  } else if constexpr (kDev) {
    __hip_atomic_store(&p.part_lse[(size_t)pidx * TH + rb + srow], lse, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    p.part_lse[(size_t)pidx * TH + rb + srow] = lse;
  }
}

// Balanced split plan for a batch of sequences of different lengths, with K
// work items per 64-row group.  Sequence b has U_b = ceil(n_b / 32) units (n_b
// = the rows its last new token sees) and gets S_b = ceil(U_b / C) splits of
// ch_b = ceil(U_b / S_b) units each (the last may be shorter), where C is the
// smallest count >= kMinUnits for which sum_b S_b <= K; the splits of the
// sequences are numbered in order, P_b being the first of sequence b.  Work
// item k is split k - P_b of the sequence with P_b <= k < P_b + S_b, or no
// work past the last.  Computed by one wave (64 lanes, sequences
// lane + 64c); with `table`, every sequence's (P_b, S_b, ch_b) is written
// there for the merge.  With min_one, a sequence with no visible row gets one
// (empty) split as well, whose work item writes its zero output.  Returns
// {b, s, S_b, ch_b, P_b, multi}, b = -1 for no work, multi = the number of
// sequences with more than one split.
constexpr int kMinUnits = 8;
struct PlanItem {
  int b, s, S_b, ch_b, P_b, multi;
};
__device__ __forceinline__ PlanItem balanced_item(const DecodeParams& p, int k, int lane,
                                                  int32_t* table, bool min_one = false) {
  const int B = p.B;
  const int K = p.num_splits;
  auto units = [&](int b) {
    if (b >= B) return 0;
    const int n = visible_rows(p.seq_lens[b], p.T, p.T - 1, p.causal, p.cap);
    return (n + UNIT - 1) / UNIT;
  };
  auto wave_sum = [](int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
  };
  auto wave_max = [](int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
    return x;
  };
  // the splits sequence b gets for a bound of C units per split (none for the
  // lanes past the last sequence)
  auto splits_of = [B, min_one](int b, int U, int C) {
    if (b >= B) return 0;
    return U == 0 ? (min_one ? 1 : 0) : (U + C - 1) / C;
  };
  long long total = 0;
  int umax = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int U = units(c0 + lane);
    total += wave_sum(U);
    umax = max(umax, wave_max(U));
  }
  // smallest feasible C in [lo, hi]; hi = max units is feasible (one split per
  // nonempty sequence, and K >= B)
  int lo = (int)max((long long)kMinUnits, (total + K - 1) / K);
  int hi = max(lo, umax);
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    int cnt = 0;
    for (int c0 = 0; c0 < B; c0 += 64) cnt += wave_sum(splits_of(c0 + lane, units(c0 + lane), mid));
    if (cnt <= K) hi = mid; else lo = mid + 1;
  }
  const int C = lo;
  PlanItem it{-1, 0, 0, 0, 0, 0};
  int base = 0;  // splits of the sequences before this chunk
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int U = units(c0 + lane);
    const int S_b = splits_of(c0 + lane, U, C);
    const int ch_b = S_b > 0 ? (U + S_b - 1) / S_b : 0;
    int incl = S_b;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int P_b = base + incl - S_b;
    it.multi += wave_sum(S_b > 1 ? 1 : 0);
    if (table != nullptr && c0 + lane < B) {
      table[4 * (c0 + lane) + 0] = P_b;
      table[4 * (c0 + lane) + 1] = S_b;
      table[4 * (c0 + lane) + 2] = ch_b;
    }
    const unsigned long long hit = __ballot(S_b > 0 && P_b <= k && k < P_b + S_b);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      it.b = c0 + l;
      it.s = k - __shfl(P_b, l);
      it.S_b = __shfl(S_b, l);
      it.ch_b = __shfl(ch_b, l);
      it.P_b = __shfl(P_b, l);
    }
    base += __shfl(incl, 63);
  }
  return it;
}

// One work item: the 64 query rows of group g (ceil(H / 64) groups per new
// token) of sequence b against cache rows s * chunk_rows .. (s + 1) *
// chunk_rows - 1 (cut at the rows the group's token sees), written as the
// final output (direct) or as partial pidx.  kDev: partials with device-scope
// stores.
template <bool kDev>
__device__ __forceinline__ void attend_range(Smem& sm, const DecodeParams& p, int g, int b, int s,
                                            int pidx, int chunk_rows, bool direct) {
  // The thread index through an opaque copy: inside the one-launch kernel's
  // item loop, the lane-dependent offsets of all three roles would otherwise
  // be hoisted out of the loop and held in registers across every role.
  int tid = threadIdx.x;
  if constexpr (kDev) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  // Wave index as a scalar: the role branches below are uniform (scalar)
  // branches, so a wave never steps through the other role's barriers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int gpt = (p.H + ROWS - 1) / ROWS;
  const int TH = p.T * p.H;
  const int t = g / gpt;                                   // the group's new token
  const int rb = t * p.H + (g - t * gpt) * ROWS;           // its first query row (t*H + h)
  const int rows_here = min(ROWS, (t + 1) * p.H - rb);     // 64, or fewer in a token's last group
  // this range starts at cache row tok0 (a multiple of UNIT)
  const int tok0 = s * chunk_rows;

  // The sequence length fixes where the range ends.  Each role first requests
  // what does not depend on it -- the score waves their queries and unit 0's
  // rotary keys, the copy waves units 0 and 1 -- and reads the length only
  // then, so that it costs no memory round trip of its own in front of the
  // first unit.  Page-table entries for those requests are looked up within
  // the table row but without the range's clamp: a unit that turns out to lie
  // past the range is copied (from a valid page) and never read.  Page ids
  // and the length are read through the constant address space: uniform
  // indexes make them scalar loads (lgkmcnt), whose waits leave the vector
  // loads and copies in flight.
  const int32_t __attribute__((address_space(4)))* ctable =
      (const int32_t __attribute__((address_space(4)))*)(p.block_table + (size_t)b * p.max_blocks);
  auto page_at = [&](int row) { return ctable[min(row / BS, p.max_blocks - 1)]; };
  // End of the range (cache rows tok0 .. tok_end-1), the same for the whole
  // workgroup: kept in scalar registers, so that the range bounds, loop counts
  // and page addresses below are scalar as well.
  auto range_end = [&]() {
    const int len = ((const int32_t __attribute__((address_space(4)))*)p.seq_lens)[b];
    const int n_valid = __builtin_amdgcn_readfirstlane(visible_rows(len, p.T, t, p.causal, p.cap));
    return min(tok0 + chunk_rows, n_valid);
  };
  // An empty range: wait for the requests in flight, and write o = 0,
  // lse = -inf when this is the final output (each wave its share).
  auto empty_range = [&]() {
    wait_vmcnt<0>();
    if (direct) {
      float* dst = p.o_lat + ((size_t)b * TH + rb) * DC;
      for (int i = tid; i < rows_here * DC; i += NT) dst[i] = 0.0f;
      if (p.lse != nullptr && tid < rows_here) p.lse[(size_t)b * TH + rb + tid] = -INFINITY;
    }
  };

  // One barrier per unit.  Barrier schedule, the same for every wave: B0, then
  // E(j) for j = -2 .. U-1, then F.  In step j (between E(j-1) and E(j)):
  //   score waves: raw scores of unit j+2 (fp32) into sm.s[(j+2) & 1];
  //   value waves: softmax of unit j+1 for their 16 rows (sm.s -> sm.p) and
  //                O += P(j) V(j), in the order of the wave, and V(j+1) into
  //                registers after the MFMAs;
  //   copy waves:  copies of unit j+4 issued, unit j+3 waited for, the stale
  //                tail of the range's last unit zeroed.
  // Latent slot u & 3 is read in step u-2 (K) and u-1 (V into registers), so
  // the 4 slots hold units j+1 .. j+4 and keep two units of copies in flight.
  // The rotary key columns (64 per row) are not staged: the score waves read
  // them from memory into registers one unit ahead.
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
      // rows past the group's last re-read it (their results are not stored)
      const int qr = min(32 * wave + 16 * rt + n16, rows_here - 1);
      const uint16_t* q = static_cast<const uint16_t*>(p.q_abs) + ((size_t)b * TH + rb + qr) * W + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < QSTEPS; ++kk)
        qf[rt][kk] = *reinterpret_cast<const bf16x8*>(q + 32 * kk);
    }
    const int raw0 = page_at(tok0), raw1 = page_at(tok0 + UNIT);
    // latent chunk c = 4kk + g4 of token n16 sits at chunk position
    // c ^ lat_sw(n16) (only the low 4 bits of c take part); token tile ti adds
    // 16 KiB
    int loff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) loff[j] = n16 * 1024 + (((4 * j + g4) ^ lat_sw(n16)) << 4);
    const uint16_t* pool = static_cast<const uint16_t*>(p.pool);
    // rotary columns 512 + 32(kk-16) + 8*g4 .. +7 of token 16ti + n16 of unit
    // u (page-table entry raw), from memory (a unit lies within one page), as
    // kr[kk - 16][ti]
    auto load_kr = [&](int u, int raw, bf16x8 (&kr)[2][2]) {
      const int tok = tok0 + u * UNIT;
      const int blk = clamp_block(raw, p.num_blocks);
      const uint16_t* rrow = pool + ((size_t)blk * BS + tok % BS + n16) * W + DC + 8 * g4;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          kr[k2][ti] = *reinterpret_cast<const bf16x8*>(rrow + ti * 16 * W + 32 * k2);
    };

    // rotary keys double-buffered by unit parity: unit 0's requested now
    bf16x8 kra[2][2], krb[2][2];
    load_kr(0, raw0, kra);

    const int tok_end = range_end();
    if (tok0 >= tok_end) {
      empty_range();
      return;
    }
    const int U = (tok_end - tok0 + UNIT - 1) / UNIT;  // 32-row units
    // Page-table entry of unit u (clamped to the range's last unit), read one
    // unit before its rotary keys so that the scalar load is not waited for.
    auto page_raw = [&](int u) { return ctable[(tok0 + min(u, U - 1) * UNIT) / BS]; };

    // scores of unit u with its rotary keys in kr; the next unit's rotary keys
    // are read into krn first
    int raw_next = raw1;  // page-table entry of unit u + 1 in scores(u)
    auto scores = [&](int u, const bf16x8 (&kr)[2][2], bf16x8 (&krn)[2][2])
                      __attribute__((always_inline)) {
      const uint8_t* lat = sm.lat[u & 3];
      auto kfrag = [&](int kk, int ti) {
        return *reinterpret_cast<const bf16x8*>(lat + loff[kk & 3] + ti * 16 * 1024 + ((kk >> 2) << 8));
      };
      f32x4 acc[2][2];  // [rt][ti]
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rt][ti][i] = 0.0f;
      constexpr int KDEPTH = 4;
      bf16x8 kf[KDEPTH][2];
#pragma unroll
      for (int kk = 0; kk < KDEPTH; ++kk) {
        kf[kk][0] = kfrag(kk, 0);
        kf[kk][1] = kfrag(kk, 1);
      }
      // the two rotary k-steps (keys already in registers) run first, while
      // the first latent fragments are still on their way from LDS; the next
      // unit's rotary keys are requested right after
#pragma unroll
      for (int i = 0; i < QSTEPS; ++i) {
        const int kk = i < QSTEPS - LSTEPS ? LSTEPS + i : i - (QSTEPS - LSTEPS);
        if (i == QSTEPS - LSTEPS && u + 1 < U) load_kr(u + 1, raw_next, krn);
        bf16x8 k0, k1;
        if (kk < LSTEPS) {
          k0 = kf[kk % KDEPTH][0];
          k1 = kf[kk % KDEPTH][1];
          if (kk + KDEPTH < LSTEPS) {
            kf[kk % KDEPTH][0] = kfrag(kk + KDEPTH, 0);
            kf[kk % KDEPTH][1] = kfrag(kk + KDEPTH, 1);
          }
        } else {
          k0 = kr[kk - LSTEPS][0];
          k1 = kr[kk - LSTEPS][1];
        }
        acc[0][0] = mfma16(k0, qf[0][kk], acc[0][0]);
        acc[1][0] = mfma16(k0, qf[1][kk], acc[1][0]);
        acc[0][1] = mfma16(k1, qf[0][kk], acc[0][1]);
        acc[1][1] = mfma16(k1, qf[1][kk], acc[1][1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The page-table entry of unit u + 2 is requested only now: a scalar
      // load in flight would turn every LDS wait of the loop above into a
      // wait for all of them.  The barrier after this unit waits for it
      // anyway, and pin_sgpr after that barrier keeps the compiler from
      // sinking the load back into the next unit's loop.
      raw_next = page_raw(u + 2);
      float* sdst = sm.s[u & 1];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          *reinterpret_cast<f32x4*>(&sdst[(32 * wave + 16 * rt + n16) * S_LD + 16 * ti + 4 * g4]) =
              acc[rt][ti];
    };

    lds_barrier();                         // B0: unit 0 landed
    // j even: unit j+2 is even, its keys in kra, the next unit's into krb
    for (int j = -2; j < U; j += 2) {
      if (j + 2 < U) scores(j + 2, kra, krb);
      lds_barrier();                       // E(j)
      pin_sgpr(raw_next);
      if (j + 1 < U) {
        if (j + 3 < U) scores(j + 3, krb, kra);
        lds_barrier();                     // E(j+1)
        pin_sgpr(raw_next);
      }
    }
    lds_barrier();                         // F
  } else if (wave >= 4 && wave < 6) {
    // =============================== copy waves ================================
    // Copy wave c fills latent rows t = c + 2i (i < 16) of a unit: 16
    // direct-to-LDS copies of 1 KiB.  Lane l fetches the 16-byte chunk that
    // belongs at LDS chunk position l of its row.
    const int c = wave - 4;
    const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
    int cl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cl[i] = (lane ^ lat_sw(c + 2 * i)) << 4;
    const uint32_t lat_base = (uint32_t)(uintptr_t)&sm.lat[0][0];
    auto issue = [&](int u, int raw) {
      const int blk = clamp_block(raw, p.num_blocks);
      const uint8_t* src = pool + (size_t)blk * TILE_BYTES + ((tok0 + u * UNIT) % BS) * ROW_BYTES;
      const uint32_t lat = lat_base + (u & 3) * (UNIT * 1024);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = c + 2 * i;
        copy16_to_lds(src + row * ROW_BYTES, (uint32_t)cl[i & 7], lat + row * 1024);
      }
    };
    // Only units 0 and 1 are requested before the first barrier, and before
    // the length is read: every workgroup starts at once, and unit 0 (scored
    // in step -2) lands sooner when it does not queue behind units 2 and 3 of
    // the whole chip.  Unit u is then issued in step u - 4, units 2 and 3 in
    // steps -2 and -1.
    const bool spec1 = chunk_rows > UNIT;  // the range may hold a unit 1
    // both page ids first, in one round trip (pinned, or the compiler sinks
    // the second load below unit 0's copies)
    const int raw0 = page_at(tok0), raw1 = page_at(tok0 + UNIT);
    pin_sgpr(raw1);
    issue(0, raw0);
    if (spec1) issue(1, raw1);
    const int tok_end = range_end();
    if (tok0 >= tok_end) {
      empty_range();
      return;
    }
    const int U = (tok_end - tok0 + UNIT - 1) / UNIT;  // 32-row units
    auto unit_valid = [&](int u) { return min(UNIT, tok_end - tok0 - u * UNIT); };
    // Page-table entry of unit u (clamped to the range's last unit, so the
    // read stays inside the range's pages); read one step ahead in the loop.
    auto page_raw = [&](int u) { return ctable[(tok0 + min(u, U - 1) * UNIT) / BS]; };
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
    };

    int raw_next = page_raw(2);
    if (spec1) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();  // unit 0 landed
    // The copy waves also run the online softmax of query rows 32 .. 63 (16
    // rows each), first in each step: its VALU work then shares a SIMD with a
    // score wave's MFMAs instead of a value wave's, which balances the four
    // SIMDs.  Copies of the next unit are issued after it; they have two
    // steps to land.
    const int grp = 2 + c;
    float m_run = -INFINITY, l_lane = 0.0f;  // reference maximum; this lane's share of the row sum
    lds_barrier();                         // B0
    for (int j = -2; j < U; ++j) {
      if (j + 1 >= 0 && j + 1 < U)
        softmax_unit(sm, j + 1, unit_valid(j + 1), grp, lane, p.scale_log2, m_run, l_lane);
      if (j + 4 < U) {
        issue(j + 4, raw_next);
        raw_next = page_raw(j + 5);
      }
      if (j + 2 >= 0 && j + 2 < U) zero_tail(j + 2);  // landed by E(j-1) (B0 for unit 0)
      // unit j+3 lands before E(j); only unit j+4 may stay in flight
      if (j + 3 < U) {
        if (j + 4 < U) wait_vmcnt<COPIES>(); else wait_vmcnt<0>();
      }
      lds_barrier();                       // E(j)
    }
    wait_vmcnt<0>();  // a unit 1 copied past a one-unit range
    softmax_finish<kDev>(sm, p, grp, lane, m_run, l_lane, direct, b, pidx, TH, rb, rows_here);
    lds_barrier();                         // F
  } else {
    // =============================== value waves ===============================
    // Value wave v owns latent columns 128v .. 128v+127 of O for all 64 rows,
    // and the softmax of query rows 16v .. 16v+15.
    const int v = (wave & 1) + 2 * (wave >> 2);
    // the softmax scale in a register of its own for the whole range (the
    // one-launch kernel would otherwise re-load it in every step)
    float c_log2 = p.scale_log2;
    if constexpr (kDev) asm volatile("" : "+s"(c_log2));
    const int tok_end = range_end();
    if (tok0 >= tok_end) {
      empty_range();
      return;
    }
    const int U = (tok_end - tok0 + UNIT - 1) / UNIT;  // 32-row units
    auto unit_valid = [&](int u) { return min(UNIT, tok_end - tok0 - u * UNIT); };
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

    float m_run = -INFINITY, l_lane = 0.0f;  // reference maximum; this lane's share of the row sum

    f32x16 o[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rt][dt][r] = 0.0f;

    bf16x8 vf[2][4];  // V of the unit whose P.V runs next
    // the 16-token half ks of V(u) into vf[ks]
    auto load_v_half = [&](int u, int ks) __attribute__((always_inline)) {
      const uint8_t* lat = sm.lat[u & 3];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const s16x4 v0 = lds_tr16(lat + voff[dt][0] + 16 * ks * 1024);
        const s16x4 v1 = lds_tr16(lat + voff[dt][1] + 16 * ks * 1024);
        vf[ks][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto load_v = [&](int u) {
      const uint8_t* lat = sm.lat[u & 3];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 v0 = lds_tr16(lat + voff[dt][0] + 16 * ks * 1024);
          const s16x4 v1 = lds_tr16(lat + voff[dt][1] + 16 * ks * 1024);
          // a plain concatenation: no instruction reads the loaded registers
          vf[ks][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    // P(u) and the rescale flags into registers (issued before the softmax of
    // the next unit so that their latency is hidden), then O = alpha(u) O +
    // P(u) V(u)
    bf16x8 pf[2][2];
    int4 fl;
    auto read_p = [&](int u) {
      const uint16_t* pp = sm.p[u & 1];
      fl = *reinterpret_cast<const int4*>(sm.flag[u & 1]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pf[ks][0] = *reinterpret_cast<const bf16x8*>(pp + poff + 16 * ks);
        pf[ks][1] = *reinterpret_cast<const bf16x8*>(pp + 32 * P_LD + poff + 16 * ks);
      }
    };
    // P(u) V(u); with `nxt` >= 0, the first half of V(nxt) replaces the first
    // half of V(u) in registers as soon as the MFMAs that read it are issued,
    // so that those reads complete under the second half's MFMAs.
    auto pv = [&](int u, int nxt) __attribute__((always_inline)) {
      if (fl.x | fl.y | fl.z | fl.w) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 al =
                *reinterpret_cast<const float4*>(&sm.alpha[u & 1][32 * rt + 8 * r4 + 4 * lhi]);
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
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          o[0][dt] = mfma32(pf[ks][0], vf[ks][dt], o[0][dt]);
          o[1][dt] = mfma32(pf[ks][1], vf[ks][dt], o[1][dt]);
        }
        if (ks == 0) {
          __builtin_amdgcn_sched_barrier(0);
          // P has arrived (the MFMAs above read it); with nothing older in
          // flight, the MFMAs below wait for none of the V reads.  The wait
          // is unconditional so that both paths reach the MFMAs in the same
          // state.
          __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (3 << 14));  // lgkmcnt(0)
          if (nxt >= 0) load_v_half(nxt, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (nxt >= 0) load_v_half(nxt, 1);
    };

    // Step j.  The softmax of unit j+1 and P(j) V(j) are independent; the two
    // value waves of a SIMD (v and v + 2) run them in opposite orders, so
    // that one wave's softmax (VALU) overlaps the other's MFMAs instead of
    // both waves contending for the same unit at the same time.  V(j+1)
    // replaces V(j) in registers right after the MFMAs that read V(j).
    auto step = [&](int j, auto pv_first) __attribute__((always_inline)) {
      const bool next = j + 1 >= 0 && j + 1 < U;
      if (j >= 0) read_p(j);
      if (pv_first) {  // the waves whose softmax rows the copy waves run
        if (j >= 0) pv(j, next ? j + 1 : -1);
        else if (next) load_v(j + 1);
      } else {
        if (next) softmax_unit(sm, j + 1, unit_valid(j + 1), v, lane, c_log2, m_run, l_lane);
        if (j >= 0) pv(j, next ? j + 1 : -1);
        else if (next) load_v(j + 1);
      }
      lds_barrier();                       // E(j)
    };
    lds_barrier();                         // B0
    if (v >= 2) {
      for (int j = -2; j < U; ++j) step(j, std::true_type{});
    } else {
      for (int j = -2; j < U; ++j) step(j, std::false_type{});
    }

    if (v < 2) softmax_finish<kDev>(sm, p, v, lane, m_run, l_lane, direct, b, pidx, TH, rb, rows_here);
    lds_barrier();                         // F
    // Streaming (non-temporal) stores: the rows are read by the next kernel,
    // not by this one, and lines left dirty in L2 would all be written back
    // at the end of the launch, which delays the next kernel's start.  A
    // split's partial is stored as bf16: it is a normalised average of cached
    // rows, so bf16 keeps 8 significant bits of every element whatever its
    // range, and the merge reads half the bytes.  kDev: partials are merged
    // in the same launch, possibly on another XCD, so they are stored with
    // device-scope stores, which do not stay in this XCD's L2.
    auto store_rows = [&](auto* dst, auto cvt) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * rt + 8 * (r >> 2) + 4 * lhi + (r & 3);
          const float inv = sm.lrow[row];
          if (row < rows_here) {  // past the token's last head: not stored
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              auto* at = &dst[(size_t)row * DC + 128 * v + 32 * dt + l32];
              if (kDev && !direct)
                __hip_atomic_store(at, cvt(o[rt][dt][r] * inv), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
              else
                __builtin_nontemporal_store(cvt(o[rt][dt][r] * inv), at);
            }
          }
        }
      }
    };
    if (direct)
      store_rows(p.o_lat + ((size_t)b * TH + rb) * DC, [](float x) { return x; });
    else
      store_rows(static_cast<uint16_t*>(p.part_o) + ((size_t)pidx * TH + rb) * DC,
                 [](float x) { return f32_to_bf16(x); });
  }
}

__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(const DecodeParams p) {
  __shared__ Smem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // 64-row groups: ceil(H / 64) per new token, the last one partial when H
  // is not a multiple of 64
  const int gpt = (p.H + ROWS - 1) / ROWS;
  const int G = p.T * gpt;
  const int S = p.num_splits;
  // Workgroup i is dispatched to XCD i % X (X XCDs, queried on the host), and
  // each XCD has its own L2.  XCD x gets a contiguous block of (sequence,
  // split) pairs, and all G 64-row groups of each: the pages of a pair and the
  // absorbed queries of a sequence then come from HBM once per XCD and from L2
  // for the other workgroups that read them.  Ids past the last full set of
  // X G keep the plain order.
  const int XCDS = p.xcds;
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
  // (sequence b, split s) of this workgroup, its partial's index and the cache
  // rows per split: the plain plan cuts every sequence at the same rows; a
  // balanced plan is computed here, by wave 0, from the sequence lengths
  int b, s, pidx, chunk_rows;
  if (p.plan == nullptr) {
    s = pair % S;
    b = pair / S;
    pidx = pair;
    chunk_rows = p.chunk_rows;
  } else {
    if (wave == 0) {
      const PlanItem it = balanced_item(p, pair, lane, g == 0 && pair == 0 ? p.plan : nullptr);
      if (lane == 0) {
        sm.item[0] = it.b;
        sm.item[1] = it.s;
        sm.item[2] = it.P_b + it.s;
        sm.item[3] = it.ch_b * UNIT;
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(sm.item[0]);
    if (b < 0) return;  // no work item: the whole workgroup
    s = __builtin_amdgcn_readfirstlane(sm.item[1]);
    pidx = __builtin_amdgcn_readfirstlane(sm.item[2]);
    chunk_rows = __builtin_amdgcn_readfirstlane(sm.item[3]);
  }

  attend_range<false>(sm, p, g, b, s, pidx, chunk_rows, S == 1 && p.plan == nullptr);
}

// ---------------------------------------------------------------- one launch
// Split-KV decode and its log-sum-exp merge in a single launch of persistent
// workgroups (one per compute unit), in the manner of the fused and
// megakernel decoders that "Research on MLA" lists for variable-length
// serving.
//  * Work items (query group, split) of the plain or balanced plan: workgroup
//    i takes item i first, then further items from a queue counter, so that a
//    workgroup that finishes early takes more.  A sequence whose rows all fit
//    one split writes its final output directly.
//  * Publishing: a split's partial rows and log-sum-exps are written with
//    device-scope stores; every wave waits for its stores to complete, then
//    one thread counts the split into its group (arrival count).
//  * Last arrival: the split that completes its group's count pushes the
//    group's kQueueSlices merge slices (8 query rows each, with the group's
//    split count) onto a ring, after the group's record (first partial, rows
//    per split) under a balanced plan; a plain plan's record follows from
//    the parameters.
//  * Merges: a workgroup that finds the item queue empty takes ring tickets,
//    waits for its ticket's entry to be pushed, and merges the slice (one row
//    per wave) with device-scope loads.  A ticket is only taken after every
//    work item has been taken by a running workgroup, and no work item waits
//    on anything, so every awaited entry is pushed; the wait is bounded all
//    the same (kSpinLimit polls; a miss sets bit 0 of the error word and
//    leaves the slice unmerged).
//  * Every counter is left zero for the next launch: the arrival count by its
//    last arrival, a ring entry by its consumer, the queue counters by the
//    last workgroup to leave.
// Device-scope stores write past the XCD's L2 and device-scope loads do not
// take lines from it, so partials written on one XCD are seen on another
// once the stores have completed (the AMDGPU memory model's agent scope).
constexpr int kCtrItems = 0, kCtrHead = 32, kCtrTail = 64, kCtrExit = 96, kCtrErr = 128;
constexpr int kCtrRing = 256;  // first word of the merge ring (8-byte entries)
constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ void st_dev(uint32_t* a, uint32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* a, uint32_t v) {
  return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Counter region (32-bit words from p.counters): the queue counters and the
// error word in the first 1 KiB, then kQueueSlices ring entries per (sequence,
// 64-row group) -- 8 bytes each: the slice + 1 and the group's split count --
// then an arrival count per group.  The group records follow the region: 8
// bytes per group, its first partial and its rows per split.
__device__ __forceinline__ uint64_t* ring_of(const DecodeParams& p) {
  return reinterpret_cast<uint64_t*>(p.counters + kCtrRing);
}
__device__ __forceinline__ uint32_t* arrive_of(const DecodeParams& p, int G) {
  return p.counters + kCtrRing + 2 * kQueueSlices * p.B * G;
}
__device__ __forceinline__ uint64_t* rec_of(const DecodeParams& p) {
  return reinterpret_cast<uint64_t*>(p.counters + kQueueCounterBytes / 4);
}

// The launch's parameters through an opaque copy of their address (the
// kernel argument block holds them at offset 0).  Inside the one-launch
// kernel's item loop, every value derived from the parameters alone would
// otherwise be hoisted out of the loop and held in scalar registers across the
// whole item, which the item's own code needs: beyond the register file, the
// compiler re-loads values inside the per-unit loops, and each such load makes
// the LDS waits there wait for it too.
typedef const __attribute__((address_space(4))) DecodeParams* ParamsPtr;
__device__ __forceinline__ const DecodeParams& params() {
  ParamsPtr kp = (ParamsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return *(const DecodeParams*)kp;
}

__global__ __launch_bounds__(NT, 1) void decode_queue_kernel(const DecodeParams) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The queue's state lives in sm.item (LDS) and is read back after each
  // item rather than held in registers across it.  sm.item: [0] sequence
  // (-1: none), [1] group, [2] split, [3] the sequence's splits, [4] its
  // first partial, [5] rows per split, [6] the sequences with more than one
  // split (-1: not known yet), [7] the workgroups of the launch.
  //
  // Work item `ticket` into sm.item (wave 0).
  auto take = [&](int ticket) {
    const DecodeParams& p = params();
    const int G = p.T * ((p.H + ROWS - 1) / ROWS);
    const int S = p.num_splits;
    const bool balanced = p.plan != nullptr;
    const int n_items = (balanced ? 1 : p.B) * S * G;
    int b = -1, g = 0, s = 0, S_b = 0, P_b = 0, ch = 0, mu = -1;
    if (ticket < n_items) {
      // item = k G + g.  The first tickets (one per workgroup) are placed as
      // in the split kernel: XCD x runs all G groups of a contiguous block of
      // (sequence, split) pairs, so that their pages come from HBM once per
      // XCD; the tickets past them are handed out in item order.
      const int grid = sm.item[7];
      const int XCDS = p.xcds;
      const int full = grid - grid % (XCDS * G);
      int k;
      if (ticket < full) {
        const int r = ticket / XCDS;
        g = r % G;
        k = (ticket % XCDS) * (full / G / XCDS) + r / G;
      } else {
        g = ticket % G;
        k = ticket / G;
      }
      if (balanced) {
        const PlanItem pi = balanced_item(p, k, lane, ticket == 0 ? p.plan : nullptr, true);
        b = pi.b;
        s = pi.s;
        S_b = pi.S_b;
        P_b = pi.P_b;
        ch = pi.ch_b * UNIT;
        mu = pi.multi;
      } else {
        b = k / S;
        s = k % S;
        S_b = S;
        P_b = b * S;
        ch = p.chunk_rows;
        mu = S > 1 ? p.B : 0;
      }
    }
    if (lane == 0) {
      sm.item[0] = b;
      sm.item[1] = g;
      sm.item[2] = s;
      sm.item[3] = S_b;
      sm.item[4] = P_b;
      sm.item[5] = ch;
      if (mu >= 0) sm.item[6] = mu;
    }
  };

  // ---- work items: the first by workgroup id, the others from the queue
  if (tid == 0) {
    sm.item[6] = -1;
    sm.item[7] = (int)gridDim.x;
  }
  __syncthreads();
  if (wave == 0) take(blockIdx.x);
  __syncthreads();
  for (;;) {
    {
      const DecodeParams& p = params();
      const int b = __builtin_amdgcn_readfirstlane(sm.item[0]);
      // no item left (tickets past the last, or a balanced plan's spare
      // items, which all come after its last real one)
      if (b < 0 || b >= p.B) break;
      const int S_b = __builtin_amdgcn_readfirstlane(sm.item[3]);
      const int s = __builtin_amdgcn_readfirstlane(sm.item[2]);
      attend_range<true>(sm, p, __builtin_amdgcn_readfirstlane(sm.item[1]), b, s,
                         __builtin_amdgcn_readfirstlane(sm.item[4]) + s,
                         __builtin_amdgcn_readfirstlane(sm.item[5]), S_b == 1);
    }
    const int S_b = __builtin_amdgcn_readfirstlane(sm.item[3]);
    if (S_b > 1) {
      wait_vmcnt<0>();  // this wave's partial stores have completed
      __syncthreads();
      if (tid == 0) {
        const DecodeParams& p = params();
        const int G = p.T * ((p.H + ROWS - 1) / ROWS);
        const int bg = sm.item[0] * G + sm.item[1];
        uint32_t* const arrive = arrive_of(p, G) + bg;
        if (add_dev(arrive, 1u) + 1 == (uint32_t)S_b) {
          // the group's last split: nothing else reads its count in this launch
          st_dev(arrive, 0u);
          if (p.plan != nullptr) {  // a plain plan's record is known to all
            st_dev64(rec_of(p) + bg,
                     (uint64_t)(uint32_t)sm.item[4] | ((uint64_t)(uint32_t)sm.item[5] << 32));
            wait_vmcnt<0>();  // the record before the ring entries
          }
          const uint32_t pos = add_dev(p.counters + kCtrTail, (uint32_t)kQueueSlices);
          for (int j = 0; j < kQueueSlices; ++j)
            st_dev64(ring_of(p) + pos + j,
                     (uint64_t)(bg * kQueueSlices + j + 1) | ((uint64_t)(uint32_t)S_b << 32));
        }
      }
    }
    __syncthreads();  // the LDS and sm.item are free for the next item
    if (wave == 0) {
      uint32_t t0 = 0;
      if (lane == 0) t0 = add_dev(params().counters + kCtrItems, 1u);
      take(sm.item[7] + (int)__shfl(t0, 0));
    }
    __syncthreads();
  }

  // ---- merges
  const DecodeParams& p = params();
  const int gpt = (p.H + ROWS - 1) / ROWS;
  const int G = p.T * gpt;
  int multi = __builtin_amdgcn_readfirstlane(sm.item[6]);
  if (multi < 0) {  // a balanced plan whose item this workgroup never computed
    if (wave == 0) {
      const PlanItem pi = balanced_item(p, 0, lane, nullptr, true);
      if (lane == 0) sm.item[6] = pi.multi;
    }
    __syncthreads();
    multi = __builtin_amdgcn_readfirstlane(sm.item[6]);
  }
  const int n_slices = multi * G * kQueueSlices;
  uint32_t* const ctr = p.counters;
  uint64_t* const ring = ring_of(p);
  const int TH = p.T * p.H;
  for (;;) {
    __syncthreads();  // sm.item is free
    if (tid == 0) {
      int task = -1;  // -1: no ticket left; -2: the entry never came
      const uint32_t t = add_dev(ctr + kCtrHead, 1u);
      if (t < (uint32_t)n_slices) {
        uint64_t e = ld_dev64(ring + t);
        for (unsigned n = 0; e == 0 && n < kSpinLimit; ++n) {
          __builtin_amdgcn_s_sleep(2);
          e = ld_dev64(ring + t);
        }
        if (e == 0) {
          __hip_atomic_fetch_or(ctr + kCtrErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          task = -2;
        } else {
          st_dev64(ring + t, 0ull);
          task = (int)(uint32_t)e - 1;
          const int bg = task / kQueueSlices;
          const int b = bg / G;
          uint64_t r;  // first partial | rows per split << 32
          if (p.plan != nullptr)
            r = ld_dev64(rec_of(p) + bg);
          else
            r = (uint64_t)(uint32_t)(b * p.num_splits) | ((uint64_t)(uint32_t)p.chunk_rows << 32);
          sm.item[1] = (int)(uint32_t)r;
          sm.item[2] = (int)(uint32_t)(e >> 32);
          sm.item[3] = (int)(uint32_t)(r >> 32);
        }
      }
      sm.item[0] = task;
    }
    __syncthreads();
    const int task = __builtin_amdgcn_readfirstlane(sm.item[0]);
    if (task == -1) break;
    if (task < 0) continue;
    const int bg = task / kQueueSlices;
    const int sl = task - bg * kQueueSlices;
    const int b = bg / G;
    const int g = bg - b * G;
    const int t = g / gpt;
    const int rb = t * p.H + (g - t * gpt) * ROWS;
    const int rows_here = min(ROWS, (t + 1) * p.H - rb);
    const int r = sl * (ROWS / kQueueSlices) + wave;  // one query row per wave
    if (r < rows_here)
      merge_row_splits<uint16_t, true>(p, (long long)b * TH + rb + r, lane,
                                       __builtin_amdgcn_readfirstlane(sm.item[1]),
                                       __builtin_amdgcn_readfirstlane(sm.item[2]),
                                       __builtin_amdgcn_readfirstlane(sm.item[3]));
  }

  // ---- leave: the last workgroup out resets the queue counters
  if (tid == 0 && add_dev(ctr + kCtrExit, 1u) + 1 == gridDim.x) {
    st_dev(ctr + kCtrItems, 0u);
    st_dev(ctr + kCtrHead, 0u);
    st_dev(ctr + kCtrTail, 0u);
    st_dev(ctr + kCtrExit, 0u);
  }
}

}  // namespace

// A 64-row group holds heads of a single query token (the causal limit is
// taken per group): ceil(H / 64) groups per token, any H and T.
bool decode_mfma_supported(int dtype, int d_c, int d_r, int block_size, int T, int H) {
  (void)T;
  return dtype == 1 && d_c == DC && d_r == DR && block_size == BS && H > 0;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  const int G = p.T * ((p.H + ROWS - 1) / ROWS);
  // plain plan: one workgroup per (sequence, split, group); balanced: per
  // (work item, group)
  const long long grid = (p.plan != nullptr ? 1LL : (long long)p.B) * p.num_splits * G;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_queue(const DecodeParams& p, int workgroups, hipStream_t stream) {
  const int G = p.T * ((p.H + ROWS - 1) / ROWS);
  const long long items = (p.plan != nullptr ? 1LL : (long long)p.B) * p.num_splits * G;
  if (items <= 0) return hipSuccess;
  if (p.counters == nullptr || items > 0x7fffffffLL ||
      (long long)p.B * G > kQueueMaxGroups || workgroups < 1)
    return hipErrorInvalidValue;
  const long long grid = items < workgroups ? items : workgroups;
  hipLaunchKernelGGL(decode_queue_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
