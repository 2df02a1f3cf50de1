// Split-KV latent-attention decode for the DeepSeek shape on CDNA4 (gfx950).
//
// One workgroup = 64 query rows (64 heads of one new token) x one contiguous
// range of 64-token cache pages of one sequence.  Per page:
//   1. the whole 64 x 576 bf16 page (72 KiB, contiguous in HBM) is copied into
//      LDS with 128-bit direct-to-LDS loads, double-buffered: the next page's
//      copies are in flight while the current page is computed;
//   2. scores S^T = K . Q^T on MFMA (v_mfma_f32_32x32x16_bf16) over all 576
//      columns: the content term (first 512) and the rotary term (last 64) of
//      the score are one dot product ("Attention, Part 2: MQA, GQA and MLA",
//      the absorbed path adds the two terms before scaling);
//   3. online softmax in the log2 domain: per-row page maxima with one
//      cross-lane exchange, merged across the two token halves through LDS.  A
//      row's reference maximum is only raised when the page maximum exceeds it
//      by more than 2^8, so the accumulator rescale is skipped on almost every
//      page; probabilities then stay below 2^8, which bf16 and fp32 carry with
//      unchanged relative precision;
//   4. values: O += P . V with V = the first 512 columns of the SAME LDS page
//      ("How DeepSeek Rewrote the Transformer", section "Absorbed projections",
//      point 3), on MFMA, with O kept in registers for the whole page range.
// The range's result is written normalised, with its log-sum-exp, either as
// the final output (one split) or as a partial for the log-sum-exp merge.
//
// Waves (8 per workgroup, two per SIMD) have fixed roles and run separate
// loops that meet at the same barriers:
//   score waves 0..3: wave w holds the absorbed queries of rows 32*(w&1)..+31
//     in registers and scores tokens 32*(w>>1)..+31 of each page;
//   value waves 4..7: wave 4+v owns latent columns 128*v..+127 of O for all 64
//     rows, and issues the page copies.
// Splitting the roles keeps the queries (144 VGPRs) and the accumulator (128)
// in different waves, so neither spills.
//
// LDS page layout: a latent region of 64 token rows (the c part, 1 KiB each,
// padded to a 1040-byte stride) and a rotary region of 64 token rows of 128 B
// (the k^R part) in which 16-byte chunk c of token t sits at position c ^ (t & 7).
// Either way, lanes of one 128-bit access that read the same chunk of 8
// consecutive tokens hit 8 different bank groups, and every latent access is a
// per-lane base plus a compile-time offset.  One 1 KiB direct-to-LDS copy fills
// exactly one latent row (or 8 rotary rows).
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DC = 512;
constexpr int DR = 64;
constexpr int W = DC + DR;
constexpr int BS = 64;                      // tokens per page
constexpr int ROWS = 64;                    // query rows per workgroup
constexpr int NT = 512;                     // threads per workgroup
constexpr int ROW_BYTES = W * 2;            // 1152
constexpr int TILE_BYTES = BS * ROW_BYTES;  // 73728
constexpr int LAT_LD = 1040;                // bytes per latent row in LDS (1 KiB + pad)
constexpr int LAT_BYTES = BS * LAT_LD;
constexpr int ROT_BYTES = BS * 128;
constexpr int P_LD = 72;                    // bf16 per row of the P tile (64 + pad)
constexpr int QK_STEPS = W / 16;            // 36
constexpr float kRescaleSlack = 8.0f;       // log2 units

struct __align__(16) Smem {
  uint8_t lat[2][LAT_BYTES];
  uint8_t rot[2][ROT_BYTES];
  uint16_t p[ROWS * P_LD];
  float red[2][ROWS];
  float alpha[ROWS];
  float mrow[ROWS];
  int rescale;
};

__device__ __forceinline__ int lat_off(int tok, int chunk) { return tok * LAT_LD + (chunk << 4); }
__device__ __forceinline__ int rot_off(int tok, int chunk) {
  return (tok << 7) + ((chunk ^ (tok & 7)) << 4);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wait_copies() {
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's page copies have landed
}

__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(const DecodeParams p) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave index as a scalar: the role branches below are then uniform (scalar)
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

  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);

  // Page copy, issued by the value waves: value wave v copies latent rows
  // t = 4i + v (i < 16) and rotary row groups j = v, v + 4 (rows 8j..8j+7).
  auto issue_page = [&](int page, int buf) {
    const int v = wave - 4;
    const int blk = clamp_block(table[page], p.num_blocks);
    const uint8_t* src = pool + (size_t)blk * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 4 * i + v;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(src + tok * ROW_BYTES + (lane << 4)),
          (void __attribute__((address_space(3)))*)(sm.lat[buf] + tok * LAT_LD), 16, 0, 0);
    }
    const int rot_lane = (lane >> 3) * ROW_BYTES + 1024 + (((lane & 7) ^ (lane >> 3)) << 4);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = v + 4 * jj;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(src + 8 * j * ROW_BYTES + rot_lane),
          (void __attribute__((address_space(3)))*)(sm.rot[buf] + j * 1024), 16, 0, 0);
    }
  };
  // Rows past the visible length of a partial page are zeroed once the page
  // has landed (value waves only): stale contents (possibly NaN) must not
  // reach P.V.
  auto zero_tail = [&](int page, int buf) {
    const int valid = n_valid - page * BS;
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4* dl = reinterpret_cast<u32x4*>(sm.lat[buf]);
    for (int q = valid * (LAT_LD / 16) + tid - 256; q < BS * (LAT_LD / 16); q += 256) dl[q] = z;
    u32x4* dr = reinterpret_cast<u32x4*>(sm.rot[buf]);
    for (int q = valid * 8 + tid - 256; q < BS * 8; q += 256) dr[q] = z;
  };
  auto partial = [&](int page) { return n_valid - page * BS < BS; };

  if (wave >= 4) issue_page(p0, 0);
  wait_copies();
  __syncthreads();
  if (partial(p0)) {
    if (wave >= 4) zero_tail(p0, 0);
    __syncthreads();
  }

  if (wave < 4) {
    // =========================== score waves ===========================
    const int ra = wave & 1;   // row half
    const int hb = wave >> 1;  // token half
    const int srow = 32 * ra + l32;

    bf16x8 qf[QK_STEPS];
    {
      const uint16_t* q = static_cast<const uint16_t*>(p.q_abs) +
                          ((size_t)b * TH + rb + srow) * W + 8 * lhi;
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(q + 16 * kk);
    }
    float m_run = -INFINITY;  // reference max (log2 units) of row srow
    float l_run = 0.0f;       // sum over this wave's token half, in that reference

    for (int pg = p0; pg < p1; ++pg) {
      const int buf = (pg - p0) & 1;
      const uint8_t* lat = sm.lat[buf];
      const uint8_t* rot = sm.rot[buf];
      const int tok = 32 * hb + l32;

      f32x16 sa, sb;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sa[r] = 0.0f; sb[r] = 0.0f; }
#pragma unroll
      for (int kk = 0; kk < DC / 16; kk += 2) {  // content term: latent columns
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(lat + lat_off(tok, 2 * kk + lhi));
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(lat + lat_off(tok, 2 * kk + 2 + lhi));
        sa = mfma32(k0, qf[kk], sa);
        sb = mfma32(k1, qf[kk + 1], sb);
      }
#pragma unroll
      for (int kk = 0; kk < DR / 16; kk += 2) {  // rotary term
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(rot + rot_off(tok, 2 * kk + lhi));
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(rot + rot_off(tok, 2 * kk + 2 + lhi));
        sa = mfma32(k0, qf[DC / 16 + kk], sa);
        sb = mfma32(k1, qf[DC / 16 + kk + 1], sb);
      }

      // mask, scale, page max of each row over this wave's 32 tokens
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tokp = 32 * hb + 8 * (r >> 2) + 4 * lhi + (r & 3);
        const float x = (pg * BS + tokp < n_valid) ? (sa[r] + sb[r]) * p.scale_log2 : -INFINITY;
        sa[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (lane < 32) sm.red[hb][srow] = mx;
      if (tid == 0) sm.rescale = 0;
      __syncthreads();  // A

      const float m_page = fmaxf(sm.red[0][srow], sm.red[1][srow]);
      const bool raise = m_page > m_run + kRescaleSlack;  // always on the first page
      const float m_new = raise ? m_page : m_run;
      const float alpha = raise ? exp2f(m_run - m_new) : 1.0f;  // 0 on the first page
      m_run = m_new;
      float sum = 0.0f;
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = exp2f(sa[r] - m_new);
        const float e1 = exp2f(sa[r + 1] - m_new);
        sum += e0 + e1;
        pk[r >> 1] = (uint32_t)f32_to_bf16(e0) | ((uint32_t)f32_to_bf16(e1) << 16);
      }
      sum += __shfl_xor(sum, 32);
      l_run = l_run * alpha + sum;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 v;
        v.x = pk[2 * g4];
        v.y = pk[2 * g4 + 1];
        *reinterpret_cast<uint2*>(sm.p + srow * P_LD + 32 * hb + 8 * g4 + 4 * lhi) = v;
      }
      if (hb == 0) {
        if (lane < 32) sm.alpha[srow] = alpha;
        if (__any(raise) && lane == 0) sm.rescale = 1;
      }
      __syncthreads();  // B: P, alpha ready for the value waves

      __syncthreads();  // C: values done, next page landed
      if (pg + 1 < p1 && partial(pg + 1)) __syncthreads();
    }

    if (lane < 32) sm.red[hb][srow] = l_run;
    if (hb == 0 && lane < 32) sm.mrow[srow] = m_run;
    __syncthreads();  // E
    if (tid < ROWS) {
      const float lt = sm.red[0][tid] + sm.red[1][tid];
      const float v = (sm.mrow[tid] + log2f(lt)) * kLn2;
      if (direct) {
        if (p.lse != nullptr) p.lse[(size_t)b * TH + rb + tid] = v;
      } else {
        p.part_lse[((size_t)b * S + s) * TH + rb + tid] = v;
      }
    }
  } else {
    // =========================== value waves ===========================
    const int v = wave - 4;
    f32x16 o[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rt][dt][r] = 0.0f;

    for (int pg = p0; pg < p1; ++pg) {
      const int buf = (pg - p0) & 1;
      const bool more = (pg + 1) < p1;
      if (more) issue_page(pg + 1, buf ^ 1);
      const uint8_t* lat = sm.lat[buf];

      __syncthreads();  // A
      __syncthreads();  // B

      if (sm.rescale) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 al =
                *reinterpret_cast<const float4*>(&sm.alpha[32 * rt + 8 * r4 + 4 * lhi]);
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
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 pf0 = *reinterpret_cast<const bf16x8*>(sm.p + l32 * P_LD + 16 * kk + 8 * lhi);
        const bf16x8 pf1 =
            *reinterpret_cast<const bf16x8*>(sm.p + (32 + l32) * P_LD + 16 * kk + 8 * lhi);
        const int tk0 = 16 * kk + 8 * lhi;  // tokens tk0..tk0+7 of the page
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int dbyte = (128 * v + 32 * dt + l32) * 2;
          uint32_t vv[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const uint16_t v0 = *reinterpret_cast<const uint16_t*>(lat + (tk0 + i) * LAT_LD + dbyte);
            const uint16_t v1 =
                *reinterpret_cast<const uint16_t*>(lat + (tk0 + i + 1) * LAT_LD + dbyte);
            vv[i >> 1] = (uint32_t)v0 | ((uint32_t)v1 << 16);
          }
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
          o[0][dt] = mfma32(pf0, vf, o[0][dt]);
          o[1][dt] = mfma32(pf1, vf, o[1][dt]);
        }
      }

      wait_copies();
      __syncthreads();  // C
      if (more && partial(pg + 1)) {
        zero_tail(pg + 1, buf ^ 1);
        __syncthreads();
      }
    }

    __syncthreads();  // E
    float* dst = direct ? p.o_lat + ((size_t)b * TH + rb) * DC
                        : p.part_o + (((size_t)b * S + s) * TH + rb) * DC;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + 8 * (r >> 2) + 4 * lhi + (r & 3);
        const float inv = 1.0f / (sm.red[0][row] + sm.red[1][row]);
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
