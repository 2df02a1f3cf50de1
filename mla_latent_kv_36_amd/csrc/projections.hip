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
// batch sizes (M = sequences x new tokens is small, each head's weight is d_n x
// d_c or d_v x d_c).  For bf16 they run on MFMA (v_mfma_f32_16x16x32_bf16):
// a workgroup reads its head's weight slice from HBM once, keeps it in
// registers, and streams the query rows through it 16 at a time.  Both
// compute the transposed tile (weight as the A operand, rows as B), so that a
// lane ends up holding 4 consecutive output columns of one row: one 8-byte
// store.  fp32 accumulation throughout; the fp32 kernels below cover fp32
// caches and shapes outside the MFMA kernels' constraints.
//
// MFMA 16x16x32 operand layout (lane l): A row l & 15, k 8(l >> 4) .. +7;
// B column l & 15, the same k; D column l & 15, rows 4(l >> 4) .. +3.
#include "common.h"
#include "launch.h"
#include "merge.h"

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

// ------------------------------------------------------------------ MFMA ---

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint16_t)))) uint16_t u16x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each 16-lane group, lane 4k + q addresses element
// [r0 + k][c0 + 4q] of a row-major bf16 tile; lane i of the group receives
// [r0 .. r0 + 3][c0 + i].
__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const f32x4& v) {
  u16x4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16(v[i]);
  *reinterpret_cast<u16x4*>(p) = h;
}

constexpr int PJ_NT = 256;        // 4 waves
constexpr int PJ_MW = 64;         // query rows per workgroup for large M (4 tiles of 16)

// Query rows per workgroup.  A workgroup's rows past the first 16 are handled
// one tile after another, each tile's loads a memory round trip of its own,
// while the weight slice is read once per workgroup (more workgroups read it
// again, from L2).  Measured at 128 query rows: two tiles per workgroup beat
// one by ~1 us; up to 64 rows every workgroup takes a single tile.
__host__ __device__ inline int pj_rows_per_wg(int M) {
  return M <= 64 ? 16 : M <= 256 ? 32 : PJ_MW;
}
constexpr int AB_CT = 128;        // latent columns per absorb workgroup (32 per wave)
constexpr int AB_KS = 6;          // at most 6 k-steps of 32: d_nope <= 192 (55 KiB staged)
constexpr int AB_LD = 2 * AB_CT + 32;  // LDS row stride (bytes) of the staged weight
constexpr int OP_VT = 64;         // value columns per out-proj workgroup (16 per wave)
constexpr int OP_KS = 16;         // at most 16 k-steps of 32: d_c <= 512

// absorb_q on MFMA.  Workgroup (h, cb, mz): latent columns cb*128 .. +127 of
// head h for query rows mz*64 .. +63.  The weight slice W^UK[h][:, cols] is
// staged in LDS (rows past d_nope zeroed, so the contraction is padded to a
// multiple of 32), then each wave takes its 32 columns x all d_nope into
// registers with transposing reads: the A operand, rows = latent columns.
//
// With ap.rows > 0 the grid has ceil(ap.rows / 4) more workgroups along x,
// placed first, that append the new cache rows instead, one row per wave (the
// append of a decode step rides along with the absorb: one launch less).
// They come first in dispatch order so that their chain of dependent loads
// (length, page id, row) runs under the absorb rather than after it.
// NKS: k-steps of 32 covering d_nope (ceil(d_nope / 32)); NT: 16-row tiles per
// workgroup (mt / 16), whose query fragments are all requested at the start.
template <int NKS, int NT>
__global__ __launch_bounds__(PJ_NT) void absorb_q_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs, int M, int H, int d_n,
    int d_c, int d_r, int mt, const AppendArgs ap) {
  extern __shared__ __align__(16) uint8_t wl[];  // [KP][AB_LD]
  const int apx = (ap.rows + PJ_NT / 64 - 1) / (PJ_NT / 64);  // append workgroups along x
  if ((int)blockIdx.x < apx) {
    // row r = b * T_new + i goes to position seq_lens[b] + i; rows whose page
    // or page id is out of range are skipped (as mla_cache_append does)
    if (blockIdx.y != 0 || blockIdx.z != 0) return;
    const int r = (int)blockIdx.x * (PJ_NT / 64) + (int)(threadIdx.x >> 6);
    if (r >= ap.rows) return;
    const int b = r / ap.T_new, i = r - b * ap.T_new;
    const int pos = ap.seq_lens[b] + i;
    const int page = pos / ap.block_size;
    if (pos < 0 || page >= ap.max_blocks) return;
    const int blk = ap.table[(size_t)b * ap.max_blocks + page];
    if (blk < 0 || blk >= ap.num_blocks) return;
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(ap.pool) +
        ((size_t)blk * ap.block_size + (pos - page * ap.block_size)) * ap.row_bytes);
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const uint8_t*>(ap.new_rows) + (size_t)r * ap.row_bytes);
    for (int k = threadIdx.x & 63; k < ap.row_bytes / 16; k += 64) dst[k] = src[k];
    return;
  }
  const int h = (int)blockIdx.x - apx, cb = blockIdx.y;
  const int mbeg = blockIdx.z * mt, mend = min(M, mbeg + mt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  constexpr int nks = NKS;
  const int W = d_c + d_r;

  // B fragments (query rows) of every tile are requested before the weight,
  // so that all of the workgroup's loads are in flight together: one memory
  // latency per workgroup, not one per tile.
  // The loads are unconditional, on a clamped row and offset, and nothing is
  // selected on the loaded values (a select, like a conditional load, makes
  // the compiler wait for the load at once): rows past mend feed outputs that
  // are not stored, k-steps past d_n are not multiplied, and k past d_n
  // within the last step meets the zero rows of the staged weight.
  auto load_q = [&](int m0, bf16x8* bq) {
    const uint16_t* qrow = q_nope + ((size_t)min(m0 + i16, mend - 1) * H + h) * d_n;
#pragma unroll
    for (int ks = 0; ks < nks; ++ks) bq[ks] = load_bf16x8(qrow + min(32 * ks + 8 * g, d_n - 8));
  };
  bf16x8 bq[NT][AB_KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_q(mbeg + 16 * t, bq[t]);  // rows past mend: clamped

  // The rotary part is carried over unchanged (by the workgroups cb == 0),
  // 16 bytes at a time.  Its first pass of pieces is requested here, with the
  // other loads, so that the copy at the end costs no memory round trip of
  // its own (every workgroup requests it; it is a few KiB, mostly from L2).
  const int chunks = d_r / 8;
  const int nrope = (mend - mbeg) * chunks;
  u32x4 rv0 = {0u, 0u, 0u, 0u};
  if (chunks > 0) {  // q_rope may be absent when d_r = 0
    const int i = min(tid, nrope - 1);
    const int m = mbeg + i / chunks, r = 8 * (i % chunks);
    rv0 = *reinterpret_cast<const u32x4*>(q_rope + ((size_t)m * H + h) * d_r + r);
  }

  // the weight slice: every piece is loaded (unconditional) before the first
  // is stored, so staging costs one memory latency; nks * 32 rows of 16
  // pieces make exactly 2 * nks pieces per thread
  const uint16_t* wsrc = w_uk + (size_t)h * d_n * d_c + cb * AB_CT;
  constexpr int ST = nks * 32 * (AB_CT / 8) / PJ_NT;
  static_assert(ST * PJ_NT == nks * 32 * (AB_CT / 8), "whole passes");
  u32x4 sv[ST];
#pragma unroll
  for (int u = 0; u < ST; ++u) {
    const int i = tid + u * PJ_NT;
    const int d = i / (AB_CT / 8), ch = i % (AB_CT / 8);
    sv[u] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)min(d, d_n - 1) * d_c + ch * 8);
  }
  // every load is issued before the first is used
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < ST; ++u) {
    const int i = tid + u * PJ_NT;
    const int d = i / (AB_CT / 8), ch = i % (AB_CT / 8);
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(wl + d * AB_LD + ch * 16) = d < d_n ? sv[u] : z;
  }
  __syncthreads();

  bf16x8 a[2][AB_KS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int ks = 0; ks < AB_KS; ++ks) {
      if (ks < nks) {
        const int col = 32 * wave + 16 * ct + 4 * (i16 & 3);
        const int d = 32 * ks + 8 * g + (i16 >> 2);
        const s16x4 v0 = lds_tr16(wl + d * AB_LD + 2 * col);
        const s16x4 v1 = lds_tr16(wl + (d + 4) * AB_LD + 2 * col);
        // a plain concatenation: no instruction reads the loaded registers
        a[ct][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }

  const int col0 = cb * AB_CT + 32 * wave + 4 * g;  // + 16 ct: this lane's 4 columns
  // one 16-row tile whose query fragments are in q
  auto tile = [&](int m0, const bf16x8 (&q)[AB_KS]) __attribute__((always_inline)) {
    const int m = m0 + i16;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < nks; ++ks) {
      acc[0] = mfma16(a[0][ks], q[ks], acc[0]);
      acc[1] = mfma16(a[1][ks], q[ks], acc[1]);
    }
    if (m < mend) {
      uint16_t* dst = q_abs + ((size_t)m * H + h) * W + col0;
      store_bf16x4(dst, acc[0]);
      store_bf16x4(dst + 16, acc[1]);
    }
  };
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (mbeg + 16 * t < mend) tile(mbeg + 16 * t, bq[t]);

  if (cb == 0) {  // the rotary part: the first pass from registers, any further ones direct
    if (tid < nrope) {
      const int m = mbeg + tid / chunks, r = 8 * (tid % chunks);
      *reinterpret_cast<u32x4*>(q_abs + ((size_t)m * H + h) * W + d_c + r) = rv0;
    }
    for (int i = tid + PJ_NT; i < nrope; i += PJ_NT) {
      const int m = mbeg + i / chunks, r = 8 * (i % chunks);
      *reinterpret_cast<u32x4*>(q_abs + ((size_t)m * H + h) * W + d_c + r) =
          *reinterpret_cast<const u32x4*>(q_rope + ((size_t)m * H + h) * d_r + r);
    }
  }
}

// absorb_q for a large M.  Workgroup (h, mz): all 512 latent columns of head
// h for query rows mz*AW_MT .. +AW_MT-1, so that each query row (and its
// rotary part) is read by one workgroup, every output row is written whole,
// and the head's weight is staged once per AW_MT rows.  Wave w takes latent
// columns 128w .. 128w+127 (8 tiles of 16) x all d_nope into registers: the A
// operand, 32 NKS VGPRs per tile.
// Everything the workgroup reads is requested at its start, by direct-to-LDS
// copies: W^UK[h] in rounds of 64 rows (one 1 KiB weight row per copy; the
// waves take their fragments from each round with transposing reads) and the
// query rows (four 256-byte rows per copy).  The 16-row tiles then run with
// no memory wait at all: on this chip one counter covers loads and stores,
// and a load waited for behind the stores of earlier tiles would wait for
// those stores too.
constexpr int AW_DC = 512;
constexpr int AW_LD = 2 * AW_DC + 32;  // bytes per staged weight row
constexpr int AW_ROWS = 64;            // weight rows per round
constexpr int AW_MT = 256;             // query rows per workgroup
constexpr int AW_QLD = 256;            // bytes per staged query row (d_nope <= 128)

// NKS: k-steps of 32 covering d_nope (<= 4).
template <int NKS>
__global__ __launch_bounds__(PJ_NT) void absorb_q_wide_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs, int M, int H, int d_n,
    int d_r) {
  extern __shared__ __align__(16) uint8_t wl[];  // [AW_ROWS][AW_LD], then [AW_MT][AW_QLD]
  uint8_t* ql = wl + AW_ROWS * AW_LD;
  const int h = blockIdx.x;
  const int mbeg = blockIdx.y * AW_MT, mend = min(M, mbeg + AW_MT);
  const int ntiles = (mend - mbeg + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int i16 = lane & 15, g = lane >> 4;
  const int W = AW_DC + d_r;
  const uint32_t wl_base = (uint32_t)(uintptr_t)wl;
  const uint16_t* wh = w_uk + (size_t)h * d_n * AW_DC;

  // weight rows r0 .. r0+63 into LDS, wave w taking rows r0 + w + 4j; rows
  // past d_n are zeroed instead (the contraction is padded to 32 NKS rows)
  auto stage = [&](int r0) {
#pragma unroll
    for (int j = 0; j < AW_ROWS / 4; ++j) {
      const int d = r0 + wave + 4 * j;
      if (d < d_n)
        copy16_to_lds(reinterpret_cast<const uint8_t*>(wh + (size_t)d * AW_DC), lane * 16,
                      wl_base + (d - r0) * AW_LD);
    }
  };
  auto zero_rows = [&](int r0) {
    const int zb = max(r0, d_n), ze = min(r0 + AW_ROWS, 32 * NKS);
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < (ze - zb) * (AW_DC / 8); i += PJ_NT)
      *reinterpret_cast<u32x4*>(wl + (zb - r0 + i / (AW_DC / 8)) * AW_LD + 16 * (i % (AW_DC / 8))) = z;
  };
  stage(0);

  // Query rows: staged row r (query row mbeg + r, clamped to mend - 1) holds
  // its 16-byte chunk c at position c ^ (r & 15), so that the 16 rows of a
  // tile read at one chunk fall in distinct banks.  A copy fills four rows;
  // lane l fills position l & 15 of row 4i + (l >> 4) with the chunk that
  // belongs there (chunks past d_nope re-read the last one: finite values that
  // meet the zeroed weight rows).
  {
    const int nch = d_n >> 3;  // chunks per row
#pragma unroll
    for (int i = 0; i < AW_MT / 16; ++i) {
      const int r = 16 * i + 4 * wave + (lane >> 4);  // this lane's staged row
      const int c = min((lane & 15) ^ (r & 15), nch - 1);
      const uint32_t voff = (uint32_t)((((size_t)min(mbeg + r, mend - 1) - mbeg) * H * d_n + 8 * c) * 2);
      copy16_to_lds(reinterpret_cast<const uint8_t*>(q_nope + ((size_t)mbeg * H + h) * d_n), voff,
                    wl_base + AW_ROWS * AW_LD + (16 * i + 4 * wave) * AW_QLD);
    }
  }

  // The rotary part of the workgroup's rows (d_r <= 64: at most 8 chunks of
  // 16 bytes per row, 2048 for 256 rows, 8 per thread), carried over
  // unchanged while the rest is on its way: all loads, then all stores.
  // Unconditional loads on clamped chunks; only the stores are predicated.
  {
    const int rch = d_r >> 3;  // rotary chunks per row
    const int nrc = (mend - mbeg) * rch;
    constexpr int RT = AW_MT * 8 / PJ_NT;
    u32x4 rv[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int i = min(tid + u * PJ_NT, nrc - 1);
      rv[u] = *reinterpret_cast<const u32x4*>(
          q_rope + ((size_t)(mbeg + i / rch) * H + h) * d_r + 8 * (i % rch));
    }
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int i = tid + u * PJ_NT;
      if (i < nrc)
        *reinterpret_cast<u32x4*>(q_abs + ((size_t)(mbeg + i / rch) * H + h) * W + AW_DC +
                                  8 * (i % rch)) = rv[u];
    }
  }

  // A fragments of k-step ks from the staged round holding weight rows r0 ..
  bf16x8 a[8][NKS];
  auto take = [&](int ks, int r0) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int col = 128 * wave + 16 * ct + 4 * (i16 & 3);
      const int d = 32 * ks - r0 + 8 * g + (i16 >> 2);
      const s16x4 v0 = lds_tr16(wl + d * AW_LD + 2 * col);
      const s16x4 v1 = lds_tr16(wl + (d + 4) * AW_LD + 2 * col);
      // a plain concatenation: no instruction reads the loaded registers
      a[ct][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // every copy of this wave has landed (and the rotary loads: the stores above
  // have read them)
  wait_vmcnt<0>();
  zero_rows(0);
  lds_barrier();
#pragma unroll
  for (int ks = 0; ks < NKS && ks < 2; ++ks) take(ks, 0);
  if (NKS > 2) {
    lds_barrier();  // every wave has its fragments of round 0
    stage(AW_ROWS);
    wait_vmcnt<0>();
    zero_rows(AW_ROWS);
    lds_barrier();
#pragma unroll
    for (int ks = 2; ks < NKS; ++ks) take(ks, AW_ROWS);
  }

  const int col0 = 128 * wave + 4 * g;  // + 16 ct: this lane's 4 columns
  // B fragments of tile t (staged row 16t + i16), read one tile ahead
  auto read_b = [&](int t, bf16x8 (&bq)[NKS]) {
    const int r = 16 * min(t, ntiles - 1) + i16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      bq[ks] = *reinterpret_cast<const bf16x8*>(ql + r * AW_QLD + 16 * ((4 * ks + g) ^ (r & 15)));
  };
  bf16x8 bn[NKS];
  read_b(0, bn);
  for (int t = 0; t < ntiles; ++t) {
    const int r = 16 * t + i16;
    bf16x8 bq[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bq[ks] = bn[ks];
    read_b(t + 1, bn);
    f32x4 acc[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = mfma16(a[ct][ks], bq[ks], acc[ct]);
    const int m = mbeg + r;
    if (m < mend) {
      uint16_t* dst = q_abs + ((size_t)m * H + h) * W + col0;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) store_bf16x4(dst + 16 * ct, acc[ct]);
    }
  }
}

// out_proj on MFMA.  Workgroup (h, vb, mz): value columns vb*64 .. +63 of head h
// for query rows mz*64 .. +63; wave w holds W^UV[h][v][:] for its 16 columns v
// (the A operand, loaded straight from HBM: both operands are contiguous along
// the latent axis).  o_lat is fp32: each element is split once, when its
// 16-row tile is staged in LDS, as hi = bf16(x), lo = bf16(x - hi), and both
// halves are multiplied, so the product keeps about 16 significant bits of
// o_lat instead of 8.  Staged rows are padded by 16 bytes so that the 16
// rows a 16-lane group reads at one latent offset fall in distinct banks.
constexpr int OP_LD = 2 * 32 * OP_KS + 16;  // bytes per staged row (d_c <= 512)

__global__ __launch_bounds__(PJ_NT) void out_proj_mfma_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
    uint16_t* __restrict__ out, int M, int H, int d_c, int d_v, int mt) {
  __shared__ __align__(16) uint8_t st[2][16 * OP_LD];  // hi, lo
  const int h = blockIdx.x, vb = blockIdx.y;
  const int mbeg = blockIdx.z * mt, mend = min(M, mbeg + mt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int nks = d_c >> 5;
  const int vrow = vb * OP_VT + 16 * wave + i16;  // A row of this lane

  // The first tile of o_lat is requested before the weight: memory loads
  // complete in issue order, so its staging below then waits for it alone
  // while the weight is still in flight.  A thread's loads (up to OP_ST, on
  // clamped rows) are all issued before the first is used.
  const int q4 = d_c >> 2;                        // float4 chunks per row
  constexpr int OP_ST = 16 * (32 * OP_KS / 4) / PJ_NT;
  f32x4 xs[OP_ST];
  auto load_x = [&](int m0) {
#pragma unroll
    for (int u = 0; u < OP_ST; ++u) {
      const int i = min(tid + u * PJ_NT, 16 * q4 - 1);
      const int r = i / q4, c4 = i - r * q4;
      xs[u] = *reinterpret_cast<const f32x4*>(
          o_lat + ((size_t)min(m0 + r, mend - 1) * H + h) * d_c + 4 * c4);
    }
  };
  load_x(mbeg);

  // W^UV fragments: unconditional loads on a clamped row and k-step.  Rows
  // past d_v only feed outputs that are not stored and k-steps past d_c are
  // not multiplied, so nothing is selected on the loaded values (a select
  // would wait for each load at once).
  bf16x8 a[OP_KS];
  const uint16_t* wrow = w_uv + ((size_t)h * d_v + min(vrow, d_v - 1)) * d_c + 8 * g;
#pragma unroll
  for (int ks = 0; ks < OP_KS; ++ks) a[ks] = load_bf16x8(wrow + 32 * min(ks, nks - 1));
  // every load is issued before the first o_lat value is used
  __builtin_amdgcn_sched_barrier(0);

  const int v0 = vb * OP_VT + 16 * wave + 4 * g;  // this lane's 4 output columns
  // one 16-row tile whose o_lat is in xs
  auto tile = [&](int m0) __attribute__((always_inline)) {
    // stage rows m0 .. m0+15 (zeros past mend) as bf16 hi / lo
    // (branch-free: a clamped index rewrites the last chunk with the same
    // values, and rows past mend are zeroed by a select; a branch here would
    // make the compiler wait for the weight loads too)
#pragma unroll
    for (int u = 0; u < OP_ST; ++u) {
      const int i = min(tid + u * PJ_NT, 16 * q4 - 1);
      const int r = i / q4, c4 = i - r * q4;
      f32x4 x = xs[u];
      if (m0 + r >= mend) x = f32x4{0.f, 0.f, 0.f, 0.f};
      u16x4 hb, lb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hb[e] = f32_to_bf16(x[e]);
        lb[e] = f32_to_bf16(x[e] - bf16_to_f32(hb[e]));
      }
      *reinterpret_cast<u16x4*>(st[0] + r * OP_LD + 8 * c4) = hb;
      *reinterpret_cast<u16x4*>(st[1] + r * OP_LD + 8 * c4) = lb;
    }
    // the next tile's o_lat is requested now, so that its load runs under
    // this tile's MFMAs
    if (m0 + 16 < mend) load_x(m0 + 16);
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int boff = i16 * OP_LD + 16 * g;
#pragma unroll
    for (int ks = 0; ks < OP_KS; ++ks) {
      if (ks < nks) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(st[0] + boff + 64 * ks);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(st[1] + boff + 64 * ks);
        acc = mfma16(a[ks], bh, acc);
        acc = mfma16(a[ks], bl, acc);
      }
    }
    const int m = m0 + i16;
    if (m < mend) {
      uint16_t* dst = out + ((size_t)m * H + h) * d_v + v0;
      if (v0 + 3 < d_v) {
        store_bf16x4(dst, acc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + i < d_v) dst[i] = f32_to_bf16(acc[i]);
      }
    }
    __syncthreads();  // the next tile overwrites the staging buffer
  };
  // The first tile is straight-line code: at a loop head the compiler would
  // wait for the weight as well before staging it.
  tile(mbeg);
  for (int m0 = mbeg + 16; m0 < mend; m0 += 16) tile(m0);
}

// The log-sum-exp merge of the split partials and out_proj in one launch.
// Workgroup (h, vb, mz): value columns vb*128 .. +127 of head h for query
// rows mz*mt .. +mt-1, in tiles of MO_TR rows; 8 waves, wave w holding
// W^UV[h][v][:] for its 16 columns v (the A operand, as in
// out_proj_mfma_kernel).  Each tile of o_lat is not read but merged from the
// bf16 split partials (the merge kernel's per-row arithmetic, lane l taking
// latent columns 8l .. 8l+7) straight into the LDS staging, MO_TR / 8 query
// rows per wave with all of their loads in flight together; with d_v <= 128
// every partial is read once.  The
// staged values are the ones the merge kernel would have written to o_lat, so
// `out` equals the two launches' bit for bit.  Workgroups of vb = 0 write
// o_lat and lse as well (o_lat: streaming stores).
constexpr int MO_NT = 512;                  // 8 waves
constexpr int MO_VT = 16 * (MO_NT / 64);    // value columns per workgroup

// MO_TR: query rows per tile, 16 or 8 (the MFMA's 16 columns, half used): at
// 16 rows or fewer, tiles of 8 make two workgroups per head, so that the
// whole chip streams the partials and W^UV (each CU's share of the memory
// bandwidth is the limit, and the pair, 128 workgroups apart, shares an XCD's
// L2 for W^UV); with more rows, tiles of 16 keep the re-reads of W^UV down.
template <int MO_TR>
__global__ __launch_bounds__(MO_NT) void merge_out_proj_kernel(const DecodeParams p,
                                                               const uint16_t* __restrict__ w_uv,
                                                               uint16_t* __restrict__ out,
                                                               int d_v, int mt) {
  __shared__ __align__(16) uint8_t st[2][16 * OP_LD];  // hi, lo
  const int H = p.H, T = p.T;
  const int M = p.B * T;
  const int h = blockIdx.x, vb = blockIdx.y;
  const int mbeg = blockIdx.z * mt, mend = min(M, mbeg + mt);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int vrow = vb * MO_VT + 16 * wave + i16;  // A row of this lane
  constexpr int MO_RW = MO_TR / (MO_NT / 64);     // query rows each wave merges per tile

  // W^UV fragments first (clamped row: rows past d_v feed outputs that are
  // not stored), so that they are in flight with the first tile's partials
  bf16x8 a[OP_KS];
  const uint16_t* wrow = w_uv + ((size_t)h * d_v + min(vrow, d_v - 1)) * 512 + 8 * g;
#pragma unroll
  for (int ks = 0; ks < OP_KS; ++ks) a[ks] = load_bf16x8(wrow + 32 * ks);

  const int v0 = vb * MO_VT + 16 * wave + 4 * g;  // this lane's 4 output columns
  if constexpr (MO_TR < 16) {  // the staged rows past the tile's stay zero
    const u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = MO_TR + wave; r < 16; r += MO_NT / 64) {
      *reinterpret_cast<u16x8*>(st[0] + r * OP_LD + 16 * lane) = z;
      *reinterpret_cast<u16x8*>(st[1] + r * OP_LD + 16 * lane) = z;
    }
  }
  for (int m0 = mbeg; m0 < mend; m0 += MO_TR) {
    // query rows m0 + MO_RW wave + i (clamped to the last row: rows past mend
    // are merged again and staged as zeros); the sequence's splits from the
    // plan, as the merge kernel takes them
    int bq[MO_RW], tq[MO_RW], P0[MO_RW], S[MO_RW], ch[MO_RW];
    bool few = true;  // at most 8 splits in each of the rows
#pragma unroll
    for (int i = 0; i < MO_RW; ++i) {
      const int m = min(m0 + MO_RW * wave + i, mend - 1);
      bq[i] = m / T;
      tq[i] = m - bq[i] * T;
      if (p.plan != nullptr) {
        // scalar loads (the index is uniform): their wait leaves the vector
        // loads in flight
        const int32_t __attribute__((address_space(4)))* e =
            (const int32_t __attribute__((address_space(4)))*)p.plan + 4 * (size_t)bq[i];
        P0[i] = e[0];
        S[i] = e[1];
        ch[i] = e[2] * 32;
      } else {
        P0[i] = bq[i] * p.num_splits;
        S[i] = p.num_splits;
        ch[i] = p.chunk_rows;
      }
      // a sequence without splits has no visible row: its loads go to split
      // 0 with a count of 1, which then merges no split (o = 0, lse = -inf)
      if (S[i] == 0) {
        P0[i] = 0;
        S[i] = 1;
        ch[i] = 32;
      }
      few = few && S[i] <= 8;
    }
    f32x4 lo[MO_RW], hi[MO_RW];
    float lse[MO_RW];
    if (few) {
      Row8Loads L[MO_RW];
#pragma unroll
      for (int i = 0; i < MO_RW; ++i)
        row8_issue<false>(p, bq[i], tq[i] * H + h, lane, P0[i], S[i], L[i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MO_RW; ++i) row8_hold(L[i]);
#pragma unroll
      for (int i = 0; i < MO_RW; ++i)
        row8_finish(p, L[i], tq[i], lane, S[i], ch[i], lo[i], hi[i], lse[i]);
    } else {
      for (int i = 0; i < MO_RW; ++i)
        row_merge512<false>(p, bq[i], tq[i] * H + h, tq[i], lane, P0[i], S[i], ch[i], lo[i],
                            hi[i], lse[i]);
    }
    // stage as bf16 hi / lo (out_proj's split of an fp32 o_lat value)
#pragma unroll
    for (int i = 0; i < MO_RW; ++i) {
      const int r = MO_RW * wave + i, m = m0 + r;
      const bool live = m < mend;
      if (live && vb == 0) {
        float* ol = p.o_lat + ((size_t)m * H + h) * 512 + 8 * lane;
        __builtin_nontemporal_store(lo[i], reinterpret_cast<f32x4*>(ol));
        __builtin_nontemporal_store(hi[i], reinterpret_cast<f32x4*>(ol + 4));
        if (lane == 0 && p.lse != nullptr) p.lse[(size_t)m * H + h] = lse[i];
      }
      u16x8 hb, lb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = live ? (e < 4 ? lo[i][e] : hi[i][e - 4]) : 0.0f;
        hb[e] = f32_to_bf16(x);
        lb[e] = f32_to_bf16(x - bf16_to_f32(hb[e]));
      }
      *reinterpret_cast<u16x8*>(st[0] + r * OP_LD + 16 * lane) = hb;
      *reinterpret_cast<u16x8*>(st[1] + r * OP_LD + 16 * lane) = lb;
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int boff = i16 * OP_LD + 16 * g;
#pragma unroll
    for (int ks = 0; ks < OP_KS; ++ks) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(st[0] + boff + 64 * ks);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(st[1] + boff + 64 * ks);
      acc = mfma16(a[ks], bh, acc);
      acc = mfma16(a[ks], bl, acc);
    }
    const int m = m0 + i16;
    if (i16 < MO_TR && m < mend && v0 < d_v) {
      uint16_t* dst = out + ((size_t)m * H + h) * d_v + v0;
      if (v0 + 3 < d_v) {
        store_bf16x4(dst, acc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + i < d_v) dst[i] = f32_to_bf16(acc[i]);
      }
    }
    __syncthreads();  // the next tile overwrites the staging buffer
  }
}

// absorb_q_mfma_kernel for ceil(d_n / 32) k-steps (1 .. AB_KS)
hipError_t launch_absorb_kernel(dim3 grid, size_t shmem, hipStream_t stream,
                                const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint16_t* w_uk, uint16_t* q_abs, int M, int H, int d_n,
                                int d_c, int d_r, int mt, const AppendArgs& ap) {
#define AB_LAUNCH_T(K, T)                                                                  \
  hipLaunchKernelGGL((absorb_q_mfma_kernel<K, T>), grid, dim3(PJ_NT), shmem, stream, q_nope, \
                     q_rope, w_uk, q_abs, M, H, d_n, d_c, d_r, mt, ap)
#define AB_LAUNCH(K)                      \
  do {                                    \
    if (mt <= 16) AB_LAUNCH_T(K, 1);      \
    else if (mt <= 32) AB_LAUNCH_T(K, 2); \
    else AB_LAUNCH_T(K, 4);               \
  } while (0)
  if (mt > PJ_MW) return hipErrorInvalidValue;
  switch ((d_n + 31) >> 5) {
    case 1: AB_LAUNCH(1); break;
    case 2: AB_LAUNCH(2); break;
    case 3: AB_LAUNCH(3); break;
    case 4: AB_LAUNCH(4); break;
    case 5: AB_LAUNCH(5); break;
    case 6: AB_LAUNCH(6); break;
    default: return hipErrorInvalidValue;
  }
#undef AB_LAUNCH
#undef AB_LAUNCH_T
  return hipGetLastError();
}

bool absorb_mfma_fits(int d_n, int d_c, int d_r) {
  return d_c % AB_CT == 0 && d_n % 8 == 0 && d_n > 0 && d_n <= 32 * AB_KS && d_r % 8 == 0;
}

// the wide absorb kernel: d_c = 512, d_nope <= 128 (A fragments of 128 columns
// in registers, 256-byte staged query rows), d_rope <= 64
bool absorb_wide_fits(int M, int H, int d_n, int d_c, int d_r) {
  // (the query rows a workgroup stages lie within 2^32 bytes of its first)
  return M > 256 && (M + AW_MT - 1) / AW_MT <= 65535 && d_c == AW_DC && d_n % 8 == 0 &&
         d_n > 0 && d_n <= 128 && d_r % 8 == 0 && d_r > 0 && d_r <= 64 &&
         (long long)AW_MT * H * d_n * 2 < (1LL << 32);
}

hipError_t launch_absorb_wide(const uint16_t* q_nope, const uint16_t* q_rope,
                              const uint16_t* w_uk, uint16_t* q_abs, int M, int H, int d_n,
                              int d_r, hipStream_t stream) {
  const dim3 grid(H, (M + AW_MT - 1) / AW_MT);
  const size_t shmem = (size_t)AW_ROWS * AW_LD + (size_t)AW_MT * AW_QLD;
#define AW_LAUNCH(K)                                                                    \
  hipLaunchKernelGGL((absorb_q_wide_kernel<K>), grid, dim3(PJ_NT), shmem, stream, q_nope, \
                     q_rope, w_uk, q_abs, M, H, d_n, d_r)
  switch ((d_n + 31) >> 5) {
    case 1: AW_LAUNCH(1); break;
    case 2: AW_LAUNCH(2); break;
    case 3: AW_LAUNCH(3); break;
    case 4: AW_LAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef AW_LAUNCH
  return hipGetLastError();
}

bool out_proj_mfma_fits(int d_c, int d_v) {
  return d_c % 32 == 0 && d_c > 0 && d_c <= 32 * OP_KS && d_v % 4 == 0;
}

}  // namespace

hipError_t launch_absorb_q(int dtype, const void* q_nope, const void* q_rope, const void* w_uk,
                           void* q_abs, int M, int H, int d_n, int d_c, int d_r,
                           hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (dtype == 1 && absorb_wide_fits(M, H, d_n, d_c, d_r))
    return launch_absorb_wide((const uint16_t*)q_nope, (const uint16_t*)q_rope,
                              (const uint16_t*)w_uk, (uint16_t*)q_abs, M, H, d_n, d_r, stream);
  if (dtype == 1 && absorb_mfma_fits(d_n, d_c, d_r)) {
    const int mt = pj_rows_per_wg(M);
    const dim3 grid(H, d_c / AB_CT, (M + mt - 1) / mt);
    const size_t shmem = (size_t)((d_n + 31) & ~31) * AB_LD;
    return launch_absorb_kernel(grid, shmem, stream, (const uint16_t*)q_nope,
                                (const uint16_t*)q_rope, (const uint16_t*)w_uk, (uint16_t*)q_abs,
                                M, H, d_n, d_c, d_r, mt, AppendArgs{});
  }
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
  if (dtype == 1 && out_proj_mfma_fits(d_c, d_v)) {
    const int mt = pj_rows_per_wg(M);
    const dim3 grid(H, (d_v + OP_VT - 1) / OP_VT, (M + mt - 1) / mt);
    hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(PJ_NT), 0, stream, o_lat,
                       (const uint16_t*)w_uv, (uint16_t*)out, M, H, d_c, d_v, mt);
    return hipGetLastError();
  }
  const dim3 grid(H, (d_v + OP_T - 1) / OP_T, (M + OP_T - 1) / OP_T);
  if (dtype == 0)
    hipLaunchKernelGGL(out_proj_kernel<float>, grid, dim3(256), 0, stream, o_lat,
                       (const float*)w_uv, (float*)out, M, H, d_c, d_v);
  else
    hipLaunchKernelGGL(out_proj_kernel<uint16_t>, grid, dim3(256), 0, stream, o_lat,
                       (const uint16_t*)w_uv, (uint16_t*)out, M, H, d_c, d_v);
  return hipGetLastError();
}

bool merge_out_proj_supported(int dtype, int d_c, int d_v) {
  return dtype == 1 && d_c == 512 && out_proj_mfma_fits(d_c, d_v);
}

hipError_t launch_merge_out_proj(const DecodeParams& p, const void* w_uv, void* out, int d_v,
                                 hipStream_t stream) {
  const int M = p.B * p.T;
  if (M <= 0) return hipSuccess;
  if (!p.part_bf16 || p.d_c != 512 || !out_proj_mfma_fits(512, d_v) || p.o_lat == nullptr)
    return hipErrorInvalidValue;
  const int mt = M <= 16 ? 8 : pj_rows_per_wg(M);
  const dim3 grid(p.H, (d_v + MO_VT - 1) / MO_VT, (M + mt - 1) / mt);
  if (M <= 16)
    hipLaunchKernelGGL(merge_out_proj_kernel<8>, grid, dim3(MO_NT), 0, stream, p,
                       (const uint16_t*)w_uv, (uint16_t*)out, d_v, mt);
  else
    hipLaunchKernelGGL(merge_out_proj_kernel<16>, grid, dim3(MO_NT), 0, stream, p,
                       (const uint16_t*)w_uv, (uint16_t*)out, d_v, mt);
  return hipGetLastError();
}

hipError_t launch_absorb_q_append(int dtype, const void* q_nope, const void* q_rope,
                                  const void* w_uk, void* q_abs, int M, int H, int d_n, int d_c,
                                  int d_r, const AppendArgs& ap, hipStream_t stream) {
  const long long extra = ((long long)ap.rows + PJ_NT / 64 - 1) / (PJ_NT / 64);
  // a large M takes the wide absorb kernel, then the append on its own
  if (M > 0 && ap.rows > 0 && dtype == 1 && !absorb_wide_fits(M, H, d_n, d_c, d_r) &&
      absorb_mfma_fits(d_n, d_c, d_r) &&
      ap.row_bytes % 16 == 0 && (long long)H + extra <= 0x7fffffffLL) {
    const int mt = pj_rows_per_wg(M);
    const dim3 grid((unsigned)(H + extra), d_c / AB_CT, (M + mt - 1) / mt);
    const size_t shmem = (size_t)((d_n + 31) & ~31) * AB_LD;
    return launch_absorb_kernel(grid, shmem, stream, (const uint16_t*)q_nope,
                                (const uint16_t*)q_rope, (const uint16_t*)w_uk, (uint16_t*)q_abs,
                                M, H, d_n, d_c, d_r, mt, ap);
  }
  hipError_t e = launch_absorb_q(dtype, q_nope, q_rope, w_uk, q_abs, M, H, d_n, d_c, d_r, stream);
  if (e != hipSuccess || ap.rows <= 0) return e;
  return launch_append(ap.pool, ap.num_blocks, ap.table, ap.max_blocks, ap.seq_lens, ap.new_rows,
                       ap.rows / ap.T_new, ap.T_new, ap.block_size, ap.row_bytes, stream);
}

}  // namespace mla
