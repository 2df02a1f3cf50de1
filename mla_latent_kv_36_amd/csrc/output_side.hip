// The output side of latent attention on CDNA4 (gfx950).
//
//   y = W^O x,  x = the per-head outputs of a token, head after head
//       ("Attention, Part 2: MQA, GQA and MLA", section "The trick that makes
//       it fast": the inference code reshapes the heads of a token into one
//       vector and applies W_o);
//   W_fold[:, h*d_c + c] = sum_v W^O[:, h*d_v + v] W^UV[h, v, c]
//       (the output-side absorption: "How DeepSeek Rewrote the Transformer",
//       section "Absorbed projections: the mathematician's shortcut", point
//       2), and y = W_fold z with z the latent outputs of a token, head after
//       head.
//
// Both projections are one product y[M, N] = X[M, K] . W[N, K]^T with both
// operands contiguous along k: X the token rows (bf16 per-head outputs, or the
// fp32 latent outputs for the folded matrix), W the weight (bf16).  At decode
// batch sizes M is small and W is the bytes that bound the call (W^O is 52 MB
// at the V2-scale width, the folded matrix 671 MB), so the kernel is a weight
// stream on v_mfma_f32_16x16x32_bf16:
//   * a workgroup owns 64 weight rows x 64 tokens over one k range, stages
//     64 x 256 chunks of both operands in LDS, and issues the next chunk's
//     loads before the current chunk's MFMAs;
//   * the weight is the A operand and the tokens the B operand, so that a
//     lane ends up with 4 consecutive outputs of one token (one 8-byte bf16
//     store, or one 16-byte partial store);
//   * tiles are numbered token tile fastest and placed XCD by XCD, so that
//     the token tiles that read one weight slice run side by side on one XCD
//     and share its L2;
//   * the k dimension is split over workgroups when the tiles alone would
//     leave compute units idle; the splits' fp32 partial sums are then added
//     in split order by a second kernel (deterministic);
//   * 17 to 128 token rows (fp32 ones rounded to bf16 first, in a launch of
//     their own) take a streaming form instead: all tokens in
//     one tile and 128 weight rows per workgroup, both operands brought in by
//     direct-to-LDS copies through a ring several chunks deep (below);
//     up to 16 tokens take a form with no LDS (below).
// fp32 token rows are rounded to bf16 when staged (the product is bf16 x bf16
// with fp32 accumulation either way).  fp32 weights and other shapes take a
// one-thread-per-output kernel.  The fold is a one-time weight preparation and
// runs on the VALU in fp32.
#include "common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int WO_TM = 64;          // tokens per workgroup tile
constexpr int WO_TN = 64;          // weight rows (outputs) per workgroup tile
constexpr int WO_KC = 256;         // k per LDS chunk (8 MFMA k-steps)
constexpr int WO_LD = WO_KC + 8;   // bf16 per LDS row: 528 B
constexpr int WO_PIECES = WO_KC / 8;               // 16-byte bf16 pieces per row
constexpr int WO_PER = WO_TM * WO_PIECES / 256;    // pieces per thread and operand
constexpr int WO_NT = 256;         // threads of the direct kernel: 4 waves x 16 weight rows
constexpr int WO_DEPTH = 4;        // direct kernel: chunks of 4 k steps in flight per wave
constexpr int WO_DC = 8;           // direct kernel: chunks per k split (32 k steps)
// 16 zero bytes in global memory (never written): the weight fragment of a
// step past the range
__device__ __align__(16) uint32_t kZero16[4] = {0u, 0u, 0u, 0u};

typedef __attribute__((__vector_size__(4 * sizeof(uint16_t)))) uint16_t u16x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive token-row elements as 8 bf16 (fp32 rows are rounded here)
__device__ __forceinline__ uint4 load_piece(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 load_piece(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(b[0]) | ((uint32_t)f32_to_bf16(b[1]) << 16);
  r.w = (uint32_t)f32_to_bf16(b[2]) | ((uint32_t)f32_to_bf16(b[3]) << 16);
  return r;
}

// With y != nullptr (one k split): y[m, n] = sum_k x[m, k] w[n, k], rounded to
// bf16.  Otherwise part[z, m, n] = the same sum over split z's k range.
// Requires K % 32 == 0 and N % 4 == 0.
template <typename XE>
__global__ __launch_bounds__(256, 2) void wo_gemm_mfma_kernel(
    const XE* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int N, int K, int steps_per_split, int xcds) {
  __shared__ __align__(16) uint16_t sx[WO_TM * WO_LD];
  __shared__ __align__(16) uint16_t sw[WO_TN * WO_LD];
  // Workgroup i runs on XCD i % xcds (queried on the host).  XCD x takes a
  // contiguous block of the tile numbers (ids past the last full set of xcds
  // keep the plain order).
  const int ntm = (M + WO_TM - 1) / WO_TM;
  const int ntn = (N + WO_TN - 1) / WO_TN;
  const int total = (int)gridDim.x;
  const int full = total - total % xcds;
  const int i = blockIdx.x;
  const int t = i < full ? (i % xcds) * (full / xcds) + i / xcds : i;
  const int m0 = (t % ntm) * WO_TM;
  const int n0 = ((t / ntm) % ntn) * WO_TN;
  const int z = t / (ntm * ntn);
  const int nk = K / 32;
  const int s_begin = z * steps_per_split;
  const int s_end = min(s_begin + steps_per_split, nk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A chunk: 64 rows x up to 256 k of both operands in 16-byte pieces, 32 per
  // row (a wave covers two rows, 1 KB contiguous per operand); the next
  // chunk's loads are issued before this chunk's MFMAs.  Every load is
  // unconditional (a conditional load makes the compiler wait for all loads
  // in flight): rows past M or N are read clamped and feed outputs that are
  // not stored, and weight pieces past the split are read from a block of
  // zeros (their token pieces, clamped, are finite).  A second chunk in
  // flight was measured slower.
  uint4 vx[WO_PER], vw[WO_PER];
  auto load_chunk = [&](int sc) {
    const int steps = min(WO_KC / 32, s_end - sc);
    const int k0 = sc * 32;
#pragma unroll
    for (int u = 0; u < WO_PER; ++u) {
      const int q = tid + 256 * u;
      const int r = q / WO_PIECES, c = q % WO_PIECES;
      const bool kin = c < steps * 4;
      const int kk = k0 + 8 * c;
      vx[u] = load_piece(x + (size_t)min(m0 + r, M - 1) * K + min(kk, K - 8));
      vw[u] = load_piece(kin ? w + (size_t)min(n0 + r, N - 1) * K + kk
                             : reinterpret_cast<const uint16_t*>(kZero16));
    }
  };
  const int l16 = lane & 15;
  const int kq = 8 * (lane >> 4);
  load_chunk(s_begin);
  for (int sc = s_begin; sc < s_end; sc += WO_KC / 32) {
    const int steps = min(WO_KC / 32, s_end - sc);
#pragma unroll
    for (int u = 0; u < WO_PER; ++u) {
      const int q = tid + 256 * u;
      const int r = q / WO_PIECES, c = q % WO_PIECES;
      *reinterpret_cast<uint4*>(&sx[r * WO_LD + 8 * c]) = vx[u];
      *reinterpret_cast<uint4*>(&sw[r * WO_LD + 8 * c]) = vw[u];
    }
    __syncthreads();
    load_chunk(sc + WO_KC / 32);   // past the split: zero weight pieces, never used
    // wave w: weight rows 16w + (l & 15) (A), tokens 16j + (l & 15) (B), k
    // 32s + 8(l >> 4) .. +7
    for (int s = 0; s < steps; ++s) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(&sw[(16 * wave + l16) * WO_LD + 32 * s + kq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sx[(16 * j + l16) * WO_LD + 32 * s + kq]);
        acc[j] = mfma16(a, b, acc[j]);
      }
    }
    __syncthreads();
  }
  // D: lane l holds token 16j + (l & 15), outputs 16w + 4(l >> 4) .. +3
  const int n = n0 + 16 * wave + 4 * (lane >> 4);
  if (n >= N) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 16 * j + l16;
    if (m >= M) continue;
    if (y != nullptr) {
      u16x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(acc[j][e]);
      *reinterpret_cast<u16x4*>(y + (size_t)m * N + n) = h;
    } else {
      *reinterpret_cast<f32x4*>(part + ((size_t)z * M + m) * N + n) = acc[j];
    }
  }
}

// The same product for at most 16 tokens, with no LDS and no barrier: each
// wave loads its own A fragments (16 weight rows, row l & 15, k 8(l >> 4) ..
// +7 of each 32-k step) and the B fragments of the 16 token rows straight
// into a register ring WO_DEPTH chunks of 4 k steps deep.  A chunk's MFMAs
// wait only for that chunk's loads; the token rows, the same for every wave,
// come from the caches.  A split is at most WO_DC chunks (the k split makes
// it so), loaded on clamped indices; the steps past the range multiply a
// weight fragment of zeros.
template <typename XE>
__global__ __launch_bounds__(WO_NT) void wo_stream_direct_kernel(
    const XE* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int N, int K, int steps_per_split, int xcds) {
  const int ntn = (N + WO_TN - 1) / WO_TN;
  const int total = (int)gridDim.x;
  const int full = total - total % xcds;
  const int i = blockIdx.x;
  const int t = i < full ? (i % xcds) * (full / xcds) + i / xcds : i;
  const int n0 = (t % ntn) * WO_TN;
  const int z = t / ntn;
  const int nk = K / 32;
  const int s_begin = z * steps_per_split;
  const int nsteps = min(s_begin + steps_per_split, nk) - s_begin;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const uint16_t* wrow = w + (size_t)min(n0 + 16 * wave + l16, N - 1) * K + 32 * s_begin + 8 * g;
  const XE* xrow = x + (size_t)min(l16, M - 1) * K + 32 * s_begin + 8 * g;
  // steps past the range read their weight fragment from a block of zeros
  // (an address select: selecting the loaded value instead would make the
  // compiler branch around the load and wait for it)
  auto load = [&](int c, bf16x8* a, bf16x8* b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int st = 4 * c + s;
      const int off = 32 * min(st, nsteps - 1);
      const uint16_t* pa = st < nsteps ? wrow + off : reinterpret_cast<const uint16_t*>(kZero16);
      a[s] = *reinterpret_cast<const bf16x8*>(pa);
      b[s] = __builtin_bit_cast(bf16x8, load_piece(xrow + off));
    }
  };
  bf16x8 wa[WO_DEPTH][4], xb[WO_DEPTH][4];
#pragma unroll
  for (int d = 0; d < WO_DEPTH; ++d) load(d, wa[d], xb[d]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // straight-line code over the split's WO_DC chunks: with a loop, the
  // compiler waits for every load in flight at the loop head
#pragma unroll
  for (int c = 0; c < WO_DC; ++c) {
    const int d = c % WO_DEPTH;
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16(wa[d][s], xb[d][s], acc);
    if (c + WO_DEPTH < WO_DC) {
      // the refill stays right here: hoisted above the MFMAs, its data
      // would be waited for at once
      __builtin_amdgcn_sched_barrier(0);
      load(c + WO_DEPTH, wa[d], xb[d]);   // clamped past the range
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const int n = n0 + 16 * wave + 4 * g;
  const int m = l16;
  if (n >= N || m >= M) return;
  if (y != nullptr) {
    u16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(acc[e]);
    *reinterpret_cast<u16x4*>(y + (size_t)m * N + n) = h;
  } else {
    *reinterpret_cast<f32x4*>(part + ((size_t)z * M + m) * N + n) = acc;
  }
}

// The same product for 16 < M <= 128 token rows (bf16, or fp32 rows rounded
// to bf16 by wo_round_x_kernel first): every token in one tile, so the
// weight is streamed once, and 128 weight rows per workgroup.
// The token rows are read again by every workgroup (from L2), half of the
// bytes a workgroup moves; in exchange the k range needs half as many splits
// for the same number of workgroups, which halves the fp32 partial sums
// written and read back (at 128 tokens and a 5,120 x 5,120 weight: 15.7 MB
// instead of 31.5 MB for 256 rows; measured 26.8 against 30.0 us, while 64
// rows, 7.9 MB of partials, took 31.7 us).  Workgroup (128 weight rows, k
// split): the k range is cut into chunks of one MFMA k-step (32 k); each
// chunk's 128 weight rows and 128 token rows (clamped to M - 1) reach LDS as
// direct-to-LDS copies (sixteen 64-byte rows per copy; 16-byte chunk c of
// row r at position
// c ^ ((r >> 2) & 3), so that the 16 rows an operand reads at one k fall in
// distinct banks) through a ring of WS_SLOTS slots, WS_SLOTS - 1 chunks ahead
// of the MFMAs: the bytes in flight per compute unit, which bound its rate
// at this latency (a deeper ring, 8 or 9 slots, was slower).  Wave w takes
// weight rows 32w .. 32w+31 (2 A tiles) against the 8 token tiles (B).
// Copies past the split's k range re-read clamped, finite values that are
// not multiplied.
constexpr int WS_AT_ = 2;                // 16-row weight tiles per wave
constexpr int WS_TN = 64 * WS_AT_;       // weight rows per workgroup (128)
constexpr int WS_TM = 128;      // token rows (all of them)
constexpr int WS_SLOTS = 6;
constexpr int WS_ROW = 64;                              // bytes per staged row (32 k)
constexpr int WS_SLOT = (WS_TM + WS_TN) * WS_ROW;       // 16 KiB
constexpr int WS_COPIES = (WS_TM + WS_TN) / 16 / 4;     // copies per wave per chunk (4)

template <int N_>
__device__ __forceinline__ void wait_copies_ahead(int ahead) {
  // this wave's copies of all but the `ahead` most recent chunks have landed
  if (ahead >= 5) wait_vmcnt<5 * N_>();
  else if (ahead == 4) wait_vmcnt<4 * N_>();
  else if (ahead == 3) wait_vmcnt<3 * N_>();
  else if (ahead == 2) wait_vmcnt<2 * N_>();
  else if (ahead == 1) wait_vmcnt<N_>();
  else wait_vmcnt<0>();
}

__global__ __launch_bounds__(256) void wo_stream_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int N, int K, int steps_per_split, int xcds) {
  extern __shared__ __align__(16) uint8_t ring[];  // [WS_SLOTS][token rows, then weight rows][64 B]
  const int ntn = (N + WS_TN - 1) / WS_TN;
  const int total = (int)gridDim.x;
  const int full = total - total % xcds;
  const int i = blockIdx.x;
  const int t = i < full ? (i % xcds) * (full / xcds) + i / xcds : i;
  const int n0 = (t % ntn) * WS_TN;
  const int z = t / ntn;
  const int nk = K / 32;
  const int s_begin = z * steps_per_split;
  const int nchunks = min(steps_per_split, nk - s_begin);  // one k-step per chunk
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t ring_base = (uint32_t)(uintptr_t)ring;

  // copies of chunk c into slot c % WS_SLOTS: staged row q < 128 is token row
  // q, q >= 128 weight row n0 + q - 128; copy j of wave w fills rows
  // 16(w + 4j) .. +15, lane l row 16(w + 4j) + (l >> 2), position l & 3
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w + (size_t)n0 * K);
  auto issue = [&](int c) {
    const int kbase = 32 * (s_begin + c);
    const uint32_t slot = ring_base + (c % WS_SLOTS) * WS_SLOT;
#pragma unroll
    for (int j = 0; j < WS_COPIES; ++j) {
      const int q0 = 16 * (wave + 4 * j);       // first staged row of this copy (uniform)
      const int q = q0 + (lane >> 2);           // this lane's row
      const int ch = (lane & 3) ^ ((q >> 2) & 3);  // the chunk that belongs at its position
      const int k = kbase + 8 * ch;
      if (q0 < WS_TM) {
        const uint32_t voff = (uint32_t)(((size_t)min(q, M - 1) * K + k) * 2);
        copy16_to_lds(xb, voff, slot + q0 * WS_ROW);
      } else {
        const uint32_t voff = (uint32_t)(((size_t)min(q - WS_TM, N - 1 - n0) * K + k) * 2);
        copy16_to_lds(wb, voff, slot + q0 * WS_ROW);
      }
    }
  };

  f32x4 acc[WS_AT_][WS_TM / 16];
#pragma unroll
  for (int at = 0; at < WS_AT_; ++at)
#pragma unroll
    for (int j = 0; j < WS_TM / 16; ++j) acc[at][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < WS_SLOTS - 1; ++c)
    if (c < nchunks) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    wait_copies_ahead<WS_COPIES>(min(WS_SLOTS - 2, nchunks - 1 - c));
    lds_barrier();  // every wave's copies of chunk c; every wave done with chunk c-1
    if (c + WS_SLOTS - 1 < nchunks) issue(c + WS_SLOTS - 1);  // into chunk c-1's slot
    const uint8_t* sl = ring + (c % WS_SLOTS) * WS_SLOT;
    // operand rows R read here have (R >> 2) & 3 == (l16 >> 2) & 3 (R = 16 k + l16)
    const int off = 16 * (g ^ ((l16 >> 2) & 3));
    bf16x8 a[WS_AT_];
#pragma unroll
    for (int at = 0; at < WS_AT_; ++at)
      a[at] = *reinterpret_cast<const bf16x8*>(
          sl + (WS_TM + 16 * WS_AT_ * wave + 16 * at + l16) * WS_ROW + off);
#pragma unroll
    for (int j = 0; j < WS_TM / 16; ++j) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sl + (16 * j + l16) * WS_ROW + off);
#pragma unroll
      for (int at = 0; at < WS_AT_; ++at) acc[at][j] = mfma16(a[at], b, acc[at][j]);
    }
  }
  // D: lane l holds token 16j + (l & 15), outputs 32w + 16at + 4(l >> 4) .. +3
#pragma unroll
  for (int at = 0; at < WS_AT_; ++at) {
    const int n = n0 + 16 * WS_AT_ * wave + 16 * at + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < WS_TM / 16; ++j) {
      const int m = 16 * j + l16;
      if (m >= M) continue;
      if (y != nullptr) {
        u16x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(acc[at][j][e]);
        *reinterpret_cast<u16x4*>(y + (size_t)m * N + n) = h;
      } else {
        *reinterpret_cast<f32x4*>(part + ((size_t)z * M + m) * N + n) = acc[at][j];
      }
    }
  }
}

// fp32 token rows rounded to bf16 (round to nearest even, as the tiled
// kernel rounds them when it stages them): 8 values per thread, n8 = n / 8.
__global__ __launch_bounds__(256) void wo_round_x_kernel(const float* __restrict__ x,
                                                         uint16_t* __restrict__ x16,
                                                         size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(x + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(x + 8 * i + 4);
  u16x8 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f32_to_bf16(a[e]);
    h[e + 4] = f32_to_bf16(b[e]);
  }
  *reinterpret_cast<u16x8*>(x16 + 8 * i) = h;
}

// y[m, n .. n+3] = sum over splits z (in order) of part[z, m, n .. n+3],
// rounded to bf16; one thread per 4 outputs.  The loads of up to 16 splits
// are issued (on clamped indices) before the first is added.
__global__ __launch_bounds__(256) void wo_finish_kernel(const float* __restrict__ part,
                                                        uint16_t* __restrict__ y, int M, int N,
                                                        int ksplit) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)M * N / 4;
  if (q >= total) return;
  const size_t MN = (size_t)M * N;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < ksplit; z0 += 16) {
    f32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = *reinterpret_cast<const f32x4*>(part + (size_t)min(z0 + k, ksplit - 1) * MN + 4 * q);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (z0 + k < ksplit) {
        s[0] += v[k][0];
        s[1] += v[k][1];
        s[2] += v[k][2];
        s[3] += v[k][3];
      }
    }
  }
  u16x4 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(s[e]);
  *reinterpret_cast<u16x4*>(y + 4 * q) = h;
}

// Any element types and shape: one thread per output, the whole dot product
// in fp32, rounded once.
template <typename XE, typename WE>
__global__ __launch_bounds__(256) void wo_gemm_generic_kernel(const XE* __restrict__ x,
                                                              const WE* __restrict__ w,
                                                              WE* __restrict__ y, int M, int N,
                                                              int K) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const WE* wr = w + (size_t)n * K;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const XE* xr = x + (size_t)m * K;
    float s = 0.0f;
    for (int k = 0; k < K; ++k) s += Elem<XE>::load(xr, k) * Elem<WE>::load(wr, k);
    Elem<WE>::store(y, (size_t)m * N + n, s);
  }
}

constexpr int FOLD_R = 16;    // rows of W^O per workgroup
constexpr int FOLD_VMAX = 256;

// W_fold[i, h*d_c + c] = sum_v W^O[i, h*d_v + v] W^UV[h, v, c] in fp32, rounded
// once.  Workgroup (c block, i block, h): thread c, rows i0 .. i0+15; the 16 x
// d_v block of W^O is staged in LDS (d_v <= 256), W^UV[h, v, c] is read along
// c (coalesced).
template <typename E>
__global__ __launch_bounds__(256) void fold_uv_o_kernel(const E* __restrict__ w_uv,
                                                        const E* __restrict__ w_o,
                                                        E* __restrict__ w_fold, int H, int d_v,
                                                        int d_c, int d) {
  __shared__ float so[FOLD_R * FOLD_VMAX];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int i0 = blockIdx.y * FOLD_R;
  const int h = blockIdx.z;
  const int rows = min(FOLD_R, d - i0);
  for (int q = threadIdx.x; q < FOLD_R * d_v; q += 256) {
    const int r = q / d_v, v = q - r * d_v;
    so[r * FOLD_VMAX + v] =
        r < rows ? Elem<E>::load(w_o, (size_t)(i0 + r) * H * d_v + (size_t)h * d_v + v) : 0.0f;
  }
  __syncthreads();
  if (c >= d_c) return;
  float acc[FOLD_R];
#pragma unroll
  for (int r = 0; r < FOLD_R; ++r) acc[r] = 0.0f;
  const E* uv = w_uv + (size_t)h * d_v * d_c + c;
  for (int v = 0; v < d_v; ++v) {
    const float u = Elem<E>::load(uv, (size_t)v * d_c);
#pragma unroll
    for (int r = 0; r < FOLD_R; ++r) acc[r] += so[r * FOLD_VMAX + v] * u;
  }
  const size_t ld = (size_t)H * d_c;
#pragma unroll
  for (int r = 0; r < FOLD_R; ++r)
    if (r < rows) Elem<E>::store(w_fold, (size_t)(i0 + r) * ld + (size_t)h * d_c + c, acc[r]);
}

}  // namespace

bool wo_gemm_mfma_supported(int dtype, int N, int K) {
  return dtype == 1 && K > 0 && K % 32 == 0 && N > 0 && N % 4 == 0;
}

// bf16 token rows, 16 < M <= 128: the weight-streaming kernel with every token
// in one tile (its 144 KiB of LDS allow one workgroup per compute unit, and a
// compute unit streams at the rate its bytes in flight allow: measured, half
// as many workgroups with twice the k range each run slower; the staged rows
// of a workgroup lie within 2^32 bytes of its first)
static bool wo_stream_lds_fits(int dtype, bool x_f32, int M, int N, int K) {
  (void)x_f32;  // fp32 token rows are rounded to bf16 first, into the workspace
  return wo_gemm_mfma_supported(dtype, N, K) && M > 16 && M <= WS_TM &&
         (long long)WS_TM * K * 2 < (1LL << 32) && (long long)WS_TN * K * 2 < (1LL << 32);
}

// Bytes of the bf16 copy of fp32 token rows that the streaming kernel reads
// (placed first in the workspace, the split partial sums after it), or 0.
// Rounding once up front lets every workgroup stream the rows as 64-byte bf16
// pieces, where the tiled kernel would re-read them as fp32 for each 64-row
// weight tile (the folded product at 128 tokens: 208 against 380 us).
static size_t wo_x16_bytes(int dtype, bool x_f32, int M, int N, int K) {
  if (!x_f32 || !wo_stream_lds_fits(dtype, x_f32, M, N, K)) return 0;
  return ((size_t)M * K * 2 + 255) / 256 * 256;
}

int wo_gemm_ksplit(int dtype, bool x_f32, int M, int N, int K, int target_workgroups) {
  if (!wo_gemm_mfma_supported(dtype, N, K) || M <= 0) return 1;
  // up to 16 tokens: the direct kernel, WO_DC chunks of 4 k steps per split
  if (M <= 16) return (K / 32 + 4 * WO_DC - 1) / (4 * WO_DC);
  if (wo_stream_lds_fits(dtype, x_f32, M, N, K)) {
    // one workgroup per compute unit (target_workgroups counts two)
    const long long tiles = (N + WS_TN - 1) / WS_TN;
    const int nk = K / 32;
    long long ks = (target_workgroups / 2) / tiles;
    if (ks < 1) ks = 1;
    if (ks > nk) ks = nk;
    const int per = (int)((nk + ks - 1) / ks);
    return (nk + per - 1) / per;
  }
  const long long tiles = (long long)((N + WO_TN - 1) / WO_TN) * ((M + WO_TM - 1) / WO_TM);
  const int nk = K / 32;
  long long ks = (target_workgroups + tiles - 1) / tiles;
  if (ks < 1) ks = 1;
  if (ks > nk) ks = nk;
  const int per = (int)((nk + ks - 1) / ks);
  return (nk + per - 1) / per;
}

size_t wo_gemm_workspace_bytes(int dtype, bool x_f32, int M, int N, int K, int ksplit) {
  const size_t parts = ksplit > 1 ? ((size_t)ksplit * M * N * sizeof(float) + 255) / 256 * 256 : 0;
  return wo_x16_bytes(dtype, x_f32, M, N, K) + parts;
}

hipError_t launch_wo_gemm(int dtype, bool x_f32, const void* x, const void* w, void* y,
                          float* part, int ksplit, int M, int N, int K, int xcds,
                          hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (xcds < 1) xcds = 1;
  if (wo_gemm_mfma_supported(dtype, N, K) && M <= 16) {
    const int nk = K / 32;
    if (ksplit != (nk + 4 * WO_DC - 1) / (4 * WO_DC)) return hipErrorInvalidValue;
    const long long tiles = (long long)((N + WO_TN - 1) / WO_TN) * ksplit;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    if (ksplit > 1 && part == nullptr) return hipErrorInvalidValue;
    uint16_t* yd = ksplit == 1 ? static_cast<uint16_t*>(y) : nullptr;
    if (x_f32)
      hipLaunchKernelGGL(wo_stream_direct_kernel<float>, dim3((unsigned)tiles), dim3(WO_NT), 0,
                         stream, static_cast<const float*>(x), static_cast<const uint16_t*>(w),
                         yd, part, M, N, K, 4 * WO_DC, xcds);
    else
      hipLaunchKernelGGL(wo_stream_direct_kernel<uint16_t>, dim3((unsigned)tiles), dim3(WO_NT), 0,
                         stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                         yd, part, M, N, K, 4 * WO_DC, xcds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ksplit == 1) return e;
    const size_t quads = (size_t)M * N / 4;
    hipLaunchKernelGGL(wo_finish_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, part, static_cast<uint16_t*>(y), M, N, ksplit);
    return hipGetLastError();
  }
  if (wo_stream_lds_fits(dtype, x_f32, M, N, K)) {
    const int nk = K / 32;
    const int per = (nk + ksplit - 1) / ksplit;
    const long long tiles = (long long)((N + WS_TN - 1) / WS_TN) * ksplit;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    const size_t x16b = wo_x16_bytes(dtype, x_f32, M, N, K);
    if ((ksplit > 1 || x16b > 0) && part == nullptr) return hipErrorInvalidValue;
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    if (x16b > 0) {  // fp32 token rows: one rounding pass into the workspace
      uint16_t* x16 = reinterpret_cast<uint16_t*>(part);
      const size_t n8 = (size_t)M * K / 8;
      hipLaunchKernelGGL(wo_round_x_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const float*>(x), x16, n8);
      hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      xs = x16;
      part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(part) + x16b);
    }
    uint16_t* yd = ksplit == 1 ? static_cast<uint16_t*>(y) : nullptr;
    hipLaunchKernelGGL(wo_stream_lds_kernel, dim3((unsigned)tiles), dim3(256),
                       (size_t)WS_SLOTS * WS_SLOT, stream, xs,
                       static_cast<const uint16_t*>(w), yd, part, M, N, K, per, xcds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ksplit == 1) return e;
    const size_t quads = (size_t)M * N / 4;
    hipLaunchKernelGGL(wo_finish_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, part, static_cast<uint16_t*>(y), M, N, ksplit);
    return hipGetLastError();
  }
  if (wo_gemm_mfma_supported(dtype, N, K)) {
    const int nk = K / 32;
    const int per = (nk + ksplit - 1) / ksplit;
    const long long tiles =
        (long long)((N + WO_TN - 1) / WO_TN) * ((M + WO_TM - 1) / WO_TM) * ksplit;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    if (ksplit > 1 && part == nullptr) return hipErrorInvalidValue;
    uint16_t* yd = ksplit == 1 ? static_cast<uint16_t*>(y) : nullptr;
    if (x_f32)
      hipLaunchKernelGGL(wo_gemm_mfma_kernel<float>, dim3((unsigned)tiles), dim3(256), 0, stream,
                         static_cast<const float*>(x), static_cast<const uint16_t*>(w), yd, part,
                         M, N, K, per, xcds);
    else
      hipLaunchKernelGGL(wo_gemm_mfma_kernel<uint16_t>, dim3((unsigned)tiles), dim3(256), 0,
                         stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                         yd, part, M, N, K, per, xcds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ksplit == 1) return e;
    const size_t quads = (size_t)M * N / 4;
    hipLaunchKernelGGL(wo_finish_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, part, static_cast<uint16_t*>(y), M, N, ksplit);
    return hipGetLastError();
  }
  if (ksplit != 1) return hipErrorInvalidValue;
  const dim3 grid((N + 255) / 256, min(M, 65535));
  if (dtype == 0) {
    if (!x_f32) return hipErrorInvalidValue;  // fp32 configurations have fp32 rows
    hipLaunchKernelGGL((wo_gemm_generic_kernel<float, float>), grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), static_cast<const float*>(w),
                       static_cast<float*>(y), M, N, K);
  } else if (x_f32) {
    hipLaunchKernelGGL((wo_gemm_generic_kernel<float, uint16_t>), grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), static_cast<const uint16_t*>(w),
                       static_cast<uint16_t*>(y), M, N, K);
  } else {
    hipLaunchKernelGGL((wo_gemm_generic_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                       static_cast<uint16_t*>(y), M, N, K);
  }
  return hipGetLastError();
}

bool fold_uv_o_supported(int d_v) { return d_v > 0 && d_v <= FOLD_VMAX; }

hipError_t launch_fold_uv_o(int dtype, const void* w_uv, const void* w_o, void* w_fold, int H,
                            int d_v, int d_c, int d, hipStream_t stream) {
  if (H <= 0 || d_c <= 0 || d <= 0) return hipSuccess;
  if (!fold_uv_o_supported(d_v) || H > 65535 || (d + FOLD_R - 1) / FOLD_R > 65535)
    return hipErrorInvalidValue;
  const dim3 grid((d_c + 255) / 256, (d + FOLD_R - 1) / FOLD_R, H);
  if (dtype == 0)
    hipLaunchKernelGGL(fold_uv_o_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(w_uv), static_cast<const float*>(w_o),
                       static_cast<float*>(w_fold), H, d_v, d_c, d);
  else
    hipLaunchKernelGGL(fold_uv_o_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(w_o),
                       static_cast<uint16_t*>(w_fold), H, d_v, d_c, d);
  return hipGetLastError();
}

}  // namespace mla
