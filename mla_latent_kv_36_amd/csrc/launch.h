// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Everything one decode launch needs; built and checked on the host.
struct DecodeParams {
  const void* q_abs;          // [B, T, H, W] storage type
  const void* pool;           // [num_blocks, block_size, W]
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* seq_lens;    // [B], rows including the T new tokens
  float* o_lat;               // [B, T, H, d_c]
  float* lse;                 // [B, T, H] or nullptr
  void* part_o;               // [B, S, T*H, d_c] when S > 1: bf16 if part_bf16, else fp32
  float* part_lse;            // [B, S, T*H]      when S > 1
  int B, T, H, d_c, d_r, block_size;
  int num_blocks, max_blocks;
  int cap;                    // host bound on rows attended per sequence
  int causal;
  int num_splits;             // S
  int chunk_rows;             // cache rows per split (a multiple of the kernel granule)
  int xcds;                   // MFMA kernel: XCDs of the device (workgroup placement)
  int part_bf16;              // partial outputs stored as bf16 (the MFMA kernel's)
  float scale_log2;           // softmax scale * log2(e)
  // Balanced plan (MFMA kernel only): when non-null, num_splits is the number
  // K of work items per 64-row group, split sizes are chosen per sequence on
  // the device, and plan[4b .. 4b+2] receives sequence b's first work item,
  // split count and units per split for the merge.  Partials are then
  // indexed by work item: part_o [K, T*H, d_c], part_lse [K, T*H].
  int32_t* plan;
  // One-launch decode (decode_queue_kernel) only: the counters of its work
  // queue and merge ring (kQueueCounterBytes, zero before the launch and left
  // zero after it), followed at once by 8 bytes per (sequence, 64-row group)
  // for the merge.
  uint32_t* counters;
};

// The one-launch decode's counter region: a 1 KiB header, then per (sequence,
// 64-row group) kQueueSlices 8-byte merge-ring entries and an arrival count.
constexpr size_t kQueueCounterBytes = (size_t)256 << 10;
constexpr int kQueueSlices = 8;
constexpr int64_t kQueueMaxGroups =
    ((int64_t)kQueueCounterBytes / 4 - 256) / (1 + 2 * kQueueSlices);

// The MFMA kernel covers bf16, d_c = 512, d_rope = 64 and 64-token pages, any
// H and T (ceil(H / 64) query groups of 64 rows per new token).
bool decode_mfma_supported(int dtype, int d_c, int d_r, int block_size, int T, int H);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
// The same decode and its merge in one launch of at most `workgroups`
// persistent workgroups (one per compute unit fits): work items from a queue,
// merges of a group's partials taken up once its last split has arrived.
hipError_t launch_decode_queue(const DecodeParams& p, int workgroups, hipStream_t stream);
// The generic kernel: a workgroup per (kGenericHeads heads of one new token,
// split).
constexpr int kGenericHeads = 8;
hipError_t launch_decode_generic(const DecodeParams& p, int dtype, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);

hipError_t launch_absorb_q(int dtype, const void* q_nope, const void* q_rope,
                           const void* w_uk, void* q_abs, int M, int H, int d_n, int d_c,
                           int d_r, hipStream_t stream);
hipError_t launch_out_proj(int dtype, const float* o_lat, const void* w_uv, void* out,
                           int M, int H, int d_c, int d_v, hipStream_t stream);
// The merge of bf16 split partials (p as for launch_combine, with o_lat) and
// out_proj in one launch: out[m, h, :] = W^UV[h] o_lat[m, h, :], o_lat and lse
// written as the merge kernel would.  bf16, d_c = 512.
bool merge_out_proj_supported(int dtype, int d_c, int d_v);
hipError_t launch_merge_out_proj(const DecodeParams& p, const void* w_uv, void* out, int d_v,
                                 hipStream_t stream);
// The cache append's arguments, for a kernel that carries the append along
// with its own work (rows == 0: no append).
struct AppendArgs {
  void* pool;
  int num_blocks;
  const int32_t* table;
  int max_blocks;
  const int32_t* seq_lens;
  const void* new_rows;
  int T_new;
  int block_size;
  int row_bytes;
  int rows;  // B * T_new
};
// absorb_q (M == 0: none) and the append in one launch where the MFMA absorb
// kernel applies, else the two launches in turn.
hipError_t launch_absorb_q_append(int dtype, const void* q_nope, const void* q_rope,
                                  const void* w_uk, void* q_abs, int M, int H, int d_n, int d_c,
                                  int d_r, const AppendArgs& ap, hipStream_t stream);
hipError_t launch_append(void* pool, int num_blocks, const int32_t* block_table,
                         int max_blocks, const int32_t* seq_lens, const void* new_rows,
                         int B, int T_new, int block_size, int row_bytes,
                         hipStream_t stream);
hipError_t launch_gather(const void* pool, int num_blocks, const int32_t* block_table,
                         int max_blocks, const int32_t* seq_lens, int B, int cap,
                         int block_size, int row_bytes, void* dense, hipStream_t stream);
// Producer step: cached rows [W^DKV h | RoPE(W^KR h)] into the pool.  `part`
// holds ksplit * M * (d_c + d_r) fp32 partial sums; ksplit comes from
// kv_produce_ksplit (1 for the generic kernel).
bool kv_proj_mfma_supported(int dtype, int d_model);
int kv_produce_ksplit(int dtype, int M, int d_model, int d_c, int d_r, int cus);
hipError_t launch_kv_produce(int dtype, const void* hidden, int d_model, const void* w_dkv,
                             const void* w_kr, float rope_base, float* part, int ksplit,
                             void* pool, int num_blocks, const int32_t* block_table,
                             int max_blocks, const int32_t* seq_lens, int B, int T_new,
                             int block_size, int d_c, int d_r, int xcds, hipStream_t stream);
hipError_t launch_rope(int dtype, void* x, const int32_t* positions, int M, int heads, int d_r,
                       float rope_base, hipStream_t stream);
// The output side (output_side.hip): y[M, N] = x[M, K] . w[N, K]^T with x bf16
// (or fp32 when x_f32) and w, y of dtype; k split over ksplit workgroups whose
// fp32 partial sums (part: ksplit * M * N floats when ksplit > 1) are added
// in split order.  wo_gemm_ksplit gives the split for a target workgroup
// count (1 for the generic kernel).  xcds: the device's XCD count (workgroup
// placement).
bool wo_gemm_mfma_supported(int dtype, int N, int K);
int wo_gemm_ksplit(int dtype, bool x_f32, int M, int N, int K, int target_workgroups);
// Workspace of one product: a bf16 copy of fp32 token rows where the
// streaming kernel takes them (first), then the split partial sums.
size_t wo_gemm_workspace_bytes(int dtype, bool x_f32, int M, int N, int K, int ksplit);
hipError_t launch_wo_gemm(int dtype, bool x_f32, const void* x, const void* w, void* y,
                          float* part, int ksplit, int M, int N, int K, int xcds,
                          hipStream_t stream);
// w_fold[d, H * d_c] from w_uv[H, d_v, d_c] and w_o[d, H * d_v] (d_v <= 256).
bool fold_uv_o_supported(int d_v);
hipError_t launch_fold_uv_o(int dtype, const void* w_uv, const void* w_o, void* w_fold, int H,
                            int d_v, int d_c, int d, hipStream_t stream);
// Reads bytes (a multiple of 16) at src once and XORs the 16-byte chunks into
// the 4 x uint32 at sink (atomically); lds: through direct-to-LDS copies.
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, bool lds,
                              hipStream_t stream);
hipError_t launch_validate(const int32_t* block_table, int B, int max_blocks,
                           const int32_t* seq_lens, int block_size, int num_blocks,
                           int32_t* err_flag, hipStream_t stream);

}  // namespace mla
