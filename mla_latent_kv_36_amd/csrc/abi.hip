// The C ABI of libmla: argument checks on the host, split planning, dispatch.
// Every check runs before the first launch, so a call that fails launches
// nothing.  No call allocates, frees or keeps device memory.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"
#include "mla.h"

namespace {

constexpr int kMaxDc = 2048;         // generic kernel: latent columns per row
constexpr int kMaxDnope = 4096;      // absorb kernel: LDS holds 16 rows of q_nope
constexpr int kMaxSplits = 65535;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == MLA_F32 ? 4 : 2; }

mla_status check_cfg(const mla_config* c) {
  if (c == nullptr) return MLA_ERR_NULL;
  if (c->dtype != MLA_F32 && c->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (c->n_heads <= 0 || c->n_heads > 65535 || c->d_c <= 0 || c->d_c > kMaxDc ||
      c->d_rope < 0 || c->d_rope > kMaxDc || c->block_size <= 0 || c->block_size > 65536 ||
      c->d_nope < 0 || c->d_v < 0)
    return MLA_ERR_DIM;
  if (!(c->softmax_scale >= 0.0f) || !isfinite(c->softmax_scale)) return MLA_ERR_DIM;
  if (c->softmax_scale == 0.0f && c->d_nope + c->d_rope <= 0) return MLA_ERR_DIM;
  return MLA_OK;
}

float softmax_scale(const mla_config* c) {
  return c->softmax_scale > 0.0f ? c->softmax_scale
                                 : 1.0f / sqrtf((float)(c->d_nope + c->d_rope));
}

bool use_mfma(const mla_config* c, int T) {
  return mla::decode_mfma_supported(c->dtype, c->d_c, c->d_rope, c->block_size, T, c->n_heads);
}

// Compute units and XCDs of the device a plan is made for: the device of
// `stream` (the current device for the null stream, or when `from_stream` is
// false, as for the sizing calls, which take no stream).  Queried at every
// call, so a partitioned or smaller device gets its own plan.  A host with no
// device to ask (sizing on a machine without a GPU) plans for one MI355X:
// 256 compute units in 8 XCDs.
struct DeviceShape {
  int cus;
  int xcds;
};
DeviceShape device_shape(hipStream_t stream, bool from_stream) {
  DeviceShape d{256, 8};
  int dev = 0;
  if (from_stream && stream != nullptr) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return d;
    dev = (int)sd;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return d;
  }
  int cus = 0, xcds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0)
    d.cus = cus;
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && xcds > 0)
    d.xcds = xcds;
  if (d.xcds > d.cus) d.xcds = 1;
  (void)hipGetLastError();
  return d;
}

// Split plan: the rows of the longest sequence are cut into `splits` ranges of
// `chunk` rows each (a multiple of the decode kernel's granule: 32 rows for
// the MFMA kernel, a page for the generic one).  Shorter sequences use the
// leading ranges only.
struct Plan {
  int splits;     // splits per sequence; a balanced plan: work items K per 64-row group
  int chunk;      // rows per split (plain plan)
  bool balanced;  // split sizes chosen per sequence on the device
};

int granule(const mla_config* c, int T) { return use_mfma(c, T) ? 32 : c->block_size; }

// 64-row query groups of the MFMA kernel: ceil(H / 64) per new token
int64_t groups_of(const mla_config* c, int T) { return (int64_t)T * ((c->n_heads + 63) / 64); }

// MFMA kernel, plain plan: units of work are (64-row query group, 32-row unit
// of the cache).  The kernel's LDS ring fits one workgroup per compute unit,
// so aim for one wave of workgroups over the chip, but keep at least 8 units
// per workgroup.  A (sequence, split) range of U units is read from HBM once
// (36,864 U bytes) while each of its T*H query rows writes a bf16 partial
// that the merge reads back: 2 * T*H * 1,024 bytes of round trip.  At the
// minimum U = 8 and T*H = 128 that is 0.89 of the range's cache bytes; at
// the V3 shape (U = 17) 0.42, which the counters confirm (16.8 MB written,
// then read, against 75.5 MB of cache).
int mfma_splits(const mla_config* c, int T, int gran_max, int64_t gran_total, int cus) {
  const int64_t work = gran_total * groups_of(c, T);
  int64_t chunk = (work + cus - 1) / cus;
  if (chunk < 8) chunk = 8;
  return (int)((gran_max + chunk - 1) / chunk);
}

int heuristic_splits(const mla_config* c, int B, int T, int gran_max, int64_t gran_total,
                     int cus) {
  if (gran_max <= 1) return 1;
  if (use_mfma(c, T)) return mfma_splits(c, T, gran_max, gran_total, cus);
  // generic kernel: a workgroup per group of heads of one new token and split
  const int64_t groups =
      (int64_t)B * T * ((c->n_heads + mla::kGenericHeads - 1) / mla::kGenericHeads);
  int64_t s = (4 * (int64_t)cus + groups - 1) / groups;
  if (s > gran_max) s = gran_max;
  return (int)(s < 1 ? 1 : s);
}

// The library's choice for the MFMA kernel when the lengths may differ (their
// total is unknown or below B x the longest): a balanced plan with one work
// item per compute unit, CUs / G per 64-row group, when that is more than
// one per sequence.  Each sequence then gets a number of splits in proportion
// to its length, so that no work item holds much more than the average.
Plan make_plan(const mla_config* c, int B, int T, int max_seq_len, int64_t total_tokens,
               int num_splits, const DeviceShape& dev) {
  const int g = granule(c, T);
  const int gran_max = max_seq_len > 0 ? (max_seq_len + g - 1) / g : 0;
  const int64_t gran_total =
      total_tokens > 0 ? (total_tokens + g - 1) / g + B : (int64_t)B * gran_max;
  if (num_splits == 0 && use_mfma(c, T) && gran_max > 1 && B > 0) {
    const bool equal = total_tokens > 0 && total_tokens >= (int64_t)B * max_seq_len;
    const int64_t K = dev.cus / groups_of(c, T);
    if (!equal && K > B) return Plan{(int)K, 0, true};
  }
  int want = num_splits > 0
                 ? num_splits
                 : heuristic_splits(c, B, T, gran_max, gran_total, dev.cus);
  if (want > gran_max) want = gran_max;
  if (want < 1) want = 1;
  const int chunk = gran_max > 0 ? (gran_max + want - 1) / want : 1;
  const int splits = gran_max > 0 ? (gran_max + chunk - 1) / chunk : 1;
  return Plan{splits, chunk * g, false};
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a split plan: partial outputs (d_c per row: bf16 from the
// MFMA kernel, fp32 from the generic one) and partial log-sum-exps (fp32) for
// B x S x T*H rows (plain plan) or K x T*H rows (a balanced plan, whose
// partials are indexed by work item), then, for a balanced plan, the
// per-sequence table of 4 int32 the merge reads; each region rounded up to
// 256 bytes.
size_t partial_bytes(const mla_config* c, int B, int T, const Plan& pl, size_t* lse_offset,
                     size_t* plan_offset) {
  const size_t rows =
      (pl.balanced ? (size_t)pl.splits : (size_t)B * pl.splits) * T * c->n_heads;
  const size_t elem = use_mfma(c, T) ? 2 : sizeof(float);
  const size_t o_bytes = round256(rows * c->d_c * elem);
  const size_t lse_bytes = round256(rows * sizeof(float));
  if (lse_offset) *lse_offset = o_bytes;
  if (plan_offset) *plan_offset = o_bytes + lse_bytes;
  return o_bytes + lse_bytes + (pl.balanced ? round256((size_t)B * 4 * sizeof(int32_t)) : 0);
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Scratch memory of mla_decode_noalloc: the split partials of one call, in a
// device array that the library owns (one copy per GPU, held until the
// process ends).  `scratch` names the array only in device code; the host
// uses its device address, looked up once per device with hipGetSymbolAddress
// while that device is current.  Calls on one GPU share the array, so calls
// that overlap in time on one GPU (different streams, or different host
// threads) race on it.  Nothing in it has to start at zero: the partial rows
// and the balanced plan's table are written before they are read in every
// call.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the device of stream s (the current
// device for the null stream).
hipError_t scratch_address(hipStream_t s, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(s, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK: success";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_DIM: return "MLA_ERR_DIM: a size or config field is out of range";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown element type";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY: sequence would not fit the block table";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported an error at launch";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    default: return "unknown mla_status";
  }
}

int32_t mla_abi_version(void) { return 2; }

// Host checks of mla_absorb_q's arguments; *work = false when there is
// nothing to launch (M == 0).
static mla_status check_absorb(const mla_config* cfg, const void* q_nope, const void* q_rope,
                               const void* w_uk, const void* q_abs, int32_t M, bool* work) {
  *work = false;
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (M < 0 || cfg->d_nope <= 0 || cfg->d_nope > kMaxDnope) return MLA_ERR_DIM;
  if (M == 0) return MLA_OK;
  if (q_nope == nullptr || w_uk == nullptr || q_abs == nullptr ||
      (cfg->d_rope > 0 && q_rope == nullptr))
    return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_abs) ||
      (q_rope != nullptr && !aligned16(q_rope)))
    return MLA_ERR_ALIGN;
  if ((int64_t)(M + 15) / 16 > 65535) return MLA_ERR_DIM;
  *work = true;
  return MLA_OK;
}

// Host checks of mla_cache_append's arguments; *work = false when there is
// nothing to launch.
static mla_status check_append(const mla_config* cfg, const void* pool, int32_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seq_lens, const void* new_rows, int32_t B,
                               int32_t T_new, int32_t max_seq_len_host, bool* work) {
  *work = false;
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (B < 0 || T_new < 0 || num_blocks <= 0 || max_blocks <= 0 || max_seq_len_host < 0)
    return MLA_ERR_DIM;
  if ((int64_t)max_seq_len_host > (int64_t)max_blocks * cfg->block_size) return MLA_ERR_CAPACITY;
  if (B == 0 || T_new == 0) return MLA_OK;
  if (pool == nullptr || block_table == nullptr || seq_lens == nullptr || new_rows == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(pool) || !aligned16(new_rows) || !aligned16(block_table) || !aligned16(seq_lens))
    return MLA_ERR_ALIGN;
  if ((int64_t)B * T_new > 0x7fffffffLL) return MLA_ERR_DIM;
  *work = true;
  return MLA_OK;
}

mla_status mla_absorb_q(const mla_config* cfg, const void* q_nope, const void* q_rope,
                        const void* w_uk, void* q_abs, int32_t M, void* stream) {
  bool work;
  mla_status st = check_absorb(cfg, q_nope, q_rope, w_uk, q_abs, M, &work);
  if (st != MLA_OK || !work) return st;
  return hip_status(mla::launch_absorb_q(cfg->dtype, q_nope, q_rope, w_uk, q_abs, M,
                                         cfg->n_heads, cfg->d_nope, cfg->d_c, cfg->d_rope,
                                         static_cast<hipStream_t>(stream)));
}

mla_status mla_cache_append(const mla_config* cfg, void* pool, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, const void* new_rows, int32_t B,
                            int32_t T_new, int32_t max_seq_len_host, void* stream) {
  bool work;
  mla_status st = check_append(cfg, pool, num_blocks, block_table, max_blocks, seq_lens, new_rows,
                               B, T_new, max_seq_len_host, &work);
  if (st != MLA_OK || !work) return st;
  const int row_bytes = (cfg->d_c + cfg->d_rope) * (int)elem_size(cfg->dtype);
  return hip_status(mla::launch_append(pool, num_blocks, block_table, max_blocks, seq_lens,
                                       new_rows, B, T_new, cfg->block_size, row_bytes,
                                       static_cast<hipStream_t>(stream)));
}

mla_status mla_absorb_q_append(const mla_config* cfg, const void* q_nope, const void* q_rope,
                               const void* w_uk, void* q_abs, int32_t M, void* pool,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               const void* new_rows, int32_t B, int32_t T_new,
                               int32_t max_seq_len_host, void* stream) {
  bool wa, wp;
  mla_status st = check_absorb(cfg, q_nope, q_rope, w_uk, q_abs, M, &wa);
  if (st != MLA_OK) return st;
  st = check_append(cfg, pool, num_blocks, block_table, max_blocks, seq_lens, new_rows, B, T_new,
                    max_seq_len_host, &wp);
  if (st != MLA_OK) return st;
  mla::AppendArgs ap{};
  if (wp) {
    ap.pool = pool;
    ap.num_blocks = num_blocks;
    ap.table = block_table;
    ap.max_blocks = max_blocks;
    ap.seq_lens = seq_lens;
    ap.new_rows = new_rows;
    ap.T_new = T_new;
    ap.block_size = cfg->block_size;
    ap.row_bytes = (cfg->d_c + cfg->d_rope) * (int)elem_size(cfg->dtype);
    ap.rows = B * T_new;
  }
  return hip_status(mla::launch_absorb_q_append(
      cfg->dtype, wa ? q_nope : nullptr, q_rope, w_uk, q_abs, wa ? M : 0, cfg->n_heads,
      cfg->d_nope, cfg->d_c, cfg->d_rope, ap, static_cast<hipStream_t>(stream)));
}

int32_t mla_decode_num_splits(const mla_config* cfg, int32_t B, int32_t T,
                              int32_t max_seq_len_host, int64_t total_tokens_host) {
  if (check_cfg(cfg) != MLA_OK || B < 0 || T < 1 || max_seq_len_host < 0) return 1;
  return make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, 0, device_shape(nullptr, false))
      .splits;
}

size_t mla_decode_workspace_size(const mla_config* cfg, int32_t B, int32_t T,
                                 int32_t max_seq_len_host, int64_t total_tokens_host,
                                 int32_t num_splits) {
  if (check_cfg(cfg) != MLA_OK || B < 0 || T < 1 || max_seq_len_host < 0 || num_splits < 0)
    return (size_t)-1;
  const Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits,
                            device_shape(nullptr, false));
  if (pl.splits <= 1) return 0;
  return partial_bytes(cfg, B, T, pl, nullptr, nullptr);
}

// Host checks of mla_decode's arguments (everything but the workspace);
// *work = false when there is nothing to launch (B == 0).
static mla_status check_decode(const mla_config* cfg, const void* q_abs, const void* pool,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               int32_t max_seq_len_host, int32_t B, int32_t T, int32_t causal,
                               int32_t num_splits, const float* o_lat, const float* lse,
                               bool* work) {
  *work = false;
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (B < 0 || T < 1 || num_blocks <= 0 || max_blocks <= 0 || max_seq_len_host < 0 ||
      num_splits < 0 || num_splits > kMaxSplits || (causal != 0 && causal != 1))
    return MLA_ERR_DIM;
  if ((int64_t)max_seq_len_host > (int64_t)max_blocks * cfg->block_size) return MLA_ERR_CAPACITY;
  if ((int64_t)B * T * cfg->n_heads > 0x7fffffffLL) return MLA_ERR_DIM;
  if (B == 0) return MLA_OK;
  if (q_abs == nullptr || pool == nullptr || block_table == nullptr || seq_lens == nullptr ||
      o_lat == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(pool) || !aligned16(o_lat) || !aligned16(block_table) ||
      !aligned16(seq_lens) || (lse != nullptr && !aligned16(lse)))
    return MLA_ERR_ALIGN;
  *work = true;
  return MLA_OK;
}

// Launches a checked decode under plan pl with its partials in `workspace`
// (at least partial_bytes(pl) bytes when pl needs a merge).
// With w_uv, out_proj follows (out = W^UV o_lat): in the merge's launch where
// the MFMA kernels apply and the plan has splits, else as a launch of its own.
static mla_status launch_decode_plan(const mla_config* cfg, const Plan& pl,
                                     const DeviceShape& dev, const void* q_abs,
                                     const void* pool, int32_t num_blocks,
                                     const int32_t* block_table, int32_t max_blocks,
                                     const int32_t* seq_lens, int32_t max_seq_len_host,
                                     int32_t B, int32_t T, int32_t causal, void* workspace,
                                     float* o_lat, float* lse, hipStream_t s,
                                     const void* w_uv = nullptr, void* out = nullptr) {
  size_t lse_off = 0;
  size_t plan_off = 0;
  const bool merge = pl.splits > 1;
  if (merge) partial_bytes(cfg, B, T, pl, &lse_off, &plan_off);

  mla::DecodeParams p{};
  p.q_abs = q_abs;
  p.pool = pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o_lat = o_lat;
  p.lse = lse;
  p.part_o = merge ? workspace : nullptr;
  p.part_bf16 = use_mfma(cfg, T) ? 1 : 0;
  p.part_lse = merge ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off)
                     : nullptr;
  p.B = B;
  p.T = T;
  p.H = cfg->n_heads;
  p.d_c = cfg->d_c;
  p.d_r = cfg->d_rope;
  p.block_size = cfg->block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks;
  p.cap = max_seq_len_host;
  p.causal = causal;
  p.num_splits = pl.splits;
  p.chunk_rows = pl.chunk;
  p.xcds = dev.xcds;
  p.scale_log2 = softmax_scale(cfg) * 1.4426950408889634f;
  p.plan = pl.balanced ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan_off)
                       : nullptr;

  hipError_t e = use_mfma(cfg, T) ? mla::launch_decode_mfma(p, s)
                                  : mla::launch_decode_generic(p, cfg->dtype, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  const bool proj = w_uv != nullptr;
  if (merge && proj && p.part_bf16 &&
      mla::merge_out_proj_supported(cfg->dtype, cfg->d_c, cfg->d_v))
    return hip_status(mla::launch_merge_out_proj(p, w_uv, out, cfg->d_v, s));
  if (merge) {
    e = mla::launch_combine(p, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  if (proj)
    return hip_status(mla::launch_out_proj(cfg->dtype, o_lat, w_uv, out, B * T, cfg->n_heads,
                                           cfg->d_c, cfg->d_v, s));
  return MLA_OK;
}

mla_status mla_decode(const mla_config* cfg, const void* q_abs, const void* pool,
                      int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                      const int32_t* seq_lens, int32_t max_seq_len_host, int32_t B,
                      int32_t T, int32_t causal, int32_t num_splits,
                      int64_t total_tokens_host, void* workspace, size_t workspace_bytes,
                      float* o_lat, float* lse, void* stream) {
  bool work;
  mla_status st = check_decode(cfg, q_abs, pool, num_blocks, block_table, max_blocks, seq_lens,
                               max_seq_len_host, B, T, causal, num_splits, o_lat, lse, &work);
  if (st != MLA_OK || !work) return st;
  if (workspace != nullptr && !aligned16(workspace)) return MLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DeviceShape dev = device_shape(s, true);
  const Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits, dev);
  const size_t need = pl.splits > 1 ? partial_bytes(cfg, B, T, pl, nullptr, nullptr) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  return launch_decode_plan(cfg, pl, dev, q_abs, pool, num_blocks, block_table, max_blocks,
                            seq_lens, max_seq_len_host, B, T, causal, workspace, o_lat, lse, s);
}

size_t mla_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

mla_status mla_decode_out_proj(const mla_config* cfg, const void* q_abs, const void* pool,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               int32_t max_seq_len_host, int32_t B, int32_t T, int32_t causal,
                               int32_t num_splits, int64_t total_tokens_host, const void* w_uv,
                               void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                               void* out, void* stream) {
  bool work;
  mla_status st = check_decode(cfg, q_abs, pool, num_blocks, block_table, max_blocks, seq_lens,
                               max_seq_len_host, B, T, causal, num_splits, o_lat, lse, &work);
  if (st != MLA_OK) return st;
  // mla_out_proj's checks, also before anything is launched
  if (cfg->d_v <= 0) return MLA_ERR_DIM;
  if ((int64_t)B * T > 0x7fffffffLL || ((int64_t)B * T + 15) / 16 > 65535 ||
      ((int64_t)cfg->d_v + 15) / 16 > 65535)
    return MLA_ERR_DIM;
  if (!work) return MLA_OK;
  if (w_uv == nullptr || out == nullptr) return MLA_ERR_NULL;
  if (!aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return MLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DeviceShape dev = device_shape(s, true);
  const Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits, dev);
  const size_t need = pl.splits > 1 ? partial_bytes(cfg, B, T, pl, nullptr, nullptr) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  return launch_decode_plan(cfg, pl, dev, q_abs, pool, num_blocks, block_table, max_blocks,
                            seq_lens, max_seq_len_host, B, T, causal, workspace, o_lat, lse, s,
                            w_uv, out);
}

// Workspace of the one-launch decode: the counter region (zero on entry), the
// per-group merge records, the balanced plan's table, then the partials as
// for mla_decode; each region rounded up to 256 bytes.
struct FusedLayout {
  size_t rec, table, part_o, part_lse, total;
};
static bool fused_layout(const mla_config* cfg, int B, int T, const Plan& pl, FusedLayout* L) {
  const int64_t BG = (int64_t)B * groups_of(cfg, T);
  if (BG > mla::kQueueMaxGroups) return false;
  L->rec = mla::kQueueCounterBytes;
  L->table = L->rec + round256((size_t)BG * 2 * sizeof(int32_t));
  L->part_o = L->table + round256((size_t)B * 4 * sizeof(int32_t));
  size_t lse_off = 0;
  const size_t pb = pl.splits > 1 ? partial_bytes(cfg, B, T, pl, &lse_off, nullptr) : 0;
  L->part_lse = L->part_o + lse_off;
  L->total = L->part_o + pb;
  return true;
}

size_t mla_decode_fused_workspace_size(const mla_config* cfg, int32_t B, int32_t T,
                                       int32_t max_seq_len_host, int64_t total_tokens_host,
                                       int32_t num_splits) {
  if (check_cfg(cfg) != MLA_OK || B < 0 || T < 1 || max_seq_len_host < 0 || num_splits < 0 ||
      !use_mfma(cfg, T))
    return (size_t)-1;
  const Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits,
                            device_shape(nullptr, false));
  FusedLayout L;
  if (!fused_layout(cfg, B, T, pl, &L)) return (size_t)-1;
  return L.total;
}

size_t mla_decode_fused_counter_bytes(void) { return mla::kQueueCounterBytes; }

mla_status mla_decode_fused(const mla_config* cfg, const void* q_abs, const void* pool,
                            int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t max_seq_len_host, int32_t B,
                            int32_t T, int32_t causal, int32_t num_splits,
                            int64_t total_tokens_host, void* workspace, size_t workspace_bytes,
                            float* o_lat, float* lse, void* stream) {
  bool work;
  mla_status st = check_decode(cfg, q_abs, pool, num_blocks, block_table, max_blocks, seq_lens,
                               max_seq_len_host, B, T, causal, num_splits, o_lat, lse, &work);
  if (st != MLA_OK) return st;
  if (!use_mfma(cfg, T)) return MLA_ERR_DIM;
  if (!work) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DeviceShape dev = device_shape(s, true);
  const Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits, dev);
  FusedLayout L;
  if (!fused_layout(cfg, B, T, pl, &L)) return MLA_ERR_DIM;
  if (workspace == nullptr || workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);

  mla::DecodeParams p{};
  p.q_abs = q_abs;
  p.pool = pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o_lat = o_lat;
  p.lse = lse;
  p.part_o = pl.splits > 1 ? ws + L.part_o : nullptr;
  p.part_lse = pl.splits > 1 ? reinterpret_cast<float*>(ws + L.part_lse) : nullptr;
  p.part_bf16 = 1;
  p.B = B;
  p.T = T;
  p.H = cfg->n_heads;
  p.d_c = cfg->d_c;
  p.d_r = cfg->d_rope;
  p.block_size = cfg->block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks;
  p.cap = max_seq_len_host;
  p.causal = causal;
  p.num_splits = pl.splits;
  p.chunk_rows = pl.chunk;
  p.xcds = dev.xcds;
  p.scale_log2 = softmax_scale(cfg) * 1.4426950408889634f;
  p.plan = pl.balanced ? reinterpret_cast<int32_t*>(ws + L.table) : nullptr;
  p.counters = reinterpret_cast<uint32_t*>(ws);  // the group records follow at L.rec
  return hip_status(mla::launch_decode_queue(p, dev.cus, s));
}

mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_abs, const void* pool,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* seq_lens,
                              int32_t max_seq_len_host, int32_t B, int32_t T, int32_t causal,
                              int32_t num_splits, int64_t total_tokens_host, float* o_lat,
                              float* lse, void* stream) {
  bool work;
  mla_status st = check_decode(cfg, q_abs, pool, num_blocks, block_table, max_blocks, seq_lens,
                               max_seq_len_host, B, T, causal, num_splits, o_lat, lse, &work);
  if (st != MLA_OK || !work) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DeviceShape dev = device_shape(s, true);
  Plan pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, num_splits, dev);
  if (pl.splits > 1 && partial_bytes(cfg, B, T, pl, nullptr, nullptr) > kScratchBytes) {
    // an explicit split count must fit as asked; the library's choice is cut
    // to the most splits whose partials fit (one split needs none)
    if (num_splits > 0) return MLA_ERR_WORKSPACE;
    const size_t per_split =
        (size_t)B * T * cfg->n_heads * ((size_t)cfg->d_c + 1) * sizeof(float) + 512;
    int fit = (int)(kScratchBytes / per_split);
    if (fit > pl.splits) fit = pl.splits;
    for (;; --fit) {
      pl = make_plan(cfg, B, T, max_seq_len_host, total_tokens_host, fit < 1 ? 1 : fit, dev);
      if (pl.splits <= 1 || partial_bytes(cfg, B, T, pl, nullptr, nullptr) <= kScratchBytes) break;
    }
  }
  void* ws = nullptr;
  if (pl.splits > 1 && scratch_address(s, &ws) != hipSuccess) return MLA_ERR_HIP;
  return launch_decode_plan(cfg, pl, dev, q_abs, pool, num_blocks, block_table, max_blocks,
                            seq_lens, max_seq_len_host, B, T, causal, ws, o_lat, lse, s);
}

mla_status mla_out_proj(const mla_config* cfg, const float* o_lat, const void* w_uv, void* out,
                        int32_t M, void* stream) {
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (M < 0 || cfg->d_v <= 0) return MLA_ERR_DIM;
  if (M == 0) return MLA_OK;
  if (o_lat == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if ((int64_t)(M + 15) / 16 > 65535 || (int64_t)(cfg->d_v + 15) / 16 > 65535)
    return MLA_ERR_DIM;
  return hip_status(mla::launch_out_proj(cfg->dtype, o_lat, w_uv, out, M, cfg->n_heads,
                                         cfg->d_c, cfg->d_v, static_cast<hipStream_t>(stream)));
}

mla_status mla_gather_rows(const mla_config* cfg, const void* pool, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t B, int32_t max_seq_len_host,
                           void* dense, void* stream) {
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (B < 0 || num_blocks <= 0 || max_blocks <= 0 || max_seq_len_host < 0 || B > 65535)
    return MLA_ERR_DIM;
  if ((int64_t)max_seq_len_host > (int64_t)max_blocks * cfg->block_size) return MLA_ERR_CAPACITY;
  if (B == 0 || max_seq_len_host == 0) return MLA_OK;
  if (pool == nullptr || block_table == nullptr || seq_lens == nullptr || dense == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(pool) || !aligned16(dense) || !aligned16(block_table) || !aligned16(seq_lens))
    return MLA_ERR_ALIGN;
  const int row_bytes = (cfg->d_c + cfg->d_rope) * (int)elem_size(cfg->dtype);
  return hip_status(mla::launch_gather(pool, num_blocks, block_table, max_blocks, seq_lens, B,
                                       max_seq_len_host, cfg->block_size, row_bytes, dense,
                                       static_cast<hipStream_t>(stream)));
}

mla_status mla_validate_block_table(const int32_t* block_table, int32_t B, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t block_size,
                                    int32_t num_blocks, int32_t* err_flag, void* stream) {
  if (B < 0 || B > 65535 || max_blocks <= 0 || block_size <= 0 || num_blocks <= 0)
    return MLA_ERR_DIM;
  if (err_flag == nullptr || (B > 0 && (block_table == nullptr || seq_lens == nullptr)))
    return MLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(err_flag) & 3u) != 0) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_validate(block_table, B, max_blocks, seq_lens, block_size,
                                         num_blocks, err_flag, static_cast<hipStream_t>(stream)));
}

mla_status mla_stream_read(const void* src, size_t bytes, void* sink, int32_t mode,
                           void* stream) {
  if (mode != 0 && mode != 1) return MLA_ERR_DIM;
  if (bytes == 0) return MLA_OK;
  if (src == nullptr || sink == nullptr) return MLA_ERR_NULL;
  if (!aligned16(src) || !aligned16(sink) || bytes % 16 != 0) return MLA_ERR_ALIGN;
  return hip_status(
      mla::launch_stream_read(src, bytes, sink, mode == 1, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
constexpr float kDefaultRopeBase = 10000.0f;
// The producer's k split aims at half the compute units: a longer k range per
// workgroup, but half the partial sums to write and add (measured faster at
// the V2-scale width than one workgroup per compute unit).
int produce_workgroups() { return device_shape(nullptr, false).cus / 2; }

// 0 selects the default base; anything else must be a finite value > 1
bool rope_base_of(float in, float* out) {
  if (in == 0.0f) {
    *out = kDefaultRopeBase;
    return true;
  }
  if (!(in > 1.0f) || !isfinite(in)) return false;
  *out = in;
  return true;
}
}  // namespace

extern "C" size_t mla_kv_produce_workspace_size(const mla_config* cfg, int32_t M,
                                                int32_t d_model) {
  if (check_cfg(cfg) != MLA_OK || M < 0 || d_model <= 0) return (size_t)-1;
  if (M == 0) return 0;
  const int ks = mla::kv_produce_ksplit(cfg->dtype, M, d_model, cfg->d_c, cfg->d_rope, produce_workgroups());
  return round256((size_t)ks * M * (cfg->d_c + cfg->d_rope) * sizeof(float));
}

extern "C" mla_status mla_kv_produce(const mla_config* cfg, const void* hidden, int32_t d_model,
                                     const void* w_dkv, const void* w_kr, float rope_base,
                                     void* pool, int32_t num_blocks, const int32_t* block_table,
                                     int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                                     int32_t T_new, int32_t max_seq_len_host, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  float base;
  if (B < 0 || T_new < 0 || d_model <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
      max_seq_len_host < 0 || (cfg->d_c & 1) || (cfg->d_rope & 1) || !rope_base_of(rope_base, &base))
    return MLA_ERR_DIM;
  if ((int64_t)max_seq_len_host > (int64_t)max_blocks * cfg->block_size) return MLA_ERR_CAPACITY;
  if ((int64_t)B * T_new > 0x7fffffffLL) return MLA_ERR_DIM;
  const int M = B * T_new;
  if (M == 0) return MLA_OK;
  if (hidden == nullptr || w_dkv == nullptr || (cfg->d_rope > 0 && w_kr == nullptr) ||
      pool == nullptr || block_table == nullptr || seq_lens == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(w_dkv) || (w_kr != nullptr && !aligned16(w_kr)) ||
      !aligned16(pool) || !aligned16(block_table) || !aligned16(seq_lens) ||
      (workspace != nullptr && !aligned16(workspace)))
    return MLA_ERR_ALIGN;
  const size_t need = mla_kv_produce_workspace_size(cfg, M, d_model);
  if (workspace == nullptr || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  const int ks = mla::kv_produce_ksplit(cfg->dtype, M, d_model, cfg->d_c, cfg->d_rope, produce_workgroups());
  return hip_status(mla::launch_kv_produce(
      cfg->dtype, hidden, d_model, w_dkv, w_kr, base, static_cast<float*>(workspace), ks, pool,
      num_blocks, block_table, max_blocks, seq_lens, B, T_new, cfg->block_size, cfg->d_c,
      cfg->d_rope, device_shape(static_cast<hipStream_t>(stream), true).xcds,
      static_cast<hipStream_t>(stream)));
}

extern "C" mla_status mla_rope(const mla_config* cfg, void* x, int32_t heads,
                               const int32_t* positions, int32_t M, float rope_base,
                               void* stream) {
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  float base;
  if (M < 0 || heads < 0 || (cfg->d_rope & 1) || !rope_base_of(rope_base, &base)) return MLA_ERR_DIM;
  if (M == 0 || heads == 0 || cfg->d_rope == 0) return MLA_OK;
  if (x == nullptr || positions == nullptr) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(positions)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_rope(cfg->dtype, x, positions, M, heads, cfg->d_rope, base,
                                     static_cast<hipStream_t>(stream)));
}

namespace {
// The output-side product aims at two workgroups per compute unit (its
// launch bounds allow two resident), splitting k when the tiles are fewer.
int output_workgroups() { return 2 * device_shape(nullptr, false).cus; }

// k of the output-side product: H * d_v for W^O, H * d_c for the folded
// matrix; 0 when it does not fit an int32.
int64_t output_k(const mla_config* c, bool folded) {
  const int64_t k = (int64_t)c->n_heads * (folded ? c->d_c : c->d_v);
  return k > 0x7fffffffLL ? 0 : k;
}

// the latent outputs are fp32; so are the per-head outputs of an fp32 configuration
bool output_x_f32(const mla_config* c, bool folded) { return folded || c->dtype == MLA_F32; }

size_t output_workspace(const mla_config* c, int M, int d_model, bool folded) {
  const int64_t K = output_k(c, folded);
  const bool x_f32 = output_x_f32(c, folded);
  const int ks = mla::wo_gemm_ksplit(c->dtype, x_f32, M, d_model, (int)K, output_workgroups());
  return mla::wo_gemm_workspace_bytes(c->dtype, x_f32, M, d_model, (int)K, ks);
}

mla_status output_args(const mla_config* cfg, int32_t M, int32_t d_model, bool folded) {
  mla_status st = check_cfg(cfg);
  if (st != MLA_OK) return st;
  if (M < 0 || d_model <= 0 || (!folded && cfg->d_v <= 0) || output_k(cfg, folded) == 0)
    return MLA_ERR_DIM;
  return MLA_OK;
}

mla_status output_call(const mla_config* cfg, bool folded, const void* x, const void* w, void* y,
                       int32_t M, int32_t d_model, void* workspace, size_t workspace_bytes,
                       void* stream) {
  mla_status st = output_args(cfg, M, d_model, folded);
  if (st != MLA_OK) return st;
  if (M == 0) return MLA_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) ||
      (workspace != nullptr && !aligned16(workspace)))
    return MLA_ERR_ALIGN;
  const int K = (int)output_k(cfg, folded);
  const bool x_f32 = output_x_f32(cfg, folded);
  const int ks = mla::wo_gemm_ksplit(cfg->dtype, x_f32, M, d_model, K, output_workgroups());
  const size_t need = output_workspace(cfg, M, d_model, folded);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(mla::launch_wo_gemm(cfg->dtype, x_f32, x, w, y, static_cast<float*>(workspace),
                                        ks, M, d_model, K, device_shape(s, true).xcds, s));
}
}  // namespace

extern "C" size_t mla_o_proj_workspace_size(const mla_config* cfg, int32_t M, int32_t d_model,
                                            int32_t folded) {
  if (output_args(cfg, M, d_model, folded != 0) != MLA_OK) return (size_t)-1;
  return M == 0 ? 0 : output_workspace(cfg, M, d_model, folded != 0);
}

extern "C" mla_status mla_o_proj(const mla_config* cfg, const void* attn, const void* w_o,
                                 void* y, int32_t M, int32_t d_model, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return output_call(cfg, false, attn, w_o, y, M, d_model, workspace, workspace_bytes, stream);
}

extern "C" mla_status mla_o_proj_folded(const mla_config* cfg, const float* o_lat,
                                        const void* w_fold, void* y, int32_t M, int32_t d_model,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return output_call(cfg, true, o_lat, w_fold, y, M, d_model, workspace, workspace_bytes, stream);
}

extern "C" mla_status mla_fold_uv_o(const mla_config* cfg, const void* w_uv, const void* w_o,
                                    void* w_fold, int32_t d_model, void* stream) {
  mla_status st = output_args(cfg, 0, d_model, false);
  if (st != MLA_OK) return st;
  if (!mla::fold_uv_o_supported(cfg->d_v) || output_k(cfg, true) == 0 ||
      (int64_t)(d_model + 15) / 16 > 65535)
    return MLA_ERR_DIM;
  if (w_uv == nullptr || w_o == nullptr || w_fold == nullptr) return MLA_ERR_NULL;
  if (!aligned16(w_uv) || !aligned16(w_o) || !aligned16(w_fold)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_fold_uv_o(cfg->dtype, w_uv, w_o, w_fold, cfg->n_heads, cfg->d_v,
                                          cfg->d_c, d_model, static_cast<hipStream_t>(stream)));
}
