/*
 * libmla: absorbed multi-head latent attention (MLA) decode on AMD CDNA4 (gfx950).
 *
 * One decode step of MLA runs as four calls, in this order:
 *   mla_absorb_q      fold each head's W^UK into its query, once per new token
 *   mla_cache_append  write the new tokens' [c | k^R] rows into the paged cache
 *   mla_decode        score the absorbed queries against every cached row,
 *                     softmax, and sum the cached latents (split-KV + merge)
 *   mla_out_proj      up-project the latent output once per head through W^UV
 *
 * (mla_absorb_q_append issues the first two as one launch), and, on the input side, mla_kv_produce (the cached row made from the token's
 * hidden vector, with RoPE on k^R, written into the cache in place of
 * mla_cache_append) and mla_rope (the same rotation for the query's rotary part);
 * on the output side, mla_o_proj (the output projection W^O over the heads) and
 * mla_fold_uv_o / mla_o_proj_folded (W^UV merged into W^O).
 *
 * The method is the inference path of "Attention, Part 2: MQA, GQA and MLA",
 * section "The trick that makes it fast: never rebuild at all": only the latent c
 * (width d_c) and the decoupled rotary key k^R (width d_rope) are cached per token
 * ("Multi-head latent attention (MLA)", sections 2 and 3); the keys and values of
 * the heads are never rebuilt.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named as device buffers are device (HBM) addresses; the caller owns
 *    every buffer.  The library never allocates, frees, or keeps a pointer after
 *    a call returns, and holds no global mutable state: calls are thread-safe.
 *    The one exception is mla_decode_noalloc, which keeps its split partials
 *    in a scratch array of its own on each GPU (see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls
 *    only enqueue work on it: MLA_OK means "validated and launched", not "done".
 *  - All arguments are checked on the host before anything is launched; a call
 *    that returns an error has launched nothing (MLA_ERR_HIP aside, which reports
 *    a failed launch).  Contents of device buffers (block ids, sequence lengths)
 *    cannot be checked on the host: see each call.
 *  - Element type: `cfg->dtype` applies to q_nope, q_rope, q_abs, W^UK, W^UV, the
 *    cache pool, new rows and mla_out_proj's output.  Accumulation is fp32; the
 *    decode outputs (o_lat, lse) are always fp32.
 *  - Row-major layouts throughout; the last dimension listed is contiguous.
 *  - Device buffers must be 16-byte aligned (err_flag: 4-byte), MLA_ERR_ALIGN
 *    otherwise.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MLA_ERR_DIM = 2,         /* a size or config field is out of range             */
  MLA_ERR_DTYPE = 3,       /* unknown element type                               */
  MLA_ERR_CAPACITY = 4,    /* sequence would not fit the block table             */
  MLA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required         */
  MLA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch        */
  MLA_ERR_ALIGN = 7        /* a device pointer is not 16-byte aligned            */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Shapes of one MLA layer.  A cached row is [c (d_c) | k^R (d_rope)], width
 * W = d_c + d_rope.  The score scale defaults to 1/sqrt(d_nope + d_rope), the
 * divisor of the page-3 absorbed path ("Attention, Part 2", section "Why position
 * needs its own key").                                                          */
typedef struct {
  int32_t n_heads;       /* H, query heads                                      */
  int32_t d_c;           /* latent width                                        */
  int32_t d_rope;        /* decoupled rotary key width d^R_h (may be 0)         */
  int32_t d_nope;        /* per-head content query width (rows of W^UK[h])      */
  int32_t d_v;           /* per-head value width (rows of W^UV[h])              */
  int32_t block_size;    /* tokens per cache page                               */
  float softmax_scale;   /* 0 => 1/sqrt(d_nope + d_rope)                        */
  int32_t dtype;         /* mla_dtype                                           */
} mla_config;

/* Human-readable text for a status code (static storage; never NULL). */
const char* mla_status_string(int32_t status);

/* Version of this interface; bumped when a signature or layout changes. */
int32_t mla_abi_version(void);

/*
 * mla_absorb_q -- query-side absorption ("Attention, Part 2", section "The trick
 * that makes it fast": the new query is multiplied once by W^UK(h)^T and then
 * compared with the cached latents; "Multi-head latent attention (MLA)",
 * section 2 and Exercise 3).
 *
 *   q_abs[m, h, 0:d_c]        = sum_d q_nope[m, h, d] * w_uk[h, d, 0:d_c]
 *   q_abs[m, h, d_c:d_c+d_r]  = q_rope[m, h, :]
 *
 * q_nope [M, H, d_nope], q_rope [M, H, d_rope], w_uk [H, d_nope, d_c] (the
 * per-head view of a linear weight of shape (H*d_nope, d_c)), q_abs [M, H, d_c +
 * d_rope]; all device, cfg->dtype.  M = sequences x new tokens.  M == 0 launches
 * nothing.  q_rope may be NULL only if d_rope == 0.
 */
mla_status mla_absorb_q(const mla_config* cfg, const void* q_nope, const void* q_rope,
                        const void* w_uk, void* q_abs, int32_t M, void* stream);

/*
 * mla_cache_append -- store the new tokens' cache rows.  Only [c | k^R] is kept
 * per token ("Attention, Part 2", section "The MLA equations": the cache per
 * token is d_c + d_r numbers).
 *
 * The cache is a pool of pages, pool [num_blocks, block_size, W] (device).  Row j
 * of sequence b lives in page block_table[b, j / block_size] (device int32
 * [B, max_blocks]) at slot j % block_size.  For i < T_new:
 *     pool[block_table[b, p / bs], p % bs, :] = new_rows[b, i, :],  p = seq_lens[b] + i
 * seq_lens (device int32 [B]) holds the lengths BEFORE the append and is not
 * modified; the caller advances it.  max_seq_len_host is the host-side bound
 * max_b(seq_lens[b]) + T_new; it must be <= max_blocks * block_size
 * (MLA_ERR_CAPACITY).  On the device, a row whose page index or page id would
 * fall outside [0, max_blocks) or [0, num_blocks) is skipped, never written.
 */
mla_status mla_cache_append(const mla_config* cfg, void* pool, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, const void* new_rows, int32_t B,
                            int32_t T_new, int32_t max_seq_len_host, void* stream);

/*
 * mla_absorb_q_append -- mla_absorb_q and mla_cache_append of one decode step
 * in one call: the two are independent (the absorbed query does not read the
 * cache), so the append's rows are copied by extra workgroups of the absorb
 * launch (one kernel launch instead of two) where the bf16 MFMA absorb kernel
 * applies, and by the two usual launches otherwise.  Arguments, checks and
 * results are exactly those of the two calls (the first failing check of
 * mla_absorb_q, then of mla_cache_append, is returned, and nothing is launched
 * then); M == 0 or B * T_new == 0 leaves out that part.
 */
mla_status mla_absorb_q_append(const mla_config* cfg, const void* q_nope, const void* q_rope,
                               const void* w_uk, void* q_abs, int32_t M, void* pool,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               const void* new_rows, int32_t B, int32_t T_new,
                               int32_t max_seq_len_host, void* stream);

/*
 * Split-KV planning for mla_decode.  Each range of cache rows is attended on
 * its own and the partial results are merged by log-sum-exp.  Two plans:
 *  - plain (num_splits > 0, or the library's choice for equal lengths): the
 *    rows of every sequence are cut at the same points into `num_splits`
 *    contiguous ranges of equal size (the last may be shorter or empty);
 *  - balanced (the library's choice for the bf16 kernel with d_c = 512,
 *    d_rope = 64 and 64-row pages, when the lengths may
 *    differ: total_tokens_host is 0 or below B x max_seq_len_host): K work
 *    items per 64-row query group (one per compute unit over the grid), and
 *    each sequence gets splits in proportion to its length, chosen on the
 *    device from seq_lens so that no item holds more than the smallest
 *    bound on 32-row units the K items allow (at least 8 units).
 * mla_decode_num_splits returns what the library would choose for this batch:
 * the split count of a plain plan (>= 1) or K for a balanced one;
 * total_tokens_host is the sum of the sequence lengths if the caller knows it,
 * else 0.
 *
 * mla_decode_workspace_size returns the device workspace mla_decode needs for a
 * given num_splits (0 = the library's choice, as above) and the same
 * total_tokens_host; 0 bytes when no merge is needed.  Returns (size_t)-1 for
 * an invalid config.
 */
int32_t mla_decode_num_splits(const mla_config* cfg, int32_t B, int32_t T,
                              int32_t max_seq_len_host, int64_t total_tokens_host);
size_t mla_decode_workspace_size(const mla_config* cfg, int32_t B, int32_t T,
                                 int32_t max_seq_len_host, int64_t total_tokens_host,
                                 int32_t num_splits);

/*
 * mla_decode -- attention in latent space ("Attention, Part 2", sections "The
 * trick that makes it fast" and "Why position needs its own key"; "How DeepSeek
 * Rewrote the Transformer", section "Absorbed projections", point 3: the values
 * are the first d_c columns of the cached row).  For every sequence b, new token
 * t < T and head h, with R_j = the j-th cached row of b:
 *
 *   n      = causal ? seq_lens[b] - T + t + 1 : seq_lens[b]   (rows visible)
 *   s_j    = scale * <q_abs[b, t, h, :], R_j>                 j < n
 *   p_j    = exp(s_j - max s) / sum_k exp(s_k - max s)
 *   o_lat[b, t, h, :] = sum_j p_j R_j[0:d_c]
 *   lse[b, t, h]      = max s + log sum_k exp(s_k - max s)    (natural log)
 *
 * A query that sees no row gets o_lat = 0 and lse = -inf.
 *
 * q_abs [B, T, H, W] (cfg->dtype), pool / block_table as in mla_cache_append,
 * seq_lens [B] (device, lengths INCLUDING the T new tokens), o_lat [B, T, H, d_c]
 * fp32, lse [B, T, H] fp32 or NULL.  max_seq_len_host >= max_b seq_lens[b] and <=
 * max_blocks * block_size; rows past it are not attended.  On the device a page
 * id outside [0, num_blocks) is clamped into range (memory safety only: the
 * result is then meaningless).  causal is 0 or 1.  num_splits: 0 = library's
 * choice, else the split count to use.  workspace: device memory of at least
 * mla_decode_workspace_size(...) bytes for the same arguments, may be NULL when
 * that size is 0.  The workspace is scratch: its contents on entry do not matter.
 */
mla_status mla_decode(const mla_config* cfg, const void* q_abs, const void* pool,
                      int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                      const int32_t* seq_lens, int32_t max_seq_len_host, int32_t B,
                      int32_t T, int32_t causal, int32_t num_splits,
                      int64_t total_tokens_host, void* workspace, size_t workspace_bytes,
                      float* o_lat, float* lse, void* stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as mla_decode, minus the
 * workspace: the split partials go to a scratch array that the library owns,
 * mla_decode_noalloc_scratch_bytes() bytes (64 MiB) on each GPU it runs on,
 * reserved with the library's code on that GPU and held until the process
 * ends.  The call itself allocates and frees nothing.
 *  - num_splits = 0: the library's split choice, cut down to the most splits
 *    whose partials fit the scratch array (one split needs none), so the
 *    results can differ from mla_decode's in rounding only.
 *  - num_splits > 0 whose partials do not fit: MLA_ERR_WORKSPACE, nothing
 *    launched.
 *  - MLA_ERR_HIP if the scratch array's device address cannot be looked up
 *    (done once per GPU, on the first call that needs it, for the device of
 *    `stream`).
 * Every call on one GPU uses the same array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give wrong results.  Calls ordered on one stream are safe.
 */
mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_abs, const void* pool,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* seq_lens,
                              int32_t max_seq_len_host, int32_t B, int32_t T, int32_t causal,
                              int32_t num_splits, int64_t total_tokens_host, float* o_lat,
                              float* lse, void* stream);
size_t mla_decode_noalloc_scratch_bytes(void);

/*
 * mla_decode_out_proj -- mla_decode followed by mla_out_proj on its o_lat
 * (out[b, t, h, :] = W^UV[h] o_lat[b, t, h, :]: "Attention, Part 2", section
 * "The trick that makes it fast", W^UV applied once per head after the sum in
 * latent space), with the log-sum-exp merge of the split partials and the
 * up-projection in one launch where they can share it (bf16, d_c = 512,
 * d_rope = 64, 64-row pages, d_v a multiple of 4, and a plan with more than
 * one split): each head's merged rows go from the partials straight into the
 * projection's operand tiles.  Otherwise the calls' own launches run in turn.
 * Arguments as mla_decode's (same workspace, mla_decode_workspace_size), plus
 * w_uv [H, d_v, d_c] and out [B*T, H, d_v] (cfg->dtype) as mla_out_proj's;
 * o_lat and lse are written as mla_decode writes them, and out equals what
 * mla_out_proj computes from that o_lat, bit for bit.  Every check of both
 * calls runs before any launch.
 */
mla_status mla_decode_out_proj(const mla_config* cfg, const void* q_abs, const void* pool,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               int32_t max_seq_len_host, int32_t B, int32_t T, int32_t causal,
                               int32_t num_splits, int64_t total_tokens_host, const void* w_uv,
                               void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                               void* out, void* stream);

/*
 * mla_decode_fused -- mla_decode's split-KV attention and its log-sum-exp
 * merge in ONE kernel launch, for batches of variable-length sequences
 * ("Research on MLA": the fused, variable-length and megakernel decoders it
 * lists; "Attention, Part 2: MQA, GQA and MLA", section "Does a smaller cache
 * make writing faster?": once the cache is small, the fixed cost of each step
 * counts).  Persistent workgroups (at most one per compute unit) take work
 * items -- a 64-row query group against one split of one sequence, under the
 * same plain or balanced plan as mla_decode -- from an on-device queue; the
 * split that arrives last in its group hands the group's merge to whichever
 * workgroups run out of work items.  A sequence whose rows fit one split is
 * written directly.  Same arguments and results as mla_decode (rounding
 * aside: partials are merged in split order, as there) for the bf16 shape
 * with d_c = 512, d_rope = 64 and 64-row pages; any other config gives
 * MLA_ERR_DIM, as does a batch with more than 3,840 (sequence, 64-row group)
 * pairs, where mla_decode_fused_workspace_size returns (size_t)-1.
 *
 * workspace: device memory of at least mla_decode_fused_workspace_size(...)
 * bytes for the same arguments (MLA_ERR_WORKSPACE otherwise; never 0).  Its
 * first mla_decode_fused_counter_bytes() bytes (256 KiB) hold the queue's
 * counters and must be zero when a call starts: fill them with zeros once,
 * after allocating the workspace; every completed call leaves them zero, so
 * calls ordered on one stream can reuse the workspace for any shape.  Calls
 * that overlap in time on one workspace race.  The rest of the workspace is
 * scratch.  The 32-bit word at byte offset 512 is an error word: bit 0 set
 * means a merge waited past its bound (only a device that stalls could cause
 * it) and some rows were not written; zero the counters again after that.
 */
size_t mla_decode_fused_workspace_size(const mla_config* cfg, int32_t B, int32_t T,
                                       int32_t max_seq_len_host, int64_t total_tokens_host,
                                       int32_t num_splits);
size_t mla_decode_fused_counter_bytes(void);
mla_status mla_decode_fused(const mla_config* cfg, const void* q_abs, const void* pool,
                            int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t max_seq_len_host, int32_t B,
                            int32_t T, int32_t causal, int32_t num_splits,
                            int64_t total_tokens_host, void* workspace, size_t workspace_bytes,
                            float* o_lat, float* lse, void* stream);

/*
 * mla_out_proj -- output-side up-projection, applied once per head after the
 * latent-space sum ("Attention, Part 2", section "The trick that makes it fast":
 * W_uv(h) is applied just once at the end).
 *
 *   out[m, h, v] = sum_c w_uv[h, v, c] * o_lat[m, h, c]
 *
 * o_lat [M, H, d_c] fp32, w_uv [H, d_v, d_c] (cfg->dtype; the per-head view of a
 * linear weight of shape (H*d_v, d_c)), out [M, H, d_v] (cfg->dtype).  M == 0
 * launches nothing.
 */
mla_status mla_out_proj(const mla_config* cfg, const float* o_lat, const void* w_uv,
                        void* out, int32_t M, void* stream);

/*
 * mla_kv_produce -- the producer step before the cache: each new token's row is
 * made from its hidden vector h and written into the paged cache, replacing
 * mla_cache_append when the rows are not already at hand.
 *
 *   c   = W^DKV h                 ("Multi-head latent attention (MLA)", section 2)
 *   k^R = RoPE(W^KR h, p)         (same page, section 3; "Attention, Part 2",
 *                                  section "The MLA equations" and its code)
 *   pool[block_table[b, p / bs], p % bs, :] = [c | k^R],  p = seq_lens[b] + i
 *
 * RoPE turns each consecutive pair (x[2i], x[2i+1]) of k^R by the angle
 * p * rope_base^(-2i/d_rope) ("Attention, Part 2", section "Why position needs
 * its own key", one pair turned by m*theta; the angle rule is RoFormer's).  The
 * latent is never rotated.  rope_base 0 selects 10000; otherwise it must be a
 * finite value > 1.
 *
 * hidden [B, T_new, d_model], w_dkv [d_c, d_model], w_kr [d_rope, d_model]
 * (cfg->dtype; the weights of linear layers d_model -> d_c and d_model -> d_rope),
 * pool / block_table / seq_lens / max_seq_len_host as for mla_cache_append
 * (seq_lens BEFORE the append, not modified; rows whose page or page id is out
 * of range are skipped on the device).  d_c and d_rope must be even.  Products
 * accumulate in fp32 and are rounded once to cfg->dtype.  workspace (device, fp32
 * partial sums) must hold mla_kv_produce_workspace_size(cfg, B * T_new, d_model)
 * bytes (MLA_ERR_WORKSPACE otherwise); its contents on entry do not matter.
 * B * T_new == 0 launches nothing.
 */
size_t mla_kv_produce_workspace_size(const mla_config* cfg, int32_t M, int32_t d_model);
mla_status mla_kv_produce(const mla_config* cfg, const void* hidden, int32_t d_model,
                          const void* w_dkv, const void* w_kr, float rope_base, void* pool,
                          int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, int32_t B, int32_t T_new,
                          int32_t max_seq_len_host, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * mla_rope -- the rotation of the query's decoupled rotary part, in place: for
 * m < M and h < heads, x[m, h, 2i .. 2i+1] is turned by positions[m] *
 * rope_base^(-2i/d_rope), the same rotation mla_kv_produce applies to k^R (the
 * score's positional term pairs the rotated query with the rotated key:
 * "Attention, Part 2", section "Why position needs its own key").  Apply it to
 * q_rope before mla_absorb_q.  x [M, heads, d_rope] (device, cfg->dtype),
 * positions [M] (device int32; for decode, token i of sequence b is at
 * seq_lens_before[b] + i).  rope_base as for mla_kv_produce; d_rope must be
 * even.  M, heads or d_rope == 0 launches nothing.
 */
mla_status mla_rope(const mla_config* cfg, void* x, int32_t heads, const int32_t* positions,
                    int32_t M, float rope_base, void* stream);

/*
 * The output side, after mla_out_proj: the model's output projection W^O, and
 * W^UV folded into it.
 *
 * mla_o_proj -- y[m, :] = W^O x_m, where x_m lists the per-head outputs
 * attn[m, h, :] head after head ("Attention, Part 2", section "The trick that
 * makes it fast": its inference code reshapes a token's heads into one vector
 * and applies W_o).
 *   attn [M, H, d_v] (cfg->dtype: mla_out_proj's output), w_o [d_model, H * d_v]
 *   (cfg->dtype; the weight of a linear layer H * d_v -> d_model), y [M, d_model]
 *   (cfg->dtype).
 *
 * mla_fold_uv_o -- the output-side absorption ("How DeepSeek Rewrote the
 * Transformer", section "Absorbed projections: the mathematician's shortcut",
 * point 2: W^UV and W^O merge into one matrix), a one-time weight preparation:
 *   w_fold[i, h * d_c + c] = sum_v w_o[i, h * d_v + v] * w_uv[h, v, c]
 *   w_uv [H, d_v, d_c], w_o [d_model, H * d_v], w_fold [d_model, H * d_c], all
 *   cfg->dtype; fp32 accumulation, rounded once.  d_v must be <= 256.
 *
 * mla_o_proj_folded -- y[m, :] = w_fold z_m, where z_m lists the latent outputs
 * o_lat[m, h, :] head after head: the same y as mla_out_proj followed by
 * mla_o_proj, in one product.
 *   o_lat [M, H, d_c] fp32 (mla_decode's output), w_fold as above, y [M, d_model]
 *   (cfg->dtype).  The bf16 kernel rounds o_lat to bf16 as it reads it.  The
 *   folded matrix holds d_c / d_v times the bytes of W^O (12.8x at the V2-scale
 *   widths), and a decode step streams its weights, so the unfolded pair is
 *   the faster route there; the folded one gives the same y.
 *
 * Both products accumulate in fp32 and round once.  When the k dimension is
 * split over workgroups, the partial sums go to `workspace` (device) and are
 * added in a fixed order (reruns are bit-exact); for 17 to 128 fp32 rows
 * (mla_o_proj_folded) the workspace also takes their bf16 copy, rounded in a
 * first launch and then streamed like bf16 rows.  It must hold
 * mla_o_proj_workspace_size(cfg, M, d_model, folded) bytes (0: none needed, NULL
 * allowed), else MLA_ERR_WORKSPACE; its contents on entry do not matter.
 * mla_o_proj_workspace_size returns (size_t)-1 for invalid arguments.  M == 0
 * launches nothing.
 */
size_t mla_o_proj_workspace_size(const mla_config* cfg, int32_t M, int32_t d_model,
                                 int32_t folded);
mla_status mla_o_proj(const mla_config* cfg, const void* attn, const void* w_o, void* y,
                      int32_t M, int32_t d_model, void* workspace, size_t workspace_bytes,
                      void* stream);
mla_status mla_fold_uv_o(const mla_config* cfg, const void* w_uv, const void* w_o,
                         void* w_fold, int32_t d_model, void* stream);
mla_status mla_o_proj_folded(const mla_config* cfg, const float* o_lat, const void* w_fold,
                             void* y, int32_t M, int32_t d_model, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Debug and test helpers.
 *
 * mla_gather_rows: dense[b, j, :] = the j-th cached row of sequence b, for
 * j < min(seq_lens[b], max_seq_len_host), through the same page addressing as
 * mla_decode.  dense [B, max_seq_len_host, W] device, cfg->dtype; rows at or past a
 * sequence's length are left untouched.
 *
 * mla_validate_block_table: checks on the device that every page a sequence
 * uses (p < ceil(seq_lens[b] / block_size)) has p < max_blocks and an id in
 * [0, num_blocks).  *err_flag (device int32) is set to 0, then bit 0 is set for a
 * bad page id and bit 1 for a sequence longer than the table.
 */
mla_status mla_gather_rows(const mla_config* cfg, const void* pool, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t B, int32_t max_seq_len_host,
                           void* dense, void* stream);
mla_status mla_validate_block_table(const int32_t* block_table, int32_t B,
                                    int32_t max_blocks, const int32_t* seq_lens,
                                    int32_t block_size, int32_t num_blocks,
                                    int32_t* err_flag, void* stream);

/*
 * Measurement helper.
 *
 * mla_stream_read: reads `bytes` of device memory at `src` once and XORs every
 * 16-byte chunk into the 16 bytes at `sink` (device, 4 x uint32, updated in
 * place with atomic XORs: sink becomes sink ^ XOR of all chunks).  It gives
 * the achievable HBM read rate that a roofline of the decode path is set
 * beside (the pages price the method by the bytes of cache it reads:
 * "Attention, Part 2: MQA, GQA and MLA", section "Why reading the cache is
 * the real cost"), and a kernel of known bytes to calibrate memory-traffic
 * counters against.  mode 0: 16-byte non-temporal loads into registers from
 * 256 x 256 threads striding over the buffer.  mode 1: direct-to-LDS copies,
 * the path the decode kernel streams the cache through: each of 256
 * workgroups streams a contiguous range in 1 KiB copies through a ring in
 * LDS (a tail under 1 KiB is read with plain loads).  src and sink 16-byte
 * aligned and bytes a multiple of 16 (MLA_ERR_ALIGN otherwise), mode 0 or 1
 * (MLA_ERR_DIM otherwise); bytes == 0 launches nothing.
 */
mla_status mla_stream_read(const void* src, size_t bytes, void* sink, int32_t mode,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
