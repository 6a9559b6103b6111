/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA absorbed-decode library.
 *
 * One decode step of DeepSeek-style Multi-Head Latent Attention with matrix
 * absorption, as four calls on one HIP stream:
 *
 *   mla_absorb_q     q_abs = [ W_UK^T q_nope ; RoPE(q_rope) ]      per head
 *   mla_decode_attn  split-K attention of every head against the shared
 *                    cached rows [c_kv ; k_rope] -> partial o_lat + lse
 *   mla_combine      log-sum-exp merge of the partials -> o_lat
 *   mla_out_proj     o = W_UV o_lat                                per head
 *
 * or as three, with mla_combine_out_proj doing the last two in one launch.
 *
 * Uncompressed per-head keys and values are never written to memory.
 *
 * Pages cited (title, section):
 *   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
 *          DeepSeek MLA Matrix Absorption and Memory Minimalism"
 *   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations,
 *          Low-Rank KV Compression, Decoupled Rotary Positional Embeddings,
 *          and Inference Matrix Absorption"
 *
 * Conventions shared by every call:
 *   - Tensor arguments are DEVICE pointers, row-major, innermost dimension
 *     contiguous, 16-byte aligned.  `dims` and the scalars are read on the
 *     host.  The caller owns all memory; no call allocates or frees.
 *   - Every call only validates its host arguments and enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the null stream).  Nothing is
 *     synchronised.  Argument errors are reported before anything is
 *     enqueued, and then nothing is enqueued.
 *   - Device-side contents (seq_lens, positions, block_table) are trusted:
 *     0 <= seq_lens[b] <= max_seq_len, block ids inside the pool.  Violations
 *     are undefined behaviour.
 *   - No call keeps state between calls; calls are reentrant.
 *   - Return value: MLA_OK or one of the error codes below.
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misalignment, bad enum  */
  MLA_ERR_UNSUPPORTED = 2, /* valid but not built (dtype mix, width limits)   */
  MLA_ERR_WORKSPACE = 3,   /* workspace pointers missing                     */
  MLA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed     */
  MLA_ERR_TOO_LARGE = 5    /* request exceeds a fixed internal buffer        */
};

/* Element types. */
enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2 /* OCP E4M3 "fn": bias 7, max 448, no inf; cache only */
};

/* Flags in mla_dims_t.flags. */
enum {
  MLA_FLAG_GENERIC = 1 /* force the plain SIMT kernels instead of MFMA ones */
};

/* Cached tokens are processed, and split-K work is divided, in tiles of
 * this many tokens; a paged cache must use blocks of this many rows
 * ([ARCH] 4.1: page blocks of 64). */
#define MLA_TILE_TOKENS 64

typedef struct mla_dims {
  int32_t batch;    /* B, sequences (0 = nothing to do)                     */
  int32_t q_len;    /* Lq, query tokens per sequence (>= 1)                  */
  int32_t heads;    /* H, attention heads                                    */
  int32_t d_nope;   /* per-head content query/key width (DeepSeek-V3: 128)   */
  int32_t d_rope;   /* decoupled RoPE width, even (64)                       */
  int32_t d_latent; /* latent width d_c (512)                                */
  int32_t d_v;      /* per-head value width (128)                            */
  int32_t q_dtype;  /* MLA_F32 or MLA_BF16: q_nope, q_rope, w_uk, w_uv,
                       o_lat, o (q_abs: fp32, or IEEE fp16 for MLA_BF16)     */
  int32_t kv_dtype; /* MLA_F32 (with q F32), MLA_BF16 or MLA_FP8_E4M3
                       (with q BF16): the cache                              */
  int32_t flags;    /* MLA_FLAG_* */
} mla_dims_t;

/*
 * mla_absorb_q -- key absorption and query RoPE.
 *
 * [ARCH] 3.1: the content score q^C . (W_UK,i c_j) is regrouped as
 * (W_UK,i^T q^C) . c_j, so each head's query is mapped once per step into the
 * latent space and scored against the raw cached latents.  [ARCH] 2.3 /
 * [MATH] "The Decoupled RoPE Solution": the positional part of the query is
 * rotated by RoPE; [MATH] reference module (apply_rope): consecutive pairs
 * (x[2k], x[2k+1]) turn by angle pos * rope_base^(-2k/d_rope).
 *
 *   q_nope    [B, Lq, H, d_nope]          q_dtype
 *   q_rope    [B, Lq, H, d_rope]          q_dtype, before rotation
 *   positions [B, Lq]                     int32, token position of each query
 *   rope_base                             e.g. 10000
 *   w_uk      [H, d_nope, d_latent]       q_dtype, W_UK,i = w_uk[i] (d_nope x d_latent)
 *   q_abs     [B, Lq, H, d_latent+d_rope] output, fp32 when q_dtype is
 *             MLA_F32 and IEEE fp16 when it is MLA_BF16:
 *             q_abs[..., :d_latent] = w_uk[h]^T q_nope   (fp32 accumulate)
 *             q_abs[..., d_latent:] = RoPE(q_rope, pos)  (angle in fp64)
 *             The fp16 form keeps 11 significant bits, so the scores of
 *             long contexts with large cached values stay within the bf16
 *             tolerance (a bf16 query moves them by ~1e-2); magnitudes
 *             beyond 65504 saturate.
 */
int mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                 const int32_t* positions, float rope_base, const void* w_uk,
                 void* q_abs, void* stream);

/*
 * mla_decode_attn -- split-K attention over the shared latent cache.
 *
 * [ARCH] 3.1 score: S_t = (q~ . c_t + q^R . k^R_t) * softmax_scale with the
 * absorbed query q~ and the decoupled key k^R shared by all heads (2.3);
 * softmax over the cached tokens; [ARCH] 3.2: the weights multiply the raw
 * latents, giving the 512-wide latent output sum_t P_t c_t.
 *
 * Cache rows.  Token t of sequence b lives in row
 *     r = block_table ? block_table[b*max_blocks_per_seq + t/64]*64 + t%64
 *                     : b*max_seq_len + t
 * with its latent at latent_cache + r*kv_row_stride (d_latent elements) and
 * its post-RoPE key at rope_cache + r*kv_row_stride (d_rope elements).  The
 * fused layout is kv_row_stride = d_latent + d_rope and
 * rope_cache = latent_cache + d_latent.  For MLA_FP8_E4M3 the stored value
 * is code * kv_scale[r] (one fp32 scale per token).
 *
 *   q_abs        [B, Lq, H, d_latent+d_rope] fp32 or fp16 (output of
 *                mla_absorb_q).  bf16 cache rows are scored and summed in
 *                fp16: every bf16 value of magnitude 2^-17 .. 65504 is an
 *                fp16 value, so the conversion is exact there; larger
 *                magnitudes saturate, smaller ones keep 2^-24 absolute
 *                precision.
 *   seq_lens     [B] int32, cached tokens per sequence
 *   block_table  [B, max_blocks_per_seq] int32, or NULL for contiguous rows
 *   block_size   must be MLA_TILE_TOKENS when block_table != NULL
 *   max_seq_len  bound on seq_lens; row pitch of the contiguous layout
 *   causal       0: every query sees all seq_lens[b] tokens; 1: query i sees
 *                tokens t <= seq_lens[b] - Lq + i
 *   num_splits   G >= 1 work units.  The 64-token tiles of all sequences,
 *                taken in order, are divided evenly: unit u covers global
 *                tiles [floor(u*T/G), floor((u+1)*T/G)) where T is the total
 *                tile count.  Each unit writes one partial per sequence it
 *                touches, into slot u + b.
 *   o_part       [G + B - 1, Lq*H, d_latent] workspace: normalised partial
 *                latent outputs (row index i*H + h), stored as fp32 when
 *                q_dtype is MLA_F32 and as IEEE fp16 otherwise (the partials
 *                are weighted averages of cached values, well inside fp16
 *                range; its 2^-11 rounding is far below the bf16 outputs')
 *   lse_part     [G + B - 1, Lq*H] fp32 workspace: natural-log LSE of each
 *                partial (-inf when the partial saw no token)
 */
int mla_decode_attn(const mla_dims_t* dims, const void* q_abs, const void* latent_cache,
                    const void* rope_cache, int64_t kv_row_stride, const float* kv_scale,
                    const int32_t* seq_lens, const int32_t* block_table,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                    int32_t causal, float softmax_scale, int32_t num_splits, void* o_part,
                    float* lse_part, void* stream);

/*
 * mla_combine -- merge the split-K partials of mla_decode_attn.
 *
 * For each sequence b and row (i, h), with the units that touched b:
 *   lse = log sum_u exp(lse_u);  o_lat = sum_u exp(lse_u - lse) o_u.
 * This is the softmax over all of b's tokens ([MATH] "Value Output Matrix
 * Absorption": softmax weights applied to the cached latents).
 *
 *   num_splits, seq_lens, o_part, lse_part: as passed to mla_decode_attn
 *   o_lat   [B, Lq, H, d_latent] q_dtype, output (0 where no token was seen)
 *   lse_out [B, Lq, H] fp32 natural-log LSE, output; may be NULL
 */
int mla_combine(const mla_dims_t* dims, int32_t num_splits, const int32_t* seq_lens,
                const void* o_part, const float* lse_part, void* o_lat, float* lse_out,
                void* stream);

/*
 * mla_out_proj -- value up-projection of the latent output.
 *
 * [ARCH] 3.2: o_i = sum_j P_ij W_UV,i c_j = W_UV,i (sum_j P_ij c_j).
 *
 *   o_lat [B, Lq, H, d_latent] q_dtype
 *   w_uv  [H, d_v, d_latent]   q_dtype, W_UV,i = w_uv[i] (d_v x d_latent)
 *   o     [B, Lq, H, d_v]      q_dtype, output (fp32 accumulate)
 */
int mla_out_proj(const mla_dims_t* dims, const void* o_lat, const void* w_uv, void* o,
                 void* stream);

/*
 * mla_combine_out_proj -- mla_combine and mla_out_proj in one call.
 *
 * Same results as mla_combine followed by mla_out_proj.  For bf16 queries,
 * d_latent 512 and d_v % 32 == 0 (without MLA_FLAG_GENERIC) one kernel
 * merges the partials of 32 query rows of a head in on-chip memory and
 * projects them right away, so the latent output makes no round trip
 * through device memory; o_lat may then be NULL (not written).  Otherwise
 * the two kernels run in turn and o_lat must be given.
 *
 *   num_splits, seq_lens, o_part, lse_part: as passed to mla_decode_attn
 *   w_uv    [H, d_v, d_latent] q_dtype
 *   o       [B, Lq, H, d_v] q_dtype, output
 *   lse_out [B, Lq, H] fp32 natural-log LSE, output; may be NULL
 *   o_lat   [B, Lq, H, d_latent] q_dtype, output; may be NULL (see above)
 */
int mla_combine_out_proj(const mla_dims_t* dims, int32_t num_splits, const int32_t* seq_lens,
                         const void* o_part, const float* lse_part, const void* w_uv, void* o,
                         float* lse_out, void* o_lat, void* stream);

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(int status);

/* Element counts of the two split-K workspaces for `num_splits` units. */
int mla_workspace_elems(const mla_dims_t* dims, int32_t num_splits, int64_t* o_part_elems,
                        int64_t* lse_part_elems);

/* Byte sizes of the two split-K workspaces (o_part elements are 4 bytes
 * when q_dtype is MLA_F32, else 2; lse_part elements are 4 bytes). */
int mla_workspace_bytes(const mla_dims_t* dims, int32_t num_splits, int64_t* o_part_bytes,
                        int64_t* lse_part_bytes);

/* A good num_splits for `device`: one work unit per compute unit and
 * block of 128 query rows.  Host-only query of device properties. */
int mla_num_splits_hint(const mla_dims_t* dims, int32_t device, int32_t* num_splits);

/*
 * mla_split_plan -- host-side view of the split-K division (no GPU use).
 *
 * For host-resident seq_lens[B], writes for every sequence b the first and
 * last unit that touch it (-1, -1 when seq_lens[b] == 0) and its first
 * global tile.  Units first_unit[b]..last_unit[b] hold b's partials in slots
 * u + b.  Useful to size and inspect the workspaces.
 */
int mla_split_plan(int32_t batch, const int32_t* seq_lens_host, int32_t num_splits,
                   int32_t* first_unit, int32_t* last_unit, int64_t* first_tile);

/*
 * Cache-append producer: the cached row of each new token ([ARCH] 2.1 and
 * 2.3; [MATH] reference module, the latent normalised before caching):
 *   c_kv   = RMSNorm(W_DKV h) * kv_norm_w   (mean square over d_latent, + eps)
 *   k_rope = RoPE(W_KR h) at positions[t]   (interleaved pairs, pair k turns
 *                                            by pos * rope_base^(-2k/d_rope))
 * written to latent_cache + cache_rows[t] * kv_row_stride (d_latent values)
 * and rope_cache + cache_rows[t] * kv_row_stride (d_rope values), the row
 * layout mla_decode_attn reads.
 *
 *   h          [n_tokens, d_model]   bf16 hidden states of the new tokens
 *   w_dkv      [d_latent, d_model]   bf16 (one row per latent channel)
 *   kv_norm_w  [d_latent]            bf16 RMSNorm weight
 *   w_kr       [d_rope, d_model]     bf16
 *   positions  [n_tokens]            int32 position of each new token
 *   cache_rows [n_tokens]            int64 destination row of each token
 *                                    (distinct rows; paging is the caller's)
 *   workspace  mla_kv_append_workspace_bytes() bytes (fp32 partial sums)
 * kv_dtype MLA_BF16 stores bf16 values (kv_scale must be NULL);
 * MLA_FP8_E4M3 stores OCP e4m3 codes of the row divided by its scale
 * amax/448 (amax over the token's 576 values, fp32) and the scale to
 * kv_scale[cache_rows[t]] (fp32), the layout mla_decode_attn reads.
 * Built for d_latent 512, d_rope 64, d_model a multiple of 512 up to 16384;
 * anything else is MLA_ERR_UNSUPPORTED.  Pointers: h, weights and workspace
 * 16-byte aligned; latent_cache 16-byte (bf16) or 8-byte (fp8) aligned,
 * rope_cache 4-byte (bf16) or 2-byte (fp8) aligned, kv_scale 4-byte
 * aligned; kv_row_stride (elements) a multiple of 8 and >= 512.
 * Asynchronous on `stream`; the caller owns all memory.
 */
typedef struct mla_append_dims {
  int32_t n_tokens;
  int32_t d_model;
  int32_t d_latent;
  int32_t d_rope;
  int32_t kv_dtype;
} mla_append_dims_t;

int mla_kv_append_workspace_bytes(const mla_append_dims_t* dims, int64_t* bytes);

int mla_kv_append(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
                  const void* kv_norm_w, const void* w_kr, const int32_t* positions,
                  float rope_base, float eps, const int64_t* cache_rows, void* latent_cache,
                  void* rope_cache, int64_t kv_row_stride, float* kv_scale, void* workspace,
                  void* stream);

/*
 * mla_kv_append_noalloc -- mla_kv_append without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, results and validation as mla_kv_append; the partial sums
 * go to a static device array of MLA_KV_APPEND_NOALLOC_SCRATCH_BYTES bytes
 * that every GPU the library runs on holds until the process ends.  A call
 * whose mla_kv_append_workspace_bytes() exceeds that size returns
 * MLA_ERR_TOO_LARGE before anything is enqueued (8 MiB: e.g. 260 new tokens
 * at hidden width 7168).  The first call on a GPU looks the array's device
 * address up on the current device (nothing is allocated, ever); call it
 * with the stream's device current.  All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and must be serialised by the caller.
 */
#define MLA_KV_APPEND_NOALLOC_SCRATCH_BYTES (8 << 20)
int mla_kv_append_noalloc(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
                          const void* kv_norm_w, const void* w_kr, const int32_t* positions,
                          float rope_base, float eps, const int64_t* cache_rows,
                          void* latent_cache, void* rope_cache, int64_t kv_row_stride,
                          float* kv_scale, void* stream);

/*
 * ---- Prefill in MHA form ([ARCH] FAQ on prefill; "DeepSeek's attention
 * evolution - [MLA]" 2.5).  In prefill every prompt token is a query, so
 * absorbing W_UK into the queries would score 512-wide latents instead of
 * 128-wide keys (~4x the attention flops); the latent is expanded into
 * per-head keys and values once instead, and ordinary causal attention runs
 * over them.  Both calls are built for bf16 (q_dtype = kv_dtype =
 * MLA_BF16), d_nope = d_v = 128, d_rope = 64, d_latent = 512, kv_row_stride
 * a multiple of 8 up to 65536, max_seq_len <= 262144 and
 * batch * ceil(max_seq_len / 128) <= 65535; anything else returns
 * MLA_ERR_UNSUPPORTED.
 */

/*
 * mla_prefill_expand -- per-head keys and values of the cached latents.
 *
 *   k_nope[b, t, h, :] = W_UK,h c_t     ([ARCH] 2.3: content key W^UK c)
 *   v[b, t, h, :]      = W_UV,h c_t     ([ARCH] 3.2: value W^UV c)
 * for every t < seq_lens[b] (fp32 accumulate, bf16 result); rows
 * t >= seq_lens[b] are not written.
 *
 *   latent_cache, kv_row_stride, seq_lens, block_table, max_blocks_per_seq,
 *   block_size, max_seq_len: the cache rows, addressed as in mla_decode_attn
 *   w_uk     [H, d_nope, d_latent] bf16
 *   w_uv     [H, d_v, d_latent]    bf16
 *   k_nope   [B, max_seq_len, H, d_nope] bf16, output
 *   v        [B, max_seq_len, H, d_v]    bf16, output
 */
int mla_prefill_expand(const mla_dims_t* dims, const void* latent_cache, int64_t kv_row_stride,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                       const void* w_uk, const void* w_uv, void* k_nope, void* v, void* stream);

/*
 * mla_prefill_attn -- attention of the prompt over the expanded keys.
 *
 * Query i of sequence b (the prompt's Lq tokens are the last Lq of its
 * seq_lens[b] cached tokens) scores every visible token t:
 *   s_t = ([q_nope ; RoPE(q_rope, pos)] . [k_nope_t ; k_rope_t]) * softmax_scale
 * ([ARCH] 2.3: decoupled query and key; 3.1: score), with t <= seq_lens[b]
 * - Lq + i when causal (else every cached token), and
 *   o = softmax(s) . v,   lse = log sum_t exp(s_t).
 * A query that sees no token gets o = 0, lse = -inf.
 *
 *   q_nope     [B, Lq, H, d_nope] bf16
 *   q_rope     [B, Lq, H, d_rope] bf16, before rotation (as mla_absorb_q)
 *   positions  [B, Lq] int32
 *   rope_base  e.g. 10000
 *   k_nope, v  outputs of mla_prefill_expand for the same cache
 *   rope_cache the post-RoPE keys, rows addressed as in mla_decode_attn
 *   causal     0 or 1
 *   o          [B, Lq, H, d_v] bf16, output
 *   lse        [B, Lq, H] fp32 natural-log LSE, output; may be NULL
 */
int mla_prefill_attn(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                     const int32_t* positions, float rope_base, const void* k_nope,
                     const void* v, const void* rope_cache, int64_t kv_row_stride,
                     const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                     int32_t causal, float softmax_scale, void* o, float* lse, void* stream);

/*
 * ---- Output-side absorption ([ARCH] 3.2 and 4.2; [MATH] "Value Output
 * Matrix Absorption").  The value up-projection W_UV,i of head i and that
 * head's d x d_v block W_O,i of the output projection W_O = [W_O,1 ... W_O,H]
 * act back to back on the latent output, so they can be multiplied once,
 * when the model is loaded, into W~_O,i = W_O,i W_UV,i (d x d_c); the
 * attention's latent outputs then map straight to the hidden width,
 *   u = sum_i W~_O,i o~_i.
 * Built for q_dtype MLA_BF16, d_latent 512, d_v <= 128, heads <= 1024,
 * d_model <= 65536 and batch * q_len * d_model < 2^31; anything else
 * returns MLA_ERR_UNSUPPORTED.  kv_dtype is not used.
 */

/* Bytes of the fused weight mla_fuse_out_weight writes:
 * ceil(d_model / 32) * 32 * H * d_latent * 2. */
int mla_fused_out_weight_bytes(const mla_dims_t* dims, int32_t d_model, int64_t* bytes);

/*
 * mla_fuse_out_weight -- the fused weight, once per layer (load time).
 *
 *   w_o      [d_model, H * d_v]   bf16, columns i*d_v .. i*d_v+d_v-1 are W_O,i
 *   w_uv     [H, d_v, d_latent]   bf16 (as in mla_out_proj)
 *   w_fused  mla_fused_out_weight_bytes() bytes, output: the values
 *            W~[n, k] = sum_j w_o[n, i*d_v + j] * w_uv[i, j, c],  k = i*d_latent + c
 *            (fp32 accumulate, one rounding to bf16), stored in 1 KB blocks
 *            in the order mla_out_proj_fused's matrix instructions read
 *            them: with K = H * d_latent, element (n, k) sits at bf16 index
 *              ((n/32 * K/16 + k/16) * 64 + ((k/8) % 2) * 32 + n % 32) * 8 + k % 8
 *            and rows n from d_model to the next multiple of 32 are zero.
 */
int mla_fuse_out_weight(const mla_dims_t* dims, int32_t d_model, const void* w_o,
                        const void* w_uv, void* w_fused, void* stream);

/* Bytes of the workspace mla_out_proj_fused needs, with M = batch * q_len:
 * 8 * M * d_model * 4 (fp32 partial sums of eight slices of the H * d_latent
 * inputs) + ceil(M / 32) * 32 * H * d_latent * 2 (o_lat repacked into the
 * order the matrix instructions read it). */
int mla_out_proj_fused_workspace_bytes(const mla_dims_t* dims, int32_t d_model, int64_t* bytes);

/*
 * mla_out_proj_fused -- the block output from the latent attention output.
 *
 *   o_lat     [B, Lq, H, d_latent] bf16 (mla_combine's o_lat)
 *   w_fused   mla_fuse_out_weight's output for the same dims and d_model
 *   workspace mla_out_proj_fused_workspace_bytes() bytes, 16-byte aligned;
 *             overwritten (no initial contents needed)
 *   out       [B, Lq, d_model] bf16, output:
 *             out[b, t, n] = sum_{i, c} W~[n, i*d_latent + c] * o_lat[b, t, i, c]
 *             (fp32 accumulate; the eight slice sums are added in a fixed
 *             order, so results repeat bit for bit)
 * batch == 0 returns MLA_OK with nothing enqueued.
 */
int mla_out_proj_fused(const mla_dims_t* dims, int32_t d_model, const void* o_lat,
                       const void* w_fused, void* workspace, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
