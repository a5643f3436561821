/*
 * libmla — Multi-head Latent Attention (MLA) decode over a latent KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is MLA as defined in the DeepSeek-V2 paper (Chinese translation
 * of the paper), section 2.1:
 *   - 2.1.2 low-rank key-value joint compression: each cached token keeps one
 *     latent c_KV of width d_c instead of per-head keys and values; keys and
 *     values are the up-projections W_UK c_KV and W_UV c_KV, and at inference
 *     W_UK can be folded into the query side and W_UV into the output side;
 *   - 2.1.3 decoupled RoPE: a rotary key k^R of width d_h^R, shared by all
 *     heads, is cached beside c_KV; a head's score is [q^C; q^R]·[k^C; k^R].
 * With both foldings a decode step for one layer is, per sequence b and head h:
 *   q_lat[b,h]  = [ W_UK[h]^T q_nope[b,h] ; q_rope[b,h] ]          (absorb)
 *   s_j         = sm_scale * q_lat[b,h] · row_j,  row_j = [c_KV_j ; k^R_j]
 *   o_lat[b,h]  = sum_j softmax(s)_j c_KV_j,  lse = log sum_j exp(s_j)  (decode)
 *   o[b,h]      = W_UV[h] o_lat[b,h]                              (out-proj)
 * Long caches may be cut into splits whose normalised partial results are
 * merged by log-sum-exp (combine).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller; the
 *     library allocates nothing and keeps no state except a thread-local copy
 *     of the last HIP error. Pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on
 *     it and the call returns without synchronising.
 *   - Arguments are validated on the host before anything is enqueued. On any
 *     failure nothing is enqueued and a negative mla_status is returned; the
 *     library never aborts and never throws across this boundary.
 *   - Layouts are dense row-major with the last index fastest.
 *   - Supported head shapes (H, d_latent, d_rope, d_nope, d_v) and dtypes:
 *       (128, 512, 64, 128, 128): MLA_BF16 tensors, cache MLA_BF16 or MLA_FP8_E4M3
 *       (4, 32, 16, 32, 32):      MLA_F32 everywhere
 *     Anything else returns MLA_ERR_UNSUPPORTED.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mla_status;
#define MLA_OK               0
#define MLA_ERR_NULL        (-1)  /* a required pointer is NULL                     */
#define MLA_ERR_SHAPE       (-2)  /* a size is negative, zero where it must not be,
                                     or inconsistent with another                 */
#define MLA_ERR_DTYPE       (-3)  /* unknown dtype or unsupported dtype combination */
#define MLA_ERR_UNSUPPORTED (-4)  /* head shape outside the compiled set, or a size
                                     beyond a documented limit                    */
#define MLA_ERR_ALIGN       (-5)  /* a pointer or stride breaks 16-byte alignment   */
#define MLA_ERR_HIP         (-6)  /* a HIP call failed; see mla_last_hip_error()    */

#define MLA_F32       0
#define MLA_BF16      1
#define MLA_FP8_E4M3  2   /* OCP e4m3 ("e4m3fn"): bias 7, max 448, no infinities */

typedef void* mla_stream;   /* a hipStream_t */

typedef struct {
  int32_t num_heads;   /* H                                  */
  int32_t d_latent;    /* d_c: width of c_KV                 */
  int32_t d_rope;      /* d_h^R: width of the rotary key     */
  int32_t d_nope;      /* per-head width of q^C and k^C      */
  int32_t d_v;         /* per-head width of v^C              */
} mla_dims;

/*
 * Rotary position frequencies (DeepSeek-V2 paper, section 2.1.3: RoPE on the
 * decoupled query and key; section 3.1.4: YaRN applied to the decoupled key to
 * extend the context, with s = 40, alpha = 1, beta = 32 over a 4K original
 * context). Feature pair (2i, 2i + 1) of a rotary vector at position p turns
 * by p * f_i:
 *   theta_i = base^(-2i / d_rope);
 *   yarn_scale == 1: f_i = theta_i (plain RoPE; the yarn_* fields are unused);
 *   yarn_scale  > 1 (YaRN, by-parts interpolation of the paper the pages
 *   cite): r_i = yarn_orig_ctx * theta_i / (2 pi) turns over the original
 *   context, g = clamp((r_i - yarn_alpha) / (yarn_beta - yarn_alpha), 0, 1),
 *   f_i = (1 - g) * theta_i / yarn_scale + g * theta_i.
 * The frequencies are computed on the host in double precision; angles
 * p * f_i are formed in double precision on the device. YaRN's length scaling
 * of the softmax is not part of the rotation: fold it into sm_scale.
 * Requires base > 0, yarn_scale >= 1 and, for yarn_scale > 1,
 * yarn_alpha < yarn_beta and yarn_orig_ctx > 0 (else MLA_ERR_SHAPE).
 */
typedef struct {
  float base;
  float yarn_scale;
  float yarn_alpha;
  float yarn_beta;
  int32_t yarn_orig_ctx;
} mla_rope;

/*
 * The latent cache of one layer (DeepSeek-V2 paper, section 2.1.3: one
 * (d_c + d_h^R)-element row per cached token).
 *
 * Token j of sequence b lives in physical row r(b, j):
 *   contiguous (page_size == 0): r = b * seq_stride + j
 *   paged      (page_size  > 0): r = block_table[b * max_pages_per_seq + j / page_size]
 *                                    * page_size + j % page_size
 * dtype MLA_BF16 / MLA_F32: `latent` holds rows of d_latent + d_rope elements,
 *   c_KV first then k^R, consecutive rows `row_stride` elements apart.
 * dtype MLA_FP8_E4M3: `latent` holds rows of d_latent e4m3 codes (`row_stride`
 *   bytes apart); `rope` holds bf16 rows of d_rope elements (`rope_stride`
 *   elements apart); `scale` holds one fp32 per row; c_KV = code * scale.
 *   Scales are zero or normal fp32 numbers (a subnormal one may flush to
 *   zero on the way through the products). The decode keeps the codes unscaled in
 *   its products (the contiguous form scores them as e4m3 against an exact
 *   two-part e4m3 split of the query) and multiplies each token's latent
 *   score, and its probability in the latent sum, by the scale in fp32.
 * Only rows of tokens j < seq_lens[b] are read; padding rows and the unused
 * tail of a sequence's last page may hold anything (NaN included).
 * page_size must be a power of two. The decode may load block-table entries
 * anywhere in row b (up to max_pages_per_seq), but it follows only those of
 * pages that hold tokens j < seq_lens[b]; the others may hold any value.
 */
typedef struct {
  int32_t dtype;
  const void* latent;
  const void* rope;                /* fp8 only, else NULL                 */
  const float* scale;              /* fp8 only, else NULL                 */
  int64_t row_stride;              /* elements (bytes for fp8 codes)      */
  int64_t rope_stride;             /* fp8 only: elements                  */
  int32_t page_size;               /* 0 = contiguous                      */
  int64_t seq_stride;              /* contiguous only: rows per sequence  */
  const int32_t* block_table;      /* paged only: [batch, max_pages_per_seq] */
  int32_t max_pages_per_seq;       /* paged only                          */
} mla_kv_cache;

/*
 * Absorb W_UK into the query (DeepSeek-V2 paper, section 2.1.2, final
 * sentences on absorption; concatenation with the rotary query from 2.1.3).
 *   q_nope [B, H, d_nope], q_rope [B, H, d_rope] (RoPE already applied),
 *   w_uk   [H, d_nope, d_latent] (the (d_nope * H) x d_latent matrix W_UK with
 *          its rows grouped by head),
 *   q_lat  [B, H, d_latent + d_rope] (output):
 *          q_lat[b,h,:d_latent] = sum_n q_nope[b,h,n] * w_uk[h,n,:],
 *          q_lat[b,h,d_latent:] = q_rope[b,h,:].
 * dtype: MLA_BF16 (bf16 in and out, fp32 accumulation) or MLA_F32.
 * batch == 0 is a no-op.
 */
mla_status mla_absorb_q(const mla_dims* dims, int32_t batch,
                        const void* q_nope, const void* q_rope, const void* w_uk,
                        void* q_lat, int32_t dtype, mla_stream stream);

/*
 * Attention of one query token per sequence over the latent cache, absorbed
 * form (DeepSeek-V2 paper, sections 2.1.2-2.1.3); softmax in fp32.
 *   q_lat    [B, H, d_latent + d_rope], bf16 for a bf16/fp8 cache, f32 for f32.
 *   seq_lens [B] int32 device array; a length outside [0, max_seq_len] is
 *            clamped to that range.
 *   sm_scale multiplies q_lat·row before the softmax (1/sqrt(d_nope + d_rope)
 *            times any length-extension factor). Any finite value is taken,
 *            zero and negative ones included (MLA_ERR_SHAPE otherwise).
 *   num_splits S >= 1 cuts the token range [0, max_seq_len) into S chunks
 *            of mla_split_chunk(max_seq_len, S) tokens; each (b, split) is
 *            computed independently (by one workgroup; when there are more
 *            of them than compute units, full chunks are handed out first,
 *            then the partly filled ones, largest first, which changes no
 *            result).
 *   S == 1: out [B, H, d_latent] in out_dtype (MLA_BF16 or MLA_F32),
 *           lse [B, H] f32 (natural log).
 *   S  > 1: out [B, S, H, d_latent] partials in out_dtype (MLA_BF16 or
 *           MLA_F32), each normalised over its own chunk; lse [B, S, H] f32.
 *           Merge them with mla_combine (same dtype as its part_dtype).
 * A sequence (or chunk) with no tokens yields out = 0 and lse = -inf.
 * Limits: row_stride (and rope_stride) at most 2^24 bytes; a chunk,
 * mla_split_chunk(max_seq_len, num_splits), of at most 2^17 tokens
 * (MLA_ERR_UNSUPPORTED above: raise num_splits). The softmax exponentials of
 * a chunk are taken against a fixed reference (the largest score of its
 * first 32 tokens) and the chunk is computed again against its true maximum
 * if a later score exceeds that reference by more than 64 (base 2). So every
 * exponential is at most 2^64 and, over at most 2^17 tokens, every sum stays
 * finite in fp32 for cache values of magnitude below 2^40.
 */
mla_status mla_decode(const mla_dims* dims, int32_t batch, const void* q_lat,
                      const mla_kv_cache* cache, const int32_t* seq_lens,
                      int32_t max_seq_len, float sm_scale, int32_t num_splits,
                      void* out, float* lse, int32_t out_dtype, mla_stream stream);

/*
 * Attention of n = tokens_per_seq new tokens per sequence in one pass (the
 * DeepSeek-V3 blog, section 3 on multi-token prediction: several future tokens
 * of one sequence are proposed together and scored together). Causal: the n
 * tokens' own cache rows are appended before the call and counted in
 * seq_lens[b]; token t of sequence b sits at position seq_lens[b] - n + t and
 * attends to the rows of tokens 0 .. seq_lens[b] - n + t (clamped to
 * [0, max_seq_len]; a token that sees no row yields out = 0, lse = -inf).
 *   batch    sequences B; the query rows are B n, row b n + t for token t.
 *   q_lat    [B n, H, d_latent + d_rope];
 *   seq_lens [B] (per sequence, as in mla_decode);
 *   out, lse as in mla_decode with B n rows: [B n, H, d_latent] and [B n, H]
 *            for S == 1, [B n, S, H, d_latent] and [B n, S, H] partials for
 *            S > 1 (mla_combine with batch B n merges them).
 * Every other argument, limit and error is that of mla_decode, which this
 * equals for tokens_per_seq == 1. tokens_per_seq < 1 is MLA_ERR_SHAPE.
 */
mla_status mla_decode_multi(const mla_dims* dims, int32_t batch, int32_t tokens_per_seq,
                            const void* q_lat, const mla_kv_cache* cache, const int32_t* seq_lens,
                            int32_t max_seq_len, float sm_scale, int32_t num_splits, void* out,
                            float* lse, int32_t out_dtype, mla_stream stream);

/*
 * Prefill: the attention of n = tokens_per_seq new tokens per sequence in the
 * non-absorbed form (DeepSeek-V2 paper, section 2.1.2: keys and values are
 * the up-projections k^C = W_UK c_KV and v^C = W_UV c_KV; section 2.1.3: a
 * head's key is [k^C ; k^R]), for scoring a prompt or a long chunk of new
 * tokens, where up-projecting each cached row once is cheaper than absorbing
 * W_UK into every query. Same causal rule as mla_decode_multi: the new
 * tokens' rows are already in the cache and counted in seq_lens[b]; token t
 * of sequence b sits at position seq_lens[b] - n + t and attends to rows
 * 0 .. seq_lens[b] - n + t (a whole prompt: seq_lens[b] == n).
 *   q_nope [B n, H, d_nope], q_rope [B n, H, d_rope] bf16 (RoPE applied;
 *          row b n + t is token t of sequence b; mla_query_proj's output);
 *   cache  a bf16 cache (contiguous or paged, any power-of-two page size);
 *   seq_lens [B], clamped to [0, max_seq_len];
 *   w_uk, w_uv [H, d_nope, d_latent] and [H, d_v, d_latent] bf16;
 *   out    [B n, H, d_v] bf16: the per-head attention output o = sum_j p_j v^C_j
 *          (W_UV already applied); lse [B n, H] f32 (natural log).
 *   workspace: mla_prefill_workspace(dims, B, max_seq_len) bytes, 16-byte
 *          aligned: the bf16 keys k^C and values v^C of every cached row
 *          [2, B, H, ceil(max_seq_len / 128) * 128, d_nope]; its contents on
 *          return are unspecified.
 * Every cached row of a sequence (its first seq_lens[b] tokens) is
 * up-projected by each call. A token that sees no row yields out = 0 and
 * lse = -inf. Softmax in fp32 with a running maximum; products on bf16 with
 * fp32 accumulation. Supported: the DeepSeek-V2 head shape with a bf16 cache
 * (else MLA_ERR_UNSUPPORTED / MLA_ERR_DTYPE). Errors as in mla_decode, plus
 * tokens_per_seq < 1 or a workspace below the required size (MLA_ERR_SHAPE).
 * The event pair of mla_time_next_launch brackets both kernels it launches.
 */
int64_t mla_prefill_workspace(const mla_dims* dims, int32_t batch, int32_t max_seq_len);
mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t tokens_per_seq,
                       const void* q_nope, const void* q_rope, const mla_kv_cache* cache,
                       const int32_t* seq_lens, int32_t max_seq_len, const void* w_uk,
                       const void* w_uv, float sm_scale, void* out, float* lse, void* workspace,
                       int64_t workspace_bytes, mla_stream stream);

/*
 * Log-sum-exp merge of split partials (the split-KV pass of mla_decode):
 *   lse[b,h] = log sum_s exp(lse_part[b,s,h]),
 *   out[b,h] = sum_s exp(lse_part[b,s,h] - lse[b,h]) * o_part[b,s,h,:].
 * Parts with lse = -inf contribute nothing; if all do, out = 0, lse = -inf.
 *   o_part [B, S, H, d_latent] in part_dtype (MLA_BF16 or MLA_F32),
 *   lse_part [B, S, H] f32, out [B, H, d_latent] in out_dtype (MLA_BF16 or
 *   MLA_F32), lse [B, H] f32 (lse may be NULL when not wanted).
 * The weighted sum runs in fp32.
 */
mla_status mla_combine(const mla_dims* dims, int32_t batch, int32_t num_splits,
                       const void* o_part, int32_t part_dtype, const float* lse_part,
                       void* out, float* lse, int32_t out_dtype, mla_stream stream);

/*
 * Apply W_UV on the output side (DeepSeek-V2 paper, section 2.1.2: W_UV
 * absorbed into the output projection).
 *   o_lat [B, H, d_latent] in o_dtype (MLA_BF16 or MLA_F32),
 *   w_uv  [H, d_v, d_latent] in w_dtype (the (d_v * H) x d_latent matrix W_UV
 *         with its rows grouped by head),
 *   out   [B, H, d_v] in out_dtype:  out[b,h,v] = sum_c w_uv[h,v,c] * o_lat[b,h,c].
 * bf16 weights: the product runs on bf16 inputs (an f32 o_lat is rounded to
 * bf16 first) with fp32 accumulation. f32 weights need f32 o_lat.
 */
mla_status mla_out_proj(const mla_dims* dims, int32_t batch, const void* o_lat,
                        int32_t o_dtype, const void* w_uv, int32_t w_dtype,
                        void* out, int32_t out_dtype, mla_stream stream);

/*
 * mla_combine followed by mla_out_proj in one pass, without the merged
 * latent output going to memory: for every (b, h) the split partials are
 * merged in fp32 with the weights exp(lse_part - lse), rounded to bf16 (the
 * values a bf16 mla_combine output would hold) and multiplied by W_UV with
 * fp32 accumulation.
 *   o_part [B, S, H, d_latent] in part_dtype, lse_part [B, S, H] f32 (as
 *          written by mla_decode with S > 1),
 *   w_uv   [H, d_v, d_latent] in w_dtype,
 *   out    [B, H, d_v] in out_dtype (MLA_BF16 or MLA_F32),
 *   lse    [B, H] f32, the merged log-sum-exp (may be NULL).
 * Parts with lse = -inf contribute nothing; if all do, out = 0, lse = -inf.
 * Only the DeepSeek-V2 head shape with bf16 partials and bf16 weights
 * (MLA_ERR_UNSUPPORTED for other shapes, MLA_ERR_DTYPE for other dtypes);
 * num_splits at most 64 (MLA_ERR_UNSUPPORTED above; mla_combine takes more).
 */
mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t num_splits,
                                const void* o_part, int32_t part_dtype, const float* lse_part,
                                const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype,
                                float* lse, mla_stream stream);

/*
 * Attention output projection (DeepSeek-V2 paper, section 2.1.1: the output
 * is W_O times the concatenated heads; section 2.1.2: W_UV may be absorbed
 * into W_O, which this library does not do, as the folded weight would be
 * d_latent / d_v times larger):
 *   u[b, :] = W_O [o[b, 0, :]; ...; o[b, H-1, :]]
 *   o     [B, H, d_v] (the heads' outputs, e.g. from mla_out_proj),
 *   w_o   [hidden, H * d_v], row-major (head-major columns),
 *   out   [B, hidden] in out_dtype.
 * dtype: MLA_BF16 for the DeepSeek-V2 shape (out MLA_BF16 or MLA_F32; hidden a
 * multiple of 32), MLA_F32 for the tiny shape (out MLA_F32). fp32
 * accumulation: within a 2048-wide part of the contraction, four 512-wide
 * ranges added in order; the parts' partial sums added in part order.
 * workspace: device memory of at least mla_o_proj_workspace() bytes, 16-byte
 * aligned, owned by the caller (the DeepSeek-V2 shape; NULL allowed for the
 * tiny one): the parts' fp32 partial sums. batch == 0 is a no-op.
 */
int64_t mla_o_proj_workspace(const mla_dims* dims, int32_t batch, int32_t hidden);
mla_status mla_o_proj(const mla_dims* dims, int32_t batch, int32_t hidden, const void* o, const void* w_o,
                      int32_t dtype, void* out, int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                      mla_stream stream);

/*
 * The cache entry of one new token per sequence (DeepSeek-V2 paper, section
 * 2.1.2: the latent is the down-projection W_DKV h of the token's hidden
 * state; section 2.1.3: the shared rotary key is RoPE(W_KR h) at the token's
 * position; section 3.1.2, model hyper-parameters: an RMS norm follows the
 * compressed latent):
 *   c_KV[b] = RMSNorm(W_DKV h[b]) = x / sqrt(mean(x^2) + rms_eps) * gain,
 *   k_R[b]  = RoPE(W_KR h[b], positions[b]): features (2i, 2i + 1) turned by
 *             positions[b] * f_i, f_i the frequencies `rope` describes (plain
 *             or YaRN; a length-extended model rotates its keys as its queries),
 * written into row positions[b] of sequence b of `cache` (the same layouts
 * mla_decode reads; this call writes through its pointers).
 *   h           [B, hidden], w_dkv [d_latent, hidden], w_kr [d_rope, hidden],
 *   norm_gain   [d_latent] or NULL (gain 1), all in `dtype`:
 *               MLA_BF16 for the DeepSeek-V2 shape (cache MLA_BF16, or
 *               MLA_FP8_E4M3: codes of c_KV / s with s = absmax(c_KV) / 448,
 *               1 for an all-zero row, rounded to nearest even, the rotary key
 *               in bf16), MLA_F32 for the tiny shape (cache MLA_F32).
 *   positions   [B] int32 device array; a position outside the cache (below
 *               0, at or beyond seq_stride, or beyond the block table's pages)
 *               writes nothing for that sequence.
 *   workspace   device memory of at least mla_cache_append_workspace() bytes,
 *               16-byte aligned, owned by the caller (fp32 partial sums).
 * Products accumulate in fp32 (bf16: 1024-wide parts of the hidden size, each
 * the in-order sum of four 256-wide ranges, the parts added in order; f32:
 * 256-wide slices added in order), the norm and rotation run in fp32 (angles
 * in fp64). hidden a multiple of 16 (bf16) or 4 (f32). batch == 0 is a no-op.
 * Errors as for mla_decode; MLA_ERR_SHAPE also for a short workspace.
 */
int64_t mla_cache_append_workspace(const mla_dims* dims, int32_t batch, int32_t hidden);
mla_status mla_cache_append(const mla_dims* dims, int32_t batch, int32_t hidden, const void* h,
                            const void* w_dkv, const void* w_kr, const void* norm_gain, int32_t dtype,
                            float rms_eps, const mla_rope* rope, const int32_t* positions,
                            const mla_kv_cache* cache, void* workspace, int64_t workspace_bytes,
                            mla_stream stream);

/*
 * mla_cache_append without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation): the fp32 partial sums go to a scratch array inside the
 * library instead, one copy on each GPU it runs on, 8 MiB, held until the
 * process ends. The call allocates nothing. Limit:
 * mla_cache_append_workspace(dims, batch, hidden) <= 8 MiB (batch up to 728
 * at hidden 5120 with the DeepSeek-V2 shape); beyond it the call returns
 * MLA_ERR_UNSUPPORTED and enqueues nothing. Every call on one GPU uses that
 * GPU's array, so calls that can run at the same time on one GPU (on
 * different streams or threads) race; the caller orders them. The first call
 * on each device resolves the array's address with that device current.
 * Arguments, results and other errors as for mla_cache_append.
 */
mla_status mla_cache_append_noalloc(const mla_dims* dims, int32_t batch, int32_t hidden, const void* h,
                                    const void* w_dkv, const void* w_kr, const void* norm_gain,
                                    int32_t dtype, float rms_eps, const mla_rope* rope,
                                    const int32_t* positions, const mla_kv_cache* cache,
                                    mla_stream stream);

/*
 * The query of one new token per sequence (DeepSeek-V2 paper, section 2.1.2:
 * the query is compressed too, c_Q = W_DQ h, and its content part is the
 * up-projection q^C = W_UQ c_Q; section 2.1.3: the rotary part of every head
 * is q^R = RoPE(W_QR c_Q) at the token's position; section 3.1.2: an RMS norm
 * follows the compressed latent, d'_c = 1536 in DeepSeek-V2):
 *   c_Q[b]      = RMSNorm(W_DQ h[b]) = x / sqrt(mean(x^2) + rms_eps) * gain,
 *   q_nope[b,h] = W_UQ[h] c_Q[b],
 *   q_rope[b,h] = RoPE(W_QR[h] c_Q[b], positions[b]) with the frequencies of `rope`,
 * the inputs mla_absorb_q takes.
 *   h      [B, hidden],  w_dq [d_qlatent, hidden],  q_norm_gain [d_qlatent] or NULL,
 *   w_uq   [H * d_nope, d_qlatent] (rows grouped by head),
 *   w_qr   [H * d_rope, d_qlatent] (rows grouped by head),
 *   positions [B] int32 device array (any value; the angle is position * f_i),
 *   q_nope [B, H, d_nope] and q_rope [B, H, d_rope] (outputs), all in `dtype`.
 * MLA_BF16 with the DeepSeek-V2 head shape only (MLA_ERR_UNSUPPORTED for the
 * tiny one); hidden a multiple of 16 and at most 20480, d_qlatent a multiple
 * of 256 and at most 4096 (MLA_ERR_UNSUPPORTED beyond). Products accumulate
 * in fp32: W_DQ h over 1024-wide parts of the contraction (four 256-wide
 * ranges added in order within a part, the parts' sums added in part order),
 * the up-projection over four equal ranges of d_qlatent added in order; the
 * norm runs in fp32 and c_Q is rounded to bf16 before the up-projection;
 * rotation angles in fp64.
 * workspace: device memory of at least mla_query_proj_workspace() bytes,
 * 16-byte aligned, owned by the caller. Three kernels are launched (the
 * timing hook's pair brackets all three). batch == 0 is a no-op.
 */
int64_t mla_query_proj_workspace(const mla_dims* dims, int32_t batch, int32_t hidden, int32_t d_qlatent);
mla_status mla_query_proj(const mla_dims* dims, int32_t batch, int32_t hidden, int32_t d_qlatent,
                          const void* h, const void* w_dq, const void* q_norm_gain, const void* w_uq,
                          const void* w_qr, int32_t dtype, float rms_eps, const mla_rope* rope,
                          const int32_t* positions, void* q_nope, void* q_rope, void* workspace,
                          int64_t workspace_bytes, mla_stream stream);

/* Tokens per split chunk that mla_decode uses for (max_seq_len, num_splits):
 * ceil(max_seq_len / num_splits) rounded up to a multiple of 32. */
int32_t mla_split_chunk(int32_t max_seq_len, int32_t num_splits);

/* A split count for mla_decode, from a cost model of this GPU. The non-empty
 * (sequence, split) items run one workgroup per compute unit, in rounds of
 * `num_cus`; each item costs its chunk of tokens plus a fixed start-up and
 * write-out of about six tiles, and every (sequence, split) pair adds a
 * partial for the merge to read. The count returned has the smallest total;
 * the number of items is exact when every sequence has max_seq_len tokens and
 * estimated from total_tokens (about total / chunk + half an item per
 * sequence, with a small margin) otherwise. Chunks are at least 256 tokens.
 * total_tokens <= 0 means batch * max_seq_len. Returns at least 1 and at most
 * the largest count mla_combine accepts. */
int32_t mla_suggest_splits(int32_t batch, int32_t max_seq_len, int64_t total_tokens,
                           int32_t num_cus);

/*
 * Measurement hook. The next kernel that an entry point of this library
 * launches from the calling thread records `start_event` when it begins
 * executing and `stop_event` when it ends (hipExtLaunchKernel's event pair),
 * so hipEventElapsedTime on the two gives that kernel's own duration, without
 * the gaps that events recorded separately on the stream add. Each entry
 * point launches one kernel, except mla_cache_append, mla_prefill and
 * mla_o_proj (bf16), which launch two, and mla_query_proj, which launches three:
 * the start event goes with the first and the stop event with the last, so
 * the pair brackets all. The events are hipEvent_t handles created by
 * the caller with timing enabled; either may be NULL. The pair is consumed
 * by that one launch; a call that fails validation launches nothing and
 * leaves it pending. Always returns MLA_OK.
 */
mla_status mla_time_next_launch(void* start_event, void* stop_event);

/*
 * Measurement helper, not part of the decode path: one streaming read of
 * `bytes` of device memory at `buf` with plain 16-byte vector loads, so that
 * a caller can time it (mla_time_next_launch) and report the decode's cache
 * bandwidth against what a read achieves on this device as well as against
 * the published peak. bytes: a multiple of 16 (0 is a no-op); buf: 16-byte
 * aligned; sink: 4 device bytes the kernel writes only if the XOR of all
 * data equals one fixed constant (so the reads cannot be optimised away).
 * Errors: NULL buf or sink MLA_ERR_NULL, bytes < 0 or not a multiple of 16
 * MLA_ERR_SHAPE, misaligned buf MLA_ERR_ALIGN.
 */
mla_status mla_read_probe(const void* buf, int64_t bytes, void* sink, mla_stream stream);

/* Static, never-NULL description of a status code. */
const char* mla_status_string(mla_status status);

/* hipError_t of the last call on this thread that returned MLA_ERR_HIP. */
int32_t mla_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
