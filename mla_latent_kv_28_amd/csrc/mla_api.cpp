// libmla C ABI: argument validation, dispatch to the compiled head shapes,
// status reporting. Nothing here allocates or synchronises.
#include "../../include/mla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
int combine_max_splits();
}

namespace {

thread_local int32_t g_last_hip_error = 0;
thread_local hipEvent_t g_next_start = nullptr, g_next_stop = nullptr;   // mla_time_next_launch

enum class Shape { kNone, kDsv2, kTiny };

Shape shape_of(const mla_dims* d) {
  if (d->num_heads == 128 && d->d_latent == 512 && d->d_rope == 64 && d->d_nope == 128 && d->d_v == 128)
    return Shape::kDsv2;
  if (d->num_heads == 4 && d->d_latent == 32 && d->d_rope == 16 && d->d_nope == 32 && d->d_v == 32)
    return Shape::kTiny;
  return Shape::kNone;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) { int k = 0; while ((int64_t(1) << k) < x) ++k; return k; }

mla_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return MLA_ERR_HIP;
}

bool valid_dtype(int32_t t) { return t == MLA_F32 || t == MLA_BF16 || t == MLA_FP8_E4M3; }

// Frequencies of the d_rope / 2 rotary pairs described by `r` (plain RoPE, or
// YaRN's by-parts interpolation), in double precision; MLA_ERR_SHAPE for
// parameters outside the documented ranges.
mla_status rope_frequencies(const mla_rope* r, int d_rope, double* out) {
  if (r == nullptr) return MLA_ERR_NULL;
  if (d_rope / 2 > mla::kMaxRopePairs) return MLA_ERR_UNSUPPORTED;
  const double base = r->base, s = r->yarn_scale;
  if (!std::isfinite(base) || base <= 0.0 || !std::isfinite(s) || s < 1.0) return MLA_ERR_SHAPE;
  const bool yarn = s > 1.0;
  if (yarn && (!std::isfinite(r->yarn_alpha) || !std::isfinite(r->yarn_beta) || !(r->yarn_alpha < r->yarn_beta) ||
               r->yarn_orig_ctx <= 0))
    return MLA_ERR_SHAPE;
  constexpr double kTwoPi = 6.283185307179586;
  for (int i = 0; i < d_rope / 2; ++i) {
    double f = std::pow(base, -2.0 * i / d_rope);
    if (yarn) {
      const double turns = r->yarn_orig_ctx * f / kTwoPi;
      const double g = std::min(1.0, std::max(0.0, (turns - r->yarn_alpha) / (r->yarn_beta - r->yarn_alpha)));
      f = (1.0 - g) * f / s + g * f;
    }
    out[i] = f;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_split_chunk(int32_t max_seq_len, int32_t num_splits) {
  if (num_splits < 1 || max_seq_len <= 0) return 0;
  const int64_t c = (static_cast<int64_t>(max_seq_len) + num_splits - 1) / num_splits;
  return static_cast<int32_t>((c + 31) / 32 * 32);
}

int32_t mla_suggest_splits(int32_t batch, int32_t max_seq_len, int64_t total_tokens, int32_t num_cus) {
  if (batch <= 0 || max_seq_len <= 0 || num_cus <= 0) return 1;
  const int64_t all_full = static_cast<int64_t>(batch) * max_seq_len;
  if (total_tokens <= 0 || total_tokens > all_full) total_tokens = all_full;
  // The (sequence, split) items run one workgroup per compute unit, in rounds
  // of num_cus; an item costs its chunk of tokens plus a fixed start-up and
  // write-out of about six tiles (192 tokens of streaming). Every (sequence,
  // split) pair also writes a partial that the merge reads back, about half a
  // token's streaming time each on this GPU. Pick the split count with the
  // smallest total. Items per split count: exact when every sequence is full
  // length, else total / chunk plus half an item per sequence (the partly
  // filled last chunk), with 3% + 2 of margin so that an estimate just under
  // a round boundary does not pick a count whose items spill into one more
  // round. Chunks are at least 256 tokens.
  constexpr double kItemOverhead = 192.0, kPartialCost = 0.43;
  int32_t best_s = 1;
  double best = 0.0;
  for (int32_t s = 1; s <= mla::combine_max_splits(); ++s) {
    const int64_t chunk = mla_split_chunk(max_seq_len, s);
    if (s > 1 && chunk < 256) break;
    const int64_t per_seq = (max_seq_len + chunk - 1) / chunk;
    const double most = static_cast<double>(batch) * per_seq;
    const double items = total_tokens == all_full
                             ? most
                             : std::min(most, 1.03 * (static_cast<double>(total_tokens) / chunk + 0.5 * batch) + 2.0);
    const double rounds = std::ceil(items / num_cus);
    const double cost = rounds * (static_cast<double>(chunk) + kItemOverhead) +
                        kPartialCost * batch * (s > 1 ? s : 0);
    if (s == 1 || cost < best) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size is negative, zero where it must not be, or inconsistent";
    case MLA_ERR_DTYPE: return "unknown dtype or unsupported dtype combination";
    case MLA_ERR_UNSUPPORTED: return "head shape outside the compiled set, or a size beyond a documented limit";
    case MLA_ERR_ALIGN: return "a pointer or stride is not 16-byte aligned";
    case MLA_ERR_HIP: return "a HIP call failed (see mla_last_hip_error)";
    default: return "unknown status";
  }
}

int32_t mla_last_hip_error(void) { return g_last_hip_error; }

mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, const void* q_nope, const void* q_rope,
                        const void* w_uk, void* q_lat, int32_t dtype, mla_stream stream) {
  if (dims == nullptr) return MLA_ERR_NULL;
  if (batch < 0) return MLA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if ((sh == Shape::kDsv2 && dtype != MLA_BF16) || (sh == Shape::kTiny && dtype != MLA_F32))
    return MLA_ERR_DTYPE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_rope || !w_uk || !q_lat) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(q_lat))
    return MLA_ERR_ALIGN;
  mla::GemmParams p{};
  p.a = q_nope;
  p.w = w_uk;
  p.c = q_lat;
  p.lda = dims->d_nope;
  p.ldc = dims->d_latent + dims->d_rope;
  p.batch = batch;
  p.heads = dims->num_heads;
  p.a_f32 = dtype == MLA_F32;
  p.c_f32 = dtype == MLA_F32;
  p.tail = q_rope;
  p.n_tail = dims->d_rope;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(sh == Shape::kDsv2 ? mla::launch_absorb_dsv2_bf16(p, s)
                                       : mla::launch_absorb_tiny_f32(p, s));
}

namespace {

// mla_decode over `batch` sequences with n query tokens each (query rows
// b n + t); n = 1 is the one-token decode.
mla_status decode_tokens(const mla_dims* dims, int32_t batch, int32_t n, const void* q_lat,
                         const mla_kv_cache* cache, const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                         int32_t num_splits, void* out, float* lse, int32_t out_dtype, mla_stream stream) {
  if (dims == nullptr || cache == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || n < 1 || max_seq_len < 0 || num_splits < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * n > 0x7fffffff) return MLA_ERR_SHAPE;
  if (!valid_dtype(cache->dtype) || (out_dtype != MLA_F32 && out_dtype != MLA_BF16)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (sh == Shape::kDsv2 && cache->dtype == MLA_F32) return MLA_ERR_DTYPE;
  if (sh == Shape::kTiny && cache->dtype != MLA_F32) return MLA_ERR_DTYPE;
  if (!std::isfinite(sm_scale)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_lat || !seq_lens || !out || !lse || !cache->latent) return MLA_ERR_NULL;
  const bool fp8 = cache->dtype == MLA_FP8_E4M3;
  if (fp8 && (!cache->rope || !cache->scale)) return MLA_ERR_NULL;
  const bool paged = cache->page_size > 0;
  if (cache->page_size < 0) return MLA_ERR_SHAPE;
  if (paged) {
    if (!cache->block_table) return MLA_ERR_NULL;
    if (!is_pow2(cache->page_size)) return MLA_ERR_SHAPE;
    const int64_t need = (static_cast<int64_t>(max_seq_len) + cache->page_size - 1) / cache->page_size;
    if (cache->max_pages_per_seq < need) return MLA_ERR_SHAPE;
  } else if (cache->seq_stride < max_seq_len) {
    return MLA_ERR_SHAPE;
  }
  const int64_t width = fp8 ? dims->d_latent : dims->d_latent + dims->d_rope;
  if (cache->row_stride < width) return MLA_ERR_SHAPE;
  const int64_t elem = cache->dtype == MLA_F32 ? 4 : (fp8 ? 1 : 2);
  if ((cache->row_stride * elem) % 16 != 0) return MLA_ERR_ALIGN;
  if (cache->row_stride * elem > (int64_t{1} << 24)) return MLA_ERR_UNSUPPORTED;
  if (fp8) {
    if (cache->rope_stride < dims->d_rope) return MLA_ERR_SHAPE;
    if ((cache->rope_stride * 2) % 16 != 0) return MLA_ERR_ALIGN;
    if (cache->rope_stride * 2 > (int64_t{1} << 24)) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(cache->rope)) return MLA_ERR_ALIGN;
  }
  if (!aligned16(q_lat) || !aligned16(cache->latent) || !aligned16(out) || !aligned16(lse))
    return MLA_ERR_ALIGN;
  if (static_cast<int64_t>(batch) * n * num_splits > 0x7fffffff) return MLA_ERR_SHAPE;
  // the fixed-reference softmax keeps its sums finite for at most 2^17 tokens a chunk
  if (mla_split_chunk(max_seq_len, num_splits) > (1 << 17)) return MLA_ERR_UNSUPPORTED;

  mla::DecodeParams p{};
  p.q_lat = q_lat;
  p.latent = cache->latent;
  p.rope = cache->rope;
  p.scale = cache->scale;
  p.row_stride = cache->row_stride;
  p.rope_stride = cache->rope_stride;
  p.seq_stride = cache->seq_stride;
  p.block_table = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.page_shift = paged ? log2i(cache->page_size) : -1;
  p.seq_lens = seq_lens;
  p.batch = batch * n;
  p.tokens_per_seq = n;
  p.max_seq_len = max_seq_len;
  p.num_splits = num_splits;
  p.chunk = mla_split_chunk(max_seq_len, num_splits);
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.out = out;
  p.lse = lse;
  p.out_bf16 = out_dtype == MLA_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (sh == Shape::kTiny) e = mla::launch_decode_tiny_f32(p, s);
  else if (fp8) e = mla::launch_decode_dsv2_fp8(p, s);
  else e = mla::launch_decode_dsv2_bf16(p, s);
  return hip_status(e);
}

}  // namespace

mla_status mla_decode(const mla_dims* dims, int32_t batch, const void* q_lat, const mla_kv_cache* cache,
                      const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, int32_t num_splits,
                      void* out, float* lse, int32_t out_dtype, mla_stream stream) {
  return decode_tokens(dims, batch, 1, q_lat, cache, seq_lens, max_seq_len, sm_scale, num_splits, out, lse,
                       out_dtype, stream);
}

mla_status mla_decode_multi(const mla_dims* dims, int32_t batch, int32_t tokens_per_seq, const void* q_lat,
                            const mla_kv_cache* cache, const int32_t* seq_lens, int32_t max_seq_len,
                            float sm_scale, int32_t num_splits, void* out, float* lse, int32_t out_dtype,
                            mla_stream stream) {
  return decode_tokens(dims, batch, tokens_per_seq, q_lat, cache, seq_lens, max_seq_len, sm_scale, num_splits,
                       out, lse, out_dtype, stream);
}

mla_status mla_combine(const mla_dims* dims, int32_t batch, int32_t num_splits, const void* o_part,
                       int32_t part_dtype, const float* lse_part, void* out, float* lse, int32_t out_dtype,
                       mla_stream stream) {
  if (dims == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || num_splits < 1) return MLA_ERR_SHAPE;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (part_dtype != MLA_F32 && part_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (shape_of(dims) == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (num_splits > mla::combine_max_splits()) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !out) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(out)) return MLA_ERR_ALIGN;
  mla::CombineParams p{};
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.splits = num_splits;
  p.heads = dims->num_heads;
  p.d_latent = dims->d_latent;
  p.out_bf16 = out_dtype == MLA_BF16;
  p.part_bf16 = part_dtype == MLA_BF16;
  return hip_status(mla::launch_combine(p, static_cast<hipStream_t>(stream)));
}

mla_status mla_out_proj(const mla_dims* dims, int32_t batch, const void* o_lat, int32_t o_dtype,
                        const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype, mla_stream stream) {
  if (dims == nullptr) return MLA_ERR_NULL;
  if (batch < 0) return MLA_ERR_SHAPE;
  if (!valid_dtype(o_dtype) || !valid_dtype(w_dtype) || !valid_dtype(out_dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (o_dtype == MLA_FP8_E4M3 || out_dtype == MLA_FP8_E4M3) return MLA_ERR_DTYPE;
  if (sh == Shape::kDsv2 && w_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (sh == Shape::kTiny && (w_dtype != MLA_F32 || o_dtype != MLA_F32 || out_dtype != MLA_F32))
    return MLA_ERR_DTYPE;
  if (batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  mla::GemmParams p{};
  p.a = o_lat;
  p.w = w_uv;
  p.c = out;
  p.lda = dims->d_latent;
  p.ldc = dims->d_v;
  p.batch = batch;
  p.heads = dims->num_heads;
  p.a_f32 = o_dtype == MLA_F32;
  p.c_f32 = out_dtype == MLA_F32;
  p.tail = nullptr;
  p.n_tail = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(sh == Shape::kDsv2 ? mla::launch_outproj_dsv2_bf16(p, s)
                                       : mla::launch_outproj_tiny_f32(p, s));
}

mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t num_splits, const void* o_part,
                                int32_t part_dtype, const float* lse_part, const void* w_uv, int32_t w_dtype,
                                void* out, int32_t out_dtype, float* lse, mla_stream stream) {
  if (dims == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || num_splits < 1) return MLA_ERR_SHAPE;
  if (!valid_dtype(part_dtype) || !valid_dtype(w_dtype) || !valid_dtype(out_dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (sh != Shape::kDsv2) return MLA_ERR_UNSUPPORTED;                  // the 16-bit DeepSeek-V2 shape only
  if (part_dtype != MLA_BF16 || w_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (out_dtype != MLA_BF16 && out_dtype != MLA_F32) return MLA_ERR_DTYPE;
  if (num_splits > mla::combine_outproj_max_splits()) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  mla::CombineOutParams p{};
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.w = w_uv;
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.splits = num_splits;
  p.heads = dims->num_heads;
  p.out_f32 = out_dtype == MLA_F32;
  return hip_status(mla::launch_combine_outproj_dsv2_bf16(p, static_cast<hipStream_t>(stream)));
}

int64_t mla_o_proj_workspace(const mla_dims* dims, int32_t batch, int32_t hidden) {
  if (dims == nullptr || batch <= 0 || hidden <= 0 || shape_of(dims) != Shape::kDsv2) return 0;
  return mla::oproj_workspace_bytes(batch, hidden, dims->num_heads * dims->d_v);
}

mla_status mla_o_proj(const mla_dims* dims, int32_t batch, int32_t hidden, const void* o, const void* w_o,
                      int32_t dtype, void* out, int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                      mla_stream stream) {
  if (dims == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || hidden <= 0) return MLA_ERR_SHAPE;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (sh == Shape::kDsv2 && (dtype != MLA_BF16 || out_dtype == MLA_FP8_E4M3)) return MLA_ERR_DTYPE;
  if (sh == Shape::kTiny && (dtype != MLA_F32 || out_dtype != MLA_F32)) return MLA_ERR_DTYPE;
  const int32_t k = dims->num_heads * dims->d_v;
  if (sh == Shape::kDsv2 && !mla::oproj_bf16_shape_ok(hidden, k)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!o || !w_o || !out) return MLA_ERR_NULL;
  if (sh == Shape::kDsv2) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < mla_o_proj_workspace(dims, batch, hidden)) return MLA_ERR_SHAPE;
  }
  if (!aligned16(o) || !aligned16(w_o) || !aligned16(out) || !aligned16(workspace)) return MLA_ERR_ALIGN;
  mla::OProjParams p{o, w_o, out, static_cast<float*>(workspace), batch, hidden, k};
  return hip_status(mla::launch_oproj(p, sh == Shape::kDsv2, out_dtype == MLA_F32, static_cast<hipStream_t>(stream)));
}

int64_t mla_cache_append_workspace(const mla_dims* dims, int32_t batch, int32_t hidden) {
  if (dims == nullptr || batch <= 0 || hidden <= 0) return 0;
  return static_cast<int64_t>(mla::append_slices(hidden, shape_of(dims) == Shape::kDsv2)) * batch *
         (dims->d_latent + dims->d_rope) *
         static_cast<int64_t>(sizeof(float));
}

}  // extern "C"

namespace {

// Validation shared by the two cache-append entry points: everything but the
// workspace. Fills `p` (work left null) and returns MLA_OK, or the status.
mla_status cache_append_params(const mla_dims* dims, int32_t batch, int32_t hidden, const void* h,
                               const void* w_dkv, const void* w_kr, const void* norm_gain, int32_t dtype,
                               float rms_eps, const mla_rope* rope, const int32_t* positions,
                               const mla_kv_cache* cache, mla::AppendParams& p, bool& dsv2) {
  if (dims == nullptr || cache == nullptr || rope == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || hidden <= 0) return MLA_ERR_SHAPE;
  if (!std::isfinite(rms_eps) || rms_eps < 0.0f) return MLA_ERR_SHAPE;
  if (!valid_dtype(dtype) || !valid_dtype(cache->dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh == Shape::kNone) return MLA_ERR_UNSUPPORTED;
  if (sh == Shape::kDsv2 && (dtype != MLA_BF16 || cache->dtype == MLA_F32)) return MLA_ERR_DTYPE;
  if (sh == Shape::kTiny && (dtype != MLA_F32 || cache->dtype != MLA_F32)) return MLA_ERR_DTYPE;
  if (hidden % (dtype == MLA_BF16 ? 16 : 4) != 0) return MLA_ERR_SHAPE;   // whole 16-wide k steps (bf16)
  {
    double f[mla::kMaxRopePairs];
    const mla_status rs = rope_frequencies(rope, dims->d_rope, f);
    if (rs != MLA_OK) return rs;
  }
  if (batch == 0) return MLA_OK;
  if (!h || !w_dkv || !w_kr || !positions || !cache->latent) return MLA_ERR_NULL;
  const bool fp8 = cache->dtype == MLA_FP8_E4M3;
  if (fp8 && (!cache->rope || !cache->scale)) return MLA_ERR_NULL;
  if (cache->page_size < 0) return MLA_ERR_SHAPE;
  const bool paged = cache->page_size > 0;
  if (paged) {
    if (!cache->block_table) return MLA_ERR_NULL;
    if (!is_pow2(cache->page_size) || cache->max_pages_per_seq < 1) return MLA_ERR_SHAPE;
  } else if (cache->seq_stride < 1) {
    return MLA_ERR_SHAPE;
  }
  const int64_t width = fp8 ? dims->d_latent : dims->d_latent + dims->d_rope;
  if (cache->row_stride < width) return MLA_ERR_SHAPE;
  const int64_t elem = cache->dtype == MLA_F32 ? 4 : (fp8 ? 1 : 2);
  if ((cache->row_stride * elem) % 16 != 0) return MLA_ERR_ALIGN;
  if (fp8) {
    if (cache->rope_stride < dims->d_rope) return MLA_ERR_SHAPE;
    if (!aligned16(cache->rope) || (reinterpret_cast<uintptr_t>(cache->scale) & 3u) != 0) return MLA_ERR_ALIGN;
  }
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(cache->latent)) return MLA_ERR_ALIGN;
  p = mla::AppendParams{};
  p.h = h;
  p.w_dkv = w_dkv;
  p.w_kr = w_kr;
  p.gain = norm_gain;
  p.positions = positions;
  p.latent = const_cast<void*>(cache->latent);
  p.rope = const_cast<void*>(cache->rope);
  p.scale = const_cast<float*>(cache->scale);
  p.row_stride = cache->row_stride;
  p.rope_stride = cache->rope_stride;
  p.seq_stride = cache->seq_stride;
  p.block_table = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.page_shift = paged ? log2i(cache->page_size) : -1;
  p.work = nullptr;
  p.batch = batch;
  p.hidden = hidden;
  p.ksplits = mla::append_slices(hidden, sh == Shape::kDsv2);
  p.d_latent = dims->d_latent;
  p.d_rope = dims->d_rope;
  p.eps = rms_eps;
  dsv2 = sh == Shape::kDsv2;
  return rope_frequencies(rope, dims->d_rope, p.freq);
}

int cache_kind_of(int32_t dtype) {
  return dtype == MLA_FP8_E4M3 ? mla::kFP8 : dtype == MLA_BF16 ? mla::kBF16 : mla::kF32;
}

}  // namespace

extern "C" {

mla_status mla_cache_append(const mla_dims* dims, int32_t batch, int32_t hidden, const void* h,
                            const void* w_dkv, const void* w_kr, const void* norm_gain, int32_t dtype,
                            float rms_eps, const mla_rope* rope, const int32_t* positions,
                            const mla_kv_cache* cache, void* workspace, int64_t workspace_bytes,
                            mla_stream stream) {
  mla::AppendParams p{};
  bool dsv2 = false;
  const mla_status st = cache_append_params(dims, batch, hidden, h, w_dkv, w_kr, norm_gain, dtype, rms_eps,
                                            rope, positions, cache, p, dsv2);
  if (st != MLA_OK || batch == 0) return st;
  if (!workspace) return MLA_ERR_NULL;
  if (workspace_bytes < mla_cache_append_workspace(dims, batch, hidden)) return MLA_ERR_SHAPE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  p.work = static_cast<float*>(workspace);
  return hip_status(mla::launch_cache_append(p, dsv2, cache_kind_of(cache->dtype), static_cast<hipStream_t>(stream)));
}

int64_t mla_query_proj_workspace(const mla_dims* dims, int32_t batch, int32_t hidden, int32_t d_qlatent) {
  if (dims == nullptr || batch <= 0 || hidden <= 0 || d_qlatent <= 0 || shape_of(dims) != Shape::kDsv2) return 0;
  int64_t cq_off = 0, total = 0;
  mla::query_workspace_layout(batch, hidden, d_qlatent, &cq_off, &total);
  return total;
}

mla_status mla_query_proj(const mla_dims* dims, int32_t batch, int32_t hidden, int32_t d_qlatent, const void* h,
                          const void* w_dq, const void* q_norm_gain, const void* w_uq, const void* w_qr,
                          int32_t dtype, float rms_eps, const mla_rope* rope, const int32_t* positions,
                          void* q_nope, void* q_rope, void* workspace, int64_t workspace_bytes, mla_stream stream) {
  if (dims == nullptr || rope == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || hidden <= 0 || d_qlatent <= 0) return MLA_ERR_SHAPE;
  if (!std::isfinite(rms_eps) || rms_eps < 0.0f) return MLA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  const Shape sh = shape_of(dims);
  if (sh != Shape::kDsv2) return MLA_ERR_UNSUPPORTED;     // the DeepSeek-V2 head shape, bf16
  if (dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (hidden % 16 != 0 || d_qlatent % 256 != 0) return MLA_ERR_SHAPE;
  if (d_qlatent > 4096 || mla::query_partial_sums(hidden) > 20) return MLA_ERR_UNSUPPORTED;
  mla::QueryParams p{};
  {
    const mla_status rs = rope_frequencies(rope, dims->d_rope, p.freq);
    if (rs != MLA_OK) return rs;
  }
  if (batch == 0) return MLA_OK;
  if (!h || !w_dq || !w_uq || !w_qr || !positions || !q_nope || !q_rope || !workspace) return MLA_ERR_NULL;
  if (workspace_bytes < mla_query_proj_workspace(dims, batch, hidden, d_qlatent)) return MLA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(w_qr) || !aligned16(q_nope) ||
      !aligned16(q_rope) || !aligned16(workspace))
    return MLA_ERR_ALIGN;
  int64_t cq_off = 0, total = 0;
  mla::query_workspace_layout(batch, hidden, d_qlatent, &cq_off, &total);
  char* ws = static_cast<char*>(workspace);
  p.h = h;
  p.w_dq = w_dq;
  p.gain = q_norm_gain;
  p.w_uq = w_uq;
  p.w_qr = w_qr;
  p.positions = positions;
  p.q_nope = q_nope;
  p.q_rope = q_rope;
  p.part1 = reinterpret_cast<float*>(ws);
  p.cq = ws + cq_off;
  p.batch = batch;
  p.hidden = hidden;
  p.dq = d_qlatent;
  p.heads = dims->num_heads;
  p.d_nope = dims->d_nope;
  p.d_rope = dims->d_rope;
  p.s1 = mla::query_partial_sums(hidden);
  p.eps = rms_eps;
  return hip_status(mla::launch_query_proj(p, static_cast<hipStream_t>(stream)));
}

int64_t mla_prefill_workspace(const mla_dims* dims, int32_t batch, int32_t max_seq_len) {
  if (dims == nullptr || batch <= 0 || max_seq_len <= 0 || shape_of(dims) != Shape::kDsv2) return 0;
  return mla::prefill_workspace_bytes(batch, dims->num_heads, max_seq_len);
}

mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t tokens_per_seq, const void* q_nope,
                       const void* q_rope, const mla_kv_cache* cache, const int32_t* seq_lens, int32_t max_seq_len,
                       const void* w_uk, const void* w_uv, float sm_scale, void* out, float* lse, void* workspace,
                       int64_t workspace_bytes, mla_stream stream) {
  if (dims == nullptr || cache == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || tokens_per_seq < 1 || max_seq_len < 0) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * tokens_per_seq > 0x7fffffff) return MLA_ERR_SHAPE;
  if (!valid_dtype(cache->dtype)) return MLA_ERR_DTYPE;
  if (shape_of(dims) != Shape::kDsv2) return MLA_ERR_UNSUPPORTED;   // the DeepSeek-V2 head shape
  if (cache->dtype != MLA_BF16) return MLA_ERR_DTYPE;               // a bf16 cache
  if (!std::isfinite(sm_scale)) return MLA_ERR_SHAPE;
  if ((static_cast<int64_t>(tokens_per_seq) + 127) / 128 > 65535) return MLA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(max_seq_len) + 127) / 128 > 0x7fffffff / 128) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_rope || !seq_lens || !w_uk || !w_uv || !out || !lse || !cache->latent) return MLA_ERR_NULL;
  const bool paged = cache->page_size > 0;
  if (cache->page_size < 0) return MLA_ERR_SHAPE;
  if (paged) {
    if (!cache->block_table) return MLA_ERR_NULL;
    if (!is_pow2(cache->page_size)) return MLA_ERR_SHAPE;
    const int64_t need = (static_cast<int64_t>(max_seq_len) + cache->page_size - 1) / cache->page_size;
    if (cache->max_pages_per_seq < need) return MLA_ERR_SHAPE;
  } else if (cache->seq_stride < max_seq_len) {
    return MLA_ERR_SHAPE;
  }
  if (cache->row_stride < dims->d_latent + dims->d_rope) return MLA_ERR_SHAPE;
  if ((cache->row_stride * 2) % 16 != 0) return MLA_ERR_ALIGN;
  if (max_seq_len > 0) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < mla_prefill_workspace(dims, batch, max_seq_len)) return MLA_ERR_SHAPE;
    if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  }
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(cache->latent) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(out))
    return MLA_ERR_ALIGN;
  mla::PrefillParams p{};
  p.q_nope = q_nope;
  p.q_rope = q_rope;
  p.latent = cache->latent;
  p.row_stride = cache->row_stride;
  p.seq_stride = cache->seq_stride;
  p.block_table = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.page_shift = paged ? log2i(cache->page_size) : -1;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.n = tokens_per_seq;
  p.heads = dims->num_heads;
  p.max_seq_len = max_seq_len;
  p.lpad = (max_seq_len + 127) / 128 * 128;
  p.w_uk = w_uk;
  p.w_uv = w_uv;
  const int64_t half = mla::prefill_workspace_bytes(batch, dims->num_heads, max_seq_len) / 2;
  p.kc = workspace;
  p.vc = static_cast<char*>(workspace) + half;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.out = out;
  p.lse = lse;
  return hip_status(mla::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

mla_status mla_cache_append_noalloc(const mla_dims* dims, int32_t batch, int32_t hidden, const void* h,
                                    const void* w_dkv, const void* w_kr, const void* norm_gain, int32_t dtype,
                                    float rms_eps, const mla_rope* rope, const int32_t* positions,
                                    const mla_kv_cache* cache, mla_stream stream) {
  mla::AppendParams p{};
  bool dsv2 = false;
  const mla_status st = cache_append_params(dims, batch, hidden, h, w_dkv, w_kr, norm_gain, dtype, rms_eps,
                                            rope, positions, cache, p, dsv2);
  if (st != MLA_OK || batch == 0) return st;
  if (mla_cache_append_workspace(dims, batch, hidden) > mla::append_scratch_bytes()) return MLA_ERR_UNSUPPORTED;
  float* scratch = nullptr;
  const hipError_t e = mla::append_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e);
  p.work = scratch;
  return hip_status(mla::launch_cache_append(p, dsv2, cache_kind_of(cache->dtype), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace mla {
void take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_next_start;
  *stop = g_next_stop;
  g_next_start = g_next_stop = nullptr;
}
}  // namespace mla

extern "C" mla_status mla_read_probe(const void* buf, int64_t bytes, void* sink, mla_stream stream) {
  if (bytes < 0 || bytes % 16 != 0) return MLA_ERR_SHAPE;
  if (bytes == 0) return MLA_OK;
  if (!buf || !sink) return MLA_ERR_NULL;
  if (!aligned16(buf)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)));
}

extern "C" mla_status mla_time_next_launch(void* start_event, void* stop_event) {
  g_next_start = static_cast<hipEvent_t>(start_event);
  g_next_stop = static_cast<hipEvent_t>(stop_event);
  return MLA_OK;
}
