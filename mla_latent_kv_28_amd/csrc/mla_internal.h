// Host-side launch interface between the C ABI (mla_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum CacheKind : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// Item order of the decode grid (set by the launcher).
enum DecodeOrder : int { kOrderPlain = 0, kOrderXcd = 1, kOrderLongestFirst = 2 };

struct DecodeParams {
  const void* q_lat;            // [B, H, DC + DR]
  const void* latent;           // cache rows (see mla_kv_cache)
  const void* rope;             // fp8 only
  const float* scale;           // fp8 only
  int64_t row_stride;           // elements (bytes for fp8 codes)
  int64_t rope_stride;          // fp8 only, elements
  int64_t seq_stride;           // contiguous only
  const int32_t* block_table;   // paged only
  int32_t max_pages;
  int32_t page_shift;           // log2(page_size); -1 = contiguous
  const int32_t* seq_lens;      // [B]
  int32_t batch;
  int32_t max_seq_len;          // lengths are clamped to [0, max_seq_len]
  int32_t num_splits;
  int32_t chunk;                // tokens per split, multiple of the tile
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // S == 1: [B, H, DC]; S > 1: [B, S, H, DC] (bf16 | f32)
  float* lse;                   // S == 1: [B, H]; S > 1: [B, S, H]
  int32_t out_bf16;             // out is bf16 (else f32)
  int32_t order;                // DecodeOrder: which item each workgroup takes
  // Query tokens per sequence (n >= 1). `batch` counts query rows bv = b n + t
  // (q_lat, out and lse are indexed by bv); the cache and seq_lens by b; token
  // t of sequence b attends to rows 0 .. seq_lens[b] - n + t.
  int32_t tokens_per_seq;
};

// Prefill of n new tokens per sequence, non-absorbed (DeepSeek-V2 shape, bf16).
struct PrefillParams {
  const void* q_nope;           // [B n, H, 128] bf16
  const void* q_rope;           // [B n, H, 64] bf16
  const void* latent;           // bf16 cache rows [c_KV | k^R]
  int64_t row_stride;           // elements
  int64_t seq_stride;           // contiguous only
  const int32_t* block_table;   // paged only
  int32_t max_pages;
  int32_t page_shift;           // -1 = contiguous
  const int32_t* seq_lens;      // [B], clamped to [0, max_seq_len]
  int32_t batch, n, heads, max_seq_len;
  int32_t lpad;                 // max_seq_len rounded up to 128
  const void* w_uk;             // [H, 128, 512] bf16
  const void* w_uv;             // [H, 128, 512] bf16
  void* kc;                     // workspace [B, H, lpad, 128] bf16
  void* vc;                     // workspace [B, H, lpad, 128] bf16
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // [B n, H, 128] bf16
  float* lse;                   // [B n, H]
};
int64_t prefill_workspace_bytes(int batch, int heads, int max_seq_len);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Compute units of the current device (cached per device; 256 if the query fails).
int device_compute_units();

// Streaming read of `bytes` (a multiple of 16) from src; sink: 4 device bytes,
// written only in the unlikely case that the XOR of the data equals a constant.
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

// Decode launchers: return the hipError_t of the launch.
hipError_t launch_decode_dsv2_bf16(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_dsv2_fp8(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_tiny_f32(const DecodeParams& p, hipStream_t s);

struct CombineParams {
  const void* o_part;    // [B, S, H, DC] (bf16 | f32)
  const float* lse_part; // [B, S, H]
  void* out;             // [B, H, DC]
  float* lse;            // [B, H] or null
  int32_t batch, splits, heads, d_latent;
  int32_t out_bf16;
  int32_t part_bf16;
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

// Rotary pairs a kernel parameter block carries frequencies for (d_rope <= 64).
constexpr int kMaxRopePairs = 32;

// Cache entry of one new token per sequence (append.hip).
struct AppendParams {
  const void* h;                // [B, hidden] (bf16 | f32)
  const void* w_dkv;            // [d_latent, hidden]
  const void* w_kr;             // [d_rope, hidden]
  const void* gain;             // [d_latent] norm gain or null
  const int32_t* positions;     // [B] position (cache row) of the new token
  void* latent;                 // cache rows (codes for e4m3)
  void* rope;                   // e4m3 only: rotary keys, bf16
  float* scale;                 // e4m3 only: per-token scale
  int64_t row_stride, rope_stride, seq_stride;
  const int32_t* block_table;   // paged only
  int32_t max_pages, page_shift;   // page_shift -1: contiguous
  float* work;                  // [ksplits, B, d_latent + d_rope] partial sums
  int32_t batch, hidden, ksplits, d_latent, d_rope;
  float eps;
  double freq[kMaxRopePairs];   // rotation frequency of feature pair i (plain or YaRN)
};
int append_slices(int hidden, bool dsv2);   // partial sums of the projection
hipError_t launch_cache_append(const AppendParams& p, bool dsv2, int cache_kind, hipStream_t s);
// The library's own per-GPU scratch for the allocation-free cache append.
int64_t append_scratch_bytes();
hipError_t append_scratch(float** ptr);   // this device's address of the array

// Query of one new token per sequence (query.hip): c_Q = RMSNorm(W_DQ h),
// q_nope = W_UQ c_Q, q_rope = RoPE(W_QR c_Q).
struct QueryParams {
  const void* h;                // [B, hidden] bf16
  const void* w_dq;             // [dq, hidden]
  const void* gain;             // [dq] or null
  const void* w_uq;             // [H * d_nope, dq]
  const void* w_qr;             // [H * d_rope, dq]
  const int32_t* positions;     // [B]
  void* q_nope;                 // [B, H, d_nope] bf16
  void* q_rope;                 // [B, H, d_rope] bf16
  float* part1;                 // [s1, B, dq] fp32 partial sums of W_DQ h
  void* cq;                     // [B, dq] bf16, the normed latent
  int32_t batch, hidden, dq, heads, d_nope, d_rope;
  int32_t s1;                   // partial sums of W_DQ h (query_partial_sums)
  float eps;
  double freq[kMaxRopePairs];
};
// Partial sums the query path keeps of W_DQ h at this hidden size (at most 16).
int query_partial_sums(int hidden);
// Workspace layout of the query path: byte offset of cq, total bytes.
void query_workspace_layout(int batch, int hidden, int dq, int64_t* cq_off, int64_t* total);
hipError_t launch_query_proj(const QueryParams& p, hipStream_t s);

// Attention output projection u[b] = W_O o[b] (oproj.hip).
struct OProjParams {
  const void* o;      // [B, k] (the heads' outputs, concatenated)
  const void* w;      // [n, k]
  void* out;          // [B, n]
  float* work;        // bf16: fp32 partial sums [parts, B, n]
  int32_t batch, n, k;
};
bool oproj_bf16_shape_ok(int n, int k);
int64_t oproj_workspace_bytes(int batch, int n, int k);
hipError_t launch_oproj(const OProjParams& p, bool bf16, bool out_f32, hipStream_t s);

// Per-head batched GEMM: C[b, h, n] = sum_k A[b, h, k] * Bm_h(k, n).
struct GemmParams {
  const void* a;         // [B, H, lda] (bf16 or f32)
  const void* w;         // absorb: [H, K, N]; out-proj: [H, N, K]
  void* c;               // [B, H, ldc]
  int64_t lda, ldc;      // elements per (b, h) row
  int32_t batch, heads;
  int32_t a_f32;         // A is f32 (bf16 weights: rounded to bf16 on load)
  int32_t c_f32;         // C is written as f32 (else bf16)
  // absorb only: copy this [B, H, n_tail] tensor into C[:, :, N:N + n_tail]
  const void* tail;
  int32_t n_tail;
};
hipError_t launch_absorb_dsv2_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_absorb_tiny_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_outproj_dsv2_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_outproj_tiny_f32(const GemmParams& p, hipStream_t s);

// Split merge and out-projection in one pass (DeepSeek-V2 shapes, bf16).
struct CombineOutParams {
  const void* o_part;    // [B, S, H, DC] bf16
  const float* lse_part; // [B, S, H]
  const void* w;         // W_UV [H, DV, DC] bf16
  void* out;             // [B, H, DV] (bf16 | f32)
  float* lse;            // [B, H] or null
  int32_t batch, splits, heads;
  int32_t out_f32;
  int32_t rows_per_block;  // set by the launcher
};
hipError_t launch_combine_outproj_dsv2_bf16(const CombineOutParams& p, hipStream_t s);
int combine_outproj_max_splits();


// Measurement: an event pair that the next kernel launch records around its
// own execution (set with mla_time_next_launch, taken by one launch).
void take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through this: with a pending event
// pair the launch carries it (hipExtLaunchKernel), otherwise a plain launch.
template <typename K, typename... Args>
inline hipError_t launch_kernel_events(K kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t e0,
                                       hipEvent_t e1, Args... args) {
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

template <typename K, typename... Args>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  return launch_kernel_events(kernel, grid, block, stream, e0, e1, args...);
}

}  // namespace mla
