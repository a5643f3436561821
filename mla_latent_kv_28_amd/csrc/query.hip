// The query of one new token per sequence.
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.2: the query is
// compressed as well, c_Q = W_DQ h, and its content part is the up-projection
// q^C = W_UQ c_Q; section 2.1.3: every head's rotary query is
// q^R = RoPE(W_QR c_Q) at the token's position; section 3.1.2: an RMS norm
// follows the compressed latent (d'_c = 1536). The rotation frequencies
// (plain RoPE or YaRN, section 3.1.4) come from the host.
//
// Four launches, bf16 in and out with fp32 accumulation:
//  1. slice_gemm_bf16 over W_DQ: [B, hidden] x [hidden, d'_c] in contraction
//     slices of 256 into fp32 partial sums (one wave per 32 x 32 output tile
//     and slice, MFMA 32x32x16, operands straight from memory);
//  2. latent_norm: one workgroup per sequence adds the slices in order, takes
//     the RMS norm and writes c_Q in bf16;
//  3. slice_gemm_bf16 over [W_UQ; W_QR]: [B, d'_c] x [d'_c, H (d_nope +
//     d_rope)], slices of 256 again;
//  4. query_finish: adds those slices in order, turns the rotary pairs and
//     writes q_nope [B, H, d_nope] and q_rope [B, H, d_rope].
// The weights (91 MB at the DeepSeek-V2 shape) are read once per 32 rows.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kQSlice = 256;   // contraction features per partial sum

struct SliceGemm {
  const __bf16* a;     // [M, K] row-major activations
  const __bf16* w0;    // rows [0, n0) of the weight, [n0, K]
  const __bf16* w1;    // rows [n0, N), [N - n0, K] (may equal w0 + n0 K)
  float* out;          // [ceil(K / 256), M, N]
  int32_t M, N, K, n0;
};

// out[s][m][n] = sum_{k in slice s} a[m][k] w[n][k]. Wave (x, y, z): columns
// 32x .. 32x + 31, slice y, rows 32z .. 32z + 31; every load of the slice goes
// out before the products.
__global__ __launch_bounds__(64) void slice_gemm_bf16(SliceGemm g) {
  const int lane = threadIdx.x, r = lane & 31, half = lane >> 5;
  const int n = blockIdx.x * 32 + r;   // B operand column (weight row); N is a multiple of 32
  const int m = blockIdx.z * 32 + r;   // A operand row
  const int k0 = blockIdx.y * kQSlice, k1 = min(k0 + kQSlice, g.K);
  const __bf16* w = n < g.n0 ? g.w0 + (int64_t)n * g.K : g.w1 + (int64_t)(n - g.n0) * g.K;
  const bool m_ok = m < g.M;
  const __bf16* a = g.a + (int64_t)(m_ok ? m : 0) * g.K;
  f32x16 acc = {};
  bf16x8 av[kQSlice / 16], bv[kQSlice / 16];
#pragma unroll
  for (int s = 0; s < kQSlice / 16; ++s) {
    const int k = k0 + 16 * s + 8 * half;
    if (k0 + 16 * s < k1) {
      av[s] = m_ok ? *(const bf16x8*)(a + k) : bf16x8{};
      bv[s] = *(const bf16x8*)(w + k);
    }
  }
#pragma unroll
  for (int s = 0; s < kQSlice / 16; ++s)
    if (k0 + 16 * s < k1) acc = mfma32x32x16(av[s], bv[s], acc);
  float* out = g.out + (int64_t)blockIdx.y * g.M * g.N;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = blockIdx.z * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (row < g.M) out[(int64_t)row * g.N + n] = acc[i];
  }
}

__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr int kMaxDqPerThread = 16;   // d'_c up to 16 x 256

// c_Q[b] = RMSNorm(sum of the slices) in bf16; one 256-thread workgroup per
// sequence, thread t owns features t, t + 256, ...
__global__ __launch_bounds__(256) void latent_norm(QueryParams p) {
  __shared__ float red[4];
  const int b = blockIdx.x, t = threadIdx.x;
  const int per = p.dq / 256;
  const int64_t slice = (int64_t)p.batch * p.dq;
  const float* src = p.part1 + (int64_t)b * p.dq;
  float x[kMaxDqPerThread];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxDqPerThread; ++j) {
    if (j < per) {
      float v = 0.0f;
      for (int s = 0; s < p.s1; ++s) v += src[s * slice + t + 256 * j];   // slice order
      x[j] = v;
      ss += v * v;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum256(ss, red) / p.dq + p.eps);
  __bf16* dst = (__bf16*)p.cq + (int64_t)b * p.dq;
#pragma unroll
  for (int j = 0; j < kMaxDqPerThread; ++j) {
    if (j < per) {
      const int c = t + 256 * j;
      const float g = p.gain != nullptr ? (float)((const __bf16*)p.gain)[c] : 1.0f;
      dst[c] = (__bf16)(x[j] * inv * g);
    }
  }
}

// q_nope / q_rope of sequence b, columns 256 blockIdx.y + t of the stacked
// [W_UQ; W_QR] product: slices added in order; a rotary column takes its
// pair partner from the neighbouring lane and turns by position * f_i.
__global__ __launch_bounds__(256) void query_finish(QueryParams p) {
  const int b = blockIdx.x, n = blockIdx.y * 256 + threadIdx.x;
  const int n_nope = p.heads * p.d_nope, N = n_nope + p.heads * p.d_rope;
  const bool ok = n < N;
  const int64_t slice = (int64_t)p.batch * N;
  const float* src = p.part2 + (int64_t)b * N + (ok ? n : 0);
  float v = 0.0f;
  for (int s = 0; s < p.s2; ++s) v += src[s * slice];   // slice order
  const float other = __shfl_xor(v, 1);                 // every lane takes part
  if (!ok) return;
  if (n < n_nope) {
    ((__bf16*)p.q_nope)[(int64_t)b * n_nope + n] = (__bf16)v;
    return;
  }
  const int c = n - n_nope;                  // head c / d_rope, feature c % d_rope
  const int f = c % p.d_rope, i = f >> 1;    // d_rope and n_nope are even: pairs stay in lane pairs
  const double ang = (double)p.positions[b] * p.freq[i];
  double sn, cs;
  sincos(ang, &sn, &cs);
  const double x0 = (f & 1) ? other : v, x1 = (f & 1) ? v : other;
  const double y = (f & 1) ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
  ((__bf16*)p.q_rope)[(int64_t)b * p.heads * p.d_rope + c] = (__bf16)(float)y;
}

}  // namespace

void query_workspace_layout(int batch, int hidden, int dq, int n2, int64_t* cq_off, int64_t* part2_off,
                            int64_t* total) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t s1 = (hidden + kQSlice - 1) / kQSlice, s2 = (dq + kQSlice - 1) / kQSlice;
  *cq_off = up(s1 * batch * dq * 4);
  *part2_off = *cq_off + up((int64_t)batch * dq * 2);
  *total = *part2_off + s2 * batch * n2 * 4;
}

// A pending event pair (mla_time_next_launch) brackets the launches: the start
// event goes with the first, the stop event with the last.
hipError_t launch_query_proj(const QueryParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  const int n2 = p.heads * (p.d_nope + p.d_rope);
  const int rb = (p.batch + 31) / 32;
  SliceGemm g1{(const __bf16*)p.h, (const __bf16*)p.w_dq, (const __bf16*)p.w_dq, p.part1, p.batch, p.dq, p.hidden,
               p.dq};
  hipError_t e = launch_kernel_events(slice_gemm_bf16, dim3(p.dq / 32, p.s1, rb), dim3(64), stream, e0, nullptr, g1);
  if (e != hipSuccess) return e;
  e = launch_kernel_events(latent_norm, dim3(p.batch), dim3(256), stream, nullptr, nullptr, p);
  if (e != hipSuccess) return e;
  SliceGemm g2{(const __bf16*)p.cq, (const __bf16*)p.w_uq, (const __bf16*)p.w_qr, p.part2, p.batch, n2, p.dq,
               p.heads * p.d_nope};
  e = launch_kernel_events(slice_gemm_bf16, dim3(n2 / 32, p.s2, rb), dim3(64), stream, nullptr, nullptr, g2);
  if (e != hipSuccess) return e;
  return launch_kernel_events(query_finish, dim3(p.batch, (n2 + 255) / 256), dim3(256), stream, nullptr, e1, p);
}

}  // namespace mla
