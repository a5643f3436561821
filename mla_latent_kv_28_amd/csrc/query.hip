// The query of one new token per sequence.
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.2: the query is
// compressed as well, c_Q = W_DQ h, and its content part is the up-projection
// q^C = W_UQ c_Q; section 2.1.3: every head's rotary query is
// q^R = RoPE(W_QR c_Q) at the token's position; section 3.1.2: an RMS norm
// follows the compressed latent (d'_c = 1536). The rotation frequencies
// (plain RoPE or YaRN, section 3.1.4) come from the host.
//
// Three launches, bf16 in and out with fp32 accumulation:
//  1. skinny_gemm over W_DQ: [B, hidden] x [hidden, d'_c] in contraction
//     parts of 1024 (four waves of 256 each), each part's sum stored as an
//     fp32 partial sum;
//  2. latent_norm: one workgroup per sequence adds those partial sums in
//     order, takes the RMS norm and writes c_Q in bf16 in the operand order
//     of the next product (fragment-major, one 1 KiB load per operand);
//  3. skinny_gemm over [W_UQ; W_QR] with the whole d'_c contraction in one
//     workgroup (four waves of d'_c / 4, their tiles added in wave order),
//     which then turns the rotary pairs (both values of a pair sit in one
//     lane; the angle position * f_i and the products in double precision)
//     and writes q_nope [B, H, d_nope] and q_rope [B, H, d_rope] directly.
// The weights (91 MB at the DeepSeek-V2 shape) are read once per 32 rows, in
// 128-byte row pieces (skinny.h).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"
#include "skinny.h"

namespace mla {
namespace {

// The rotary finish of the second product: the columns of W_UQ c_Q go to
// q_nope as they are; the columns of W_QR c_Q are turned in pairs (2i, 2i + 1)
// by position * f_i (angle and products in double precision) into q_rope.
// Lane values v[0..3] are columns n .. n + 3 of row b: two whole pairs.
struct EpiQuery {
  void* q_nope;
  void* q_rope;
  const int32_t* positions;
  int32_t M, heads, d_nope, d_rope;
  double freq[kMaxRopePairs];
  __device__ __forceinline__ void operator()(int b, int n, int, const f32x4& v) const {
    if (b >= M) return;
    const int n_nope = heads * d_nope;
    if (n < n_nope) {
      *(u32x2*)((__bf16*)q_nope + (int64_t)b * n_nope + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      return;
    }
    const int c = n - n_nope, f = c % d_rope;
    float y[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const double ang = (double)positions[b] * freq[f / 2 + q];
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double x0 = v[2 * q], x1 = v[2 * q + 1];
      y[2 * q] = (float)(x0 * cs - x1 * sn);
      y[2 * q + 1] = (float)(x0 * sn + x1 * cs);
    }
    *(u32x2*)((__bf16*)q_rope + (int64_t)b * heads * d_rope + c) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  }
};

constexpr int kQWaves = 4, kQNa = 2;      // waves per workgroup, 16-row weight groups per workgroup
constexpr int kQ1Depth = 4, kQ2Depth = 3; // macro steps in flight per wave (W_DQ; [W_UQ; W_QR])
constexpr int kQ1Kw = 256;                // W_DQ: contraction features per wave

constexpr int kMaxParts = 20;   // partial sums of W_DQ h (hidden up to 20 x 1024)

// c_Q[b] = RMSNorm(sum of the partial sums) in bf16; one workgroup of d'_c / 4
// threads per sequence, thread t owns features 4t .. 4t + 3 and adds their
// partial sums in order (all loads issued first). c_Q is stored
// fragment-major (frag_offset), the operand layout of the up-projection.
__global__ __launch_bounds__(1024) void latent_norm(QueryParams p) {
  __shared__ float red[16];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6, waves = blockDim.x >> 6;
  const int64_t part = (int64_t)p.batch * p.dq;
  const float* src = p.part1 + (int64_t)b * p.dq + 4 * t;
  f32x4 v[kMaxParts];
#pragma unroll
  for (int s = 0; s < kMaxParts; ++s)
    if (s < p.s1) v[s] = *(const f32x4*)(src + s * part);
  f32x4 x = v[0];
#pragma unroll
  for (int s = 1; s < kMaxParts; ++s)
    if (s < p.s1) x += v[s];   // in order
  float ss = (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < waves; ++w) tot += red[w];   // in wave order
  const float inv = 1.0f / sqrtf(tot / p.dq + p.eps);
  float g[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if (p.gain != nullptr) {
    const u32x2 gw = *(const u32x2*)((const __bf16*)p.gain + 4 * t);
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = bf16_bits_to_f32((gw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
  }
  *(u32x2*)((__bf16*)p.cq + frag_offset(b, 4 * t, p.dq)) =
      u32x2{pack_bf16x2(x[0] * inv * g[0], x[1] * inv * g[1]), pack_bf16x2(x[2] * inv * g[2], x[3] * inv * g[3])};
}

}  // namespace

int query_partial_sums(int hidden) {
  return (hidden + kQWaves * kQ1Kw - 1) / (kQWaves * kQ1Kw);
}

void query_workspace_layout(int batch, int hidden, int dq, int64_t* cq_off, int64_t* total) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  *cq_off = up((int64_t)query_partial_sums(hidden) * batch * dq * 4);
  *total = *cq_off + up((int64_t)(batch + 31) / 32 * 32 * dq * 2);   // c_Q fragment-major, rows padded to 32
}

// A pending event pair (mla_time_next_launch) brackets the launches: the start
// event goes with the first, the stop event with the last.
hipError_t launch_query_proj(const QueryParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  const int n2 = p.heads * (p.d_nope + p.d_rope);
  const int rb = (p.batch + 31) / 32;
  const dim3 block(64 * kQWaves);
  // 1. W_DQ h in s1 contraction parts of kQWaves * kQ1Kw features
  SkParams g1{p.h, p.w_dq, p.w_dq, p.hidden, p.dq, p.batch, p.dq, p.hidden, kQ1Kw, p.s1};
  const EpiPartial ep1{p.part1, p.batch, p.dq};
  const bool tail1 = p.s1 * kQWaves * kQ1Kw != p.hidden;
  const dim3 grid1(p.dq / (16 * kQNa) * p.s1, rb);
  hipError_t e = tail1 ? launch_kernel_events(skinny_gemm<kQWaves, kQ1Depth, kQNa, kXRowLds, true, EpiPartial>, grid1, block,
                                              stream, e0, nullptr, g1, ep1)
                       : launch_kernel_events(skinny_gemm<kQWaves, kQ1Depth, kQNa, kXRowLds, false, EpiPartial>, grid1, block,
                                              stream, e0, nullptr, g1, ep1);
  if (e != hipSuccess) return e;
  // 2. c_Q = RMSNorm of their sum, blocked by 16 features
  e = launch_kernel_events(latent_norm, dim3(p.batch), dim3(p.dq / 4), stream, nullptr, nullptr, p);
  if (e != hipSuccess) return e;
  // 3. [W_UQ; W_QR] c_Q over the whole d'_c in one workgroup, rotary finish
  const int kw2 = (p.dq / kQWaves + 64 * kQ2Depth - 1) / (64 * kQ2Depth) * (64 * kQ2Depth);
  SkParams g2{p.cq, p.w_uq, p.w_qr, 0, p.heads * p.d_nope, p.batch, n2, p.dq, kw2, 1};
  EpiQuery ep2{p.q_nope, p.q_rope, p.positions, p.batch, p.heads, p.d_nope, p.d_rope, {}};
  for (int i = 0; i < kMaxRopePairs; ++i) ep2.freq[i] = p.freq[i];
  const dim3 grid2(n2 / (16 * kQNa), rb);
  if (kw2 * kQWaves != p.dq)
    return launch_kernel_events(skinny_gemm<kQWaves, kQ2Depth, kQNa, kXFrag, true, EpiQuery>, grid2, block, stream, nullptr,
                                e1, g2, ep2);
  return launch_kernel_events(skinny_gemm<kQWaves, kQ2Depth, kQNa, kXFrag, false, EpiQuery>, grid2, block, stream, nullptr, e1,
                              g2, ep2);
}

}  // namespace mla
