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
//  1. qgemm over W_DQ: [B, hidden] x [hidden, d'_c]; a workgroup of five
//     waves per (32 output features, 1280 contraction features, 32 rows),
//     each wave one 256-wide slice (MFMA 32x32x16, operands straight from
//     memory, every load of a slice issued before its products); the five
//     partial tiles are added through LDS in wave order and stored as one
//     fp32 partial sum;
//  2. latent_norm: one workgroup per sequence adds those partial sums in
//     order, takes the RMS norm and writes c_Q in bf16;
//  3. qgemm over [W_UQ; W_QR] with the whole d'_c contraction in one
//     workgroup (up to eight waves, each taking every eighth 256-wide slice,
//     their tiles added through LDS in wave order), which then turns the rotary pairs (the partner value from the
//     neighbouring lane, the angle position * f_i in double precision) and
//     writes q_nope [B, H, d_nope] and q_rope [B, H, d_rope] directly.
// The weights (91 MB at the DeepSeek-V2 shape) are read once per 32 rows.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kQSlice = 256;     // contraction features per wave and pass
constexpr int kQMaxWaves = 8;    // waves per workgroup
constexpr int kQ1Slices = 5;     // slices per workgroup over W_DQ

struct QGemm {
  const __bf16* a;     // [M, K] row-major activations
  const __bf16* w0;    // rows [0, n0) of the weight, [n0, K]
  const __bf16* w1;    // rows [n0, N), [N - n0, K]
  float* out;          // FINISH == false: [gridDim.y, M, N] partial sums
  int32_t M, N, K, n0;
  int32_t slices;      // 256-wide slices per workgroup
};

// Workgroup (x, y, z): columns 32x .. 32x + 31, slices y * slices .. of the
// contraction, rows 32z .. 32z + 31; wave w takes slices w, w + waves, ...
// of them. The waves' tiles are added in wave order through LDS; FINISH
// turns the rotary columns and writes the query.
template <bool FINISH>
__global__ __launch_bounds__(64 * kQMaxWaves) void qgemm(QGemm g, QueryParams p) {
  __shared__ __attribute__((aligned(16))) float red[kQMaxWaves][64 * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int n = blockIdx.x * 32 + r;   // B operand column (weight row); N is a multiple of 32
  const int m = blockIdx.z * 32 + r;   // A operand row
  const __bf16* w = n < g.n0 ? g.w0 + (int64_t)n * g.K : g.w1 + (int64_t)(n - g.n0) * g.K;
  const bool m_ok = m < g.M;
  const __bf16* a = g.a + (int64_t)(m_ok ? m : 0) * g.K;
  f32x16 acc = {};
  for (int sl = wave; sl < g.slices; sl += waves) {
    const int k0 = (blockIdx.y * g.slices + sl) * kQSlice, k1 = min(k0 + kQSlice, g.K);
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
  }
  // fixed-order sum of the waves' tiles: lane l of every wave holds the same
  // 16 positions, so the sum is elementwise
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(f32x4*)&red[wave][lane * 16 + 4 * i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
  __syncthreads();
  if (wave != 0) return;
  for (int v = 1; v < waves; ++v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 x = *(const f32x4*)&red[v][lane * 16 + 4 * i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * i + e] += x[e];
    }
  }
  // accumulator i: row 32z + 8 (i / 4) + 4 half + i % 4, column n
  if constexpr (!FINISH) {
    float* out = g.out + (int64_t)blockIdx.y * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = blockIdx.z * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < g.M) out[(int64_t)row * g.N + n] = acc[i];
    }
  } else {
    const int n_nope = p.heads * p.d_nope;
    const bool rot = n >= n_nope;
    const int c = n - n_nope;                    // head c / d_rope, feature c % d_rope
    const int f = rot ? c % p.d_rope : 0, pair = f >> 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = blockIdx.z * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      const float v = acc[i];
      const float other = __shfl_xor(v, 1);     // d_rope and n_nope are even: pairs stay in lane pairs
      if (row >= g.M) continue;
      if (!rot) {
        ((__bf16*)p.q_nope)[(int64_t)row * n_nope + n] = (__bf16)v;
        continue;
      }
      const double ang = (double)p.positions[row] * p.freq[pair];
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double x0 = (f & 1) ? other : v, x1 = (f & 1) ? v : other;
      const double y = (f & 1) ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
      ((__bf16*)p.q_rope)[(int64_t)row * p.heads * p.d_rope + c] = (__bf16)(float)y;
    }
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
constexpr int kMaxParts = 16;         // partial sums of W_DQ h (hidden up to 16 x 1280)

// c_Q[b] = RMSNorm(sum of the partial sums) in bf16; one 256-thread
// workgroup per sequence, thread t owns features t, t + 256, ...; every load
// of a feature's partial sums is issued before they are added in order.
__global__ __launch_bounds__(256) void latent_norm(QueryParams p) {
  __shared__ float red[4];
  const int b = blockIdx.x, t = threadIdx.x;
  const int per = p.dq / 256;
  const int64_t part = (int64_t)p.batch * p.dq;
  const float* src = p.part1 + (int64_t)b * p.dq;
  float x[kMaxDqPerThread];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxDqPerThread; ++j) {
    if (j < per) {
      float parts[kMaxParts];
#pragma unroll
      for (int s = 0; s < kMaxParts; ++s) parts[s] = s < p.s1 ? src[s * part + t + 256 * j] : 0.0f;
      float v = 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxParts; ++s)
        if (s < p.s1) v += parts[s];   // in order
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

}  // namespace

int query_partial_sums(int hidden) {
  const int slices = (hidden + kQSlice - 1) / kQSlice;
  return (slices + kQ1Slices - 1) / kQ1Slices;
}

void query_workspace_layout(int batch, int hidden, int dq, int64_t* cq_off, int64_t* total) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  *cq_off = up((int64_t)query_partial_sums(hidden) * batch * dq * 4);
  *total = *cq_off + up((int64_t)batch * dq * 2);
}

// A pending event pair (mla_time_next_launch) brackets the launches: the start
// event goes with the first, the stop event with the last.
hipError_t launch_query_proj(const QueryParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  const int n2 = p.heads * (p.d_nope + p.d_rope);
  const int rb = (p.batch + 31) / 32;
  QGemm g1{(const __bf16*)p.h, (const __bf16*)p.w_dq, (const __bf16*)p.w_dq, p.part1, p.batch, p.dq, p.hidden,
           p.dq, kQ1Slices};
  hipError_t e = launch_kernel_events(qgemm<false>, dim3(p.dq / 32, p.s1, rb), dim3(64 * kQ1Slices), stream, e0,
                                      nullptr, g1, p);
  if (e != hipSuccess) return e;
  e = launch_kernel_events(latent_norm, dim3(p.batch), dim3(256), stream, nullptr, nullptr, p);
  if (e != hipSuccess) return e;
  const int s2 = p.dq / kQSlice;
  QGemm g2{(const __bf16*)p.cq, (const __bf16*)p.w_uq, (const __bf16*)p.w_qr, nullptr, p.batch, n2, p.dq,
           p.heads * p.d_nope, s2};
  return launch_kernel_events(qgemm<true>, dim3(n2 / 32, 1, rb), dim3(64 * std::min(s2, kQMaxWaves)), stream,
                              nullptr, e1, g2, p);
}

}  // namespace mla
