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
//     each wave one 256-wide slice (MFMA 32x32x16); the five partial tiles
//     are added through LDS in wave order and stored as one fp32 partial sum;
//  2. latent_norm: one workgroup per sequence adds those partial sums in
//     order, takes the RMS norm and writes c_Q in bf16, blocked by 16
//     features ([d'_c / 16][rows][16]) so that the next product's operand
//     loads are whole 1 KiB rows;
//  3. qgemm over [W_UQ; W_QR] with the whole d'_c contraction in one
//     workgroup (waves of two 256-wide slices, at most eight, their tiles
//     added through LDS in wave order), which then turns the
//     rotary pairs (the partner value from the neighbouring lane, the angle
//     position * f_i in double precision) and writes q_nope [B, H, d_nope]
//     and q_rope [B, H, d_rope] directly.
// A wave's weight slice (32 rows x 512 bytes) goes HBM -> LDS with direct
// 16-byte loads, two whole rows per instruction, and its MFMA fragments are
// read back from LDS: loading the fragments straight from memory touched 32
// rows per instruction, and [W_UQ; W_QR] took 37 us at batch 32 against
// 29 us staged (three waves of two slices a workgroup; one wave a slice,
// whose six waves' 96 KB of LDS left one workgroup per compute unit, 36 us).
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
constexpr int kQStage = 32 * kQSlice * 2;   // LDS bytes of one wave's weight slice

struct QGemm {
  const __bf16* a;     // activations: [M, K] row-major, or blocked [K / 16][Mpad][16]
  const __bf16* w0;    // rows [0, n0) of the weight, [n0, K]
  const __bf16* w1;    // rows [n0, N), [N - n0, K]
  float* out;          // FINISH == false: [gridDim.y, M, N] partial sums
  int32_t M, N, K, n0;
  int32_t slices;      // 256-wide slices per workgroup
};

// Workgroup (x, y, z): columns 32x .. 32x + 31, slices y * slices .. of the
// contraction, rows 32z .. 32z + 31; wave w takes slices w, w + waves, ...
// of them. Weight row j of the tile sits at LDS bytes 512 j .. with its
// 16-byte chunk c at position c ^ (j & 31), so the 32 rows that one fragment
// read touches cover every bank group. The waves' tiles are added in wave
// order through LDS; FINISH turns the rotary columns and writes the query.
template <bool FINISH, bool A_BLOCKED, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void qgemm(QGemm g, QueryParams p) {
  __shared__ __attribute__((aligned(16))) char stage[WAVES * kQStage];   // at most blockDim.x / 64 used
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int n0 = blockIdx.x * 32;       // N is a multiple of 32; a tile lies in one weight
  const int n = n0 + r;                 // B operand column (weight row)
  const int m = blockIdx.z * 32 + r;    // A operand row
  const int mpad = gridDim.z * 32;
  const __bf16* wt = n0 < g.n0 ? g.w0 + (int64_t)n0 * g.K : g.w1 + (int64_t)(n0 - g.n0) * g.K;
  const auto res = buffer_rsrc(wt, (uint32_t)(32 * g.K * 2));   // reads past the tile return zero
  const bool m_ok = m < g.M;
  const __bf16* a = g.a + (int64_t)(m_ok ? m : 0) * g.K;
  MLA_LDS char* st = (MLA_LDS char*)stage + wave * kQStage;
  f32x16 acc = {};
  for (int sl = wave; sl < g.slices; sl += waves) {
    const int k0 = (blockIdx.y * g.slices + sl) * kQSlice;
    if (k0 >= g.K) break;              // uniform in the wave
    const int kn = min(kQSlice, g.K - k0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the previous slice's fragments are read
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 2 * i + half;
      const int chunk = (lane & 31) ^ (row & 31);
      buf_load16_to_lds(res, (uint32_t)(row * g.K * 2 + k0 * 2 + 16 * chunk), 0u, st + i * 1024);
    }
    bf16x8 av[kQSlice / 16];
#pragma unroll
    for (int s = 0; s < kQSlice / 16; ++s) {
      if (16 * s < kn) {
        bf16x8 v;
        if constexpr (A_BLOCKED) v = *(const bf16x8*)(g.a + ((int64_t)(k0 / 16 + s) * mpad + m) * 16 + 8 * half);
        else v = *(const bf16x8*)(a + k0 + 16 * s + 8 * half);
        av[s] = m_ok ? v : bf16x8{};
      }
    }
    wait_vmem();
#pragma unroll
    for (int s = 0; s < kQSlice / 16; ++s) {
      if (16 * s < kn) {
        const bf16x8 bv = *(const MLA_LDS bf16x8*)(st + r * 512 + 16 * ((2 * s + half) ^ r));
        acc = mfma32x32x16(av[s], bv, acc);
      }
    }
  }
  // fixed-order sum of the waves' tiles: lane l of every wave holds the same
  // 16 positions, so the sum is elementwise; each wave parks its tile in its
  // own staging region
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  MLA_LDS float* mine = (MLA_LDS float*)st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(MLA_LDS f32x4*)(mine + lane * 16 + 4 * i) = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
  __syncthreads();
  if (wave != 0) return;
  for (int v = 1; v < waves; ++v) {
    const MLA_LDS float* other = (const MLA_LDS float*)((MLA_LDS char*)stage + v * kQStage);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 x = *(const MLA_LDS f32x4*)(other + lane * 16 + 4 * i);
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
constexpr int kFastParts = 4;         // hidden up to 4 x 1280: every load issued before any sum

// c_Q[b] = RMSNorm(sum of the partial sums) in bf16; one 256-thread
// workgroup per sequence, thread t owns features t, t + 256, ...; the
// partial sums of a feature are added in order. c_Q is stored blocked:
// feature c of row b at ((c / 16) * Mpad + b) * 16 + c % 16.
__global__ __launch_bounds__(256) void latent_norm(QueryParams p) {
  __shared__ float red[4];
  const int b = blockIdx.x, t = threadIdx.x;
  const int per = p.dq / 256;
  const int64_t part = (int64_t)p.batch * p.dq;
  const float* src = p.part1 + (int64_t)b * p.dq;
  float x[kMaxDqPerThread];
  float ss = 0.0f;
  if (p.s1 <= kFastParts) {
    float v[kMaxDqPerThread][kFastParts];
#pragma unroll
    for (int j = 0; j < kMaxDqPerThread; ++j)
#pragma unroll
      for (int s = 0; s < kFastParts; ++s) v[j][s] = (j < per && s < p.s1) ? src[s * part + t + 256 * j] : 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxDqPerThread; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int s = 0; s < kFastParts; ++s)
        if (s < p.s1) a += v[j][s];   // in order
      x[j] = a;
      if (j < per) ss += a * a;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxDqPerThread; ++j) {
      float a = 0.0f;
      if (j < per)
        for (int s = 0; s < p.s1; ++s) a += src[s * part + t + 256 * j];   // in order
      x[j] = a;
      if (j < per) ss += a * a;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum256(ss, red) / p.dq + p.eps);
  const int mpad = (p.batch + 31) / 32 * 32;
  __bf16* dst = (__bf16*)p.cq;
#pragma unroll
  for (int j = 0; j < kMaxDqPerThread; ++j) {
    if (j < per) {
      const int c = t + 256 * j;
      const float g = p.gain != nullptr ? (float)((const __bf16*)p.gain)[c] : 1.0f;
      dst[((int64_t)(c >> 4) * mpad + b) * 16 + (c & 15)] = (__bf16)(x[j] * inv * g);
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
  *total = *cq_off + up((int64_t)(batch + 31) / 32 * 32 * dq * 2);   // c_Q blocked, rows padded to 32
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
  hipError_t e = launch_kernel_events(qgemm<false, false, kQ1Slices>, dim3(p.dq / 32, p.s1, rb),
                                      dim3(64 * kQ1Slices), stream, e0, nullptr, g1, p);
  if (e != hipSuccess) return e;
  e = launch_kernel_events(latent_norm, dim3(p.batch), dim3(256), stream, nullptr, nullptr, p);
  if (e != hipSuccess) return e;
  const int s2 = p.dq / kQSlice;
  QGemm g2{(const __bf16*)p.cq, (const __bf16*)p.w_uq, (const __bf16*)p.w_qr, nullptr, p.batch, n2, p.dq,
           p.heads * p.d_nope, s2};
  // two slices a wave: three waves for d'_c = 1536, whose 48 KB of LDS let
  // three workgroups share a compute unit (one wave a slice: 36 us; three:
  // 29 us at batch 32)
  const dim3 grid2(n2 / 32, 1, rb);
  if (s2 <= 6)
    return launch_kernel_events(qgemm<true, true, 3>, grid2, dim3(64 * ((s2 + 1) / 2)), stream, nullptr, e1, g2, p);
  return launch_kernel_events(qgemm<true, true, kQMaxWaves>, grid2, dim3(64 * std::min((s2 + 1) / 2, kQMaxWaves)),
                              stream, nullptr, e1, g2, p);
}

}  // namespace mla
