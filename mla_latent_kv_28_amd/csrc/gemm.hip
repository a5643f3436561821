// Per-head batched projections on MFMA: the two absorbed weight products of
// MLA decode (DeepSeek-V2 paper, Chinese translation, section 2.1.2: W_UK is
// folded into the query side and W_UV into the output side).
//   absorb:   q_lat[b,h,n] = sum_k q_nope[b,h,k] * W_UK[h,k,n]   (W stored [K][N])
//   out-proj: o[b,h,n]     = sum_k o_lat[b,h,k]  * W_UV[h,n,k]   (W stored [N][K])
// For every head this is a (batch x K) . (K x N) product. One wave computes a
// 32-row x NT-column block with v_mfma_f32_32x32x16_bf16 (or eight fp32
// 32x32x2 per 16-wide k block); the weights are streamed once per 32 rows.
//
// A weight stored [K][N] (absorb) has N contiguous, but an MFMA B operand
// needs eight consecutive k of one column per lane. Each lane therefore reads
// eight rows k of eight consecutive columns (8 x 16 bytes) and transposes them
// in registers with byte permutes into eight fragments; fragment m's column c
// is n0 + 8c + m, which puts eight consecutive columns of one output row in
// one lane (one 16-byte store).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

template <bool F32, bool W_KN, int K, int N>
struct GemmCfg {
  static constexpr int NT = F32 ? 32 : (W_KN ? 256 : 128);   // columns per wave
  static constexpr int NFRAG = NT / 32;
  static constexpr int KC = K / 16;                          // 16-wide k blocks
  static_assert(K % 16 == 0 && N % NT == 0, "shape");
};

// A fragment: row b (lane r), k = 16*kc + 8*hh + 0..7; zero for rows >= batch.
template <bool F32>
struct AFrag;
template <>
struct AFrag<false> { bf16x8 v; };
template <>
struct AFrag<true> { float v[8]; };

__device__ __forceinline__ bf16x8 load_a_bf16(const void* row, int k0, bool ok, bool a_f32) {
  if (!ok) return bf16x8{};
  if (!a_f32) return *(const bf16x8*)((const __bf16*)row + k0);
  const f32x4 x0 = *(const f32x4*)((const float*)row + k0);
  const f32x4 x1 = *(const f32x4*)((const float*)row + k0 + 4);
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = (__bf16)x0[e]; v[4 + e] = (__bf16)x1[e]; }
  return v;
}

template <bool F32, bool W_KN, int K, int N>
__global__ __launch_bounds__(64) void head_gemm(GemmParams p) {
  using G = GemmCfg<F32, W_KN, K, N>;
  const int h = blockIdx.x, n0 = blockIdx.y * G::NT, b0 = blockIdx.z * 32;
  const int lane = threadIdx.x, hh = lane >> 5, r = lane & 31;
  const int brow = b0 + r;
  const bool row_ok = brow < p.batch;
  const int64_t arow = ((int64_t)(row_ok ? brow : 0) * p.heads + h) * p.lda;
  const char* wbase = (const char*)p.w + (int64_t)h * K * N * (F32 ? 4 : 2);

  f32x16 acc[G::NFRAG];
#pragma unroll
  for (int f = 0; f < G::NFRAG; ++f) acc[f] = f32x16{};

#pragma unroll 4
  for (int kc = 0; kc < G::KC; ++kc) {
    const int k0 = 16 * kc + 8 * hh;
    if constexpr (!F32) {
      const bf16x8 a = load_a_bf16((const char*)p.a + arow * (p.a_f32 ? 4 : 2), k0, row_ok, p.a_f32);
      if constexpr (W_KN) {
        // rows k0 .. k0+7, columns n0 + 8r .. +7
        u32x4 rows[8];
        const __bf16* w = (const __bf16*)wbase + (int64_t)k0 * N + n0 + 8 * r;
#pragma unroll
        for (int e = 0; e < 8; ++e) rows[e] = load16(w + (int64_t)e * N);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          u32x4 f;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            f[d] = (m & 1) ? pack_hi16(rows[2 * d][m >> 1], rows[2 * d + 1][m >> 1])
                           : pack_lo16(rows[2 * d][m >> 1], rows[2 * d + 1][m >> 1]);
          acc[m] = mfma32x32x16(a, __builtin_bit_cast(bf16x8, f), acc[m]);
        }
      } else {
#pragma unroll
        for (int g = 0; g < G::NFRAG; ++g) {
          const bf16x8 bw = *(const bf16x8*)((const __bf16*)wbase + (int64_t)(n0 + 32 * g + r) * K + k0);
          acc[g] = mfma32x32x16(a, bw, acc[g]);
        }
      }
    } else {
      float a[8];
      {
        const float* ar = (const float*)p.a + arow + k0;
        const f32x4 x0 = *(const f32x4*)ar, x1 = *(const f32x4*)(ar + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = row_ok ? x0[e] : 0.f; a[4 + e] = row_ok ? x1[e] : 0.f; }
      }
      float bw[8];
      const float* wf = (const float*)wbase;
      if constexpr (W_KN) {
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = wf[(int64_t)(k0 + e) * N + n0 + r];
      } else {
        const f32x4 x0 = *(const f32x4*)(wf + (int64_t)(n0 + r) * K + k0);
        const f32x4 x1 = *(const f32x4*)(wf + (int64_t)(n0 + r) * K + k0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { bw[e] = x0[e]; bw[4 + e] = x1[e]; }
      }
      acc[0] = mfma32x32x16_f32(a, bw, acc[0]);
    }
  }

  // C layout: lane (hh, c), accumulator i -> row 8*(i/4) + 4*hh + i%4.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = b0 + 8 * (i >> 2) + 4 * hh + (i & 3);
    if (b >= p.batch) continue;
    const int64_t crow = ((int64_t)b * p.heads + h) * p.ldc;
    if constexpr (!F32 && W_KN) {
      // fragment m holds column n0 + 8r + m: eight consecutive columns
      u32x4 v;
#pragma unroll
      for (int d = 0; d < 4; ++d) v[d] = pack_bf16x2(acc[2 * d][i], acc[2 * d + 1][i]);
      *(u32x4*)((__bf16*)p.c + crow + n0 + 8 * r) = v;
    } else {
#pragma unroll
      for (int g = 0; g < G::NFRAG; ++g) {
        const int n = n0 + 32 * g + r;
        if (p.c_f32) ((float*)p.c)[crow + n] = acc[g][i];
        else ((__bf16*)p.c)[crow + n] = (__bf16)acc[g][i];
      }
    }
  }

  // absorb: append the rotary query after the latent part
  if (p.tail != nullptr && blockIdx.y == 0) {
    const int nt = p.n_tail;
    for (int idx = lane; idx < 32 * nt; idx += 64) {
      const int rr = idx / nt, j = idx % nt, b = b0 + rr;
      if (b >= p.batch) continue;
      const int64_t src = ((int64_t)b * p.heads + h) * nt + j;
      const int64_t dst = ((int64_t)b * p.heads + h) * p.ldc + N + j;
      if (F32) ((float*)p.c)[dst] = ((const float*)p.tail)[src];
      else ((__bf16*)p.c)[dst] = ((const __bf16*)p.tail)[src];
    }
  }
}

template <bool F32, bool W_KN, int K, int N>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  using G = GemmCfg<F32, W_KN, K, N>;
  if (p.batch == 0) return hipSuccess;
  dim3 grid(p.heads, N / G::NT, (p.batch + 31) / 32);
  hipLaunchKernelGGL((head_gemm<F32, W_KN, K, N>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_dsv2_bf16(const GemmParams& p, hipStream_t s) {
  return launch<false, true, 128, 512>(p, s);
}
hipError_t launch_absorb_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, true, 32, 32>(p, s);
}
hipError_t launch_outproj_dsv2_bf16(const GemmParams& p, hipStream_t s) {
  return launch<false, false, 512, 128>(p, s);
}
hipError_t launch_outproj_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, false, 32, 32>(p, s);
}

}  // namespace mla
