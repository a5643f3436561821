// Log-sum-exp merge of split-KV partials.
//
// Each split s of a sequence produced o_s (softmax-normalised over its own
// tokens) and lse_s = log sum exp(scores) over those tokens. Attention over
// the union is   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
// Splits with no tokens carry lse_s = -inf and contribute nothing.
//
// One workgroup per (sequence, head). The merge weights are computed once per
// workgroup into LDS; each thread then owns one 16-byte vector of latent
// features (4 fp32 or 8 bf16 partial values) and sums it over the splits with
// four loads in flight.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxSplitsLds = 1024;

template <bool PART_BF16>
struct PartVec {
  static constexpr int N = PART_BF16 ? 8 : 4;   // features per 16-byte vector
  __device__ static void unpack(const u32x4& x, float (&v)[N]) {
    if constexpr (PART_BF16) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[2 * d] = bf16_bits_to_f32(x[d] & 0xffffu);
        v[2 * d + 1] = bf16_bits_to_f32(x[d] >> 16);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w = x[d];   // __builtin_bit_cast of a vector element itself reads element 0
        v[d] = __builtin_bit_cast(float, w);
      }
    }
  }
};

template <bool PART_BF16>
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  using V = PartVec<PART_BF16>;
  constexpr int ESZ = PART_BF16 ? 2 : 4;
  __shared__ float wts[kMaxSplitsLds];
  __shared__ float red[2];
  const int bh = blockIdx.x;
  const int b = bh / p.heads, h = bh % p.heads;
  const int S = p.splits;
  const float* lse_p = p.lse_part + (int64_t)b * S * p.heads + h;     // stride heads
  if (threadIdx.x < 64) {
    float m = -INFINITY;
    for (int s = threadIdx.x; s < S; s += 64) m = fmaxf(m, lse_p[(int64_t)s * p.heads]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float z = 0.0f;
    for (int s = threadIdx.x; s < S; s += 64) {
      const float l = lse_p[(int64_t)s * p.heads];
      const float w = (m == -INFINITY || l == -INFINITY) ? 0.0f : fast_exp2((l - m) * kLog2e);
      wts[s] = w;
      z += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    if (threadIdx.x == 0) { red[0] = m; red[1] = z; }
  }
  __syncthreads();
  const float m = red[0], z = red[1];
  const bool empty = (m == -INFINITY);
  const float inv = empty ? 0.0f : 1.0f / z;
  if (threadIdx.x == 0 && p.lse != nullptr)
    p.lse[(int64_t)b * p.heads + h] = empty ? -INFINITY : m + fast_log2(z) * kLn2;

  const int nvec = p.d_latent / V::N;
  const int64_t split_stride = (int64_t)p.heads * p.d_latent * ESZ;
  const char* part = (const char*)p.o_part + ((int64_t)b * S * p.heads + h) * p.d_latent * ESZ;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    const char* src = part + v * 16;
    float acc[V::N];
#pragma unroll
    for (int e = 0; e < V::N; ++e) acc[e] = 0.0f;
    // a split with weight 0 is skipped element-wise, so whatever it holds
    // (an empty split's zeros or anything else) cannot reach the sum
    auto add = [&](const u32x4& x, float w) {
      float xv[V::N];
      V::unpack(x, xv);
#pragma unroll
      for (int e = 0; e < V::N; ++e) acc[e] += w == 0.0f ? 0.0f : w * xv[e];
    };
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      u32x4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = load16(src + (s + i) * split_stride);
#pragma unroll
      for (int i = 0; i < 4; ++i) add(x[i], wts[s + i]);
    }
    for (; s < S; ++s) add(load16(src + s * split_stride), wts[s]);

    const int64_t o = ((int64_t)b * p.heads + h) * p.d_latent + V::N * v;
#pragma unroll
    for (int q = 0; q < V::N / 4; ++q) {
      const f32x4 r = {acc[4 * q] * inv, acc[4 * q + 1] * inv, acc[4 * q + 2] * inv, acc[4 * q + 3] * inv};
      if (p.out_bf16) {
        u32x2 pk;
        pk[0] = pack_bf16x2(r[0], r[1]);
        pk[1] = pack_bf16x2(r[2], r[3]);
        *(u32x2*)((__bf16*)p.out + o + 4 * q) = pk;
      } else {
        *(f32x4*)((float*)p.out + o + 4 * q) = r;
      }
    }
  }
}

}  // namespace

int combine_max_splits() { return kMaxSplitsLds; }

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const int vec = p.part_bf16 ? 8 : 4;
  const int threads = p.d_latent / vec >= 128 ? 128 : 64;   // >= 64: one full wave computes the weights
  if (p.part_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(p.batch * p.heads), dim3(threads), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(p.batch * p.heads), dim3(threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
