// Log-sum-exp merge of split-KV partials.
//
// Each split s of a sequence produced o_s (softmax-normalised over its own
// tokens) and lse_s = log sum exp(scores) over those tokens. Attention over
// the union is   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
// Splits with no tokens carry lse_s = -inf and contribute nothing.
//
// One workgroup per (sequence, head); each thread owns four latent features.
// The merge weights are computed once per workgroup into LDS.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxSplitsLds = 1024;

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
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

  const int nvec = p.d_latent / 4;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float w = wts[s];
      if (w == 0.0f) continue;
      const f32x4 x = *(const f32x4*)(p.o_part + (((int64_t)b * S + s) * p.heads + h) * p.d_latent + 4 * v);
      acc += w * x;
    }
    acc *= inv;
    const int64_t o = ((int64_t)b * p.heads + h) * p.d_latent + 4 * v;
    if (p.out_bf16) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[0], acc[1]);
      pk[1] = pack_bf16x2(acc[2], acc[3]);
      *(u32x2*)((__bf16*)p.out + o) = pk;
    } else {
      *(f32x4*)((float*)p.out + o) = acc;
    }
  }
}

}  // namespace

int combine_max_splits() { return kMaxSplitsLds; }

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const int threads = p.d_latent / 4 >= 128 ? 128 : 64;
  hipLaunchKernelGGL(combine_kernel, dim3(p.batch * p.heads), dim3(threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
