// The attention output projection: u[b] = W_O [o[b,1]; ...; o[b,H]].
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.1: the attention
// output of token t is W_O times the concatenation of the heads' outputs;
// section 2.1.2: W_UV can be absorbed into W_O. Folding W_UV into W_O makes
// the weight d x (H d_c), four times larger than W_O at d_c = 512, so the
// library keeps the two products (mla_out_proj / mla_combine_out_proj, then
// this one).
//
// bf16, two kernels:
//  1. skinny_gemm (skinny.h): one workgroup of four waves per (32 output
//     features, 2048-wide contraction part), 160 x 8 = 1280 at d = 5120 and
//     H d_v = 16384; each wave streams its 512-wide range of 32 weight rows
//     and of the 32 rows of o in 128-byte row pieces, puts both into operand
//     order through its LDS buffer, and the four waves' tiles, added in
//     order, go to the caller's workspace as the part's fp32 partial sums;
//  2. oproj_reduce: adds the parts in order (deterministic) and rounds.
// W_O dominates the bytes (168 MB at d = 5120, H d_v = 16384); it is read once
// per 32 batch rows.
// fp32 (tiny shape): one thread per output feature, plain fma.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"
#include "skinny.h"

namespace mla {
namespace {

constexpr int kOpWaves = 4, kOpDepth = 4;   // waves per workgroup, macro steps in flight per wave
constexpr int kOpNa = 2;                    // 16-row weight groups per workgroup
constexpr int kOpKw = 512;                  // contraction features per wave
constexpr int kOpPart = kOpWaves * kOpKw;   // contraction features per workgroup

__host__ __device__ int oproj_parts(int k) { return (k + kOpPart - 1) / kOpPart; }

// out[b][n] = the parts' partial sums added in part order; four outputs a
// thread (n is a multiple of 32), every part's load issued before the sum.
constexpr int kOpMaxParts = 16;
template <bool OUT_F32>
__global__ __launch_bounds__(256) void oproj_reduce(OProjParams p) {
  const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (e >= (int64_t)p.batch * p.n) return;
  const int parts = oproj_parts(p.k);
  const int64_t stride = (int64_t)p.batch * p.n;
  f32x4 v[kOpMaxParts];
#pragma unroll
  for (int s = 0; s < kOpMaxParts; ++s)
    if (s < parts) v[s] = *(const f32x4*)(p.work + s * stride + e);
  f32x4 sum = v[0];
#pragma unroll
  for (int s = 1; s < kOpMaxParts; ++s)
    if (s < parts) sum += v[s];
  for (int s = kOpMaxParts; s < parts; ++s) sum += *(const f32x4*)(p.work + s * stride + e);
  if constexpr (OUT_F32) {
    *(f32x4*)((float*)p.out + e) = sum;
  } else {
    *(u32x2*)((__bf16*)p.out + e) = u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
  }
}

__global__ __launch_bounds__(128) void oproj_f32(OProjParams p) {
  const int b = blockIdx.y, n = blockIdx.x * 128 + threadIdx.x;
  if (n >= p.n) return;
  const float* o = (const float*)p.o + (int64_t)b * p.k;
  const float* w = (const float*)p.w + (int64_t)n * p.k;
  float s = 0.0f;
  for (int k = 0; k < p.k; ++k) s = fmaf(o[k], w[k], s);
  ((float*)p.out)[(int64_t)b * p.n + n] = s;
}

}  // namespace

// bf16: n a multiple of 32, k a multiple of 1024.
bool oproj_bf16_shape_ok(int n, int k) { return n % 32 == 0 && k % 1024 == 0; }

// Workspace: the parts' fp32 partial sums.
int64_t oproj_workspace_bytes(int batch, int n, int k) { return (int64_t)oproj_parts(k) * batch * n * 4; }

hipError_t launch_oproj(const OProjParams& p, bool bf16, bool out_f32, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (!bf16) return launch_kernel(oproj_f32, dim3((p.n + 127) / 128, p.batch), dim3(128), stream, p);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);      // a pending event pair brackets both kernels
  const int parts = oproj_parts(p.k);
  const SkParams g{p.o, p.w, p.w, p.k, p.n, p.batch, p.n, p.k, kOpKw, parts};
  const EpiPartial ep{p.work, p.batch, p.n};
  const dim3 grid0(p.n / (16 * kOpNa) * parts, (p.batch + 31) / 32), block0(64 * kOpWaves);
  hipError_t e =
      parts * kOpPart != p.k
          ? launch_kernel_events(skinny_gemm<kOpWaves, kOpDepth, kOpNa, kXRowLds, true, EpiPartial>, grid0, block0, stream,
                                 e0, nullptr, g, ep)
          : launch_kernel_events(skinny_gemm<kOpWaves, kOpDepth, kOpNa, kXRowLds, false, EpiPartial>, grid0, block0, stream,
                                 e0, nullptr, g, ep);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(((int64_t)p.batch * p.n / 4 + 255) / 256));
  if (out_f32) return launch_kernel_events(oproj_reduce<true>, grid, dim3(256), stream, nullptr, e1, p);
  return launch_kernel_events(oproj_reduce<false>, grid, dim3(256), stream, nullptr, e1, p);
}

}  // namespace mla
