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
//  1. oproj_partial: one workgroup of 5 waves per (160 output features,
//     1024-wide K slice, 32 batch rows), 512 at d = 5120 and B <= 32 (8, 4 or
//     1 waves where 160 does not divide the features). Wave w streams the
//     slice of its 32 weight rows through three register buffers of eight
//     k-steps (two in flight while one is multiplied), while the slice of o
//     sits in LDS (rows padded against bank
//     conflicts); MFMA 32x32x16; the fp32 tile goes to slice s of the caller's
//     workspace. All the register space holds weights, which come from HBM.
//  2. oproj_reduce: adds the slices in order (deterministic) and rounds.
// W_O dominates the bytes (168 MB at d = 5120, H d_v = 16384); it is read once
// per 32 batch rows.
// fp32 (tiny shape): one thread per output feature, plain fma.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kOpSlice = 1024;  // K per workgroup
constexpr int kOpSteps = 8;     // k-steps of 16 per register buffer
constexpr int kOpRow = kOpSlice + 8;   // LDS row of o (elements), padded against bank conflicts

// Partial sums of one K slice: work[slice][b][n].
// WAVES waves per workgroup, 32 output features each.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void oproj_partial(OProjParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 o_lds[32 * kOpRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 31, half = lane >> 5;
  const int k0 = blockIdx.y * kOpSlice, b0 = blockIdx.z * 32;
  const int n = blockIdx.x * (32 * WAVES) + wave * 32 + r;   // output feature of this lane's B operand
  const __bf16* b_row = (const __bf16*)p.w + (int64_t)n * p.k + k0 + 8 * half;
  f32x16 acc = {};
  constexpr int kBatches = kOpSlice / 16 / kOpSteps;
  // three register buffers: two batches of weights stay in flight while one is
  // multiplied (the loop is unrolled, so every buffer index is a constant)
  bf16x8 w[3][kOpSteps];
  auto load = [&](bf16x8 (&u)[kOpSteps], int s0) {
#pragma unroll
    for (int s = 0; s < kOpSteps; ++s) u[s] = *(const bf16x8*)(b_row + 16 * (s0 + s));
  };
  load(w[0], 0);                     // the weights first: they come from HBM
  load(w[1], kOpSteps);
  // the slice of o (32 batch rows x kOpSlice) into LDS; rows past the batch are zero
  for (int e = threadIdx.x; e < 32 * kOpSlice / 8; e += 64 * WAVES) {
    const int row = e / (kOpSlice / 8), c = (e % (kOpSlice / 8)) * 8;
    const bf16x8 v = b0 + row < p.batch ? *(const bf16x8*)((const __bf16*)p.o + (int64_t)(b0 + row) * p.k + k0 + c)
                                        : bf16x8{};
    *(bf16x8*)(o_lds + row * kOpRow + c) = v;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kBatches; ++t) {
    if (t + 2 < kBatches) load(w[(t + 2) % 3], (t + 2) * kOpSteps);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kOpSteps; ++s) {
      const bf16x8 a = *(const bf16x8*)(o_lds + r * kOpRow + 16 * (t * kOpSteps + s) + 8 * half);
      acc = mfma32x32x16(a, w[t % 3][s], acc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float* out = p.work + (int64_t)blockIdx.y * p.batch * p.n;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = b0 + 8 * (i >> 2) + 4 * half + (i & 3);   // D[row][col], col = lane % 32
    if (row < p.batch) out[(int64_t)row * p.n + n] = acc[i];
  }
}

// out[b][n] = the slices' partial sums added in slice order.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void oproj_reduce(OProjParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)p.batch * p.n) return;
  const int slices = p.k / kOpSlice;
  const int64_t stride = (int64_t)p.batch * p.n;
  float v[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) v[s] = s < slices ? p.work[s * stride + e] : 0.0f;   // loads together
  float sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 16; ++s) sum += v[s];
  for (int s = 16; s < slices; ++s) sum += p.work[s * stride + e];
  if constexpr (OUT_F32)
    ((float*)p.out)[e] = sum;
  else
    ((__bf16*)p.out)[e] = (__bf16)sum;
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

// bf16: n a multiple of 32, k a multiple of kOpSlice.
bool oproj_bf16_shape_ok(int n, int k) { return n % 32 == 0 && k % kOpSlice == 0; }

int64_t oproj_workspace_bytes(int batch, int n, int k) { return (int64_t)(k / kOpSlice) * batch * n * 4; }

hipError_t launch_oproj(const OProjParams& p, bool bf16, bool out_f32, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (!bf16) return launch_kernel(oproj_f32, dim3((p.n + 127) / 128, p.batch), dim3(128), stream, p);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);      // a pending event pair brackets both kernels
  // Workgroups of 5 waves (160 features) where they divide the features:
  // at d = 5120 that makes 32 x 16 = 512 workgroups, two per compute unit in
  // one round (8-wave workgroups left 64 units with two of 320); else 8, 4 or 1.
  const dim3 g0(0, p.k / kOpSlice, (p.batch + 31) / 32);
  hipError_t e;
  if (p.n % 160 == 0)
    e = launch_kernel_events(oproj_partial<5>, dim3(p.n / 160, g0.y, g0.z), dim3(320), stream, e0, nullptr, p);
  else if (p.n % 256 == 0)
    e = launch_kernel_events(oproj_partial<8>, dim3(p.n / 256, g0.y, g0.z), dim3(512), stream, e0, nullptr, p);
  else if (p.n % 128 == 0)
    e = launch_kernel_events(oproj_partial<4>, dim3(p.n / 128, g0.y, g0.z), dim3(256), stream, e0, nullptr, p);
  else
    e = launch_kernel_events(oproj_partial<1>, dim3(p.n / 32, g0.y, g0.z), dim3(64), stream, e0, nullptr, p);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(((int64_t)p.batch * p.n + 255) / 256));
  if (out_f32) return launch_kernel_events(oproj_reduce<true>, grid, dim3(256), stream, nullptr, e1, p);
  return launch_kernel_events(oproj_reduce<false>, grid, dim3(256), stream, nullptr, e1, p);
}

}  // namespace mla
