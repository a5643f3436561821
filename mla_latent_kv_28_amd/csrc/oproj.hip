// The attention output projection: u[b] = W_O [o[b,1]; ...; o[b,H]].
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.1: the attention
// output of token t is W_O times the concatenation of the heads' outputs;
// section 2.1.2: W_UV can be absorbed into W_O. Folding W_UV into W_O makes
// the weight d x (H d_c), four times larger than W_O at d_c = 512, so the
// library keeps the two products (mla_out_proj / mla_combine_out_proj, then
// this one).
//
// bf16: one workgroup of 16 waves per (32 output features, 32 batch rows),
// 160 workgroups at d = 5120. K = H d_v goes in batches of 64; wave w takes
// every sixteenth batch, so the waves read neighbouring pieces of the same
// weight rows together, and contracts them with MFMA 32x32x16 on operands
// loaded straight from memory, the next batch requested before the current
// one is multiplied. The 16 partial tiles are added in wave order through
// LDS. W_O dominates the bytes (168 MB at d = 5120, H d_v = 16384) and is
// read once per 32 batch rows.
// fp32 (tiny shape): one thread per output feature, plain fma.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kOpWaves = 16;
constexpr int kOpSteps = 4;   // k-steps of 16 per register buffer

template <bool OUT_F32>
__global__ __launch_bounds__(64 * kOpWaves) void oproj_bf16(OProjParams p) {
  __shared__ float tile[kOpWaves][16][64];   // each wave's 32 x 32 fp32 tile, MFMA lane order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 31, half = lane >> 5;
  const int n = blockIdx.x * 32 + r;         // output feature of this lane's B operand
  const int m = blockIdx.y * 32 + r;         // batch row of this lane's A operand
  // rows past the batch read row 0 instead: an MFMA row only reaches its own
  // output row, and those are not stored
  const __bf16* a_row = (const __bf16*)p.o + (int64_t)(m < p.batch ? m : 0) * p.k + 8 * half;
  const __bf16* b_row = (const __bf16*)p.w + (int64_t)n * p.k + 8 * half;
  f32x16 acc = {};
  // K in batches of kBatch; wave w takes batches w, w + 16, ..., so the 16
  // waves read neighbouring pieces of the same 32 weight rows at a time. Two
  // register buffers: the next batch is requested before the current one is
  // multiplied (each wave has an even number of batches).
  constexpr int kBatch = 16 * kOpSteps;
  const int nb = p.k / (kOpWaves * kBatch);
  auto at = [&](int t) { return (t * kOpWaves + wave) * kBatch; };
  bf16x8 a0[kOpSteps], b0[kOpSteps], a1[kOpSteps], b1[kOpSteps];
  auto load = [&](bf16x8 (&a)[kOpSteps], bf16x8 (&b)[kOpSteps], int k0) {
#pragma unroll
    for (int s = 0; s < kOpSteps; ++s) {
      a[s] = *(const bf16x8*)(a_row + k0 + 16 * s);
      b[s] = *(const bf16x8*)(b_row + k0 + 16 * s);
    }
  };
  auto mul = [&](const bf16x8 (&a)[kOpSteps], const bf16x8 (&b)[kOpSteps]) {
#pragma unroll
    for (int s = 0; s < kOpSteps; ++s) acc = mfma32x32x16(a[s], b[s], acc);
  };
  load(a0, b0, at(0));
  for (int t = 0; t < nb; t += 2) {
    load(a1, b1, at(t + 1));
    __builtin_amdgcn_sched_barrier(0);
    mul(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    load(a0, b0, at(min(t + 2, nb - 1)));   // unconditional: the last pass reloads a batch
    __builtin_amdgcn_sched_barrier(0);
    mul(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) tile[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kOpWaves; ++w) v += tile[w][i][lane];   // wave order: deterministic
    const int row = blockIdx.y * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (row < p.batch) {
      if constexpr (OUT_F32)
        ((float*)p.out)[(int64_t)row * p.n + n] = v;
      else
        ((__bf16*)p.out)[(int64_t)row * p.n + n] = (__bf16)v;
    }
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

// k must be a multiple of 16 waves x 2 batches x 16 x kOpSteps for bf16 (each
// wave an even number of whole batches of k-steps) and n a multiple of 32.
bool oproj_bf16_shape_ok(int n, int k) { return n % 32 == 0 && k % (kOpWaves * 2 * 16 * kOpSteps) == 0; }

hipError_t launch_oproj(const OProjParams& p, bool bf16, bool out_f32, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (!bf16) return launch_kernel(oproj_f32, dim3((p.n + 127) / 128, p.batch), dim3(128), stream, p);
  const dim3 grid(p.n / 32, (p.batch + 31) / 32);
  if (out_f32) return launch_kernel(oproj_bf16<true>, grid, dim3(64 * kOpWaves), stream, p);
  return launch_kernel(oproj_bf16<false>, grid, dim3(64 * kOpWaves), stream, p);
}

}  // namespace mla
