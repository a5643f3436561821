// Log-sum-exp merge of split-KV partials.
//
// Each split s of a sequence produced o_s (softmax-normalised over its own
// tokens) and lse_s = log sum exp(scores) over those tokens. Attention over
// the union is   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
// Splits with no tokens carry lse_s = -inf and contribute nothing.
//
// One wave per (sequence, head), four heads per workgroup. Each lane owns
// 16-byte vectors of latent features (4 fp32 or 8 bf16 partial values).
// Splits are taken 64 at a time: lane l holds the LSE and merge weight of
// split 64g + l, and the weights reach the other lanes by v_readlane (scalar
// registers), so no LDS and no barrier. The first eight splits' vectors are
// requested before the LSEs, so both round trips overlap; loads use clamped
// (always valid) addresses instead of branches and surplus slots weigh 0.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxSplits = 1024;
constexpr int kWaves = 4;     // heads per workgroup
constexpr int kChunk = 8;     // split vectors in flight per lane

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

__device__ __forceinline__ float lane_value(float v, int l) {   // l uniform
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {   // in-row lane permutation (every source lane valid)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Wave-wide reductions on the vector unit: within each row of 16 lanes by
// DPP (swap neighbours, swap pairs, mirror halves, mirror the row), then the
// four rows through v_readlane.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp<0xb1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4e>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp<0x141>(v));   // row_half_mirror
  v = op(v, dpp<0x140>(v));   // row_mirror
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

template <bool PART_BF16>
__global__ __launch_bounds__(64 * kWaves) void combine_kernel(CombineParams p) {
  using V = PartVec<PART_BF16>;
  constexpr int ESZ = PART_BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (bh >= p.batch * p.heads) return;           // whole waves
  const int b = bh / p.heads, h = bh % p.heads;
  const int S = p.splits;
  const int nvec = p.d_latent / V::N;
  const int64_t split_stride = (int64_t)p.heads * p.d_latent * ESZ;
  const char* part = (const char*)p.o_part + ((int64_t)b * S * p.heads + h) * p.d_latent * ESZ;
  const float* lse_p = p.lse_part + (int64_t)b * S * p.heads + h;       // split stride: heads
  const int vl = min(lane, nvec - 1);            // lanes past the features repeat the last vector

  // LSEs of the first 64 splits, then the first vectors: waiting for the
  // LSEs (an older load) leaves the vectors in flight
  const float lse0 = lane < S ? lse_p[(int64_t)lane * p.heads] : -INFINITY;
  u32x4 first[kChunk];
#pragma unroll
  for (int i = 0; i < kChunk; ++i) first[i] = load16(part + min(i, S - 1) * split_stride + vl * 16);

  // maximum LSE over all splits
  float m = lse0;
  for (int g = 64; g < S; g += 64) m = fmaxf(m, g + lane < S ? lse_p[(int64_t)(g + lane) * p.heads] : -INFINITY);
  m = wave_max(m);
  const bool empty = (m == -INFINITY);

  for (int v0 = 0; v0 < nvec; v0 += 64) {     // uniform trip count: the wave-wide steps need every lane
    const int v = v0 + lane;
    const bool own = v < nvec;
    const char* src = part + min(v, nvec - 1) * 16;
    float acc[V::N];
#pragma unroll
    for (int e = 0; e < V::N; ++e) acc[e] = 0.0f;
    float z = 0.0f;
    for (int g = 0; g < S; g += 64) {
      const float l = g == 0 ? lse0 : g + lane < S ? lse_p[(int64_t)(g + lane) * p.heads] : -INFINITY;
      const float w = (empty || l == -INFINITY) ? 0.0f : fast_exp2((l - m) * kLog2e);
      z += wave_sum(w);
      const int n = min(64, S - g);
      for (int s0 = 0; s0 < n; s0 += kChunk) {
        u32x4 x[kChunk];
        if (g == 0 && s0 == 0 && v0 == 0) {
#pragma unroll
          for (int i = 0; i < kChunk; ++i) x[i] = first[i];
        } else {
#pragma unroll
          for (int i = 0; i < kChunk; ++i) x[i] = load16(src + min(g + s0 + i, S - 1) * split_stride);
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          // a split with weight 0 (empty, or past S) is skipped element-wise,
          // so whatever it holds cannot reach the sum
          const float wi = s0 + i < n ? lane_value(w, s0 + i) : 0.0f;
          float xv[V::N];
          V::unpack(x[i], xv);
#pragma unroll
          for (int e = 0; e < V::N; ++e) acc[e] += wi == 0.0f ? 0.0f : wi * xv[e];
        }
      }
    }
    const float inv = empty ? 0.0f : 1.0f / z;
    if (v0 == 0 && lane == 0 && p.lse != nullptr)
      p.lse[(int64_t)b * p.heads + h] = empty ? -INFINITY : m + fast_log2(z) * kLn2;
    if (!own) continue;
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

int combine_max_splits() { return kMaxSplits; }

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const int waves = p.batch * p.heads;
  const dim3 grid((waves + kWaves - 1) / kWaves);
  if (p.part_bf16) return launch_kernel(combine_kernel<true>, grid, dim3(64 * kWaves), s, p);
  return launch_kernel(combine_kernel<false>, grid, dim3(64 * kWaves), s, p);
}

}  // namespace mla
