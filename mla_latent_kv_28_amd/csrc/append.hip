// The cache entry of one new token per sequence.
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.2: the cached latent is
// the down-projection c_KV = W_DKV h of the token's hidden state; section
// 2.1.3: the shared rotary key is k_R = RoPE(W_KR h) at the token's position;
// section 3.1.2 (model hyper-parameters): an RMS norm follows the compressed
// latent. Norm: x / sqrt(mean(x^2) + eps), times an optional gain. Rotation:
// pairs (2i, 2i + 1) turned by position * f_i, the frequencies (plain RoPE or
// YaRN, section 3.1.4) computed on the host.
//
// Two kernels:
//  1. the projection [B, d] x [d, d_c + d_R] into fp32 partial sums
//     work[part][b][n]: bf16, skinny_gemm (skinny.h) over [W_DKV; W_KR] in
//     1024-wide contraction parts (four waves of 256 each, weights and hidden
//     states in 128-byte row pieces through each wave's LDS buffer); fp32
//     (tiny shape), append_project_f32 in 256-wide slices, one thread per
//     output column, plain fma. The weights are read once per 32 batch rows;
//     they dominate the bytes.
//  2. append_finish: one workgroup per sequence sums the slices in a fixed
//     order, applies the norm and the rotation in fp32 (angles in fp64), and
//     writes the row
//     of its position: bf16 or fp32 [c_KV ; k_R], or e4m3 codes of c_KV with a
//     per-token scale absmax / 448 and the rotary key in bf16.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "mla_device.h"
#include "mla_internal.h"
#include "skinny.h"

namespace mla {
namespace {

constexpr int kSlice = 256;   // hidden features per partial sum (fp32 projection)
constexpr int kApWaves = 4, kApDepth = 4, kApKw = 256;   // bf16 projection: 1024-wide parts

typedef short i16x2 __attribute__((ext_vector_type(2)));

// ---- 1. projection -------------------------------------------------------------

__global__ __launch_bounds__(64) void append_project_f32(AppendParams p) {
  const int N = p.d_latent + p.d_rope;
  const int b = blockIdx.z, k0 = blockIdx.y * kSlice, k1 = min(k0 + kSlice, p.hidden);
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const float* w = n < p.d_latent ? (const float*)p.w_dkv + (int64_t)n * p.hidden
                                  : (const float*)p.w_kr + (int64_t)(n - p.d_latent) * p.hidden;
  const float* h = (const float*)p.h + (int64_t)b * p.hidden;
  float s = 0.0f;
  for (int k = k0; k < k1; ++k) s = fmaf(h[k], w[k], s);
  p.work[((int64_t)blockIdx.y * p.batch + b) * N + n] = s;
}

// ---- 2. norm, rotation, store ----------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

// Cache row of position pos of sequence b, or -1 outside the cache.
__device__ __forceinline__ int64_t entry_row(const AppendParams& p, int b, int pos) {
  if (pos < 0) return -1;
  if (p.page_shift < 0) return pos < p.seq_stride ? (int64_t)b * p.seq_stride + pos : -1;
  const int lp = pos >> p.page_shift;
  if (lp >= p.max_pages) return -1;
  const int64_t page = p.block_table[(int64_t)b * p.max_pages + lp];
  return (page << p.page_shift) + (pos & ((1 << p.page_shift) - 1));
}

// DC latent features, DR rotary ones; lanes own PER consecutive latent
// features. Four waves sum every fourth slice each (their loads go out
// together); wave 0 adds the four sums in wave order and finishes the row.
constexpr int kFinishWaves = 4;

template <int DC, int DR, int KIND>
__global__ __launch_bounds__(64 * kFinishWaves) void append_finish(AppendParams p) {
  static_assert(DR <= 64 && DR % 2 == 0 && DR / 2 <= kMaxRopePairs, "one rotary feature per lane");
  constexpr int PER = DC >= 64 ? DC / 64 : 1;
  static_assert(DC >= 64 ? DC % 64 == 0 : true, "latent width");
  __shared__ float red[kFinishWaves - 1][PER + 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, b = blockIdx.x;
  const int N = DC + DR;
  const int pos = p.positions[b];
  const bool lat_ok = DC >= 64 || lane < DC;
  const int c0 = DC >= 64 ? lane * PER : lane;
  const float* part = p.work + (int64_t)b * N;
  const int64_t slice_stride = (int64_t)p.batch * N;

  float x[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) x[j] = 0.0f;
  float kr = 0.0f;
  // this wave's slices in order; the loads of U of them go out together
  constexpr int U = 8;
  for (int t0 = 0; wave + kFinishWaves * t0 < p.ksplits; t0 += U) {
    float v[U][PER], vk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = min(wave + kFinishWaves * (t0 + u), p.ksplits - 1);
      const float* ps = part + (int64_t)sl * slice_stride;
      if constexpr (PER % 4 == 0) {
#pragma unroll
        for (int j = 0; j < PER; j += 4) {
          const f32x4 t = *(const f32x4*)(ps + c0 + j);
          v[u][j] = t[0], v[u][j + 1] = t[1], v[u][j + 2] = t[2], v[u][j + 3] = t[3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) v[u][j] = lat_ok ? ps[c0 + j] : 0.0f;
      }
      vk[u] = lane < DR ? ps[DC + lane] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wave + kFinishWaves * (t0 + u) < p.ksplits) {
#pragma unroll
        for (int j = 0; j < PER; ++j) x[j] += v[u][j];
        kr += vk[u];
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) red[wave - 1][j][lane] = x[j];
    red[wave - 1][PER][lane] = kr;
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kFinishWaves - 1; ++w) {
#pragma unroll
    for (int j = 0; j < PER; ++j) x[j] += red[w][j][lane];
    kr += red[w][PER][lane];
  }
  const int64_t row = entry_row(p, b, pos);
  if (row < 0) return;                                  // outside the cache: nothing written
  // RMS norm of the latent
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < PER; ++j) ss += lat_ok ? x[j] * x[j] : 0.0f;
  const float inv = 1.0f / sqrtf(wave_sum(ss) / DC + p.eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    float g = 1.0f;
    if (p.gain != nullptr && lat_ok)
      g = KIND == kF32 ? ((const float*)p.gain)[c0 + j] : (float)((const __bf16*)p.gain)[c0 + j];
    x[j] = x[j] * inv * g;
  }
  // rotation of the pair (2i, 2i + 1), angle in fp64
  const float other = __shfl_xor(kr, 1);
  float k_out = 0.0f;
  if (lane < DR) {
    const int i = lane >> 1;
    const double ang = (double)pos * p.freq[i];
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x0 = (lane & 1) ? other : kr, x1 = (lane & 1) ? kr : other;
    k_out = (float)((lane & 1) ? x0 * sn + x1 * cs : x0 * cs - x1 * sn);
  }

  if constexpr (KIND == kF32) {
    float* dst = (float*)p.latent + row * p.row_stride;
    if (lat_ok) {
#pragma unroll
      for (int j = 0; j < PER; ++j) dst[c0 + j] = x[j];
    }
    if (lane < DR) dst[DC + lane] = k_out;
  } else if constexpr (KIND == kBF16) {
    static_assert(PER == 8, "16-byte row pieces");
    __bf16* dst = (__bf16*)p.latent + row * p.row_stride;
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    *(u32x4*)(dst + c0) = v;
    if (lane < DR) dst[DC + lane] = (__bf16)k_out;
  } else {
    static_assert(PER == 8, "8-byte code pieces");
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = wave_max(amax);
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    float y[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) y[j] = fminf(fmaxf(x[j] / scale, -448.0f), 448.0f);   // keeps codes finite
    // OCP e4m3, round to nearest even (scale operand 1); two codes per call,
    // into the low or the high half of a 32-bit word
    i16x2 w0 = {0, 0}, w1 = {0, 0};
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, y[0], y[1], 1.0f, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, y[2], y[3], 1.0f, true);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, y[4], y[5], 1.0f, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, y[6], y[7], 1.0f, true);
    *(u32x2*)((uint8_t*)p.latent + row * p.row_stride + c0) =
        u32x2{__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1)};
    if (lane == 0) p.scale[row] = scale;
    if (lane < DR) ((__bf16*)p.rope)[row * p.rope_stride + lane] = (__bf16)k_out;
  }
}

}  // namespace

int append_slices(int hidden, bool dsv2) {
  const int part = dsv2 ? kApWaves * kApKw : kSlice;
  return (hidden + part - 1) / part;
}

// Scratch of the allocation-free entry point: the fp32 partial sums that
// mla_cache_append keeps in the caller's workspace, here in a device array of
// the library's own (one copy on each GPU the library runs on, held until the
// process ends). Every element a call reads was written by that call's
// projection, so nothing needs clearing between calls.
constexpr int64_t kAppendScratchBytes = int64_t{8} << 20;
static __device__ __align__(256) float scratch[kAppendScratchBytes / sizeof(float)];

int64_t append_scratch_bytes() { return kAppendScratchBytes; }

// Device address of the current GPU's copy of `scratch`, resolved with
// hipGetSymbolAddress the first time a device asks (with that device current)
// and kept per device. Host code passes this address to kernels, never the
// array's name (which on the host is only a stand-in).
hipError_t append_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* ptr = addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (q == nullptr) return hipErrorInvalidSymbol;
    ptr = static_cast<float*>(q);
    addr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

// A pending event pair (mla_time_next_launch) brackets both kernels: the
// start event goes with the projection, the stop event with the finish.
hipError_t launch_cache_append(const AppendParams& p, bool dsv2, int cache_kind, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  const int N = p.d_latent + p.d_rope;
  hipError_t e;
  if (dsv2) {
    const SkParams g{p.h, p.w_dkv, p.w_kr, p.hidden, p.d_latent, p.batch, N, p.hidden, kApKw, p.ksplits};
    const EpiPartial ep{p.work, p.batch, N};
    const dim3 grid(N / 32 * p.ksplits, (p.batch + 31) / 32), block(64 * kApWaves);
    e = p.ksplits * kApWaves * kApKw != p.hidden
            ? launch_kernel_events(skinny_gemm<kApWaves, kApDepth, 2, kXRowLds, true, EpiPartial>, grid, block,
                                   stream, e0, nullptr, g, ep)
            : launch_kernel_events(skinny_gemm<kApWaves, kApDepth, 2, kXRowLds, false, EpiPartial>, grid, block,
                                   stream, e0, nullptr, g, ep);
    if (e != hipSuccess) return e;
    if (cache_kind == kFP8)
      return launch_kernel_events((append_finish<512, 64, kFP8>), dim3(p.batch), dim3(64 * kFinishWaves), stream,
                                  nullptr, e1, p);
    return launch_kernel_events((append_finish<512, 64, kBF16>), dim3(p.batch), dim3(64 * kFinishWaves), stream,
                                nullptr, e1, p);
  }
  e = launch_kernel_events(append_project_f32, dim3((N + 63) / 64, p.ksplits, p.batch), dim3(64), stream, e0,
                           nullptr, p);
  if (e != hipSuccess) return e;
  return launch_kernel_events((append_finish<32, 16, kF32>), dim3(p.batch), dim3(64 * kFinishWaves), stream, nullptr,
                              e1, p);
}

}  // namespace mla
