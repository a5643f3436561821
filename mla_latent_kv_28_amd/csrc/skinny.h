// Products with few rows and a large weight, Y[M, N] = X[M, K] W[N, K]^T
// for M <= 32 per row block (one decode token per sequence), bf16 operands
// and fp32 sums: the weight is read once per 32 rows and dominates the bytes,
// so the kernel is a stream of the weight through the vector memory path.
//
// Workgroup of WAVES waves per (16 NA weight rows, contraction part); wave w
// takes a contiguous kw-wide range of the part and walks it in macro steps of
// 64 features, each two 32-wide k steps of v_mfma_f32_16x16x32_bf16 with the
// weight as the A operand (NA groups of 16 rows) and the activations as the B
// operand (two 16-row halves of the batch).
//  - Weights: every load instruction reads 8 whole 128-byte row pieces (1 KiB
//    of consecutive lines per 8 rows); the wave writes them to its own LDS
//    buffer and reads the MFMA fragments back (lane 16 g + c: row c, 16 bytes
//    at k + 8 g). A wave's LDS operations run in order, so the buffer needs
//    no barrier, and one buffer serves every macro step.
//  - Activations: either fragment-major (one 1 KiB load per k step and batch
//    half, laid out by frag_offset below) or row-major, read like the
//    weights into a second region of the wave's buffer.
// The loads of the next D macro steps are in flight while one is multiplied.
// The waves' 2 NA 16x16 tiles are added through LDS in wave order
// (deterministic) and handed to the epilogue: lane (g, c) of tile (na, bb)
// holds Y[16 bb + c][16 na + 4 g + i], i = 0..3 (batch rows from 32 times the
// row block, weight rows from the tile's first).
#pragma once

#include <hip/hip_runtime.h>

#include "mla_device.h"

namespace mla {
namespace {

// Activation layouts of skinny_gemm: fragment-major (frag_offset; one 1 KiB
// load a fragment), or row-major read like the weights (8 rows x 128 bytes a
// load) and put into fragment order through the wave's LDS buffer. (Row-major
// activations read straight into fragments, 16 rows x 64 bytes a load, cost
// far more than their bytes when the rows lie far apart.)
constexpr int kXFrag = 1, kXRowLds = 2;

struct SkParams {
  const void* x;       // kXFrag: fragment-major (frag_offset); kXRowLds: row-major [M][ldx]
  const void* w0;      // weight rows [0, n0), [n0][K] row-major
  const void* w1;      // weight rows [n0, N)
  int32_t ldx;         // row-major activations: elements per row
  int32_t n0, M, N, K;
  int32_t kw;          // contraction features per wave (a multiple of 64 D)
  int32_t kparts;      // contraction parts (workgroups per 16 NA weight rows)
};

// Fragment-major activations: element (b, k) of an [M, K] matrix, with
// b = 32 rb + 16 bb + c and k = 32 t + 8 g + j, sits at element
// (((rb * K / 32 + t) * 2 + bb) * 64 + 16 g + c) * 8 + j, so that the B
// fragment of k step t and batch half bb is one 1 KiB block in lane order.
// Rows are padded to a multiple of 32.
__host__ __device__ __forceinline__ int64_t frag_offset(int b, int k, int K) {
  const int rb = b >> 5, bb = (b >> 4) & 1, c = b & 15, t = k >> 5, g = (k >> 3) & 3, j = k & 7;
  return ((((int64_t)rb * (K / 32) + t) * 2 + bb) * 64 + 16 * g + c) * 8 + j;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_b128(const __amdgpu_buffer_rsrc_t& r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// LDS position (bytes) of 16-byte piece p (0..7) of weight row r in a wave's
// buffer of 128-byte row pieces. Two rows share a 256-byte window of 16 slots;
// the slot is ((r & 1) 8 + p) ^ (r >> 1 & 7), so the 16 rows one fragment read
// touches at one piece, and the 2 rows x 8 pieces one write touches per 16
// lanes, land on 16 distinct slots.
__device__ __forceinline__ int sk_lds_pos(int r, int p) {
  return (r >> 1) * 256 + ((((r & 1) << 3) | p) ^ ((r >> 1) & 7)) * 16;
}

// TAIL: the contraction parts reach past K; the operands of k >= K are zeroed
// (reads past either operand's buffer return zero, and reads inside it are
// discarded). NA: 16-row groups of weight rows per workgroup (2 or 4).
template <int WAVES, int D, int NA, int XL, bool TAIL, class EPI>
__global__ __launch_bounds__(64 * WAVES) void skinny_gemm(SkParams g, EPI epi) {
  constexpr int TILES = 2 * NA;        // 16x16 tiles per wave: (weight group, batch half)
  constexpr int WLD = 2 * NA;          // weight loads per macro step (8 rows each)
  static_assert(WAVES >= 4 && TILES % 4 == 0, "the tiles split evenly over four finishing waves");
  // a wave's weight buffer (and, XL == kXRowLds, its activation rows after
  // the weight rows), then (after its loop) its tiles for the sum
  constexpr int XROWS = XL == kXRowLds ? 32 : 0;
  constexpr int WB = (16 * NA + XROWS) * 128;
  __shared__ __attribute__((aligned(16))) char wbuf[WAVES][WB];
  static_assert(WB >= TILES * 64 * 16, "a wave's tiles fit its buffer");
  const int lane = threadIdx.x & 63, c = lane & 15, grp = lane >> 4;
  auto red = [&](int w, int a) -> MLA_LDS f32x4& { return ((MLA_LDS f32x4*)wbuf[w])[a * 64 + lane]; };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntile = blockIdx.x / g.kparts, kpart = blockIdx.x - ntile * g.kparts;
  const int n0 = 16 * NA * ntile, rb = blockIdx.y;
  const char* wt = n0 < g.n0 ? (const char*)g.w0 + (int64_t)n0 * g.K * 2
                             : (const char*)g.w1 + (int64_t)(n0 - g.n0) * g.K * 2;
  const auto wres = buffer_rsrc(wt, (uint32_t)(16 * NA * g.K * 2));
  // weight load i of a macro step: rows 8 i + lane / 8, piece lane % 8
  const uint32_t wv = (uint32_t)((lane >> 3) * g.K * 2 + 16 * (lane & 7));
  MLA_LDS char* wl = (MLA_LDS char*)wbuf[wave];
  static_assert(XL == kXFrag || XL == kXRowLds, "activation layout");
  __amdgpu_buffer_rsrc_t xres;
  uint32_t xv0 = 0, xvr[4] = {};
  if constexpr (XL == kXFrag) {
    xres = buffer_rsrc(g.x, (uint32_t)((int64_t)(g.M + 31) / 32 * 32 * g.K * 2));
    xv0 = (uint32_t)(rb * (g.K / 32) * 2048 + 16 * lane);   // batch half 1: + 1024
  } else {
    // like the weights: load i reads row 8 i + lane / 8 of the row block
    // (clamped to the batch; rows past it are not stored), piece lane % 8
    xres = buffer_rsrc(g.x, (uint32_t)((int64_t)g.M * g.ldx * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xvr[i] = (uint32_t)(min(32 * rb + 8 * i + (lane >> 3), g.M - 1) * g.ldx * 2 + 16 * (lane & 7));
  }
  const int kbeg = kpart * (g.kw * WAVES) + wave * g.kw;
  const int nm = g.kw / 64;   // macro steps, a multiple of D

  bf16x8 wr[D][WLD], xb[D][2][2];   // [slot][load], [slot][k step][batch half]
  auto load = [&](int m, int j) {
    const int k = kbeg + 64 * m;
#pragma unroll
    for (int i = 0; i < WLD; ++i) wr[j][i] = load_b128(wres, wv + (uint32_t)(8 * i * g.K * 2), (uint32_t)(2 * k));
    if constexpr (XL == kXRowLds) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xb[j][i >> 1][i & 1] = load_b128(xres, xvr[i], (uint32_t)(2 * k));
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t xs = (uint32_t)((k / 32 + t) * 2048);
        xb[j][t][0] = load_b128(xres, xv0, xs);
        xb[j][t][1] = load_b128(xres, xv0 + 1024, xs);
      }
    }
  };
  f32x4 acc[TILES] = {};
  auto mma = [&](int m, int j) {
    // weights (and activation rows) of this macro step through the wave's
    // buffer into fragment order
#pragma unroll
    for (int i = 0; i < WLD; ++i) *(MLA_LDS bf16x8*)(wl + sk_lds_pos(8 * i + (lane >> 3), lane & 7)) = wr[j][i];
    if constexpr (XL == kXRowLds) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(MLA_LDS bf16x8*)(wl + sk_lds_pos(16 * NA + 8 * i + (lane >> 3), lane & 7)) = xb[j][i >> 1][i & 1];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 a[NA];
#pragma unroll
      for (int na = 0; na < NA; ++na) a[na] = *(const MLA_LDS bf16x8*)(wl + sk_lds_pos(16 * na + c, 4 * t + grp));
      bf16x8 b0, b1;
      if constexpr (XL == kXRowLds) {
        b0 = *(const MLA_LDS bf16x8*)(wl + sk_lds_pos(16 * NA + c, 4 * t + grp));
        b1 = *(const MLA_LDS bf16x8*)(wl + sk_lds_pos(16 * NA + 16 + c, 4 * t + grp));
      } else {
        b0 = xb[j][t][0];
        b1 = xb[j][t][1];
      }
      if constexpr (TAIL) {
        if (kbeg + 64 * m + 32 * t + 8 * grp >= g.K) {
          b0 = b1 = bf16x8{};
#pragma unroll
          for (int na = 0; na < NA; ++na) a[na] = bf16x8{};
        }
      }
#pragma unroll
      for (int na = 0; na < NA; ++na) {
        acc[2 * na] = mfma16x16x32(a[na], b0, acc[2 * na]);
        acc[2 * na + 1] = mfma16x16x32(a[na], b1, acc[2 * na + 1]);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) load(j, j);
  int m0 = 0;
  for (; m0 + D < nm; m0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      mma(m0 + j, j);
      load(m0 + j + D, j);
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j) mma(m0 + j, j);

  // the waves' tiles added in wave order; wave w < 4 finishes tiles w, w + 4, ...
#pragma unroll
  for (int a = 0; a < TILES; ++a) red(wave, a) = acc[a];
  __syncthreads();
  if (wave >= 4) return;
#pragma unroll
  for (int a = wave; a < TILES; a += 4) {
    f32x4 v = red(0, a);
#pragma unroll
    for (int u = 1; u < WAVES; ++u) {
      const f32x4 o = red(u, a);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += o[i];
    }
    const int b = 32 * rb + 16 * (a & 1) + c;
    const int n = n0 + 16 * (a >> 1) + 4 * grp;
    epi(b, n, kpart, v);
  }
}

// Partial sums of one contraction part: out[kpart][b][n] (fp32).
struct EpiPartial {
  float* out;
  int32_t M, N;
  __device__ __forceinline__ void operator()(int b, int n, int kpart, const f32x4& v) const {
    if (b < M) *(f32x4*)(out + ((int64_t)kpart * M + b) * N + n) = v;
  }
};

}  // namespace
}  // namespace mla
