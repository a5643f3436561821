// Per-head batched projections on MFMA: the two absorbed weight products of
// MLA decode (DeepSeek-V2 paper, Chinese translation, section 2.1.2: W_UK is
// folded into the query side and W_UV into the output side).
//   absorb:   q_lat[b,h,n] = sum_k q_nope[b,h,k] * W_UK[h,k,n]   (W stored [K][N])
//   out-proj: o[b,h,n]     = sum_k o_lat[b,h,k]  * W_UV[h,n,k]   (W stored [N][K])
// For every head this is a (batch x K) . (K x N) product with a small batch:
// the time goes into reading the weights (16.8 MB per call at the
// DeepSeek-V2 shapes), so the bf16 kernels spread each head's weights over a
// 256-thread workgroup whose four waves split K, issue all their weight loads
// at once, keep the weight fragments in registers while they loop over
// 32-row batch blocks, and add their K-partials through LDS.
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

// ---- bf16 absorb: W [K=128][N=512] per head, one workgroup per (head, 256 columns)
constexpr int kAbsK = 128, kAbsN = 512, kAbsNT = 256;

__global__ __launch_bounds__(256, 1) void absorb_bf16_kernel(GemmParams p) {
  // K-partials of the four waves: [wave][i][lane][m] fp32, m = fragment
  __shared__ __attribute__((aligned(16))) float part[4 * 16 * 64 * 8];
  const int h = blockIdx.x, n0 = blockIdx.y * kAbsNT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  constexpr int KCW = kAbsK / 16 / 4;                     // 16-wide k blocks per wave (2)
  constexpr int TAIL_CH = 64 / 8;                         // 16-byte chunks of a 64-wide rotary row
  const bool do_tail = blockIdx.y == 0 && p.tail != nullptr;

  // Everything the first batch block needs is requested up front, in one
  // round trip: the weights, this wave's query rows and the rotary rows.
  u32x4 raw[KCW][8];
  const __bf16* wh = (const __bf16*)p.w + (int64_t)h * kAbsK * kAbsN;
#pragma unroll
  for (int q = 0; q < KCW; ++q) {
    const int k0 = 16 * (wave * KCW + q) + 8 * hh;
#pragma unroll
    for (int e = 0; e < 8; ++e) raw[q][e] = load16(wh + (int64_t)(k0 + e) * kAbsN + n0 + 8 * r);
  }
  auto load_a = [&](int b0, bf16x8 (&a)[KCW]) {
    const int brow = b0 + r;
    const bool ok = brow < p.batch;
    const __bf16* arow = (const __bf16*)p.a + ((int64_t)(ok ? brow : 0) * p.heads + h) * p.lda;
#pragma unroll
    for (int q = 0; q < KCW; ++q) {
      a[q] = *(const bf16x8*)(arow + 16 * (wave * KCW + q) + 8 * hh);
      if (!ok) a[q] = bf16x8{};
    }
  };
  // rotary rows: one 16-byte chunk per thread (32 rows x 8 chunks)
  auto load_tail = [&](int b0) -> u32x4 {
    const int row = min(b0 + tid / TAIL_CH, p.batch - 1);
    return load16((const __bf16*)p.tail + ((int64_t)row * p.heads + h) * 64 + 8 * (tid % TAIL_CH));
  };
  bf16x8 a_next[KCW];
  load_a(0, a_next);
  u32x4 tail_next = do_tail ? load_tail(0) : u32x4{};

  bf16x8 wf[KCW][8];
#pragma unroll
  for (int q = 0; q < KCW; ++q)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      u32x4 f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        f[d] = (m & 1) ? pack_hi16(raw[q][2 * d][m >> 1], raw[q][2 * d + 1][m >> 1])
                       : pack_lo16(raw[q][2 * d][m >> 1], raw[q][2 * d + 1][m >> 1]);
      wf[q][m] = __builtin_bit_cast(bf16x8, f);
    }

  for (int b0 = 0; b0 < p.batch; b0 += 32) {
    bf16x8 a[KCW];
#pragma unroll
    for (int q = 0; q < KCW; ++q) a[q] = a_next[q];
    const u32x4 tail = tail_next;
    if (b0 + 32 < p.batch) {          // the next block's rows go out before this block's math
      load_a(b0 + 32, a_next);
      if (do_tail) tail_next = load_tail(b0 + 32);
    }
    f32x16 acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = f32x16{};
#pragma unroll
    for (int q = 0; q < KCW; ++q)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = mfma32x32x16(a[q], wf[q][m], acc[m]);
    // accumulator i of lane (hh, c): row 8(i/4) + 4hh + i%4, columns n0 + 8c + m
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float* dst = part + ((wave * 16 + i) * 64 + lane) * 8;
      *(f32x4*)dst = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *(f32x4*)(dst + 4) = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
    __syncthreads();
    // each thread sums four (i, lane) pairs over the waves: eight consecutive
    // columns of one row, one 16-byte store
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pr = k * 256 + tid, i = pr >> 6, ln = pr & 63;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* src = part + ((w * 16 + i) * 64 + ln) * 8;
        const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] += x0[e]; v[4 + e] += x1[e]; }
      }
      const int row = b0 + 8 * (i >> 2) + 4 * (ln >> 5) + (i & 3);
      if (row < p.batch) {
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(v[2 * d], v[2 * d + 1]);
        *(u32x4*)((__bf16*)p.c + ((int64_t)row * p.heads + h) * p.ldc + n0 + 8 * (ln & 31)) = o;
      }
    }
    // the rotary query goes after the latent part
    if (do_tail) {
      const int row = b0 + tid / TAIL_CH;
      if (row < p.batch)
        *(u32x4*)((__bf16*)p.c + ((int64_t)row * p.heads + h) * p.ldc + kAbsN + 8 * (tid % TAIL_CH)) = tail;
    }
    __syncthreads();
  }
}

// ---- bf16 out-proj: W [N=128][K=512] per head, one workgroup per (head, 32 columns)
constexpr int kOutK = 512, kOutN = 128, kOutNT = 32;

template <bool A_F32>
__global__ __launch_bounds__(256, 2) void outproj_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) float part[4 * 64 * 16];   // [wave][lane][i]
  const int h = blockIdx.x, n0 = blockIdx.y * kOutNT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  constexpr int KCW = kOutK / 16 / 4;                     // 16-wide k blocks per wave (8)

  // B fragments: W[n0 + r][k .. k + 7] is contiguous
  bf16x8 wf[KCW];
  const __bf16* wrow = (const __bf16*)p.w + ((int64_t)h * kOutN + n0 + r) * kOutK;
#pragma unroll
  for (int q = 0; q < KCW; ++q) wf[q] = *(const bf16x8*)(wrow + 16 * (wave * KCW + q) + 8 * hh);

  for (int b0 = 0; b0 < p.batch; b0 += 32) {
    const int brow = b0 + r;
    const bool ok = brow < p.batch;
    const int64_t aoff = ((int64_t)(ok ? brow : 0) * p.heads + h) * p.lda;
    bf16x8 a[KCW];
#pragma unroll
    for (int q = 0; q < KCW; ++q) {
      const int k0 = 16 * (wave * KCW + q) + 8 * hh;
      a[q] = load_a_bf16((const char*)p.a + aoff * (A_F32 ? 4 : 2), k0, ok, A_F32);
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int q = 0; q < KCW; ++q) acc = mfma32x32x16(a[q], wf[q], acc);
    float* dst = part + (wave * 64 + lane) * 16;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(dst + 4 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    __syncthreads();
    // thread t: row t / 8 of the block, columns n0 + 4 (t % 8) .. + 3
    {
      const int rr = tid >> 3, c0 = 4 * (tid & 7);
      const int i = 4 * (rr >> 3) + (rr & 3), hh2 = (rr >> 2) & 1;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += part[(w * 64 + 32 * hh2 + c0 + e) * 16 + i];
      const int row = b0 + rr;
      if (row < p.batch) {
        const int64_t o = ((int64_t)row * p.heads + h) * p.ldc + n0 + c0;
        if (p.c_f32) {
          *(f32x4*)((float*)p.c + o) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          u32x2 pk;
          pk[0] = pack_bf16x2(v[0], v[1]);
          pk[1] = pack_bf16x2(v[2], v[3]);
          *(u32x2*)((__bf16*)p.c + o) = pk;
        }
      }
    }
    __syncthreads();
  }
}

// ---- split merge + out-proj in one pass: W [N=128][K=512] per head, bf16
// partials, at most kCoMaxSplits splits. One 512-thread workgroup per (head,
// 64 columns), per 32-row batch block:
//   1. merge weights e^(lse_s - max) / z per (row, split) into LDS;
//   2. the merge: wave w takes rows w, w + 8, w + 16, w + 24, each wave
//      instruction reading one split's whole 1 KiB row (64 lanes x 16 bytes),
//      so the weights are wave-uniform; fp32 sums, times 1/z, rounded to
//      bf16 (the values a bf16 mla_combine output would hold) and stored to
//      LDS with 16-byte chunks XOR-swizzled by the row;
//   3. wave w reads its k range (64w .. 64w + 63) of all 32 rows as MFMA A
//      fragments, multiplies by W_UV and the eight K-partials are added
//      through LDS.
// The merged latent rows never go to memory.
constexpr int kCoK = 512, kCoN = 128, kCoNT = 64, kCoWaves = 8, kCoMaxSplits = 64;

template <bool OUT_F32>
__global__ __launch_bounds__(64 * kCoWaves, 1) void combine_outproj_kernel(CombineOutParams p) {
  __shared__ __attribute__((aligned(16))) float part[kCoWaves * 64 * 32];   // [wave][lane][fragment][16]
  __shared__ __attribute__((aligned(16))) uint16_t olat[32 * kCoK];         // merged rows, bf16, swizzled
  __shared__ float wts[32 * kCoMaxSplits];                                  // [row][split]
  __shared__ float inv_z[32];
  const int h = blockIdx.x, n0 = blockIdx.y * kCoNT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  constexpr int KCW = kCoK / 16 / kCoWaves;               // 16-wide k blocks per wave (4)
  const int S = p.splits, H = p.heads;
  const int kw = 16 * KCW * wave + 8 * hh;                // this lane's first k in the products

  // W_UV fragments of the two 32-column fragments: W[h][n0 + 32f + r][kw + 16q ..]
  bf16x8 wf[2][KCW];
  {
    const __bf16* wrow = (const __bf16*)p.w + ((int64_t)h * kCoN + n0 + r) * kCoK + kw;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < KCW; ++q) wf[f][q] = *(const bf16x8*)(wrow + (int64_t)32 * f * kCoK + 16 * q);
  }
  const int64_t split_stride = (int64_t)H * kCoK * 2;      // bytes between two splits of one (b, h)
  const int64_t row_stride = (int64_t)S * split_stride;    // bytes between two batch rows

  for (int b0 = 0; b0 < p.batch; b0 += 32) {
    // 1. merge weights: thread (row = tid / 16, lane group s16 = tid % 16)
    //    takes splits s16, s16 + 16, ...
    {
      const int row = tid >> 4, s16 = tid & 15;
      const int b = min(b0 + row, p.batch - 1);
      const float* lse_row = p.lse_part + (int64_t)b * S * H + h;
      float l[kCoMaxSplits / 16];
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < kCoMaxSplits / 16; ++k) {
        const int sp = s16 + 16 * k;
        l[k] = sp < S ? lse_row[(int64_t)sp * H] : -INFINITY;
        m = fmaxf(m, l[k]);
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const bool empty = (m == -INFINITY);
      float z = 0.0f;
#pragma unroll
      for (int k = 0; k < kCoMaxSplits / 16; ++k) {
        const int sp = s16 + 16 * k;
        const float w = (empty || l[k] == -INFINITY) ? 0.0f : fast_exp2((l[k] - m) * kLog2e);
        if (sp < S) wts[row * kCoMaxSplits + sp] = w;
        z += w;
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) z += __shfl_xor(z, off);
      if (s16 == 0) {
        inv_z[row] = empty ? 0.0f : 1.0f / z;
        if (blockIdx.y == 0 && b0 + row < p.batch && p.lse != nullptr)
          p.lse[(int64_t)(b0 + row) * H + h] = empty ? -INFINITY : m + fast_log2(z) * kLn2;
      }
    }
    __syncthreads();

    // 2. merge: wave w, rows w + 8j; lane = 16-byte chunk of the row
    {
      const char* base = (const char*)p.o_part + (int64_t)h * kCoK * 2 + lane * 16;
      float acc[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
      constexpr int SC = 4;                                // splits in flight
      for (int s0 = 0; s0 < S; s0 += SC) {
        u32x4 x[SC][4];
#pragma unroll
        for (int i = 0; i < SC; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = min(b0 + wave + 8 * j, p.batch - 1);
            x[i][j] = load16(base + b * row_stride + min(s0 + i, S - 1) * split_stride);
          }
#pragma unroll
        for (int i = 0; i < SC; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // a split with weight 0 (empty, or past S) has its words zeroed,
            // so whatever it holds cannot reach the sum
            const float w = s0 + i < S ? wts[(wave + 8 * j) * kCoMaxSplits + s0 + i] : 0.0f;
            const bool skip = (w == 0.0f);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t v = skip ? 0u : (uint32_t)x[i][j][d];
              acc[j][2 * d] = fmaf(w, __builtin_bit_cast(float, v << 16), acc[j][2 * d]);
              acc[j][2 * d + 1] = fmaf(w, __builtin_bit_cast(float, v & 0xffff0000u), acc[j][2 * d + 1]);
            }
          }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wave + 8 * j;
        const float inv = inv_z[row];
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[j][2 * d] * inv, acc[j][2 * d + 1] * inv);
        *(u32x4*)(olat + row * kCoK + 8 * (lane ^ (row & 15))) = o;
      }
    }
    __syncthreads();

    // 3. products: A fragment (row r, k block q) of this wave's k range
    f32x16 c[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int q = 0; q < KCW; ++q) {
      const int chunk = (kw + 16 * q) >> 3;
      const bf16x8 a = *(const bf16x8*)(olat + r * kCoK + 8 * (chunk ^ (r & 15)));
#pragma unroll
      for (int f = 0; f < 2; ++f) c[f] = mfma32x32x16(a, wf[f][q], c[f]);
    }
    float* dst = part + (wave * 64 + lane) * 32;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dst + 16 * f + 4 * g) = f32x4{c[f][4 * g], c[f][4 * g + 1], c[f][4 * g + 2], c[f][4 * g + 3]};
    __syncthreads();
    {
      // thread t: lane t % 64, fragment f and accumulator group j from t / 64;
      // accumulator 4j + i of lane (hh, c) is row 8j + 4hh + i, column n0 + 32f + c
      const int ln = tid & 63, grp = tid >> 6, f = grp >> 2, j = grp & 3;
      f32x4 v = f32x4{};
#pragma unroll
      for (int w = 0; w < kCoWaves; ++w) v += *(const f32x4*)(part + (w * 64 + ln) * 32 + 16 * f + 4 * j);
      const int col = n0 + 32 * f + (ln & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = b0 + 8 * j + 4 * (ln >> 5) + i;
        if (row < p.batch) {
          const int64_t o = ((int64_t)row * H + h) * kCoN + col;
          if constexpr (OUT_F32) ((float*)p.out)[o] = v[i];
          else ((__bf16*)p.out)[o] = (__bf16)v[i];
        }
      }
    }
    __syncthreads();
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
  if (p.batch == 0) return hipSuccess;
  if (p.tail != nullptr && p.n_tail != 64) return hipErrorInvalidValue;   // 64-wide rotary rows
  hipLaunchKernelGGL(absorb_bf16_kernel, dim3(p.heads, kAbsN / kAbsNT), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_absorb_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, true, 32, 32>(p, s);
}
hipError_t launch_outproj_dsv2_bf16(const GemmParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (p.a_f32)
    hipLaunchKernelGGL(outproj_bf16_kernel<true>, dim3(p.heads, kOutN / kOutNT), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(outproj_bf16_kernel<false>, dim3(p.heads, kOutN / kOutNT), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_outproj_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, false, 32, 32>(p, s);
}
int combine_outproj_max_splits() { return kCoMaxSplits; }
hipError_t launch_combine_outproj_dsv2_bf16(const CombineOutParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (p.splits > kCoMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(p.heads, kCoN / kCoNT), block(64 * kCoWaves);
  if (p.out_f32)
    hipLaunchKernelGGL(combine_outproj_kernel<true>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(combine_outproj_kernel<false>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
