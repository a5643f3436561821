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
//
// The workgroup's 128 x 256 block of W_UK goes to LDS with direct loads (two
// 512-byte rows per wave instruction). Wave w then owns columns n0 + 64w ..
// + 63 over the whole k range: its B operands (8 consecutive k of one column
// per lane) come from transposing LDS reads, so no k-partials have to be
// added across waves. Row k's 16-byte chunks are XOR-swizzled by 4 (k & 3):
// the eight rows and four chunks of one transposing read then cover every
// bank group exactly twice. Results go through LDS so that every global
// store writes 16 bytes.
constexpr int kAbsK = 128, kAbsN = 512, kAbsNT = 256;
constexpr int kAbsRow = kAbsNT * 2;                      // bytes of one staged W row

__device__ __forceinline__ int abs_w_off(int k, int chunk) { return k * kAbsRow + 16 * (chunk ^ (4 * (k & 3))); }

__global__ __launch_bounds__(256, 1) void absorb_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kAbsK * kAbsRow + 32 * kAbsRow];   // W block + result tile
  MLA_LDS char* wl = (MLA_LDS char*)smem;
  MLA_LDS char* cl = wl + kAbsK * kAbsRow;
  const int h = blockIdx.x, n0 = blockIdx.y * kAbsNT;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int KB = kAbsK / 16;                          // 16-wide k blocks
  constexpr int TAIL_CH = 64 / 8;                         // 16-byte chunks of a 64-wide rotary row
  const bool do_tail = blockIdx.y == 0 && p.tail != nullptr;

  // A operands: lane (hh, r) holds row b0 + r, k = 16 kb + 8 hh .. + 7
  auto load_a = [&](int b0, bf16x8 (&a)[KB]) {
    const int brow = b0 + r;
    const bool ok = brow < p.batch;
    const __bf16* arow = (const __bf16*)p.a + ((int64_t)(ok ? brow : 0) * p.heads + h) * p.lda + 8 * hh;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      a[kb] = *(const bf16x8*)(arow + 16 * kb);
      if (!ok) a[kb] = bf16x8{};
    }
  };
  // rotary rows: one 16-byte chunk per thread (32 rows x 8 chunks)
  auto load_tail = [&](int b0) -> u32x4 {
    const int row = min(b0 + tid / TAIL_CH, p.batch - 1);
    return load16((const __bf16*)p.tail + ((int64_t)row * p.heads + h) * 64 + 8 * (tid % TAIL_CH));
  };
  bf16x8 a_next[KB];
  load_a(0, a_next);
  u32x4 tail_next = do_tail ? load_tail(0) : u32x4{};
  {
    // W rows k = 2i, 2i + 1: lane c of the instruction fills physical chunk
    // c & 31 of row 2i + c / 32 with the logical chunk it stands for
    const char* wsrc = (const char*)p.w + (int64_t)h * kAbsK * kAbsN * 2 + n0 * 2;
#pragma unroll
    for (int i = 0; i < kAbsK / 2 / 4; ++i) {
      const int pair = wave * (kAbsK / 8) + i, k = 2 * pair + hh;
      load16_to_lds(wsrc + (int64_t)k * kAbsN * 2 + 16 * ((lane & 31) ^ (4 * (k & 3))), wl + 2 * pair * kAbsRow);
    }
  }
  // transposing reads: source lane (a4, e4) of 16-lane group (hh, sub)
  // points at row 16 kb + 8 hh + 4 q + e4, columns 64w + 32f + 16 sub + 4 a4
  // .. + 3; lane (hh, r) receives column 64w + 32f + r, rows 8 hh + 4 q .. + 3
  const int s16 = lane & 15, a4 = s16 & 3, e4 = s16 >> 2, sub = (lane >> 4) & 1;
  auto w_frag = [&](int kb, int f) -> bf16x8 {
    const int lc = 8 * wave + 4 * f + 2 * sub + (a4 >> 1);
    const bf16x4 v0 = lds_read_tr16(wl + abs_w_off(16 * kb + 8 * hh + e4, lc) + 8 * (a4 & 1));
    const bf16x4 v1 = lds_read_tr16(wl + abs_w_off(16 * kb + 8 * hh + 4 + e4, lc) + 8 * (a4 & 1));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  wait_vmem();
  __syncthreads();

  for (int b0 = 0; b0 < p.batch; b0 += 32) {
    bf16x8 a[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) a[kb] = a_next[kb];
    const u32x4 tail = tail_next;
    if (b0 + 32 < p.batch) {          // the next block's rows go out before this block's math
      load_a(b0 + 32, a_next);
      if (do_tail) tail_next = load_tail(b0 + 32);
    }
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[f] = mfma32x32x16(a[kb], w_frag(kb, f), acc[f]);
    // accumulator i of lane (hh, r): row 8(i/4) + 4hh + i%4, column 64w + 32f + r
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * hh + (i & 3);
        *(MLA_LDS __bf16*)(cl + row * kAbsRow + 2 * (64 * wave + 32 * f + r)) = (__bf16)acc[f][i];
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32 * kAbsRow / 16 / 256; ++j) {
      const int c = j * 256 + tid, row = c / (kAbsRow / 16), ch = c % (kAbsRow / 16);
      const u32x4 v = *(const MLA_LDS u32x4*)(cl + row * kAbsRow + 16 * ch);
      if (b0 + row < p.batch)
        *(u32x4*)((__bf16*)p.c + ((int64_t)(b0 + row) * p.heads + h) * p.ldc + n0 + 8 * ch) = v;
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
// block of batch rows): 16 rows up to batch 32, else about half the batch
// rounded up to 32-row passes, so that there are about 256 workgroups, every
// partial row is read once and the head's W_UV once per block. Per pass:
//   1. the loads are requested at once: the partial LSEs, the first splits'
//      partial rows (wave w takes rows w + 8j, each wave instruction one
//      split's whole 1 KiB row through a buffer descriptor with the row and
//      split in the scalar offset) and, in the first pass, the head's W_UV
//      rows (wave w takes rows 16w .. 16w + 15, one 1 KiB row per instruction);
//   2. merge weights e^(lse_s - max) per (row, split) stay in the lanes that
//      computed them (lane 16j + s of wave w: row w + 8j, split s) and are
//      read with readlane;
//   3. the merge: fp32 sums, times 1/z, rounded to bf16 (the values a bf16
//      mla_combine output would hold) and stored to LDS, as are the W_UV rows
//      in the first pass;
//   4. wave w multiplies the pass's rows by columns 32(w % 4) .. + 31 of
//      W_UV over k half w / 4 (a 32-row MFMA; in a 16-row pass rows 16..31
//      are not stored), both operands read from LDS; the two k halves are
//      added through LDS.
// LDS rows of 1 KiB (W_UV rows and merged rows) have their 16-byte chunks
// XOR-swizzled by the row, so 16 consecutive rows read at one chunk hit 16
// different bank groups.
constexpr int kCoK = 512, kCoN = 128, kCoWaves = 8, kCoMaxSplits = 64;
static_assert(kCoMaxSplits % 16 == 0, "split chunks");
constexpr int kCoRow = kCoK * 2;                          // bytes of one bf16 row
constexpr int kCoLds = kCoN * kCoRow + 32 * kCoRow;      // W_UV rows + 32 MFMA rows: 160 KiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ int co_chunk(int row, int chunk) { return row * kCoRow + 16 * (chunk ^ (row & 15)); }
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {   // in-row lane permutation (every source lane valid)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Reduction over each row of 16 lanes by DPP (swap neighbours, swap pairs,
// mirror halves, mirror the row); every lane of the row gets the same value.
template <class Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
  v = op(v, dpp_move<0xb1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4e>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  return op(v, dpp_move<0x140>(v));   // row_mirror
}

// RPW merged rows per wave and pass: 2 (16-row passes) or 4 (32-row passes).
template <bool OUT_F32, int RPW>
__global__ __launch_bounds__(64 * kCoWaves, 1) void combine_outproj_kernel(CombineOutParams p) {
  static_assert(RPW == 2 || RPW == 4, "16- or 32-row passes");
  constexpr int PR = kCoWaves * RPW;                      // rows per pass
  constexpr int SC = 16 / RPW;                            // splits in flight per row
  static_assert(kCoMaxSplits % SC == 0 && 16 % SC == 0, "split chunks");
  __shared__ __attribute__((aligned(16))) char smem[kCoLds];
  MLA_LDS char* wl = (MLA_LDS char*)smem;                 // W_UV rows of the head
  MLA_LDS char* ol = wl + kCoN * kCoRow;                  // merged rows; then the k-half sums
  const int h = blockIdx.x, b_first = blockIdx.y * p.rows_per_block;
  const int b_end = min(b_first + p.rows_per_block, p.batch);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = p.splits, H = p.heads;
  const int split_stride = H * kCoRow;                    // bytes between two splits of one (b, h)
  const int row_stride = S * split_stride;                // bytes between two batch rows
  // A block of at most 4 rows with more splits than one chunk runs split-
  // parallel: slot (wave w, j) takes row (w + 8j) & 3 and split group
  // (w + 8j) >> 2, i.e. every fourth chunk of SC splits; the four groups'
  // fp32 sums of a row are added through LDS before the rounding.
  const bool spm = RPW == 2 && b_end - b_first <= 4 && S > SC;
  auto real_row = [&](int vrow) { return spm ? (vrow & 3) : vrow; };
  auto group = [&](int vrow) { return spm ? (vrow >> 2) : 0; };
  const int chunk_step = spm ? 4 * SC : SC;               // splits between a slot's chunks
  const int j16 = lane >> 4, s16 = lane & 15;             // weight lanes: row wave + 8 j16, split s16 + 16k
  const int lrow = real_row(wave + 8 * (RPW == 2 ? (j16 & 1) : j16));   // (16-row passes: lanes 32..63 repeat)

  // partial LSEs of a pass (splits past S read split S - 1 and are masked
  // after the load, so no branch surrounds it)
  auto issue_lse = [&](float (&l)[kCoMaxSplits / 16], int b0, int rows) {
    const float* lse_row = p.lse_part + (int64_t)(b0 + min(lrow, rows - 1)) * S * H + h;
#pragma unroll
    for (int k = 0; k < kCoMaxSplits / 16; ++k) {
      const int sp = s16 + 16 * k;
      const float v = lse_row[(int64_t)min(sp, S - 1) * H];
      l[k] = sp < S ? v : -INFINITY;
    }
  };
  // partial rows of a pass: byte offset row * row_stride + split *
  // split_stride from the head's first row (below 2^31 for 32 rows of at
  // most 64 splits of 128 heads)
  auto part_rsrc = [&](int b0, int rows) {
    return buffer_rsrc((const char*)p.o_part + ((int64_t)b0 * S * H + h) * kCoRow, rows * row_stride - h * kCoRow);
  };
  auto issue = [&](u32x4 (&x)[SC][RPW], const __amdgpu_buffer_rsrc_t& rs, int rows, int s0) {
#pragma unroll
    for (int i = 0; i < SC; ++i)
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int vrow = wave + 8 * j;
        const int rr = min(real_row(vrow), rows - 1), sp = min(s0 + group(vrow) * SC + i, S - 1);
        x[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, rr * row_stride + sp * split_stride, 0);
      }
  };

  // 1. the first pass's loads, then the head's W_UV rows (coalesced 1 KiB rows
  //    into registers, requested last: needed last)
  float l[kCoMaxSplits / 16];
  u32x4 x[SC][RPW];
  issue_lse(l, b_first, min(PR, b_end - b_first));
  issue(x, part_rsrc(b_first, min(PR, b_end - b_first)), min(PR, b_end - b_first), 0);
  u32x4 wrow[kCoN / kCoWaves];
  {
    const char* wh = (const char*)p.w + ((int64_t)h * kCoN + wave * (kCoN / kCoWaves)) * kCoRow + lane * 16;
#pragma unroll
    for (int k = 0; k < kCoN / kCoWaves; ++k) wrow[k] = load16(wh + k * kCoRow);
  }

  // one pass over rows b0 .. b0 + rows - 1 whose LSEs and first splits are in l, x
  auto pass_body = [&](auto first_pass, int b0, int rows) {
    constexpr bool FIRST = decltype(first_pass)::value;
    const __amdgpu_buffer_rsrc_t part_rs = part_rsrc(b0, rows);
    // 2. merge weights of (row lrow, splits s16 + 16k)
    float wk[kCoMaxSplits / 16], inv;
    {
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < kCoMaxSplits / 16; ++k) m = fmaxf(m, l[k]);
      m = row16_reduce(m, [](float u, float v) { return fmaxf(u, v); });
      const bool empty = (m == -INFINITY);
      float z = 0.0f;
#pragma unroll
      for (int k = 0; k < kCoMaxSplits / 16; ++k) {
        wk[k] = (empty || l[k] == -INFINITY) ? 0.0f : fast_exp2((l[k] - m) * kLog2e);
        z += wk[k];
      }
      z = row16_reduce(z, [](float u, float v) { return u + v; });
      inv = empty ? 0.0f : 1.0f / z;
      if (s16 == 0 && j16 < RPW && wave + 8 * j16 < rows && p.lse != nullptr)   // each real row once
        p.lse[(int64_t)(b0 + lrow) * H + h] = empty ? -INFINITY : m + fast_log2(z) * kLn2;
    }

    // 3. merge: wave w, rows w + 8j; lane = 16-byte chunk of the row
    float acc[RPW][8];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    auto merge = [&](int s0) {
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        // splits c0 .. c0 + SC - 1 of this slot share one weight register, c0 / 16
        const int c0 = s0 + group(wave + 8 * j) * SC, kk = c0 >> 4, lo = c0 & 15;
        const float wsel = kk == 0 ? wk[0] : kk == 1 ? wk[1] : kk == 2 ? wk[2] : wk[3];
#pragma unroll
        for (int i = 0; i < SC; ++i) {
          // a split with weight 0 (empty, or past S) has its words zeroed,
          // so whatever it holds cannot reach the sum: the byte selectors and
          // the mask are wave-uniform
          const float w = c0 + i < S ? lane_value(wsel, 16 * j + lo + i) : 0.0f;
          const bool skip = (w == 0.0f);
          const uint32_t sel_lo = skip ? 0x0c0c0c0cu : 0x01000c0cu;   // (v & 0xffff) << 16, or 0
          const uint32_t mask_hi = skip ? 0u : 0xffff0000u;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t v = x[i][j][d];
            acc[j][2 * d] = fmaf(w, __builtin_bit_cast(float, __builtin_amdgcn_perm(v, v, sel_lo)), acc[j][2 * d]);
            acc[j][2 * d + 1] = fmaf(w, __builtin_bit_cast(float, v & mask_hi), acc[j][2 * d + 1]);
          }
        }
      }
    };
    merge(0);
    for (int s0 = chunk_step; s0 < S; s0 += chunk_step) {
      issue(x, part_rs, rows, s0);
      merge(s0);
    }
    if (FIRST && spm) {   // (a block of at most 4 rows has one pass)
      // add the four split groups of each row (slot sums through the W_UV
      // area, still free): rows 0..3 end up in slot 0 of waves 0..3
      MLA_LDS f32x4* sum = (MLA_LDS f32x4*)wl;               // [vrow][lane][2]
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        sum[((wave + 8 * j) * 64 + lane) * 2] = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
        sum[((wave + 8 * j) * 64 + lane) * 2 + 1] = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
      }
      __syncthreads();
      if (wave < 4) {
#pragma unroll
        for (int g = 1; g < 4; ++g) {
          const f32x4 u0 = sum[((wave + 4 * g) * 64 + lane) * 2], u1 = sum[((wave + 4 * g) * 64 + lane) * 2 + 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) { acc[0][e] += u0[e]; acc[0][4 + e] += u1[e]; }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int row = wave + 8 * j;
      const float iv = lane_value(inv, 16 * j);
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[j][2 * d] * iv, acc[j][2 * d + 1] * iv);
      *(MLA_LDS u32x4*)(ol + co_chunk(row, lane)) = o;
    }
    if constexpr (FIRST) {
#pragma unroll
      for (int k = 0; k < kCoN / kCoWaves; ++k) {
        const int n = wave * (kCoN / kCoWaves) + k;
        *(MLA_LDS u32x4*)(wl + co_chunk(n, lane)) = wrow[k];
      }
    }
    __syncthreads();

    // 4. products: columns 32f .. 32f + 31 over k blocks 16kq .. 16kq + 15
    const int f = wave & 3, kq = wave >> 2, n = 32 * f + r;
    f32x16 c = f32x16{};
#pragma unroll
    for (int q = 0; q < kCoK / 32; ++q) {
      const int chunk = 2 * (16 * kq + q) + hh;
      const bf16x8 a = *(const MLA_LDS bf16x8*)(ol + co_chunk(r, chunk));
      const bf16x8 bw = *(const MLA_LDS bf16x8*)(wl + co_chunk(n, chunk));
      c = mfma32x32x16(a, bw, c);
    }
    __syncthreads();
    constexpr int G = PR / 8;                                // accumulator groups holding pass rows
    MLA_LDS f32x4* red = (MLA_LDS f32x4*)ol;                // [f][g][lane]
    if (kq == 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) red[(f * G + g) * 64 + lane] = f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
    }
    __syncthreads();
    if (kq == 0) {
      // accumulator 4g + i of lane (hh, r) is row 8g + 4hh + i, column 32f + r
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const f32x4 o = red[(f * G + g) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * g + 4 * hh + i;
          const float v = c[4 * g + i] + o[i];
          if (row < rows) {
            const int64_t off = ((int64_t)(b0 + row) * H + h) * kCoN + n;
            if constexpr (OUT_F32) ((float*)p.out)[off] = v;
            else ((__bf16*)p.out)[off] = (__bf16)v;
          }
        }
      }
    }
    __syncthreads();   // the merged-row area is refilled by the next pass
  };

  pass_body(std::true_type{}, b_first, min(PR, b_end - b_first));
  for (int b0 = b_first + PR; b0 < b_end; b0 += PR) {
    const int rows = min(PR, b_end - b0);
    issue_lse(l, b0, rows);
    issue(x, part_rsrc(b0, rows), rows, 0);
    pass_body(std::false_type{}, b0, rows);
  }
}

template <bool F32, bool W_KN, int K, int N>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  using G = GemmCfg<F32, W_KN, K, N>;
  if (p.batch == 0) return hipSuccess;
  dim3 grid(p.heads, N / G::NT, (p.batch + 31) / 32);
  return launch_kernel((head_gemm<F32, W_KN, K, N>), grid, dim3(64), s, p);
}

}  // namespace

hipError_t launch_absorb_dsv2_bf16(const GemmParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (p.tail != nullptr && p.n_tail != 64) return hipErrorInvalidValue;   // 64-wide rotary rows
  return launch_kernel(absorb_bf16_kernel, dim3(p.heads, kAbsN / kAbsNT), dim3(256), s, p);
}
hipError_t launch_absorb_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, true, 32, 32>(p, s);
}
hipError_t launch_outproj_dsv2_bf16(const GemmParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (p.a_f32) return launch_kernel(outproj_bf16_kernel<true>, dim3(p.heads, kOutN / kOutNT), dim3(256), s, p);
  return launch_kernel(outproj_bf16_kernel<false>, dim3(p.heads, kOutN / kOutNT), dim3(256), s, p);
}
hipError_t launch_outproj_tiny_f32(const GemmParams& p, hipStream_t s) {
  return launch<true, false, 32, 32>(p, s);
}
int combine_outproj_max_splits() { return kCoMaxSplits; }
hipError_t launch_combine_outproj_dsv2_bf16(const CombineOutParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (p.splits > kCoMaxSplits) return hipErrorInvalidValue;
  // rows per workgroup: 16 up to batch 32; else half the batch rounded up to
  // whole 32-row passes (about 256 workgroups, W_UV read once per block)
  CombineOutParams q = p;
  q.rows_per_block = p.batch <= 32 ? 16 : (((p.batch + 1) / 2 + 31) / 32) * 32;
  const dim3 grid(p.heads, (p.batch + q.rows_per_block - 1) / q.rows_per_block), block(64 * kCoWaves);
  if (q.rows_per_block == 16) {
    if (p.out_f32) return launch_kernel(combine_outproj_kernel<true, 2>, grid, block, s, q);
    return launch_kernel(combine_outproj_kernel<false, 2>, grid, block, s, q);
  }
  if (p.out_f32) return launch_kernel(combine_outproj_kernel<true, 4>, grid, block, s, q);
  return launch_kernel(combine_outproj_kernel<false, 4>, grid, block, s, q);
}

}  // namespace mla
