// MLA decode over the latent cache, absorbed form.
//
// Method: DeepSeek-V2 paper (Chinese translation), section 2.1.2 (only the
// latent c_KV is cached; W_UK folds into the query and W_UV into the output)
// and section 2.1.3 (a shared rotary key k^R is cached beside c_KV and the
// score is the dot product of the concatenations). With the foldings every
// head scores its absorbed query q_lat = [W_UK^T q^C ; q^R] against the same
// (d_c + d_h^R)-wide cache rows and sums the c_KV part of those rows weighted
// by the softmax. All heads of a sequence read one shared row per token, so
// the work is a dense contraction like multi-query attention:
//   S^T[tokens x heads] = Rows[tokens x 576] . Q^T[576 x heads]      (MFMA)
//   O^T[512 x heads]   += C_KV^T[512 x tokens] . P^T[tokens x heads]  (MFMA)
//
// One workgroup handles one (sequence, split) for all heads: wave w owns heads
// 32w .. 32w+31 (its query fragments stay in VGPRs, its 32 x 512 output in
// AGPRs). Tiles of 32 tokens are streamed HBM -> LDS with direct 16-byte
// loads, double buffered, and every tile is read from HBM exactly once for
// all heads. The softmax is the streaming form in fp32 and base 2 against a
// fixed per-head reference maximum (see kHeadroom).
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

template <int H_, int DC_, int DR_, int KIND_>
struct Cfg {
  static constexpr int H = H_, DC = DC_, DR = DR_, W = DC_ + DR_;
  static constexpr int KIND = KIND_;
  static constexpr bool F32 = KIND_ == kF32;
  static constexpr bool FP8 = KIND_ == kFP8;
  static constexpr int T = 32;                          // tokens per tile
  static constexpr int WAVES = (H + 31) / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int ESZ = F32 ? 4 : 2;               // LDS element bytes
  static constexpr int LAT_CH = DC * ESZ / 16;          // 16-byte chunks per LDS latent row
  static constexpr int ROPE_CH = DR * ESZ / 16;
  static constexpr int LAT_BYTES = T * DC * ESZ;
  static constexpr int ROPE_BYTES = T * DR * ESZ;
  static constexpr int SCALE_BYTES = FP8 ? T * 4 : 0;
  static constexpr int BUF_BYTES = LAT_BYTES + ROPE_BYTES + SCALE_BYTES;
  static constexpr int NKC_LAT = DC / 16, NKC_ROPE = DR / 16, NKC = NKC_LAT + NKC_ROPE;
  static constexpr int NFRAG = DC / 32;                 // 32-feature output fragments
  static_assert(DC % 32 == 0 && DR % 16 == 0, "head shape");
};

// XOR swizzle of 16-byte chunks within an LDS row. The key moves chunk pairs
// (t & 3 -> 0, 2, 4, 6) so that the transposing reads of 4 consecutive tokens
// hit distinct banks, and the low bit (t >> 2 & 1) separates rows 4 apart for
// the row-wise reads of 8 consecutive tokens.
template <int CH>
__device__ __forceinline__ int swz(int t) {
  if constexpr (CH >= 8) return ((t & 3) << 1) | ((t >> 2) & 1);
  else return 0;
}

template <class C>
__device__ __forceinline__ int lat_off(int t, int byte) {   // byte offset in a tile buffer
  return t * (C::DC * C::ESZ) + ((((byte >> 4) ^ swz<C::LAT_CH>(t))) << 4) + (byte & 15);
}
template <class C>
__device__ __forceinline__ int rope_off(int t, int byte) {
  return C::LAT_BYTES + t * (C::DR * C::ESZ) + ((((byte >> 4) ^ swz<C::ROPE_CH>(t))) << 4) + (byte & 15);
}

template <bool PAGED>
__device__ __forceinline__ int64_t row_of(const DecodeParams& p, int b, int tok) {
  if constexpr (!PAGED) {
    return (int64_t)b * p.seq_stride + tok;
  } else {
    const int page = p.block_table[(int64_t)b * p.max_pages + (tok >> p.page_shift)];
    return ((int64_t)page << p.page_shift) + (tok & ((1 << p.page_shift) - 1));
  }
}

// Staging registers of the fp8 loader (codes and scales pass through VGPRs).
template <class C>
struct Fp8Stage {
  static constexpr int CODE_CH = C::T * C::DC / 16;     // 16-code chunks per tile
  static constexpr int ROUNDS = (CODE_CH + C::THREADS - 1) / C::THREADS;
  static_assert(!C::FP8 || CODE_CH % C::THREADS == 0, "fp8 loader covers whole rounds");
  u32x4 codes[C::FP8 ? ROUNDS : 1];
  float scale;
};

// Per-lane direct loads of a region whose rows hold CH 16-byte chunks
// (CH < 64: several rows per wave instruction).
template <class C, bool PAGED, int CH>
__device__ __forceinline__ void issue_rows_lanewise(const DecodeParams& p, const char* src,
                                                    int64_t src_row_bytes, MLA_LDS char* dst, int b,
                                                    int tile_base, int start, int end) {
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int TOT = C::T * CH;
#pragma unroll
  for (int k = 0; k < (TOT + C::THREADS - 1) / C::THREADS; ++k) {
    const int pc = k * C::THREADS + tid;
    if (TOT % C::THREADS == 0 || pc < TOT) {
      const int t = pc / CH;
      const int c = (pc % CH) ^ swz<CH>(t);
      int tok = tile_base + t;
      tok = tok < end ? tok : start;
      load16_to_lds(src + row_of<PAGED>(p, b, tok) * src_row_bytes + c * 16,
                    dst + (k * C::THREADS + wave * 64) * 16);
    }
  }
}

// Start the HBM -> LDS transfer of tile rows [tile_base, tile_base + T).
// Rows past `end` are replaced by row `start` (always valid); their scores are
// masked, so they only need to be finite.
template <class C, bool PAGED>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, MLA_LDS char* buf, int b,
                                           int tile_base, int start, int end, Fp8Stage<C>& st) {
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (!C::FP8) {
    const char* base = (const char*)p.latent;
    const int64_t rs = p.row_stride * C::ESZ;
    if constexpr (C::LAT_CH == 64) {
      // one 1 KiB latent row per wave instruction: the row address is
      // wave-uniform (scalar registers), each lane adds its swizzled chunk
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
      for (int k = 0; k < C::T / C::WAVES; ++k) {
        const int t = k * C::WAVES + wave;
        int tok = tile_base + t;
        tok = tok < end ? tok : start;
        const char* g = base + row_of<PAGED>(p, b, tok) * rs + ((lane ^ swz<64>(t)) << 4);
        load16_to_lds(g, buf + t * (C::DC * C::ESZ));
      }
    } else {
      issue_rows_lanewise<C, PAGED, C::LAT_CH>(p, base, rs, buf, b, tile_base, start, end);
    }
    issue_rows_lanewise<C, PAGED, C::ROPE_CH>(p, base + C::DC * C::ESZ, rs, buf + C::LAT_BYTES, b,
                                              tile_base, start, end);
  } else {
    // e4m3 codes: 16 per chunk, staged in VGPRs and widened to bf16 later.
    const char* codes = (const char*)p.latent;
    constexpr int CPR = C::DC / 16;                      // code chunks per row
#pragma unroll
    for (int k = 0; k < Fp8Stage<C>::ROUNDS; ++k) {
      const int pc = k * C::THREADS + tid;
      const int t = pc / CPR, c = pc % CPR;
      int tok = tile_base + t;
      tok = tok < end ? tok : start;
      st.codes[k] = load16(codes + row_of<PAGED>(p, b, tok) * p.row_stride + c * 16);
    }
    issue_rows_lanewise<C, PAGED, C::ROPE_CH>(p, (const char*)p.rope, p.rope_stride * 2,
                                              buf + C::LAT_BYTES, b, tile_base, start, end);
    if (tid < C::T) {
      int tok = tile_base + tid;
      tok = tok < end ? tok : start;
      st.scale = p.scale[row_of<PAGED>(p, b, tok)];
    }
  }
}

// fp8 only: widen the staged codes to bf16 and store them with the scales.
template <class C>
__device__ __forceinline__ void commit_tile(MLA_LDS char* buf, const Fp8Stage<C>& st) {
  if constexpr (C::FP8) {
    const int tid = threadIdx.x;
    constexpr int CPR = C::DC / 16;
#pragma unroll
    for (int k = 0; k < Fp8Stage<C>::ROUNDS; ++k) {
      const int pc = k * C::THREADS + tid;
      const int t = pc / CPR, c = pc % CPR;
      const u32x4 w = st.codes[k];
      u32x4 lo, hi;   // 16 codes -> 16 bf16 = two 16-byte LDS chunks (2c, 2c + 1)
      lo[0] = e4m3x2_to_bf16x2<false>(w[0]); lo[1] = e4m3x2_to_bf16x2<true>(w[0]);
      lo[2] = e4m3x2_to_bf16x2<false>(w[1]); lo[3] = e4m3x2_to_bf16x2<true>(w[1]);
      hi[0] = e4m3x2_to_bf16x2<false>(w[2]); hi[1] = e4m3x2_to_bf16x2<true>(w[2]);
      hi[2] = e4m3x2_to_bf16x2<false>(w[3]); hi[3] = e4m3x2_to_bf16x2<true>(w[3]);
      *(MLA_LDS u32x4*)(buf + lat_off<C>(t, (2 * c) * 16)) = lo;
      *(MLA_LDS u32x4*)(buf + lat_off<C>(t, (2 * c + 1) * 16)) = hi;
    }
    if (tid < C::T) *(MLA_LDS float*)(buf + C::LAT_BYTES + C::ROPE_BYTES + tid * 4) = st.scale;
  }
}

// Per-lane LDS byte offsets, computed once. Every LDS read of the tile loop is
// one of these plus a compile-time constant, so the reads use the DS
// instruction's immediate offset instead of one address register per read.
// (The XOR key only touches the low 3 bits of a chunk index.)
template <class C>
struct LaneOffs {
  int qk_lat[4];    // latent k block kc:  qk_lat[kc & 3] + 128 * (kc >> 2)
  int qk_rope[4];   // rotary k block kk:  qk_rope[kk]
  int pv[2];        // C_KV^T fragment f, k step u, half q:
                    //   pv[f & 1] + ROWB * (16u + 8q) + 128 * (f >> 1)
};

template <class C>
__device__ __forceinline__ LaneOffs<C> lane_offsets() {
  LaneOffs<C> o;
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  constexpr int ROWB = C::DC * C::ESZ;
  const int kr = swz<C::LAT_CH>(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) o.qk_lat[j] = r * ROWB + 16 * ((2 * j + hh) ^ kr);
  const int kq = swz<C::ROPE_CH>(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) o.qk_rope[j] = C::LAT_BYTES + r * (C::DR * C::ESZ) + 16 * ((2 * j + hh) ^ kq);
  const int s16 = lane & 15, a4 = s16 & 3, e4 = s16 >> 2, sub = (lane >> 4) & 1;
  const int kt = swz<C::LAT_CH>(4 * hh + e4);     // equals the key of 16u + 8q + 4hh + e4
#pragma unroll
  for (int fp = 0; fp < 2; ++fp)
    o.pv[fp] = (4 * hh + e4) * ROWB + 16 * ((4 * fp + 2 * sub + (a4 >> 1)) ^ kt) + 8 * (a4 & 1);
  return o;
}

template <class C>
struct QFrag {
  // bf16: one 8-element vector per 16-wide k block; f32: eight floats.
  typename std::conditional<C::F32, float[C::NKC][8], bf16x8[C::NKC]>::type v;
};

template <class C>
struct State {
  f32x16 o[C::NFRAG];
  float m_ref;     // reference maximum the exponentials are taken against
  float m_max;     // largest base-2 scaled score seen so far
  float l;         // this lane's share of the softmax denominator
  bool overflow;   // a score exceeded m_ref by more than kHeadroom
};

// Scores may exceed the reference maximum by up to 2^kHeadroom before the
// exponentials could overflow fp32: with at most 2^17 tokens per split and
// |c_KV| < 2^9 every sum stays below 2^90. The reference is fixed at the first
// tile's maximum, so the accumulators are never rescaled inside the loop; in
// the rare case that a later score exceeds it by more than the headroom, the
// split is recomputed with the true maximum as reference.
constexpr float kHeadroom = 64.0f;

// One tile: scores, online softmax, weighted latent sum.
template <class C>
__device__ __forceinline__ void compute_tile(const MLA_LDS char* buf, const QFrag<C>& q, State<C>& s,
                                             const LaneOffs<C>& lo, int tile_base, int end,
                                             float scale_log2) {
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;

  // ---- S^T = Rows . Q^T : lane (hh, c) gets tokens 8j + 4hh + i of head c ----
  f32x16 sl = {}, sr = {};
#pragma unroll
  for (int kc = 0; kc < C::NKC; ++kc) {
    const bool rope_part = kc >= C::NKC_LAT;
    const int kk = rope_part ? kc - C::NKC_LAT : kc;
    if constexpr (C::F32) {
      float a[8];
      const int byte = (16 * kk + 8 * hh) * 4;
      const int o0 = rope_part ? rope_off<C>(r, byte) : lat_off<C>(r, byte);
      const int o1 = rope_part ? rope_off<C>(r, byte + 16) : lat_off<C>(r, byte + 16);
      const f32x4 x0 = *(const MLA_LDS f32x4*)(buf + o0);
      const f32x4 x1 = *(const MLA_LDS f32x4*)(buf + o1);
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = x0[e]; a[4 + e] = x1[e]; }
      sl = mfma32x32x16_f32(a, q.v[kc], sl);
    } else {
      const int off = rope_part ? lo.qk_rope[kk] : lo.qk_lat[kk & 3] + 128 * (kk >> 2);
      const bf16x8 a = *(const MLA_LDS bf16x8*)(buf + off);
      if (C::FP8 && rope_part) sr = mfma32x32x16(a, q.v[kc], sr);
      else sl = mfma32x32x16(a, q.v[kc], sl);
    }
  }

  // ---- online softmax (base 2) ----
  float x[16];
  float tok_scale[16];
  if constexpr (C::FP8) {
    const MLA_LDS float* sc = (const MLA_LDS float*)(buf + C::LAT_BYTES + C::ROPE_BYTES);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = *(const MLA_LDS f32x4*)(sc + 8 * j + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) tok_scale[4 * j + i] = v[i];
    }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = tile_base + 8 * (i >> 2) + 4 * hh + (i & 3);
    float v = C::FP8 ? (tok_scale[i] * sl[i] + sr[i]) : sl[i];
    v *= scale_log2;
    x[i] = tok < end ? v : -INFINITY;
    mt = fmaxf(mt, x[i]);
  }
  mt = wave_max32(mt);
  if (s.m_ref == -INFINITY) s.m_ref = mt;     // first tile of the first pass
  s.m_max = fmaxf(s.m_max, mt);
  s.overflow = s.overflow || (mt > s.m_ref + kHeadroom);
  float pr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pr[i] = x[i] == -INFINITY ? 0.0f : fast_exp2(x[i] - s.m_ref);
    s.l += pr[i];
    if constexpr (C::FP8) pr[i] *= tok_scale[i];
  }

  // ---- O^T += C_KV^T . P^T over two 16-token k steps ----
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (C::F32) {
      float pb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = pr[8 * u + e];
#pragma unroll
      for (int f = 0; f < C::NFRAG; ++f) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 16 * u + 8 * (e >> 2) + 4 * hh + (e & 3);
          a[e] = *(const MLA_LDS float*)(buf + lat_off<C>(t, (32 * f + r) * 4));
        }
        s.o[f] = mfma32x32x16_f32(a, pb, s.o[f]);
      }
    } else {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pr[8 * u + e];
      // transposing reads: source lane s = a + 4e of each 16-lane group points
      // at token 16u + 8q + 4hh + e, features 32f + 16*sub + 4a .. +3
      constexpr int ROWB = C::DC * C::ESZ;
#pragma unroll
      for (int f = 0; f < C::NFRAG; ++f) {
        const int off = lo.pv[f & 1] + ROWB * 16 * u + 128 * (f >> 1);
        const bf16x4 v0 = lds_read_tr16(buf + off);
        const bf16x4 v1 = lds_read_tr16(buf + off + ROWB * 8);
        const bf16x8 a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        s.o[f] = mfma32x32x16(a, pb, s.o[f]);
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void write_result(const DecodeParams& p, int b, int split, const State<C>& s,
                                             bool empty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int head = wave * 32 + r;
  const float l_tot = s.l + __shfl_xor(s.l, 32);   // lanes r and r + 32 hold one head
  if (head >= C::H) return;
  float inv = empty ? 0.0f : 1.0f / l_tot;
  float lse = empty ? -INFINITY : (s.m_ref + fast_log2(l_tot)) * kLn2;
  const bool split_out = p.num_splits > 1;
  const int64_t row = split_out ? (((int64_t)b * p.num_splits + split) * C::H + head)
                                : ((int64_t)b * C::H + head);
  if (hh == 0) p.lse[row] = lse;
  if (split_out || !p.out_bf16) {
    float* o = (float*)p.out + row * C::DC;
#pragma unroll
    for (int f = 0; f < C::NFRAG; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = empty ? 0.0f : s.o[f][4 * j + i] * inv;
        *(f32x4*)(o + 32 * f + 8 * j + 4 * hh) = v;
      }
  } else {
    uint16_t* o = (uint16_t*)p.out + row * C::DC;
#pragma unroll
    for (int f = 0; f < C::NFRAG; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 v;
        float w0 = empty ? 0.0f : s.o[f][4 * j + 0] * inv, w1 = empty ? 0.0f : s.o[f][4 * j + 1] * inv;
        float w2 = empty ? 0.0f : s.o[f][4 * j + 2] * inv, w3 = empty ? 0.0f : s.o[f][4 * j + 3] * inv;
        v[0] = pack_bf16x2(w0, w1);
        v[1] = pack_bf16x2(w2, w3);
        *(u32x2*)(o + 32 * f + 8 * j + 4 * hh) = v;
      }
  }
}

template <class C, bool PAGED>
__global__ __launch_bounds__(C::THREADS, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char buf0[C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char buf1[C::BUF_BYTES];

  int w = blockIdx.x;
  if (p.xcd_remap) w = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int b = w / p.num_splits, split = w % p.num_splits;
  const int L = max(0, min(p.seq_lens[b], p.max_seq_len));
  const int start = split * p.chunk;
  const int end = min(start + p.chunk, L);

  State<C> s;
#pragma unroll
  for (int f = 0; f < C::NFRAG; ++f) s.o[f] = f32x16{};
  s.m_ref = -INFINITY;
  s.m_max = -INFINITY;
  s.l = 0.0f;
  s.overflow = false;
  if (start >= end) {             // uniform over the workgroup
    write_result<C>(p, b, split, s, true);
    return;
  }

  // Absorbed query fragments of this wave's 32 heads (B operand of S^T).
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int head = wave * 32 + r;
  QFrag<C> q;
  {
    const bool ok = head < C::H;
    if constexpr (C::F32) {
      const float* qr = (const float*)p.q_lat + ((int64_t)b * C::H + (ok ? head : 0)) * C::W;
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
        const f32x4 x0 = *(const f32x4*)(qr + 16 * kc + 8 * hh);
        const f32x4 x1 = *(const f32x4*)(qr + 16 * kc + 8 * hh + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { q.v[kc][e] = ok ? x0[e] : 0.f; q.v[kc][4 + e] = ok ? x1[e] : 0.f; }
      }
    } else {
      const __bf16* qr = (const __bf16*)p.q_lat + ((int64_t)b * C::H + (ok ? head : 0)) * C::W;
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
        bf16x8 v = *(const bf16x8*)(qr + 16 * kc + 8 * hh);
        q.v[kc] = ok ? v : bf16x8{};
      }
    }
  }

  Fp8Stage<C> st;
  const LaneOffs<C> lo = lane_offsets<C>();
  const int ntiles = (end - start + C::T - 1) / C::T;
  MLA_LDS char* B0 = (MLA_LDS char*)buf0;
  MLA_LDS char* B1 = (MLA_LDS char*)buf1;
  __shared__ int redo_flag[C::WAVES];

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {   // recompute with the true maximum as reference
#pragma unroll
      for (int f = 0; f < C::NFRAG; ++f) s.o[f] = f32x16{};
      s.l = 0.0f;
      s.m_ref = s.m_max;
    }
    issue_tile<C, PAGED>(p, B0, b, start, start, end, st);
    wait_vmem();
    commit_tile<C>(B0, st);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      MLA_LDS char* cur = (it & 1) ? B1 : B0;
      MLA_LDS char* nxt = (it & 1) ? B0 : B1;
      const bool more = it + 1 < ntiles;
      if (more) issue_tile<C, PAGED>(p, nxt, b, start + (it + 1) * C::T, start, end, st);
      compute_tile<C>(cur, q, s, lo, start + it * C::T, end, p.scale_log2);
      if (more) { wait_vmem(); commit_tile<C>(nxt, st); }
      __syncthreads();
    }
    if (pass == 1) break;
    const bool wave_overflow = __ballot(s.overflow) != 0;
    if ((threadIdx.x & 63) == 0) redo_flag[threadIdx.x >> 6] = wave_overflow ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) any |= redo_flag[w];
    if (!any) break;    // uniform over the workgroup
  }
  write_result<C>(p, b, split, s, false);
}

template <class C>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  const int grid = p.batch * p.num_splits;
  if (grid == 0) return hipSuccess;
  DecodeParams q = p;
  q.xcd_remap = (grid % 8 == 0 && p.num_splits > 1) ? 1 : 0;
  if (p.page_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<C, true>), dim3(grid), dim3(C::THREADS), 0, stream, q);
  else
    hipLaunchKernelGGL((decode_kernel<C, false>), dim3(grid), dim3(C::THREADS), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_dsv2_bf16(const DecodeParams& p, hipStream_t s) {
  return launch<Cfg<128, 512, 64, kBF16>>(p, s);
}
hipError_t launch_decode_dsv2_fp8(const DecodeParams& p, hipStream_t s) {
  return launch<Cfg<128, 512, 64, kFP8>>(p, s);
}
hipError_t launch_decode_tiny_f32(const DecodeParams& p, hipStream_t s) {
  return launch<Cfg<4, 32, 16, kF32>>(p, s);
}

}  // namespace mla
