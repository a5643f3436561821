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
// One workgroup handles one (sequence, split) for all heads, and every cache
// tile is read from HBM once for all heads. Tiles of 32 tokens stream
// HBM -> LDS with direct 16-byte loads into a ring of LDS buffers (two tiles
// in flight while a third is computed). Wave w:
//   - scores its 32 heads 32w..32w+31 (their query fragments stay in VGPRs),
//     runs the softmax for them and writes P^T of those heads to LDS;
//   - after one workgroup barrier, accumulates latent features
//     w*d_c/waves .. (w+1)*d_c/waves - 1 for ALL heads (its O^T slice lives in
//     AGPRs), reading P^T of every head from LDS and its own C_KV^T slice with
//     transposing reads.
// Splitting the latent sum by features (not by heads) means each wave reads
// only its slice of the tile through the slower transposing LDS path.
// The softmax is the streaming form in fp32 and base 2 against a fixed
// per-head reference maximum (see kHeadroom), so the accumulators are never
// rescaled inside the loop.
#include <atomic>
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
  static constexpr int WAVES = (H + 31) / 32;           // = head blocks of 32
  static constexpr int HB = WAVES;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int FPW = DC / WAVES;                // latent features per wave (latent sum)
  static constexpr int NFJ = FPW / 32;                  // 32-feature fragments per wave
  static constexpr int ESZ = F32 ? 4 : 2;               // LDS element bytes
  static constexpr int LAT_CH = DC * ESZ / 16;          // 16-byte chunks per LDS latent row
  static constexpr int ROPE_CH = DR * ESZ / 16;
  static constexpr int LAT_BYTES = T * DC * ESZ;
  static constexpr int ROPE_BYTES = T * DR * ESZ;
  static constexpr int SCALE_BYTES = FP8 ? T * 4 : 0;
  static constexpr int BUF_BYTES = LAT_BYTES + ROPE_BYTES + SCALE_BYTES;
  static constexpr int NBUF = FP8 ? 3 : 4;              // tile ring
  static constexpr int AHEAD = NBUF - 2;                // tiles in flight beyond the next one
  static constexpr int PROW = T * ESZ;                  // bytes of one head's P^T row
  static constexpr int P_BYTES = HB * 32 * PROW;
  static constexpr int NKC_LAT = DC / 16, NKC_ROPE = DR / 16, NKC = NKC_LAT + NKC_ROPE;
  static constexpr int LDS_BYTES = NBUF * BUF_BYTES + 2 * P_BYTES;
  static_assert(DC % (32 * WAVES) == 0 && DR % 16 == 0, "head shape");
  static_assert(FPW % 128 == 0 || F32, "a wave's feature slice starts on a swizzle period");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// XOR swizzle of 16-byte chunks within an LDS row (the LDS serves 256 bytes,
// i.e. 16 chunks, per cycle).
//  - 1 KiB latent rows (64 chunks): key = (t & 3) << 2 | (t >> 2) & 3, a
//    bijection on t mod 16. Sixteen consecutive rows read at the same chunk
//    (the row-wise score reads) land on 16 distinct chunk slots, and the
//    transposing reads of 4 consecutive tokens x 4 consecutive chunks also
//    cover all 16 slots (the token's low bits select the slot's high bits).
//  - 128-byte rotary rows (8 chunks): key = (t >> 1) & 7; two rows share a
//    256-byte window, so sixteen rows again cover 16 distinct slots.
template <int CH>
__device__ __forceinline__ int swz(int t) {
  if constexpr (CH >= 16) return ((t & 3) << 2) | ((t >> 2) & 3);
  else if constexpr (CH == 8) return (t >> 1) & 7;
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
// P^T row of head h, chunk k (16 bytes): bf16 rows hold four chunks (four
// rows per 256-byte window), swizzled by (h >> 2) & 3 so that sixteen
// consecutive heads at one chunk cover 16 distinct slots; f32 rows are plain.
template <class C>
__device__ __forceinline__ int p_off(int h, int k) {
  if constexpr (C::F32) return h * C::PROW + 16 * k;
  else return h * C::PROW + 16 * (k ^ ((h >> 2) & 3));
}

// Physical cache rows of the tokens of one tile. Tiles start on multiples of
// 32 tokens; a token past the split's end is replaced by the tile's first
// token (always valid), whose score is masked later. With pages of at least
// 16 tokens a tile touches at most two pages, looked up once per tile with
// scalar loads; smaller pages are looked up per token.
// Where one sequence's rows live, computed once per workgroup.
struct SeqView {
  int64_t seq_row;          // contiguous: first row of the sequence
  const int32_t* bt_row;    // paged: the sequence's block-table row
};

// Query row bv = b n + t (n query tokens per sequence): the cache sequence b
// whose rows it reads, and how many of them it attends to (token t sees rows
// 0 .. L_b - n + t, so one query token per sequence sees all L_b).
__device__ __forceinline__ int cache_seq(const DecodeParams& p, int bv) {
  return p.tokens_per_seq > 1 ? bv / p.tokens_per_seq : bv;
}
__device__ __forceinline__ int query_len(const DecodeParams& p, int bv) {
  if (p.tokens_per_seq <= 1) return p.seq_lens[bv];
  const int n = p.tokens_per_seq, b = bv / n;
  return p.seq_lens[b] - (n - 1 - (bv - b * n));
}

template <bool PAGED>
__device__ __forceinline__ SeqView seq_view(const DecodeParams& p, int bv) {
  SeqView v;
  const int b = cache_seq(p, bv);
  v.seq_row = PAGED ? 0 : (int64_t)b * p.seq_stride;
  v.bt_row = PAGED ? p.block_table + (int64_t)b * p.max_pages : nullptr;
  return v;
}

template <bool PAGED>
struct TileRows {
  int tile_base, end;
  int64_t seq_row;         // contiguous: first row of the sequence
  int shift, lp0;          // paged: log2(page size), first logical page of the tile
  int64_t pg0, pg1;        // paged, big pages: physical pages of the tile
  bool small_pages;
  const int32_t* bt_row;

  __device__ __forceinline__ TileRows(const DecodeParams& p, const SeqView& sv, int tile_base_, int end_)
      : tile_base(tile_base_), end(end_) {
    if constexpr (!PAGED) {
      seq_row = sv.seq_row;
    } else {
      shift = p.page_shift;
      bt_row = sv.bt_row;
      lp0 = tile_base >> shift;
      small_pages = shift < 4;
      if (!small_pages) {
        pg0 = bt_row[lp0];
        pg1 = (shift == 4 && tile_base + 16 < end) ? (int64_t)bt_row[lp0 + 1] : pg0;
      }
    }
  }
  __device__ __forceinline__ int64_t row(int t) const {   // t: token index within the tile
    int tok = tile_base + t;
    tok = tok < end ? tok : tile_base;
    if constexpr (!PAGED) {
      return seq_row + tok;
    } else {
      const int mask = (1 << shift) - 1;
      if (!small_pages) {
        const int64_t pg = ((tok >> shift) == lp0) ? pg0 : pg1;
        return (pg << shift) + (tok & mask);
      }
      return ((int64_t)bt_row[tok >> shift] << shift) + (tok & mask);
    }
  }
};

// Per-lane global byte offsets of the fast tile loader (see issue_tile).
struct DmaOffs {
  int lat;         // latent chunk of row 4k + wave: lat ^ 16 (k & 3)
  int rope;        // this thread's rotary chunk, bytes from the tile's first row
  int rope_chunk;  // the same chunk, bytes from the start of its own row
};

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
template <class C, int CH, class Rows>
__device__ __forceinline__ void issue_rows_lanewise(const Rows& tr, const char* src, int64_t src_row_bytes,
                                                    MLA_LDS char* dst) {
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int TOT = C::T * CH;
#pragma unroll
  for (int k = 0; k < (TOT + C::THREADS - 1) / C::THREADS; ++k) {
    const int pc = k * C::THREADS + tid;
    if (TOT % C::THREADS == 0 || pc < TOT) {
      const int t = pc / CH;
      const int c = (pc % CH) ^ swz<CH>(t);
      load16_to_lds(src + tr.row(t) * src_row_bytes + c * 16, dst + (k * C::THREADS + wave * 64) * 16);
    }
  }
}

// Vector-memory instructions one tile costs each thread (for vmcnt waits).
template <class C>
constexpr int loads_per_tile() {
  constexpr int lat = C::FP8 ? Fp8Stage<C>::ROUNDS
                             : (C::LAT_CH == 64 ? C::T / C::WAVES
                                                : (C::T * C::LAT_CH + C::THREADS - 1) / C::THREADS);
  constexpr int rope = (C::T * C::ROPE_CH + C::THREADS - 1) / C::THREADS;
  return lat + rope;
}

// Start the HBM -> LDS transfer of tile rows [tile_base, tile_base + T).
template <class C, bool PAGED>
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const SeqView& sv, const DmaOffs& dma,
                                           MLA_LDS char* buf, int tile_base, int end, Fp8Stage<C>& st) {
  const int tid = threadIdx.x;
  const TileRows<PAGED> tr(p, sv, tile_base, end);
  if constexpr (!C::FP8 && C::LAT_CH == 64) {
    // Fast path: a full tile whose 32 rows are consecutive in memory (a
    // contiguous cache, or pages of at least 32 tokens). Row addresses are
    // wave-uniform scalar values; lanes add their swizzled chunk offsets.
    const bool consecutive = !PAGED || p.page_shift >= 5;
    if (consecutive && tile_base + C::T <= end) {
      const int64_t rs = p.row_stride * C::ESZ;
      const char* tile = (const char*)p.latent + tr.row(0) * rs;
      const auto res = buffer_rsrc(tile, (uint32_t)(C::T * rs));   // rows are at most 2^24 bytes apart
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
      static_assert(C::WAVES == 4, "row 4k + wave has swizzle key (wave << 2) | (k & 3)");
      // rotary keys: 8 lanes per row, one instruction for the whole tile
      static_assert(C::T * C::ROPE_CH == C::THREADS, "one rotary chunk per thread");
      buf_load16_to_lds(res, (uint32_t)dma.rope, 0u, buf + C::LAT_BYTES + wave * 64 * 16);
      // latent rows wave, wave + 4, ...
      MLA_LDS char* dst = buf + wave * (C::DC * C::ESZ);
#pragma unroll
      for (int k = 0; k < C::T / C::WAVES; ++k) {
        buf_load16_to_lds(res, (uint32_t)(dma.lat ^ (16 * (k & 3))), (uint32_t)((k * C::WAVES + wave) * rs), dst);
        dst += C::WAVES * (C::DC * C::ESZ);
      }
      return;
    }
  }
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
        const char* g = base + tr.row(t) * rs + (uint32_t)(dma.lat ^ (16 * (k & 3)));
        load16_to_lds(g, buf + t * (C::DC * C::ESZ));
      }
    } else {
      issue_rows_lanewise<C, C::LAT_CH>(tr, base, rs, buf);
    }
    issue_rows_lanewise<C, C::ROPE_CH>(tr, base + C::DC * C::ESZ, rs, buf + C::LAT_BYTES);
  } else {
    // e4m3 codes: 16 per chunk, staged in VGPRs and widened to bf16 later.
    const char* codes = (const char*)p.latent;
    constexpr int CPR = C::DC / 16;                      // code chunks per row
#pragma unroll
    for (int k = 0; k < Fp8Stage<C>::ROUNDS; ++k) {
      const int pc = k * C::THREADS + tid;
      const int t = pc / CPR, c = pc % CPR;
      st.codes[k] = load16(codes + tr.row(t) * p.row_stride + c * 16);
    }
    issue_rows_lanewise<C, C::ROPE_CH>(tr, (const char*)p.rope, p.rope_stride * 2, buf + C::LAT_BYTES);
    if (tid < C::T) st.scale = p.scale[tr.row(tid)];
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

// Per-lane LDS byte offsets of the tile-buffer reads (16-bit cache layouts).
// The swizzle keys only flip address bits below the bits that select the
// fragment, so every read of the loop is one of these bases XOR a constant
// (the fragment's position inside a 256-byte window) plus a constant (the
// DS instruction's immediate offset). Five registers instead of one per read.
template <class C>
struct LaneOffs {
  int lat;     // latent score operand of k block kc:  (lat ^ 32 (kc & 7)) + 256 (kc >> 3)
  int rope;    // rotary score operand of k block kk:  rope ^ 32 kk
  int pv[2];   // C_KV^T fragment j, k step u, half q: (pv[q] ^ 64 (j & 3)) + ROWB 16u + 256 (j >> 2)
  int p;       // P^T of head 32 hb + r, k step u:     (p ^ 32 u) + 32 hb PROW
};

template <class C>
__device__ __forceinline__ LaneOffs<C> lane_offsets(int wave) {
  LaneOffs<C> o{};
  if constexpr (!C::F32) {
    static_assert(C::LAT_CH == 64 && C::ROPE_CH == 8 && C::DR * C::ESZ == 128 && C::PROW == 64,
                  "the XOR forms below assume 1 KiB latent rows, 128-byte rotary rows, 64-byte P rows");
    const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
    constexpr int ROWB = C::DC * C::ESZ;
    // chunk (2 kb + hh) ^ key = 2 kb ^ (hh ^ key): the k block flips bits 5.. of the byte offset
    o.lat = r * ROWB + 16 * (hh ^ swz<C::LAT_CH>(r));
    o.rope = C::LAT_BYTES + r * (C::DR * C::ESZ) + 16 * (hh ^ swz<C::ROPE_CH>(r));
    // transposing reads: source lane (a, e) of 16-lane group `sub` points at
    // token 16u + 8q + 4hh + e, features wave*FPW + 32j + 16*sub + 4a .. +3,
    // i.e. chunk (4j + 2 sub + a/2) ^ key: j flips bits 6..7 of the byte offset
    const int s16 = lane & 15, a4 = s16 & 3, e4 = s16 >> 2, sub = (lane >> 4) & 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tok = 8 * q + 4 * hh + e4;
      o.pv[q] = tok * ROWB + 16 * ((2 * sub + (a4 >> 1)) ^ swz<C::LAT_CH>(tok)) + 8 * (a4 & 1) +
                2 * wave * C::FPW;
    }
    o.p = r * C::PROW + 16 * (hh ^ ((r >> 2) & 3));
  }
  return o;
}

// The bases are made opaque once per tile so that the compiler recomputes the
// XORs next to their reads instead of keeping every offset live in a register.
template <class C>
__device__ __forceinline__ void refresh(LaneOffs<C>& lo) {
  asm volatile("" : "+v"(lo.lat), "+v"(lo.rope), "+v"(lo.pv[0]), "+v"(lo.pv[1]), "+v"(lo.p));
}

template <class C>
__device__ __forceinline__ int pv_off(const LaneOffs<C>& lo, int q, int j, int u) {
  return (lo.pv[q] ^ (64 * (j & 3))) + C::DC * C::ESZ * 16 * u + 256 * (j >> 2);
}
template <class C>
__device__ __forceinline__ int p_rd_off(const LaneOffs<C>& lo, int hb, int u) {
  return (lo.p ^ (32 * u)) + 32 * hb * C::PROW;
}

template <class C>
struct QFrag {
  // bf16: one 8-element vector per 16-wide k block; f32: eight floats.
  typename std::conditional<C::F32, float[C::NKC][8], bf16x8[C::NKC]>::type v;
};

// Query fragments through LDS (16-bit layouts with 32 heads per wave). Lane
// (hh, r) needs 16-byte chunks 2kc + hh of head r's row for every k block kc;
// loading them directly touches 32 cache lines per instruction (one 32-byte
// piece of each head's row). Staged, each wave copies its 32 head rows with
// direct-to-LDS loads of consecutive bytes, in two halves of 36 chunks per
// row, each row padded to 37 chunks so that the 16 rows read by a quarter
// wave land on 16 distinct bank slots; then it reads its fragments.
template <class C>
struct QStage {
  static constexpr int CH = C::W * 2 / 16;            // 16-byte chunks per row
  static constexpr int HALF = CH / 2;
  static constexpr int PITCH = HALF + 1;
  static constexpr int CHUNKS = 32 * PITCH;           // per wave and half
  static constexpr int LOADS = (CHUNKS + 63) / 64;    // load instructions per half
  static constexpr int BYTES = CHUNKS * 16;
  static_assert(C::F32 || (CH % 2 == 0 && HALF % 2 == 0 && C::NKC * 2 == CH), "two halves of whole k blocks");
};

template <class C>
__device__ __forceinline__ void stage_q_issue(const DecodeParams& p, int b, int half, MLA_LDS char* region) {
  using Q = QStage<C>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* rows = (const char*)p.q_lat + ((int64_t)b * C::H + 32 * wave) * (C::W * 2) + half * Q::HALF * 16;
  const auto res = buffer_rsrc(rows, 32 * (C::W * 2));
  // LDS chunk 64 i + lane holds padded row r, chunk c; stepping i moves the
  // position by 64 = STEP_R rows + STEP_C chunks
  constexpr int STEP_R = 64 / Q::PITCH, STEP_C = 64 % Q::PITCH;
  int r = lane / Q::PITCH, c = lane % Q::PITCH;
#pragma unroll
  for (int i = 0; i < Q::LOADS; ++i) {
    const uint32_t off = r * (C::W * 2) + min(c, Q::HALF - 1) * 16;   // the pad re-reads a real chunk
    if (Q::CHUNKS % 64 == 0 || i + 1 < Q::LOADS || lane < Q::CHUNKS - 64 * (Q::LOADS - 1))
      buf_load16_to_lds(res, off, 0u, region + 64 * 16 * i);
    r += STEP_R;
    c += STEP_C;
    if (c >= Q::PITCH) { c -= Q::PITCH; r += 1; }
    asm volatile("" : "+v"(r), "+v"(c));   // computed in turn, not all up front
  }
}

template <class C, class QF>
__device__ __forceinline__ void stage_q_read(QF& q, int half, const MLA_LDS char* region) {
  using Q = QStage<C>;
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
#pragma unroll
  for (int k = 0; k < Q::HALF / 2; ++k)
    q.v[half * (Q::HALF / 2) + k] = *(const MLA_LDS bf16x8*)(region + (r * Q::PITCH + 2 * k + hh) * 16);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the region is refilled
}

template <class C>
struct State {
  f32x16 o[C::NFJ][C::HB];   // O^T: this wave's feature fragments x all head blocks
  float m_ref;     // reference maximum the exponentials are taken against (own heads)
  float m_max;     // this lane's largest base-2 scaled score
  float l;         // this lane's share of the softmax denominator
  bool overflow;   // one of this lane's scores exceeded m_ref by more than kHeadroom
};

// Scores may exceed the reference maximum by up to 2^kHeadroom before the
// exponentials could overflow fp32: with at most 2^17 tokens per split and
// |c_KV| < 2^9 every sum stays below 2^90. The reference is fixed at the first
// tile's maximum, so the accumulators are never rescaled inside the loop; in
// the rare case that a later score exceeds it by more than the headroom, the
// split is recomputed with the true maximum as reference.
constexpr float kHeadroom = 64.0f;

// Byte offset of the per-wave overflow flags in the buffer that holds the
// softmax denominators at the end of a pass (after 128 floats).
constexpr int kFinFlags = 512;

// Raw scores of one tile for this wave's 32 heads: lane (hh, c) holds tokens
// 8j + 4hh + i (accumulator 4j + i) of head 32*wave + c. The e4m3 cache keeps
// the latent part apart: it still has to be multiplied by the token's scale.
template <class C>
struct Scores {
  f32x16 lat, rope;
};

template <class C>
__device__ __forceinline__ bf16x8 qk_operand(const MLA_LDS char* buf, const LaneOffs<C>& lo, int kc) {
  const int off = kc >= C::NKC_LAT ? (lo.rope ^ (32 * (kc - C::NKC_LAT)))
                                   : (lo.lat ^ (32 * (kc & 7))) + 256 * (kc >> 3);
  return *(const MLA_LDS bf16x8*)(buf + off);
}

// One latent-sum accumulator lives in VGPRs. A wave's latent-sum accumulators
// would fill all 256 AGPRs, and the MFMA builtins keep every accumulator in
// AGPRs, so the score accumulator would not fit and the register allocator
// would shuttle accumulators between the register files every tile. The
// product for the last fragment is therefore issued with VGPR operands.
// Dependent products that accumulate into exactly the same registers need no
// wait states; VALU reads of the result wait for vgpr_acc_drain().
// The compiler inserts no wait states before inline asm, so the MFMA is
// preceded by enough of them for operands that vector instructions wrote just
// before (an MFMA reading such a register at once gets its old value).
__device__ __forceinline__ void mfma_vgpr_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 5\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The same product starting from zero (no accumulator input); the result
// registers must not overlap the operands, which the product reads over
// several passes.
__device__ __forceinline__ void mfma_vgpr_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 5\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// More wait states than the longest MFMA needs before VALU reads its result.
__device__ __forceinline__ void vgpr_acc_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

template <class C>
__device__ __forceinline__ void pv_mfma(State<C>& s, int j, int hb, const bf16x8& a, const bf16x8& b) {
  if (j == C::NFJ - 1 && hb == C::HB - 1) mfma_vgpr_acc(s.o[j][hb], a, b);
  else s.o[j][hb] = mfma32x32x16(a, b, s.o[j][hb]);
}

template <class C>
__device__ __forceinline__ void qk_mfma(Scores<C>& sc, const bf16x8& a, const QFrag<C>& q, int kc) {
  if (C::FP8 && kc >= C::NKC_LAT) sc.rope = mfma32x32x16(a, q.v[kc], sc.rope);
  else sc.lat = mfma32x32x16(a, q.v[kc], sc.lat);
}



// S^T = Rows . Q^T for one tile (k = all d_c + d_rope columns).
template <class C>
__device__ __forceinline__ Scores<C> qk_tile(const MLA_LDS char* __restrict__ buf, const QFrag<C>& q,
                                             const LaneOffs<C>& lo) {
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  Scores<C> sc;
  sc.lat = f32x16{};
  sc.rope = f32x16{};
  if constexpr (C::F32) {
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      const bool rope_part = kc >= C::NKC_LAT;
      const int kk = rope_part ? kc - C::NKC_LAT : kc;
      float a[8];
      const int byte = (16 * kk + 8 * hh) * 4;
      const int o0 = rope_part ? rope_off<C>(r, byte) : lat_off<C>(r, byte);
      const int o1 = rope_part ? rope_off<C>(r, byte + 16) : lat_off<C>(r, byte + 16);
      const f32x4 x0 = *(const MLA_LDS f32x4*)(buf + o0);
      const f32x4 x1 = *(const MLA_LDS f32x4*)(buf + o1);
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = x0[e]; a[4 + e] = x1[e]; }
      sc.lat = mfma32x32x16_f32(a, q.v[kc], sc.lat);
    }
  } else {
    // operands are read three k blocks ahead of the MFMA that consumes them
    bf16x8 a0 = qk_operand<C>(buf, lo, 0), a1 = qk_operand<C>(buf, lo, 1), a2 = qk_operand<C>(buf, lo, 2);
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      const bf16x8 a3 = kc + 3 < C::NKC ? qk_operand<C>(buf, lo, kc + 3) : bf16x8{};
      qk_mfma<C>(sc, a0, q, kc);
      a0 = a1; a1 = a2; a2 = a3;
    }
  }
  return sc;
}

// O^T[this wave's features, all heads] += C_KV^T . P^T for one tile.
template <class C>
__device__ __forceinline__ void latent_sum_tile(const MLA_LDS char* __restrict__ buf,
                                                const MLA_LDS char* __restrict__ pbuf, State<C>& s,
                                                const LaneOffs<C>& lo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (C::F32) {
#pragma unroll
      for (int j = 0; j < C::NFJ; ++j) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 16 * u + 8 * (e >> 2) + 4 * hh + (e & 3);
          a[e] = *(const MLA_LDS float*)(buf + lat_off<C>(t, (wave * C::FPW + 32 * j + r) * 4));
        }
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) {
          float pb[8];
          const f32x4 x0 = *(const MLA_LDS f32x4*)(pbuf + p_off<C>(32 * hb + r, 4 * u + 2 * hh));
          const f32x4 x1 = *(const MLA_LDS f32x4*)(pbuf + p_off<C>(32 * hb + r, 4 * u + 2 * hh + 1));
#pragma unroll
          for (int e = 0; e < 4; ++e) { pb[e] = x0[e]; pb[4 + e] = x1[e]; }
          s.o[j][hb] = mfma32x32x16_f32(a, pb, s.o[j][hb]);
        }
      }
    } else {
      constexpr int ROWB = C::DC * C::ESZ;
      bf16x8 a[C::NFJ];
#pragma unroll
      for (int j = 0; j < C::NFJ; ++j) {
        const bf16x4 v0 = lds_read_tr16(buf + pv_off<C>(lo, 0, j, u));
        const bf16x4 v1 = lds_read_tr16(buf + pv_off<C>(lo, 1, j, u));
        a[j] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int hb = 0; hb < C::HB; ++hb) {
        const bf16x8 pb = *(const MLA_LDS bf16x8*)(pbuf + p_rd_off<C>(lo, hb, u));
#pragma unroll
        for (int j = 0; j < C::NFJ; ++j) pv_mfma<C>(s, j, hb, a[j], pb);
      }
    }
  }
}

// Streaming softmax of one tile (base 2, fixed reference) and P^T to LDS.
//
// Rows past the end of a partial tile hold copies of valid rows; their
// scores are replaced by -inf. `first` (uniform): the first tile of the
// first pass sets the reference. With LATENT_SUM, the latent-sum products of the
// previous tile (`prev`, probabilities in `pr`) are issued between the
// softmax's vector instructions: they are independent, and the matrix cores
// work through them while the vector unit runs the softmax.
template <class C, bool LATENT_SUM>
__device__ __forceinline__ void softmax_tile(const MLA_LDS char* __restrict__ buf, MLA_LDS char* __restrict__ pbuf,
                                             const MLA_LDS char* __restrict__ prev,
                                             const MLA_LDS char* __restrict__ pr, const Scores<C>& sc,
                                             State<C>& s, const LaneOffs<C>& lo, int nvalid, float scale_log2,
                                             bool first) {
  // every rounding step as written, whatever the surrounding code: the
  // contiguous and paged kernels give bit-identical results
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  constexpr bool INTERLEAVE = LATENT_SUM && !C::F32;
  if constexpr (LATENT_SUM && C::F32) latent_sum_tile<C>(prev, pr, s, lo);

  // latent-sum operands and products of k step u (16 tokens of the previous tile)
  bf16x8 va[C::NFJ];
  auto pv_load = [&](int u) {
#pragma unroll
    for (int j = 0; j < C::NFJ; ++j) {
      const bf16x4 v0 = lds_read_tr16(prev + pv_off<C>(lo, 0, j, u));
      const bf16x4 v1 = lds_read_tr16(prev + pv_off<C>(lo, 1, j, u));
      va[j] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto pv_block = [&](int u, int hb) {
    const bf16x8 pb = *(const MLA_LDS bf16x8*)(pr + p_rd_off<C>(lo, hb, u));
#pragma unroll
    for (int j = 0; j < C::NFJ; ++j) pv_mfma<C>(s, j, hb, va[j], pb);
  };
  float tok_scale[16];
  if constexpr (C::FP8) {
    const MLA_LDS float* scl = (const MLA_LDS float*)(buf + C::LAT_BYTES + C::ROPE_BYTES);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = *(const MLA_LDS f32x4*)(scl + 8 * j + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) tok_scale[4 * j + i] = v[i];
    }
  }
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = C::FP8 ? (tok_scale[i] * sc.lat[i] + sc.rope[i]) : sc.lat[i];
    x[i] = v * scale_log2;
  }
  // tokens past the end of a partial tile (uniform) score -inf: they take
  // part in neither the maxima nor the sums
  if (nvalid < C::T) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
      x[i] = tok < nvalid ? x[i] : -INFINITY;
    }
  }
  // from here on one basic block: the scheduler can interleave the softmax
  // with the latent-sum MFMAs
  if constexpr (INTERLEAVE) { pv_load(0); pv_block(0, 0); }
  if constexpr (INTERLEAVE) pv_block(0, 1);
  float mt = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mt = fmaxf(mt, x[i]);
  const float m_first = wave_max32(mt);   // lanes r and r + 32 hold one head
  s.m_ref = first ? m_first : s.m_ref;
  s.m_max = fmaxf(s.m_max, mt);
  s.overflow = s.overflow || (mt > s.m_ref + kHeadroom);
  if constexpr (INTERLEAVE) pv_block(0, 2);
  float pr_[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) pr_[i] = fast_exp2(x[i] - s.m_ref);
  if constexpr (INTERLEAVE) { pv_block(0, 3); pv_load(1); pv_block(1, 0); }
#pragma unroll
  for (int i = 8; i < 16; ++i) pr_[i] = fast_exp2(x[i] - s.m_ref);
  if constexpr (INTERLEAVE) pv_block(1, 1);
  float q4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q4[j] = (pr_[4 * j] + pr_[4 * j + 1]) + (pr_[4 * j + 2] + pr_[4 * j + 3]);
  s.l += (q4[0] + q4[1]) + (q4[2] + q4[3]);
  if constexpr (C::FP8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) pr_[i] *= tok_scale[i];
  }
  if constexpr (INTERLEAVE) pv_block(1, 2);

  // P^T rows of this wave's heads: element e of k step u is token
  // 16u + 8(e/4) + 4hh + e%4, i.e. pr_[8u + e].
  const int head = 32 * wave + r;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (C::F32) {
      f32x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) { v0[e] = pr_[8 * u + e]; v1[e] = pr_[8 * u + 4 + e]; }
      *(MLA_LDS f32x4*)(pbuf + p_off<C>(head, 4 * u + 2 * hh)) = v0;
      *(MLA_LDS f32x4*)(pbuf + p_off<C>(head, 4 * u + 2 * hh + 1)) = v1;
    } else {
      u32x4 v;
#pragma unroll
      for (int d = 0; d < 4; ++d) v[d] = pack_bf16x2(pr_[8 * u + 2 * d], pr_[8 * u + 2 * d + 1]);
      *(MLA_LDS u32x4*)(pbuf + p_off<C>(head, 2 * u + hh)) = v;
    }
  }
  if constexpr (INTERLEAVE) pv_block(1, 3);
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if constexpr (N == 27) asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
  else static_assert(N == 0, "add the vmcnt value here");
}

// Workgroup barrier for the tile loop. LDS stores of this wave are drained
// first; the direct HBM->LDS loads are waited for explicitly by the caller
// (s_waitcnt vmcnt), so no fence has to drain every load still in flight.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One step of the software-pipelined tile loop, t = 0 .. ntiles - 1:
//   (bf16) start loading tile t + 2 into the slot freed by tile t - 2;
//   scores of tile t;
//   softmax of tile t, P^T(t) to LDS, interleaved with the latent sum of
//   tile t - 1 (t > 0);
//   make tile t + 1 resident (e4m3: widen it into its slot and start tile t + 2);
//   barrier.
// The ring slots are distinct buffers (for the three-slot e4m3 ring, `fill`
// and `prev` share a slot, but only the rotary/scale part of `fill` and only
// the latent part of `prev` are touched). __restrict__ tells the compiler
// that LDS reads of one slot need not wait for the loads into another; the
// explicit vmcnt wait before the barrier is what makes tile t + 1 resident.
template <class C, bool PAGED, bool FIRST>
__device__ __forceinline__ void tile_step(const DecodeParams& p, const MLA_LDS char* __restrict__ cur,
                                          const MLA_LDS char* __restrict__ prev, MLA_LDS char* __restrict__ next,
                                          MLA_LDS char* __restrict__ fill, MLA_LDS char* __restrict__ pw,
                                          const MLA_LDS char* __restrict__ pr, const QFrag<C>& q, State<C>& s,
                                          LaneOffs<C>& lo, const SeqView& sv, DmaOffs& dma, Fp8Stage<C>& st,
                                          int t, int ntiles, int start, int end, bool first) {
  constexpr int LPT = loads_per_tile<C>();
  refresh<C>(lo);
  asm volatile("" : "+v"(dma.lat));
  if constexpr (!C::FP8)
    if (t + 2 < ntiles) issue_tile<C, PAGED>(p, sv, dma, fill, start + (t + 2) * C::T, end, st);
  const Scores<C> sc = qk_tile<C>(cur, q, lo);
  softmax_tile<C, !FIRST>(cur, pw, prev, pr, sc, s, lo, end - (start + t * C::T), p.scale_log2, first);
  if (t + 1 < ntiles) {
    if constexpr (C::FP8) {
      wait_vmem_le<0>();
      commit_tile<C>(next, st);
      if (t + 2 < ntiles) issue_tile<C, PAGED>(p, sv, dma, fill, start + (t + 2) * C::T, end, st);
    } else {
      if (t + 2 < ntiles) wait_vmem_le<LPT>();
      else wait_vmem_le<0>();
    }
  }
  tile_barrier();
}

// The partner lane 32 away (lanes r and r + 32 hold the two token halves of
// one head): v_permlane32_swap, a vector instruction, no LDS round trip.
__device__ __forceinline__ float lane32_partner(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  // lanes 0..31 find the upper half's value in the second result, lanes
  // 32..63 the lower half's in the first
  return __builtin_bit_cast(float, (uint32_t)((threadIdx.x & 32) ? sw[0] : sw[1]));
}

// Exchange between the two halves of the wave: lane r + 32's `lo` becomes
// lane r's `hi`, and lane r's `hi` becomes lane r + 32's `lo`
// (v_permlane32_swap of `lo` in the upper half with `hi` in the lower half).
__device__ __forceinline__ void swap_lane_halves(uint32_t& lo, uint32_t& hi) {
  const auto sw = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
  lo = sw[0];
  hi = sw[1];
}

// The 32 latent-sum MFMAs of one tile, m = 0..31 (k step u = m / 16, head
// block hb = m / 4 % 4, feature fragment j = m % 4), with their operand reads
// scheduled ahead of use: the P^T operand of head block b + 1 at MFMA 4b, the
// C_KV^T operands of k step 1 at MFMAs 10..13. va[0] and pb[0] are read by the
// caller before MFMA 0.
template <class C, bool CODES = false>
struct PvSched {
  State<C>& s;
  bf16x8 (&va)[2][C::NFJ];
  bf16x8 (&pb)[2];
  const MLA_LDS char* __restrict__ prev;
  const MLA_LDS char* __restrict__ pr;
  const LaneOffs<C>& lo;
  i32x2 raw1[C::NFJ];   // e4m3 codes of k step 1, widened at their first use
  __device__ __forceinline__ void read_pb(int blk) {
    pb[blk & 1] = *(const MLA_LDS bf16x8*)(pr + p_rd_off<C>(lo, blk & 3, blk >> 2));
  }
  __device__ __forceinline__ void read_va(int u, int j) {
    if constexpr (CODES) {
      const i32x2 w = lds_read_tr8(prev + ((lo.pv[0] ^ (32 * j)) + C::DC * 16 * u));
      if (u == 0) va[0][j] = e4m3x8_to_bf16x8(w);
      else raw1[j] = w;
    } else {
      const bf16x4 v0 = lds_read_tr16(prev + pv_off<C>(lo, 0, j, u));
      const bf16x4 v1 = lds_read_tr16(prev + pv_off<C>(lo, 1, j, u));
      va[u][j] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  __device__ __forceinline__ void step(int m) {
    if (m % 4 == 0 && m / 4 + 1 < 8) read_pb(m / 4 + 1);
    if (m >= 10 && m < 14) read_va(1, m - 10);
    if constexpr (CODES) {
      // k step 1's operands replace k step 0's, which are dead from MFMA 16 on
      if (m >= 16 && m < 20) va[0][m - 16] = e4m3x8_to_bf16x8(raw1[m - 16]);
      pv_mfma<C>(s, m & 3, (m >> 2) & 3, va[0][m & 3], pb[(m >> 2) & 1]);
    } else {
      pv_mfma<C>(s, m & 3, (m >> 2) & 3, va[m >> 4][m & 3], pb[(m >> 2) & 1]);
    }
  }
};

// Latent-sum MFMAs of tile t - 1 that may be issued in the tail of the score
// phase of tile t (bound by LDS reads, so the matrix cores have room); the
// rest run in phase two. Measured on MI355X, moving some of them early was no
// faster than none, so none are.
constexpr int kPvEarly = 0;

// Phase two of the streaming step: the softmax of tile t on the vector unit,
// interleaved group by group with the remaining latent-sum MFMAs of tile
// t - 1. A wave issues in order, so a run of MFMAs holds back the vector work
// queued behind it; here each MFMA is followed by a few vector instructions
// that execute while it runs, and scheduling barriers keep the compiler from
// regrouping them. The arithmetic is that of softmax_tile in the same order,
// so contiguous and paged caches give identical bits.
// E4M3: the scores are fs (s_t lat + rope) (see QF8), with the tile's
// per-token scales s_t in `scl` (token 8 w + i at float 64 w + i), and the
// probabilities enter the latent sum times s_t once the denominator has taken
// them. `scale_log2` is fs there; fs >= 0, so the maximum is taken over the
// unscaled scores and each probability is exp2(fma(score, fs, -m)), one
// instruction fewer per score.
template <class C, bool E4M3, class PS>
__device__ __forceinline__ void softmax_pv_stream(PS& pvs, MLA_LDS char* __restrict__ pw, const Scores<C>& sc,
                                                  State<C>& s, int nvalid, float scale_log2, bool first,
                                                  const MLA_LDS float* __restrict__ scl, f32x4 sg_next = {}) {
#pragma clang fp contract(off)
  static_assert(!C::F32 && !C::FP8 && C::NFJ == 4 && C::HB == 4, "32 latent-sum MFMAs, 16 scores per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  auto sync = [] { __builtin_amdgcn_sched_barrier(0); };
  // vector group g runs beside latent-sum MFMA kPvEarly + g (if any is left)
  auto mfma = [&](int g) {
    if (kPvEarly + g < 32) pvs.step(kPvEarly + g);
  };
  float x[16], a[8], pv[16];
  // scaled scores (e4m3: times the token's r, element i of group g being
  // token 8 g + 4 hh + i)
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    mfma(g);
    if constexpr (E4M3) {
      // scales of tokens 8 g + 4 hh + 0..3, read one group ahead (the
      // caller reads group 0's)
      const f32x4 sg = sg_next;
      if (g < 3) sg_next = *(const MLA_LDS f32x4*)(scl + 64 * (g + 1) + 4 * hh);
#pragma unroll
      for (int i = 4 * g; i < 4 * g + 4; ++i) x[i] = __builtin_fmaf(sc.lat[i], sg[i - 4 * g], sc.rope[i]);
    } else {
#pragma unroll
      for (int i = 4 * g; i < 4 * g + 4; ++i) x[i] = sc.lat[i] * scale_log2;
    }
    sync();
  }
  // maximum over this lane's 16 tokens (exact in any order)
  mfma(4);
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = fmaxf(x[2 * k], x[2 * k + 1]);
  sync();
  mfma(5);
#pragma unroll
  for (int k = 4; k < 8; ++k) a[k] = fmaxf(x[2 * k], x[2 * k + 1]);
  sync();
  mfma(6);
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = fmaxf(a[2 * k], a[2 * k + 1]);
  sync();
  mfma(7);
  // e4m3: the maximum of the unscaled scores times fs >= 0 (see split_query_f8)
  const float mt = E4M3 ? fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])) * scale_log2
                       : fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
  sync();
  mfma(8);
  const float m_first = fmaxf(mt, lane32_partner(mt));
  s.m_ref = first ? m_first : s.m_ref;
  s.m_max = fmaxf(s.m_max, mt);
  s.overflow = s.overflow || (mt > s.m_ref + kHeadroom);
  sync();
  // probabilities, two per MFMA
  f32x4 sj_next = {};
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    mfma(9 + g);
    if (E4M3 && g == 6) sj_next = *(const MLA_LDS f32x4*)(scl + 4 * hh);
    pv[2 * g] = E4M3 ? fast_exp2(__builtin_fmaf(x[2 * g], scale_log2, -s.m_ref)) : fast_exp2(x[2 * g] - s.m_ref);
    pv[2 * g + 1] = E4M3 ? fast_exp2(__builtin_fmaf(x[2 * g + 1], scale_log2, -s.m_ref))
                         : fast_exp2(x[2 * g + 1] - s.m_ref);
    sync();
  }
  if (nvalid < C::T) {    // partial tile (uniform): tokens past the end weigh nothing
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
      pv[i] = tok < nvalid ? pv[i] : 0.0f;
    }
  }
  sync();
  float q4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mfma(17 + j);
    q4[j] = (pv[4 * j] + pv[4 * j + 1]) + (pv[4 * j + 2] + pv[4 * j + 3]);
    if constexpr (E4M3) {
      // the denominator has taken them; the latent sum takes them times
      // their tokens' scales (tokens 8 j + 4 hh + 0..3, read one group ahead)
      const f32x4 sj = sj_next;
      if (j < 3) sj_next = *(const MLA_LDS f32x4*)(scl + 64 * (j + 1) + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[4 * j + i] *= sj[i];
    }
    sync();
  }
  mfma(21);
  s.l += (q4[0] + q4[1]) + (q4[2] + q4[3]);
  sync();
  // P^T rows of this wave's heads: element e of k step u is token
  // 16u + 8(e/4) + 4hh + e%4, i.e. pv[8u + e]
  u32x4 pk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    mfma(22 + u);
#pragma unroll
    for (int d = 0; d < 4; ++d) pk[u][d] = pack_bf16x2(pv[8 * u + 2 * d], pv[8 * u + 2 * d + 1]);
    sync();
  }
  mfma(24);
  const int head = 32 * wave + r;
#pragma unroll
  for (int u = 0; u < 2; ++u) *(MLA_LDS u32x4*)(pw + p_off<C>(head, 2 * u + hh)) = pk[u];
  sync();
#pragma unroll
  for (int g = 25; g < 32; ++g) mfma(g);
}

// Where the streamed tiles of one split start. A contiguous cache adds the
// tile's first token to the sequence's first row. A paged cache with pages of
// at least 32 tokens (so that no tile straddles two pages) looks the page up
// in `pages`, which holds the split's physical page ids one per lane (lane i:
// logical page lp0 + i), loaded once per workgroup and read with readlane.
struct TileBase {
  const char* base;   // contiguous: the sequence's first row; paged: the pool's
  int shift, lp0;     // paged: log2(page size), the split's first logical page
  int pages;          // paged: this lane's physical page id
};

// Loads of one tile of a 16-bit cache (32 consecutive rows): a scalar tile
// address plus 32-bit lane offsets. Tiles past the end of the split are
// clamped to its last tile, and rows past the split's end repeat its last
// row, so every tile costs every thread the same nine loads.
template <class C>
struct StreamTile {
  __amdgpu_buffer_rsrc_t res;   // the tile's 32 rows
  int last, rs;
  template <bool PAGED>
  __device__ __forceinline__ StreamTile(const DecodeParams& p, const TileBase& tbase, int t, int ntiles, int start,
                                        int end, std::integral_constant<bool, PAGED>) {
    const int tb = start + min(t, ntiles - 1) * C::T;
    last = min(end - tb, C::T) - 1;
    rs = (int)(p.row_stride * C::ESZ);
    const char* tile;
    if constexpr (PAGED) {
      const int64_t pg = __builtin_amdgcn_readlane(tbase.pages, (tb >> tbase.shift) - tbase.lp0);
      tile = tbase.base + ((pg << tbase.shift) + (tb & ((1 << tbase.shift) - 1))) * rs;
    } else {
      tile = tbase.base + (int64_t)tb * rs;
    }
    res = buffer_rsrc(tile, (uint32_t)(C::T * rs));   // rows are at most 2^24 bytes apart
  }
  // latent row 4k + wave (one 1 KiB row per wave instruction)
  __device__ __forceinline__ void latent(const DmaOffs& dma, MLA_LDS char* fill, int wave, int k) const {
    const int row = min(k * C::WAVES + wave, last);
    buf_load16_to_lds(res, (uint32_t)(dma.lat ^ (16 * (k & 3))), (uint32_t)(row * rs),
                      fill + (k * C::WAVES + wave) * (C::DC * C::ESZ));
  }
  // rotary parts: 8 lanes per row, rows tid / 8
  __device__ __forceinline__ void rope(const DmaOffs& dma, MLA_LDS char* fill, int wave) const {
    const int row = min((int)(threadIdx.x >> 3), last);
    buf_load16_to_lds(res, (uint32_t)(row * rs + dma.rope_chunk), 0u, fill + C::LAT_BYTES + wave * 64 * 16);
  }
  __device__ __forceinline__ void all(const DmaOffs& dma, MLA_LDS char* fill, int wave) const {
#pragma unroll
    for (int k = 0; k < C::T / C::WAVES; ++k) latent(dma, fill, wave, k);
    rope(dma, fill, wave);
  }
};

// An e4m3 cache streamed as codes (contiguous layout). The codes stay e4m3 in
// LDS: the scores take them directly as fp8 MFMA operands against an exact
// two-part e4m3 split of the query (QF8), and the latent sum widens them in
// registers (exact) after a byte-transposing read. The per-token scale s
// multiplies each token's latent score and, after the denominator has taken
// the probabilities, each probability that enters the latent sum.
// LDS: the two P^T buffers first, then a ring of NSLOT tile slots, each
//   codes:  32 rows x 512 bytes, 16-byte chunk c of row t at c ^ key8(t);
//   rotary: the bf16 rows in the 16-bit tile's layout;
//   scales: one 256-byte row per wave, token 8 w + i at float 64 w + i.
// The query is staged from the third slot on, clear of tiles 0 and 1, and the
// bf16 output rows are staged after the P^T buffers (where the denominators
// are) at the end.
template <class C>
struct F8Ring {
  static constexpr int CODES = C::T * C::DC;                  // one byte per code
  static constexpr int ROPE = CODES;                          // offset of the rotary rows in a slot
  static constexpr int SCL = ROPE + C::ROPE_BYTES;            // offset of the scales
  static constexpr int SLOT = SCL + C::WAVES * 256;
  static constexpr int NSLOT = 5, AHEAD = NSLOT - 2;          // tiles in flight beyond the next one
  static constexpr int P = 0, S0 = 2 * C::P_BYTES;            // P^T buffers, first slot
  static constexpr int LPT = 6;                               // loads per thread and tile
  static constexpr int QROPE = S0 + NSLOT * SLOT;             // per wave: the query's rotary fragments
  static constexpr int QROPE_BYTES = C::NKC_ROPE * 64 * 16;
  static constexpr int STAGE = S0;                            // output staging at the end
  static_assert(!C::F32 && !C::FP8 && C::WAVES == 4 && C::T == 32 && C::DC == 512, "DeepSeek-V2 shapes");
  static_assert(QROPE + C::WAVES * QROPE_BYTES <= C::LDS_BYTES, "LDS budget");
  static_assert(S0 + 2 * SLOT + C::WAVES * QStage<C>::BYTES <= C::LDS_BYTES, "staged query after slots 0, 1");
  static_assert(CODES == C::THREADS * 4 * 16, "four 16-byte code chunks per thread");
};

// Swizzle key of code row t (512-byte rows, 16-byte chunks): bits (3, 1, 0, 2)
// of t mod 16. The score reads (16 consecutive rows at one chunk) and the
// transposing reads of the latent sum (8 rows of one 4-row parity at two
// neighbouring chunks, or 16 rows at one chunk) all land on distinct slots.
__device__ __forceinline__ int key8(int t) { return (t & 8) | ((t & 3) << 1) | ((t >> 2) & 1); }

// Loads of one e4m3 tile: wave w, lane i loads code chunk i % 32 of rows
// 8w + 2k + i / 32 (k = 0..3: two whole 512-byte rows per instruction), the
// scales of rows 8w .. 8w + 7 (lanes 0..7, repeated) and the rotary chunks of
// rows 8w .. 8w + 7. Rows past the split's end repeat its last row (their
// scores repeat a valid score, so the maxima are unchanged, and the softmax
// zeroes their probabilities); a tile past the end has an empty buffer and
// reads nothing.
template <class C>
struct F8Tile {
  __amdgpu_buffer_rsrc_t codes_res, scale_res, rope_res;
  int rs, rs2, last;
  __device__ __forceinline__ F8Tile(const DecodeParams& p, int64_t seq_row, int t, int start, int end) {
    // uniform by construction; stated, so that the resources stay scalar
    // (a resource the compiler takes for divergent costs a loop per load)
    const int tb = __builtin_amdgcn_readfirstlane(start + t * C::T);
    const int nv = __builtin_amdgcn_readfirstlane(max(0, min(end - tb, C::T)));   // rows inside the split
    last = max(nv - 1, 0);
    const int64_t row0 = (int64_t)__builtin_amdgcn_readfirstlane((int)seq_row) +
                         ((int64_t)__builtin_amdgcn_readfirstlane((int)(seq_row >> 32)) << 32) + tb;
    rs = (int)p.row_stride;
    rs2 = (int)(p.rope_stride * 2);
    codes_res = buffer_rsrc((const char*)p.latent + row0 * p.row_stride, (uint32_t)(nv * rs));
    scale_res = buffer_rsrc(p.scale + row0, (uint32_t)(nv * 4));
    rope_res = buffer_rsrc((const char*)p.rope + row0 * (p.rope_stride * 2), (uint32_t)(nv * rs2));
  }
  // lane (h, c) fills LDS row r = 8w + 2k + h, chunk c, with code chunk
  // c ^ key8(r) = (c ^ 2h) ^ K, K = 8 (w & 1) | 4 (k & 1) | k / 2, of cache
  // row min(r, last); lo16 = 16 (c ^ 2h) and h come from the caller
  __device__ __forceinline__ void codes(MLA_LDS char* slot, int wave, int k, int lo16, int h) const {
    const int K = 8 * (wave & 1) | 4 * (k & 1) | (k >> 1);
    const int r0 = 8 * wave + 2 * k;
    const uint32_t row = (uint32_t)min(r0 + h, last);
    buf_load16_to_lds(codes_res, __umul24(row, (uint32_t)rs) + (uint32_t)(lo16 ^ (16 * K)), 0u, slot + r0 * C::DC);
  }
  // row8 = 8w + lane % 8
  __device__ __forceinline__ void scales(MLA_LDS char* slot, int wave, int row8) const {
    buf_load4_to_lds(scale_res, (uint32_t)(4 * min(row8, last)), 0u, slot + F8Ring<C>::SCL + wave * 256);
  }
  // row = tid / 8, chunk = this thread's swizzled rotary chunk (bytes)
  __device__ __forceinline__ void rope(MLA_LDS char* slot, int wave, int row, int chunk) const {
    buf_load16_to_lds(rope_res, __umul24((uint32_t)min(row, last), (uint32_t)rs2) + (uint32_t)chunk, 0u,
                      slot + F8Ring<C>::ROPE + wave * 64 * 16);
  }
};

// Per-lane load offsets of the e4m3 tiles (constant over the loop).
struct F8LoadOffs {
  int lo16;    // 16 ((lane % 32) ^ 2 (lane / 32))
  int h;       // lane / 32
  int row8;    // 8 wave + lane % 8
  int rrow;    // tid / 8
  int rchunk;  // this thread's swizzled rotary chunk (bytes)
};

template <class C>
__device__ __forceinline__ F8LoadOffs f8_load_offsets(const DmaOffs& dma) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  F8LoadOffs o;
  o.lo16 = 16 * ((lane & 31) ^ (2 * h));
  o.h = h;
  o.row8 = 8 * wave + (lane & 7);
  o.rrow = tid >> 3;
  o.rchunk = dma.rope_chunk - C::DC * C::ESZ;
  return o;
}

// Per-lane LDS offsets of the e4m3 loop (the LaneOffs fields, reused):
//  lat:   score operand of latent block b (64 codes), half x: (lat ^ 64 b) ^ 16 x
//         (lane (g, r): row r, bytes 64 b + 32 g .. + 31);
//  rope:  rotary score operand of k block kk: rope ^ 32 kk (as the 16-bit tile);
//  pv[0]: transposing read of C_KV^T fragment j, k step u: (pv[0] ^ 32 j) + 8 KiB u;
//  p:     P^T reads, as in the 16-bit loop.
// Transposing reads: source lane (a, k) of 16-lane group G = 2 hh + sub points
// at token 8 (k / 4) + 4 hh + k % 4 (+ 16 u) and bytes 128 w + 32 j + 16 sub
// + 8 a .. + 7, so that lane (G, x) receives feature 128 w + 32 j + 16 sub + x
// of the tokens that element e of the P^T operand of lane half hh stands for.
template <class C>
__device__ __forceinline__ LaneOffs<C> lane_offsets_f8(int wave) {
  LaneOffs<C> o = lane_offsets<C>(wave);
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  o.lat = r * C::DC + 16 * ((2 * hh) ^ key8(r));
  o.rope = o.rope - C::LAT_BYTES + F8Ring<C>::ROPE;
  const int G = lane >> 4, x = lane & 15, sub = G & 1, hg = G >> 1, k = x >> 1, a = x & 1;
  const int tok = 8 * (k >> 2) + 4 * hg + (k & 3);
  o.pv[0] = (tok * C::DC + 16 * (sub ^ key8(tok)) + 8 * a) ^ (128 * wave);
  o.pv[1] = 0;
  return o;
}

// Block b's chunks sit at base ^ 64 b: the base holds no bit 8 (the key
// flips chunk bits 0..3), so the high bit of b is an offset of 256 bytes.
template <class T>
__device__ __forceinline__ T* opaque_lds(T* p) {
  uint32_t v = (uint32_t)(size_t)p;
  asm volatile("" : "+s"(v));
  return (T*)(size_t)v;
}

__device__ __forceinline__ i32x8 code_operand(const MLA_LDS char* buf, int base, int b) {
  const int o = (base ^ (64 * (b & 3))) + 256 * (b >> 2);
  const int o1 = (base ^ (64 * (b & 3)) ^ 16) + 256 * (b >> 2);
  const u32x4 x0 = *(const MLA_LDS u32x4*)(buf + o);
  const u32x4 x1 = *(const MLA_LDS u32x4*)(buf + o1);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <class C>
__device__ __forceinline__ bf16x8 pv_operand_f8(const MLA_LDS char* buf, const LaneOffs<C>& lo, int j, int u) {
  return e4m3x8_to_bf16x8(lds_read_tr8(buf + ((lo.pv[0] ^ (32 * j)) + C::DC * 16 * u)));
}

// The absorbed query of this wave's 32 heads as operands of the fp8 score
// products (the rotary fragments, 16 bytes per lane and k block, go to the
// wave's F8Ring::QROPE region, lane l's fragment kk at 16 (64 kk + l)). Head n's latent part is split exactly as q = 2^e (hi + 2^-4 lo)
// with hi, lo e4m3 and e per head (its largest |q| / 2^e in [128, 256)): hi
// rounds q / 2^e to four significant bits, and what a bf16 value has beyond
// them, at most four more bits, is lo (exact for values down to 2^13 below
// the head's largest; smaller ones round to e4m3's subnormal spacing). The
// rotary part stays bf16, times 2^-e, so that the scaled score of token t is
// fs (s_t (hi + 2^-4 lo) . codes + 2^-e q_R . k_R) with one factor fs = 2^e
// |scale| log2(e) per lane (a negative scale negates the query instead).
template <class C>
struct QF8 {
  i32x8 hi[C::DC / 64], lo[C::DC / 64];   // block b: lane (g, n) holds k = 64 b + 32 g .. + 31 of head n
  float fs;
};

// The staged bf16 query as read from LDS: latent block b, 16-byte chunk c of
// lane (g, n) is chunk 8 b + 4 g + c of head n's row; the rotary fragments as
// the 16-bit loop reads them.
template <class C>
struct QRaw {
  u32x4 v[C::DC / 64][4];
  bf16x8 rope[C::NKC_ROPE];
};

// One staged half (chunks 0 .. 35 or 36 .. 71 of each head row). The block
// that straddles the halves (b = 4) is chunks 32 .. 35 for lane half g = 0
// and 36 .. 39 for g = 1: each lane keeps the read from its own half.
template <class C>
__device__ __forceinline__ void stage_q_read_f8(QRaw<C>& q, int half, const MLA_LDS char* region) {
  using Q = QStage<C>;
  const int lane = threadIdx.x & 63, g = lane >> 5, r = lane & 31;
  auto rd = [&](int chunk) { return *(const MLA_LDS u32x4*)(region + (r * Q::PITCH + chunk) * 16); };
#pragma unroll
  for (int b = 0; b < C::DC / 64; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch0 = 8 * b + c;   // chunk of lane half 0; half 1 adds 4
      if (ch0 + 4 < Q::HALF) {
        if (half == 0) q.v[b][c] = rd(ch0 + 4 * g);
      } else if (ch0 >= Q::HALF) {
        if (half == 1) q.v[b][c] = rd(ch0 + 4 * g - Q::HALF);
      } else if (half == 0) {
        const u32x4 x = rd(min(ch0 + 4 * g, Q::HALF - 1));
        if (g == 0) q.v[b][c] = x;
      } else {
        const u32x4 x = rd(max(ch0 + 4 * g - Q::HALF, 0));
        if (g == 1) q.v[b][c] = x;
      }
    }
  if (half == 1) {
#pragma unroll
    for (int kk = 0; kk < C::NKC_ROPE; ++kk)
      q.rope[kk] = *(const MLA_LDS bf16x8*)(region + (r * Q::PITCH + 2 * (C::NKC_LAT + kk) + g - Q::HALF) * 16);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the region is refilled
}

__device__ __forceinline__ float pow2i(int e) {   // 2^e, -126 <= e <= 127
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

template <class C>
__device__ __forceinline__ void split_query_f8(QF8<C>& q, const QRaw<C>& raw, float scale_log2,
                                               MLA_LDS char* __restrict__ qrope) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  // largest magnitude of the head (latent and rotary parts): bf16 magnitudes
  // order as 15-bit integers
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int b = 0; b < C::DC / 64; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, raw.v[b][c][d] & 0x7fff7fffu));
#pragma unroll
  for (int kk = 0; kk < C::NKC_ROPE; ++kk) {
    const u32x4 w = __builtin_bit_cast(u32x4, raw.rope[kk]);
#pragma unroll
    for (int d = 0; d < 4; ++d) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[d] & 0x7fff7fffu));
  }
  uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]);
  m = max(m, (uint32_t)__shfl_xor((int)m, 32));   // lanes n and n + 32 hold one head
  // largest / 2^e in [128, 256): e = exponent(largest) - 7
  const int e = max((int)(m >> 7) - 134, -120);
  // a negative softmax scale is carried by the query (every sign flipped), so
  // that fs = 2^e |scale| log2 e is never negative
  const uint32_t flip = scale_log2 < 0.0f ? 0x80008000u : 0u;
  const float sh = pow2i(e), sl = pow2i(e - 4), inv = pow2i(-e);
#pragma unroll
  for (int b = 0; b < C::DC / 64; ++b) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w0 = raw.v[b][d >> 1][2 * (d & 1)] ^ flip, w1 = raw.v[b][d >> 1][2 * (d & 1) + 1] ^ flip;
      const float x0 = __builtin_bit_cast(float, w0 << 16), x1 = __builtin_bit_cast(float, w0 & 0xffff0000u);
      const float x2 = __builtin_bit_cast(float, w1 << 16), x3 = __builtin_bit_cast(float, w1 & 0xffff0000u);
      i16x2v h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2v{0, 0}, x0, x1, sh, false);
      h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x2, x3, sh, true);
      const int hw = __builtin_bit_cast(int, h);
      const f32x2 b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, sh, false);
      const f32x2 b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, sh, true);
      i16x2v l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2v{0, 0}, x0 - b01[0], x1 - b01[1], sl, false);
      l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x2 - b23[0], x3 - b23[1], sl, true);
      q.hi[b][d] = hw;
      q.lo[b][d] = __builtin_bit_cast(int, l);
    }
  }
#pragma unroll
  for (int kk = 0; kk < C::NKC_ROPE; ++kk) {
    const u32x4 w = __builtin_bit_cast(u32x4, raw.rope[kk]) ^ flip;
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      o[d] = pack_bf16x2(bf16_bits_to_f32(w[d] & 0xffffu) * inv, bf16_bits_to_f32(w[d] >> 16) * inv);
    *(MLA_LDS u32x4*)(qrope + (kk * 64 + (threadIdx.x & 63)) * 16) = o;
  }
  q.fs = sh * fabsf(scale_log2);
}

struct NoF8Ring {   // stands in where no e4m3 ring is used
  static constexpr int S0 = 0, P = 0, SLOT = 0, NSLOT = 1, AHEAD = 0, LPT = 0, STAGE = 0, QROPE = 0,
                       QROPE_BYTES = 0;
};

// Steady state for a contiguous 16-bit cache: one basic block per tile.
// The nine direct loads of tile t + 2 are spread through the score MFMAs of
// tile t, so the load issue overlaps the LDS reads and the matrix cores; the
// latent-sum MFMAs of tile t - 1 then run while the vector unit computes the
// softmax of tile t. Past the end of the split the loads fetch the last tile
// again (its rows are still in L2 and its slot is not read), which keeps the
// per-thread load count, and with it the vmcnt wait, the same for every tile.
template <class C, bool PAGED>
__device__ __forceinline__ void tile_step_stream(const DecodeParams& p, const MLA_LDS char* __restrict__ cur,
                                                 const MLA_LDS char* __restrict__ prev,
                                                 MLA_LDS char* __restrict__ fill, MLA_LDS char* __restrict__ pw,
                                                 const MLA_LDS char* __restrict__ pr, const QFrag<C>& q,
                                                 State<C>& s, LaneOffs<C>& lo, DmaOffs& dma, const TileBase& tbase,
                                                 int t, int ntiles, int start, int end, bool first) {
  static_assert(!C::F32 && !C::FP8 && C::LAT_CH == 64 && C::WAVES == 4, "16-bit DeepSeek-V2 layout");
  constexpr int LPT = loads_per_tile<C>();
  static_assert(LPT == C::T / C::WAVES + 1, "nine loads per tile");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  refresh<C>(lo);
  asm volatile("" : "+v"(dma.lat), "+v"(dma.rope_chunk));

  const StreamTile<C> ld(p, tbase, t + 2, ntiles, start, end, std::integral_constant<bool, PAGED>{});   // tile t + 2
  Scores<C> sc;
  sc.lat = f32x16{};
  sc.rope = f32x16{};
  constexpr int LAT_LOADS = C::T / C::WAVES;
  static_assert(C::NKC >= 4 * LAT_LOADS + 1, "one latent load every four score MFMAs");
  bf16x8 va[2][C::NFJ], pb[2];
  PvSched<C> pvs{s, va, pb, prev, pr, lo};
  // operands of the first latent-sum MFMAs are read during the score MFMAs
  constexpr int PV0 = C::NKC - kPvEarly;      // score step of the first early latent-sum MFMA
  constexpr int PF = PV0 - 8;                 // score step of the first operand read
  static_assert(PF >= 0, "room for the operand reads");
  bf16x8 a0 = qk_operand<C>(cur, lo, 0), a1 = qk_operand<C>(cur, lo, 1), a2 = qk_operand<C>(cur, lo, 2);
#pragma unroll
  for (int kc = 0; kc < C::NKC; ++kc) {
    if (kc % 4 == 0 && kc / 4 < LAT_LOADS) ld.latent(dma, fill, wave, kc / 4);
    if (kc == 4 * LAT_LOADS) ld.rope(dma, fill, wave);
    if (kc >= PF + 2 && kc < PF + 6) pvs.read_va(0, kc - (PF + 2));
    if (kc == PF + 6) pvs.read_pb(0);
    const bf16x8 a3 = kc + 3 < C::NKC ? qk_operand<C>(cur, lo, kc + 3) : bf16x8{};
    qk_mfma<C>(sc, a0, q, kc);
    a0 = a1; a1 = a2; a2 = a3;
    if (kc >= PV0) pvs.step(kc - PV0);
  }
  __builtin_amdgcn_sched_barrier(0);
  softmax_pv_stream<C, false>(pvs, pw, sc, s, end - (start + t * C::T), p.scale_log2, first, nullptr);
  wait_vmem_le<LPT>();
  tile_barrier();
}

// Steady state for a contiguous e4m3 cache (F8Ring), one basic block per
// tile. Step t requests tile t + AHEAD (its six loads spread through the
// score products), scores tile t with fp8 products of the codes against the
// split query (eight latent blocks of 64 codes, hi and lo, then the four
// rotary blocks in bf16), and runs the softmax of tile t beside the
// latent-sum MFMAs of tile t - 1, whose operands are widened from the codes
// in registers. Tile t + 1 is resident once only the loads of tiles
// t + 2 .. t + AHEAD are outstanding.
template <class C>
__device__ __forceinline__ void tile_step_f8(const DecodeParams& p, const MLA_LDS char* __restrict__ cur,
                                             const MLA_LDS char* __restrict__ prev, MLA_LDS char* __restrict__ fill,
                                             MLA_LDS char* __restrict__ pw, const MLA_LDS char* __restrict__ pr,
                                             const QF8<C>& q, const MLA_LDS char* __restrict__ qrope, State<C>& s,
                                             LaneOffs<C>& lo, F8LoadOffs& lof, int64_t seq_row, int t, int start,
                                             int end, bool first) {
  using R = F8Ring<C>;
  constexpr int NB = C::DC / 64;
  static_assert(NB == 8 && C::NKC_ROPE == 4 && R::LPT == 6, "eight latent blocks, six loads");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  asm volatile("" : "+v"(lo.lat), "+v"(lo.rope), "+v"(lo.pv[0]), "+v"(lo.p));
  asm volatile("" : "+v"(lof.lo16), "+v"(lof.h), "+v"(lof.row8), "+v"(lof.rrow), "+v"(lof.rchunk));
  // slot addresses as plain scalars: folded back into the ring arithmetic,
  // they leave offsets that the LDS instructions' immediate field cannot hold
  cur = opaque_lds(cur);
  prev = opaque_lds(prev);
  pr = opaque_lds(pr);
  const F8Tile<C> ld(p, seq_row, t + R::AHEAD, start, end);
  Scores<C> sc;
  sc.lat = f32x16{};
  bf16x8 va[2][C::NFJ], pb[2];
  PvSched<C, true> pvs{s, va, pb, prev, pr, lo};
  // the rotary products first, into VGPRs (the AGPRs hold the latent sums
  // and the latent score)
  bf16x8 r0 = qk_operand<C>(cur, lo, C::NKC_LAT), r1 = qk_operand<C>(cur, lo, C::NKC_LAT + 1);
  // the order below is pinned (scheduling barriers): left to itself, the
  // compiler moves each operand read next to its MFMA, and the chain of
  // score products then waits out every LDS read
  auto sync = [] { __builtin_amdgcn_sched_barrier(0); };
  const int lane = threadIdx.x & 63;
  f32x4 sg0;    // the softmax's first scales (tokens 4 hh + 0..3)
  i32x8 a[2];   // code operands, one block ahead
  a[0] = code_operand(cur, lo.lat, 0);
  bf16x8 qr[2];
  qr[0] = *(const MLA_LDS bf16x8*)(qrope);
  qr[1] = *(const MLA_LDS bf16x8*)(qrope + 64 * 16);
  sync();
#pragma unroll
  for (int kk = 0; kk < C::NKC_ROPE; ++kk) {
    bf16x8 r2 = {}, q2 = {};
    if (kk + 2 < C::NKC_ROPE) {
      r2 = qk_operand<C>(cur, lo, C::NKC_LAT + kk + 2);
      q2 = *(const MLA_LDS bf16x8*)(qrope + (kk + 2) * 64 * 16);
    }
    if (kk == 0) mfma_vgpr_first(sc.rope, r0, qr[0]);
    else mfma_vgpr_acc(sc.rope, r0, qr[kk & 1]);
    r0 = r1;
    r1 = r2;
    qr[kk & 1] = q2;
    sync();
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b + 1 < NB) a[(b + 1) & 1] = code_operand(cur, lo.lat, b + 1);
    if (b < 4) ld.codes(fill, wave, b, lof.lo16, lof.h);
    else if (b == 4) ld.scales(fill, wave, lof.row8);
    else if (b == 5) ld.rope(fill, wave, lof.rrow, lof.rchunk);
    if (b >= 5 && b < 7) {
      pvs.read_va(0, 2 * (b - 5));
      pvs.read_va(0, 2 * (b - 5) + 1);
    }
    if (b == 7) pvs.read_pb(0);
    if (b == 7) sg0 = *(const MLA_LDS f32x4*)((const MLA_LDS char*)cur + R::SCL + 16 * (lane >> 5));
    sc.lat = mfma32x32x64_e4m3<127>(a[b & 1], q.hi[b], sc.lat);
    sc.lat = mfma32x32x64_e4m3<123>(a[b & 1], q.lo[b], sc.lat);   // lo carries 2^-4
    sync();
  }
  vgpr_acc_drain(sc.rope);
  __builtin_amdgcn_sched_barrier(0);
  softmax_pv_stream<C, true>(pvs, pw, sc, s, end - (start + t * C::T), q.fs, first,
                             (const MLA_LDS float*)(cur + R::SCL), sg0);
  wait_vmem_le<(R::AHEAD - 1) * R::LPT>();
  tile_barrier();
}

// O^T += C_KV^T . P^T for one tile of e4m3 codes (the last tile of a pass).
template <class C>
__device__ __forceinline__ void latent_sum_tile_f8(const MLA_LDS char* __restrict__ buf,
                                                   const MLA_LDS char* __restrict__ pbuf, State<C>& s,
                                                   const LaneOffs<C>& lo) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    bf16x8 a[C::NFJ];
#pragma unroll
    for (int j = 0; j < C::NFJ; ++j) a[j] = pv_operand_f8<C>(buf, lo, j, u);
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) {
      const bf16x8 pb = *(const MLA_LDS bf16x8*)(pbuf + p_rd_off<C>(lo, hb, u));
#pragma unroll
      for (int j = 0; j < C::NFJ; ++j) pv_mfma<C>(s, j, hb, a[j], pb);
    }
  }
}

// Which (sequence, split) item a workgroup takes. Workgroups reach the XCDs
// round-robin and, within one XCD, its compute units in index order, one per
// compute unit at a time.
//  kOrderPlain: index = b * S + split.
//  kOrderXcd:   a sequence's splits on one XCD (one round of equal items).
//  kOrderLongestFirst (grids of several rounds): every full chunk first
//    (sequence-major), then the partly filled last chunks in eight bands of
//    remainder, largest first, then the empty items; longest-first list
//    scheduling, which keeps uneven lengths from leaving a ragged last round.
//    Every wave derives the same item from the lengths, 64 sequences a pass
//    (a separate kernel instance, so the index orders keep their prologue).
struct Item {
  int b, split, len;
};

struct SeqCounts {
  int len, full, rem, band, empty;   // band: 0 = largest remainder .. 7; -1 none
};

__device__ __forceinline__ SeqCounts seq_counts(const DecodeParams& p, int b) {
  SeqCounts c{0, 0, 0, -1, 0};
  if (b < p.batch) {
    c.len = query_len(p, b);
    const int L = p.chunk > 0 ? max(0, min(c.len, p.max_seq_len)) : 0;
    if (L > 0) {
      c.full = min(L / p.chunk, p.num_splits);
      c.rem = L - c.full * p.chunk;   // 0 once every split is full
      if (c.rem > 0) c.band = (p.chunk - c.rem) / (p.chunk >> 3);   // chunks are multiples of 32
    }
    c.empty = p.num_splits - c.full - (c.rem > 0 ? 1 : 0);
  }
  return c;
}

__device__ __forceinline__ int wave_inclusive_sum(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ Item longest_first_item(const DecodeParams& p, int k) {
  const int lane = threadIdx.x & 63;
  // class sizes: full chunks, the eight remainder bands
  const SeqCounts first = seq_counts(p, lane);   // reused by both sweeps
  int full_total = 0;
  int band_total[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const SeqCounts c = b0 == 0 ? first : seq_counts(p, b0 + lane);
    full_total += __builtin_amdgcn_readlane(wave_inclusive_sum(c.full, lane), 63);
#pragma unroll
    for (int q = 0; q < 8; ++q) band_total[q] += __popcll(__ballot(c.band == q));
  }
  // the class that holds position k, and k's rank within it
  int cls = 0;   // 0 full, 1 + q band q, 9 empty
  if (k >= full_total) {
    k -= full_total;
    cls = 9;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (cls == 9) {
        if (k < band_total[q]) cls = 1 + q;
        else k -= band_total[q];
      }
    }
  }
  Item it{0, 0, 0};
  int base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const SeqCounts c = b0 == 0 ? first : seq_counts(p, b0 + lane);
    const int n = cls == 0 ? c.full : cls == 9 ? c.empty : (c.band == cls - 1 ? 1 : 0);
    const int incl = wave_inclusive_sum(n, lane);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (k < base + total) {
      const uint64_t hit = __ballot(n > 0 && base + incl > k);
      const int ln = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      const int off = k - base - (__builtin_amdgcn_readlane(incl, ln) - __builtin_amdgcn_readlane(n, ln));
      const int full = __builtin_amdgcn_readlane(c.full, ln);
      const int rem = __builtin_amdgcn_readlane(c.rem, ln);
      it.b = b0 + ln;
      it.split = cls == 0 ? off : cls == 9 ? full + (rem > 0 ? 1 : 0) + off : full;
      it.len = __builtin_amdgcn_readlane(c.len, ln);
      break;
    }
    base += total;
  }
  return it;
}

template <class C>
__device__ __forceinline__ int64_t out_row(const DecodeParams& p, int b, int split, int head) {
  return p.num_splits > 1 ? (((int64_t)b * p.num_splits + split) * C::H + head)
                          : ((int64_t)b * C::H + head);
}

template <class C, bool PAGED, bool PSTREAM, bool E4M3, bool LONGEST_FIRST>
__global__ __launch_bounds__(C::THREADS, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  static_assert(!E4M3 || (!PAGED && !C::F32 && !C::FP8), "e4m3 tiles stream through the contiguous 16-bit loop");
  using R8 = typename std::conditional<E4M3, F8Ring<C>, NoF8Ring>::type;

  int b, split, len_b;
  if constexpr (LONGEST_FIRST) {
    const Item it = longest_first_item(p, blockIdx.x);
    b = it.b;
    split = it.split;
    len_b = it.len;
  } else {
    int w = blockIdx.x;
    if (p.order == kOrderXcd) w = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    b = w / p.num_splits;
    split = w % p.num_splits;
    len_b = query_len(p, b);   // a scalar load, requested before the loads into LDS
  }
  MLA_LDS char* lds = (MLA_LDS char*)smem;
  auto slot = [&](int x) -> MLA_LDS char* {   // x >= 0
    if constexpr (E4M3) return lds + R8::S0 + (x % R8::NSLOT) * R8::SLOT;
    else return lds + (x % C::NBUF) * C::BUF_BYTES;
  };

  // 16-bit caches, contiguous or with pages of at least 32 tokens (PSTREAM),
  // stream whole tiles and stage the query through LDS (slots 2..3 and the
  // P^T buffers); its first half is requested before anything else, since
  // it depends on nothing but the sequence. A paged split's page ids follow.
  constexpr bool STREAM = !C::F32 && !C::FP8 && (!PAGED || PSTREAM);
  static_assert(!PSTREAM || PAGED, "PSTREAM is the paged streaming form");
  MLA_LDS char* qreg = slot(2) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * QStage<C>::BYTES;
  if constexpr (STREAM) stage_q_issue<C>(p, b, 0, qreg);
  TileBase tbase{(const char*)p.latent, 0, 0, 0};
  if constexpr (PAGED && STREAM) {
    tbase.shift = p.page_shift;
    tbase.lp0 = (split * p.chunk) >> p.page_shift;
    const int32_t* bt = p.block_table + (int64_t)cache_seq(p, b) * p.max_pages;
    tbase.pages = bt[min(tbase.lp0 + (int)(threadIdx.x & 63), p.max_pages - 1)];
  }

  const int L = max(0, min(len_b, p.max_seq_len));
  const int start = split * p.chunk;
  const int end = min(start + p.chunk, L);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int head = wave * 32 + r;
  MLA_LDS char* pbase = lds + (E4M3 ? R8::P : C::NBUF * C::BUF_BYTES);
  const bool f32_out = !p.out_bf16;

  if (start >= end) {             // uniform over the workgroup: no tokens
    if constexpr (STREAM) wait_vmem_le<0>();   // nothing may land in LDS after the workgroup ends
    if (head < C::H) {
      const int64_t row = out_row<C>(p, b, split, head);
      if (hh == 0) p.lse[row] = -INFINITY;
      for (int f = hh; f < C::DC / 4; f += 2) {
        if (f32_out) *(f32x4*)((float*)p.out + row * C::DC + 4 * f) = f32x4{};
        else *(u32x2*)((uint16_t*)p.out + row * C::DC + 4 * f) = u32x2{};
      }
    }
    return;
  }

  State<C> s;
#pragma unroll
  for (int j = 0; j < C::NFJ; ++j)
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) s.o[j][hb] = f32x16{};
  s.m_ref = -INFINITY;
  s.m_max = -INFINITY;
  s.l = 0.0f;
  s.overflow = false;

  // Absorbed query fragments of this wave's 32 heads (B operand of S^T).
  QFrag<C> q;
  auto load_q = [&]() {
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
  };
  Fp8Stage<C> st;
  LaneOffs<C> lo;
  if constexpr (E4M3) lo = lane_offsets_f8<C>(wave);
  else lo = lane_offsets<C>(wave);
  typename std::conditional<E4M3, QF8<C>, int>::type q8{};   // the e4m3 loop's split query
  const SeqView sv = seq_view<PAGED>(p, b);
  DmaOffs dma;
  {
    const int tr_ = threadIdx.x / C::ROPE_CH, cr = (threadIdx.x % C::ROPE_CH) ^ swz<C::ROPE_CH>(tr_);
    dma.lat = (lane ^ (wave << 2)) << 4;
    dma.rope_chunk = C::DC * C::ESZ + cr * 16;
    dma.rope = (int)(tr_ * (p.row_stride * C::ESZ)) + dma.rope_chunk;
  }
  const int ntiles = (end - start + C::T - 1) / C::T;
  constexpr int LPT = loads_per_tile<C>();
  if constexpr (!PAGED) tbase.base = (const char*)p.latent + sv.seq_row * (p.row_stride * C::ESZ);
  auto pslot = [&](int x) -> MLA_LDS char* { return pbase + (x & 1) * C::P_BYTES; };
  // End of a pass over the split. The last step left the P^T buffer
  // pslot(ntiles) free: every wave writes its heads' softmax denominators
  // (lanes r and r + 32 hold halves of one head's) and its overflow flag
  // there, runs the latent sum of the last tile, and one barrier publishes
  // both for the normalisation and the recompute decision.
  auto finish_pass = [&]() {
    MLA_LDS char* fin = pslot(ntiles);
    const float l_tot = s.l + __shfl_xor(s.l, 32);
    if (hh == 0) ((MLA_LDS float*)fin)[head] = l_tot;
    const bool wave_overflow = __ballot(s.overflow) != 0;
    if (lane == 0) ((MLA_LDS int*)(fin + kFinFlags))[wave] = wave_overflow ? 1 : 0;
    if constexpr (E4M3) latent_sum_tile_f8<C>(slot(ntiles - 1), pslot(ntiles - 1), s, lo);
    else latent_sum_tile<C>(slot(ntiles - 1), pslot(ntiles - 1), s, lo);
    if constexpr (!C::F32) vgpr_acc_drain(s.o[C::NFJ - 1][C::HB - 1]);
    __syncthreads();
  };
  static_assert(kFinFlags >= 32 * C::WAVES * 4 && kFinFlags + 4 * C::WAVES <= C::P_BYTES, "denominators and flags fit");

  if constexpr (!STREAM) load_q();

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {   // recompute with the true maximum as reference
#pragma unroll
      for (int j = 0; j < C::NFJ; ++j)
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) s.o[j][hb] = f32x16{};
      s.l = 0.0f;
      s.m_ref = fmaxf(s.m_max, __shfl_xor(s.m_max, 32));
      s.overflow = false;
    }
    if constexpr (STREAM && E4M3) {
      // prologue: tiles 0 and 1 land beside the staged query (first pass:
      // requested after its first half); tile 2 goes to the slot the query
      // occupies, so (first pass) it is requested once every wave has read
      // the query, and the query is split while it loads
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      F8LoadOffs lof = f8_load_offsets<C>(dma);
      auto issue8 = [&](int x) {
        const F8Tile<C> ld(p, sv.seq_row, x, start, end);
#pragma unroll
        for (int k = 0; k < 4; ++k) ld.codes(slot(x), wv, k, lof.lo16, lof.h);
        ld.scales(slot(x), wv, lof.row8);
        ld.rope(slot(x), wv, lof.rrow, lof.rchunk);
      };
      static_assert(R8::AHEAD == 2 || R8::AHEAD == 3, "tiles 0 .. AHEAD - 1 in the prologue");
      issue8(0);
      issue8(1);
      if (pass == 0) {
        QRaw<C> raw;
        wait_vmem_le<2 * R8::LPT>();              // query half 0
        stage_q_read_f8<C>(raw, 0, qreg);
        stage_q_issue<C>(p, b, 1, qreg);
        wait_vmem_le<0>();                        // tiles 0, 1 and query half 1
        stage_q_read_f8<C>(raw, 1, qreg);
        tile_barrier();                           // every wave is done with the staged query
        if constexpr (R8::AHEAD == 3) issue8(2);
        split_query_f8<C>(q8, raw, p.scale_log2, lds + R8::QROPE + wv * R8::QROPE_BYTES);
      } else {
        if constexpr (R8::AHEAD == 3) issue8(2);
        wait_vmem_le<(R8::AHEAD - 1) * R8::LPT>();   // tile 0
      }
      static_assert(C::P_BYTES == C::THREADS * 32, "two 16-byte zero stores per thread");
      *(MLA_LDS u32x4*)(pslot(1) + threadIdx.x * 32) = u32x4{};
      *(MLA_LDS u32x4*)(pslot(1) + threadIdx.x * 32 + 16) = u32x4{};
      tile_barrier();
      // step 0 runs its latent sum over tile 0's codes with the zeroed P^T
      // buffer, which adds exactly zero
#pragma clang loop unroll(disable)
      for (int t = 0; t < ntiles; ++t) {
        const int tp = max(t - 1, 0), first = pass == 0 && t == 0;
        tile_step_f8<C>(p, slot(t), slot(tp), slot(t + R8::AHEAD), pslot(t), pslot(t - 1), q8,
                        lds + R8::QROPE + wv * R8::QROPE_BYTES + 16 * lane, s, lo, lof, sv.seq_row, t, start,
                        end, first != 0);
      }
      finish_pass();
    } else if constexpr (STREAM) {
      // prologue: tiles 0 and 1, and (first pass) the second half of the
      // query once the first is read
      static_assert(C::NBUF == 4 && 4 * QStage<C>::BYTES <= 2 * C::BUF_BYTES + 2 * C::P_BYTES, "query staging");
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      StreamTile<C>(p, tbase, 0, ntiles, start, end, std::integral_constant<bool, PAGED>{}).all(dma, slot(0), wv);
      if (pass == 0) {
        wait_vmem_le<LPT>();                      // query half 0
        stage_q_read<C>(q, 0, qreg);
        stage_q_issue<C>(p, b, 1, qreg);
      }
      StreamTile<C>(p, tbase, 1, ntiles, start, end, std::integral_constant<bool, PAGED>{}).all(dma, slot(1), wv);
      wait_vmem_le<LPT>();                        // tile 0 (and query half 1)
      if (pass == 0) stage_q_read<C>(q, 1, qreg);
      static_assert(C::P_BYTES == C::THREADS * 32, "two 16-byte zero stores per thread");
      *(MLA_LDS u32x4*)(pslot(1) + threadIdx.x * 32) = u32x4{};
      *(MLA_LDS u32x4*)(pslot(1) + threadIdx.x * 32 + 16) = u32x4{};
      tile_barrier();
      // step t loads tile t + 2 (the last tile again past the end). Step 0
      // has no previous tile: its latent sum runs over tile 0's rows with the
      // zeroed P^T buffer, which adds exactly zero.
      // one copy of the step for every t: not peeled, not unrolled
#pragma clang loop unroll(disable)
      for (int t = 0; t < ntiles; ++t) {
        const int tp = max(t - 1, 0), first = pass == 0 && t == 0;
        tile_step_stream<C, PAGED>(p, slot(t), slot(tp), slot(t + 2), pslot(t), pslot(t - 1), q, s, lo, dma, tbase, t,
                            ntiles, start, end, first != 0);
      }
      finish_pass();
    } else {
    // prologue: tile 0 resident, tile 1 in flight
    issue_tile<C, PAGED>(p, sv, dma, slot(0), start, end, st);
    if constexpr (C::FP8) {
      wait_vmem_le<0>();
      commit_tile<C>(slot(0), st);
      if (ntiles > 1) issue_tile<C, PAGED>(p, sv, dma, slot(1), start + C::T, end, st);
    } else {
      if (ntiles > 1) {
        issue_tile<C, PAGED>(p, sv, dma, slot(1), start + C::T, end, st);
        wait_vmem_le<LPT>();
      } else {
        wait_vmem_le<0>();
      }
    }
    tile_barrier();

    tile_step<C, PAGED, true>(p, slot(0), slot(C::NBUF - 1), slot(1), slot(2), pslot(0), pslot(1), q, s, lo,
                              sv, dma, st, 0, ntiles, start, end, pass == 0);
    for (int t = 1; t < ntiles; ++t)
      tile_step<C, PAGED, false>(p, slot(t), slot(t - 1), slot(t + 1), slot(t + 2), pslot(t), pslot(t - 1), q,
                                 s, lo, sv, dma, st, t, ntiles, start, end, false);
    finish_pass();
    }
    if (pass == 1) break;
    // did any lane's scores outrun the headroom? (uniform decision)
    int any = 0;
#pragma unroll
    for (int v = 0; v < C::WAVES; ++v) any |= ((const MLA_LDS int*)(pslot(ntiles) + kFinFlags))[v];
    if (!any) break;
    __syncthreads();   // every wave has read the flags before the second pass reuses the buffers
  }

  // ---- normalise and store; every head's denominator is in LDS already ----
  const MLA_LDS float* lden = (const MLA_LDS float*)pslot(ntiles);
  const float l_tot = s.l + __shfl_xor(s.l, 32);   // every lane takes part in the exchange
  if (hh == 0 && head < C::H) p.lse[out_row<C>(p, b, split, head)] = (s.m_ref + fast_log2(l_tot)) * kLn2;
  // staging of the bf16 rows below: one region of H padded rows per wave,
  // all clear of the P^T buffers (where the denominators are)
  constexpr int SROW = C::FPW * 2 + 16;
  constexpr int STAGE_AT = E4M3 ? R8::STAGE : 0;
  constexpr bool STAGE = !C::F32 && (E4M3 ? R8::STAGE + C::WAVES * C::H * SROW <= C::LDS_BYTES
                                          : C::WAVES * C::H * SROW <= C::NBUF * C::BUF_BYTES);
  if constexpr (STAGE) {
    if (!f32_out) {
      // Lanes r and r + 32 hold alternating runs of four features of head
      // 32 hb + r. Packed to bf16 pairs, half of them are exchanged between
      // the two lanes (v_permlane32_swap), after which lane r holds features
      // 0..15 and lane r + 32 features 16..31 of each 32-feature fragment.
      // Each wave stages its own feature slice of every head (128 heads x
      // FPW features, rows padded by 16 bytes against bank conflicts) in a
      // region of its own, then reads it back so that every 16 lanes hold
      // one head's slice and each store writes whole 256-byte row segments.
      static_assert(C::FPW * 2 == 16 * 16, "16 lanes a row");
      MLA_LDS char* stage = lds + STAGE_AT + wave * (C::H * SROW);
#pragma unroll
      for (int hb = 0; hb < C::HB; ++hb) {
        const int h = 32 * hb + r;
        const float inv = 1.0f / lden[h];
#pragma unroll
        for (int j = 0; j < C::NFJ; ++j) {
          uint32_t pk[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(s.o[j][hb][2 * k] * inv, s.o[j][hb][2 * k + 1] * inv);
#pragma unroll
          for (int k = 0; k < 4; ++k) swap_lane_halves(pk[k], pk[k + 4]);
          MLA_LDS char* dst = stage + h * SROW + (32 * j + 16 * hh) * 2;
          *(MLA_LDS u32x4*)dst = u32x4{pk[0], pk[1], pk[4], pk[5]};
          *(MLA_LDS u32x4*)(dst + 16) = u32x4{pk[2], pk[3], pk[6], pk[7]};
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's own staging
      // 16 lanes per head, four heads per instruction; eight reads in flight
      const int c = lane & 15;
      const MLA_LDS char* src = stage + (lane >> 4) * SROW + 16 * c;
      uint16_t* dst = (uint16_t*)p.out + out_row<C>(p, b, split, lane >> 4) * C::DC + wave * C::FPW + 8 * c;
#pragma unroll
      for (int i0 = 0; i0 < C::H / 4; i0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = *(const MLA_LDS u32x4*)(src + 4 * (i0 + k) * SROW);
#pragma unroll
        for (int k = 0; k < 8; ++k) *(u32x4*)(dst + (int64_t)4 * (i0 + k) * C::DC) = v[k];
      }
      return;
    }
  }
#pragma unroll
  for (int hb = 0; hb < C::HB; ++hb) {
    const int h = 32 * hb + r;
    if (h >= C::H) continue;
    const float inv = 1.0f / lden[h];
    const int64_t row = out_row<C>(p, b, split, h);
#pragma unroll
    for (int j = 0; j < C::NFJ; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int feat = wave * C::FPW + 32 * j + 8 * jj + 4 * hh;
        const float v0 = s.o[j][hb][4 * jj + 0] * inv, v1 = s.o[j][hb][4 * jj + 1] * inv;
        const float v2 = s.o[j][hb][4 * jj + 2] * inv, v3 = s.o[j][hb][4 * jj + 3] * inv;
        if (f32_out) {
          *(f32x4*)((float*)p.out + row * C::DC + feat) = f32x4{v0, v1, v2, v3};
        } else {
          u32x2 v;
          v[0] = pack_bf16x2(v0, v1);
          v[1] = pack_bf16x2(v2, v3);
          *(u32x2*)((uint16_t*)p.out + row * C::DC + feat) = v;
        }
      }
  }
}

}  // namespace

// Compute units of the current device, queried once per device (the item
// order only; any value gives correct results).
int device_compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

template <class C, bool LF>
hipError_t launch_order(const DecodeParams& q, int grid, hipStream_t stream) {
  if (q.page_shift >= 0) {
    // pages of at least one tile, a split's pages within one wave's lanes
    const bool stream_pages = q.page_shift >= 5 && ((q.chunk + (1 << q.page_shift) - 1) >> q.page_shift) + 1 <= 64;
    if constexpr (C::KIND == kBF16) {
      if (stream_pages)
        return launch_kernel((decode_kernel<C, true, true, false, LF>), dim3(grid), dim3(C::THREADS), stream, q);
    }
    return launch_kernel((decode_kernel<C, true, false, false, LF>), dim3(grid), dim3(C::THREADS), stream, q);
  }
  if constexpr (C::FP8 && C::H == 128 && C::DC == 512 && C::DR == 64) {
    // contiguous e4m3: codes streamed into fp8 score products (F8Ring)
    using CB = Cfg<C::H, C::DC, C::DR, kBF16>;
    return launch_kernel((decode_kernel<CB, false, false, true, LF>), dim3(grid), dim3(CB::THREADS), stream, q);
  }
  return launch_kernel((decode_kernel<C, false, false, false, LF>), dim3(grid), dim3(C::THREADS), stream, q);
}

template <class C>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  const int grid = p.batch * p.num_splits;
  if (grid == 0) return hipSuccess;
  DecodeParams q = p;
  if (grid > device_compute_units()) {
    q.order = kOrderLongestFirst;
    return launch_order<C, true>(q, grid, stream);
  }
  q.order = (grid % 8 == 0 && p.num_splits > 1) ? kOrderXcd : kOrderPlain;
  return launch_order<C, false>(q, grid, stream);
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
