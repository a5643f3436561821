// Prefill of n new tokens per sequence in the non-absorbed form.
//
// DeepSeek-V2 paper (Chinese translation), section 2.1.2: keys and values are
// the up-projections k^C = W_UK c_KV and v^C = W_UV c_KV of the cached
// latents; section 2.1.3: a head's key is [k^C ; k^R] with the shared rotary
// key k^R. When many queries of one sequence are scored together (a prompt)
// the up-projection is paid once per cached token instead of once per query,
// and the attention is ordinary multi-head attention with head width
// d_nope + d_rope = 192 for scores and d_v = 128 for values.
//
// Two launches:
//  1. upproj_kernel: K^C and V^C of every cached row of every sequence,
//     [B, H, Lpad, 128] bf16 each in the caller's workspace. One 256-thread
//     workgroup per (128 tokens, head, K or V): out^T[128 d x 128 t] =
//     W[h] . rows^T over k = d_c = 512 in chunks of 64 staged through LDS
//     (rows padded to 144 bytes, conflict-free 16-byte reads), the next
//     chunk's loads in flight during the current chunk's MFMAs.
//  2. prefill_attn_kernel: one 256-thread workgroup per (128 new tokens,
//     head, sequence), wave w owning tokens 32w .. 32w + 31. Key blocks of 64
//     tokens, [K^C | k^R] and V^C staged through LDS, scores as
//     S^T[keys x tokens] = K . Q^T (the queries stay in VGPRs), causal mask,
//     online softmax in fp32 and base 2 with the running maximum, and
//     O^T[d_v x tokens] += V^T . P^T where P^T comes straight from the score
//     accumulators: the transposing LDS reads of V deliver the keys of each
//     16-wide k step in exactly the order the accumulators hold them.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDC = 512, kDN = 128, kDR = 64, kDV = 128, kDQK = kDN + kDR;
constexpr int kUpTile = 128;      // tokens (and features) per up-projection workgroup
constexpr int kUpK = 64;          // contraction chunk
constexpr int kUpRow = 144;       // LDS bytes per staged row (128 + 16 padding)
constexpr int kUpTileBytes = kUpTile * kUpRow;
constexpr int kQBlock = 128;      // new tokens per attention workgroup
constexpr int kKBlock = 64;       // keys per step
constexpr int kKRow = 400;        // LDS bytes per key row: 384 (K^C | k^R) + 16 padding
constexpr int kVRow = 256;        // LDS bytes per value row (16-byte chunks XOR-swizzled)
constexpr int kKTile = kKBlock * kKRow, kVTile = kKBlock * kVRow;

__device__ __forceinline__ int clamp_len(const PrefillParams& p, int b) {
  return max(0, min(p.seq_lens[b], p.max_seq_len));
}

// Physical cache row of token j of sequence b.
__device__ __forceinline__ int64_t cache_row(const PrefillParams& p, int b, int j) {
  if (p.page_shift < 0) return (int64_t)b * p.seq_stride + j;
  const int32_t page = p.block_table[(int64_t)b * p.max_pages + (j >> p.page_shift)];
  return ((int64_t)page << p.page_shift) + (j & ((1 << p.page_shift) - 1));
}

__global__ __launch_bounds__(256, 2) void upproj_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kUpTileBytes];
  MLA_LDS char* lds = (MLA_LDS char*)smem;
  const int h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const int L = clamp_len(p, b);
  const int t0 = blockIdx.x * kUpTile;
  if (t0 >= L) return;   // uniform: no cached token in this tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, r = lane & 31;
  const __bf16* w = (const __bf16*)(which ? p.w_uv : p.w_uk) + (int64_t)h * kDN * kDC;

  // Thread tid stages pieces tid + 256 i (i < 4) of each 128 x 64 chunk:
  // row (idx >> 3), 16-byte piece (idx & 7). Tokens past the end repeat the
  // last valid token (their columns are never read back).
  const char* wsrc[4];
  const char* asrc[4];
  int loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
    wsrc[i] = (const char*)(w + (int64_t)row * kDC) + 16 * piece;
    const int j = min(t0 + row, L - 1);
    asrc[i] = (const char*)p.latent + cache_row(p, b, j) * p.row_stride * 2 + 16 * piece;
    loff[i] = row * kUpRow + 16 * piece;
  }
  u32x4 wr[4], ar[4];
  auto load = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wr[i] = load16(wsrc[i] + kc * kUpK * 2);
      ar[i] = load16(asrc[i] + kc * kUpK * 2);
    }
  };
  auto store = [&](int stage) {
    MLA_LDS char* base = lds + stage * 2 * kUpTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(MLA_LDS u32x4*)(base + loff[i]) = wr[i];
      *(MLA_LDS u32x4*)(base + kUpTileBytes + loff[i]) = ar[i];
    }
  };

  // wave (wm, wn): features 64 wm .. +63 (A operand, weight rows), tokens
  // 64 wn .. +63 (B operand, cache rows)
  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2] = {};
  load(0);
  store(0);
  __syncthreads();
  constexpr int NK = kDC / kUpK;
  for (int kc = 0; kc < NK; ++kc) {
    if (kc + 1 < NK) load(kc + 1);
    const MLA_LDS char* base = lds + (kc & 1) * 2 * kUpTileBytes;
#pragma unroll
    for (int ks = 0; ks < kUpK / 16; ++ks) {
      const int off = 32 * ks + 16 * hh;
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const MLA_LDS bf16x8*)(base + (64 * wm + 32 * i + r) * kUpRow + off);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bb[j] = *(const MLA_LDS bf16x8*)(base + kUpTileBytes + (64 * wn + 32 * j + r) * kUpRow + off);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], bb[j], acc[i][j]);
    }
    if (kc + 1 < NK) store((kc + 1) & 1);
    __syncthreads();
  }

  // acc[i][j] element 4 jj + ii: feature 64 wm + 32 i + 8 jj + 4 hh + ii of
  // token t0 + 64 wn + 32 j + r; four consecutive features per 8-byte store.
  __bf16* out = (__bf16*)(which ? p.vc : p.kc) + ((int64_t)b * p.heads + h) * p.lpad * kDN;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 64 * wn + 32 * j + r;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 64 * wm + 32 * i + 8 * jj + 4 * hh;
        u32x2 v;
        v[0] = pack_bf16x2(acc[i][j][4 * jj], acc[i][j][4 * jj + 1]);
        v[1] = pack_bf16x2(acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]);
        *(u32x2*)(out + (int64_t)t * kDN + d) = v;
      }
  }
}

// POS_SCALE (a positive softmax scale, the usual case): the running maximum is
// taken over the raw scores and each probability is exp2(fma(s, scale, -m)),
// one instruction fewer per score than scaling first; otherwise every score is
// scaled before the maximum.
template <bool POS_SCALE>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kKTile + kVTile];
  MLA_LDS char* ktile = (MLA_LDS char*)smem;
  MLA_LDS char* vtile = ktile + kKTile;
  const int n = p.n;
  const int nqb = (n + kQBlock - 1) / kQBlock;
  const int qb = nqb - 1 - (int)blockIdx.x;   // the longest key ranges first
  const int h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(p, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, r = lane & 31;
  const int q0 = qb * kQBlock;
  const int t = q0 + 32 * wave + r;            // this lane's new token (both lane halves)
  const bool valid = t < n;
  const int pos = L - n + t;                   // its position: it sees keys 0 .. pos
  const int64_t bv = (int64_t)b * n + (valid ? t : 0);

  // every token of this wave valid, and the position of its first token
  // (the lowest: every lane sees at least keys 0 .. wave_pos0)
  const bool wave_full = q0 + 32 * wave + 31 < n;
  const int wave_pos0 = L - n + q0 + 32 * wave;
  // keys the workgroup needs: up to the position of its last valid token
  const int kmax = L - n + min(q0 + kQBlock - 1, n - 1);
  const int nkb = kmax >= 0 ? kmax / kKBlock + 1 : 0;

  // query fragments: k step s covers features 16 s .. 16 s + 15 of [q^C ; q^R]
  bf16x8 qf[kDQK / 16];
  {
    const __bf16* qn = (const __bf16*)p.q_nope + (bv * p.heads + h) * kDN;
    const __bf16* qr = (const __bf16*)p.q_rope + (bv * p.heads + h) * kDR;
#pragma unroll
    for (int s = 0; s < kDQK / 16; ++s) {
      const int d = 16 * s + 8 * hh;
      const bf16x8 v = d < kDN ? *(const bf16x8*)(qn + d) : *(const bf16x8*)(qr + d - kDN);
      qf[s] = valid ? v : bf16x8{};
    }
  }

  // staging: thread tid moves pieces tid + 256 i of each block; K^C and V^C
  // rows are 16 pieces, k^R rows 8
  const __bf16* kc_base = (const __bf16*)p.kc + ((int64_t)b * p.heads + h) * p.lpad * kDN;
  const __bf16* vc_base = (const __bf16*)p.vc + ((int64_t)b * p.heads + h) * p.lpad * kDN;
  u32x4 kreg[4], rreg[2], vreg[4];
  auto load = [&](int kb) {
    const int j0 = kb * kKBlock;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, piece = idx & 15;
      const int j = min(j0 + row, L - 1);
      kreg[i] = load16(kc_base + (int64_t)j * kDN + 8 * piece);
      vreg[i] = load16(vc_base + (int64_t)j * kDN + 8 * piece);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
      const int j = min(j0 + row, L - 1);
      rreg[i] = load16((const char*)p.latent + cache_row(p, b, j) * p.row_stride * 2 + kDC * 2 + 16 * piece);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, piece = idx & 15;
      *(MLA_LDS u32x4*)(ktile + row * kKRow + 16 * piece) = kreg[i];
      *(MLA_LDS u32x4*)(vtile + row * kVRow + 16 * (piece ^ ((row & 3) << 1))) = vreg[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, piece = idx & 7;
      *(MLA_LDS u32x4*)(ktile + row * kKRow + 16 * (16 + piece)) = rreg[i];
    }
  };

  // transposing reads of V^T: source lane (a, e) of 16-lane group `sub`
  // addresses key 16 u + 8 q + 4 hh + e, features 32 jb + 16 sub + 4 a .. +3
  const int s16 = lane & 15, a4 = s16 & 3, e4 = s16 >> 2, sub = (lane >> 4) & 1;
  auto v_off = [&](int u, int q, int jb) {
    const int key = 16 * u + 8 * q + 4 * hh + e4;
    const int chunk = 4 * jb + 2 * sub + (a4 >> 1);
    return key * kVRow + 16 * (chunk ^ ((key & 3) << 1)) + 8 * (a4 & 1);
  };

  float m = -INFINITY, l = 0.0f;
  f32x16 o[kDV / 32] = {};
  if (nkb > 0) load(0);
  for (int kb = 0; kb < nkb; ++kb) {
    store();
    __syncthreads();
    if (kb + 1 < nkb) load(kb + 1);
    const int j0 = kb * kKBlock;

    // S^T[64 keys x 32 tokens] in two 32-key blocks
    f32x16 sc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      sc[kk] = f32x16{};
#pragma unroll
      for (int s = 0; s < kDQK / 16; ++s) {
        const bf16x8 a = *(const MLA_LDS bf16x8*)(ktile + (32 * kk + r) * kKRow + 16 * (2 * s + hh));
        sc[kk] = mfma32x32x16(a, qf[s], sc[kk]);
      }
    }
    // element 4 jj + ii of sc[kk]: key j0 + 32 kk + 8 jj + 4 hh + ii; a
    // block that every token of the wave sees whole takes no mask (uniform)
    float x[2][16];
    float mt = -INFINITY;
    const bool whole = wave_full && j0 + kKBlock - 1 <= wave_pos0;
    if (POS_SCALE && whole) {
      // raw scores
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          x[kk][e] = sc[kk][e];
          mt = fmaxf(mt, x[kk][e]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.scale_log2;
    } else if (POS_SCALE) {
      // raw scores; masked keys become -inf (exp2(fma(-inf, scale, -ref)) = 0)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + 32 * kk + 8 * (e >> 2) + 4 * hh + (e & 3);
          x[kk][e] = (valid && key <= pos) ? sc[kk][e] : -INFINITY;
          mt = fmaxf(mt, x[kk][e]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.scale_log2;
    } else if (whole) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          x[kk][e] = sc[kk][e] * p.scale_log2;
          mt = fmaxf(mt, x[kk][e]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + 32 * kk + 8 * (e >> 2) + 4 * hh + (e & 3);
          const float v = sc[kk][e] * p.scale_log2;
          x[kk][e] = (valid && key <= pos) ? v : -INFINITY;
          mt = fmaxf(mt, x[kk][e]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
    }
    const float m_new = fmaxf(m, mt);
    const float ref = m_new == -INFINITY ? 0.0f : m_new;   // a token with no key yet
    const float alpha = fast_exp2(m - ref);                 // 0 on the first block that has keys
    m = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[kk][e] = POS_SCALE ? fast_exp2(__builtin_fmaf(x[kk][e], p.scale_log2, -ref)) : fast_exp2(x[kk][e] - ref);
        psum += x[kk][e];
      }
    l = l * alpha + psum;
    if (__ballot(alpha != 1.0f)) {   // uniform: no lane's maximum moved, nothing to rescale
#pragma unroll
      for (int jb = 0; jb < kDV / 32; ++jb) o[jb] *= alpha;
    }

    // O^T += V^T . P^T, four 16-key steps; element e of step u is key
    // 16 u + 8 (e / 4) + 4 hh + e % 4 = accumulator 8 (u & 1) + e of block u / 2
#pragma unroll
    for (int u = 0; u < kKBlock / 16; ++u) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)x[u >> 1][8 * (u & 1) + e];
#pragma unroll
      for (int jb = 0; jb < kDV / 32; ++jb) {
        const bf16x4 v0 = lds_read_tr16(vtile + v_off(u, 0, jb));
        const bf16x4 v1 = lds_read_tr16(vtile + v_off(u, 1, jb));
        const bf16x8 a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[jb] = mfma32x32x16(a, pb, o[jb]);
      }
    }
    __syncthreads();
  }

  // o[jb] element 4 jj + ii: feature 32 jb + 8 jj + 4 hh + ii of this token
  const float l_tot = l + __shfl_xor(l, 32);
  if (!valid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  __bf16* out = (__bf16*)p.out + (bv * p.heads + h) * kDV;
#pragma unroll
  for (int jb = 0; jb < kDV / 32; ++jb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v;
      v[0] = pack_bf16x2(o[jb][4 * jj] * inv, o[jb][4 * jj + 1] * inv);
      v[1] = pack_bf16x2(o[jb][4 * jj + 2] * inv, o[jb][4 * jj + 3] * inv);
      *(u32x2*)(out + 32 * jb + 8 * jj + 4 * hh) = v;
    }
  if (hh == 0) p.lse[bv * p.heads + h] = l_tot > 0.0f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

int64_t prefill_workspace_bytes(int batch, int heads, int max_seq_len) {
  const int64_t lpad = ((int64_t)max_seq_len + kUpTile - 1) / kUpTile * kUpTile;
  return 2 * (int64_t)batch * heads * lpad * kDN * 2;
}

// A pending event pair (mla_time_next_launch) brackets both launches.
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.n == 0) return hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_launch_events(&e0, &e1);
  hipError_t e = hipSuccess;
  if (p.lpad > 0) {
    e = launch_kernel_events(upproj_kernel, dim3(p.lpad / kUpTile, p.heads, 2 * p.batch), dim3(256), stream, e0,
                             nullptr, p);
    if (e != hipSuccess) return e;
    e0 = nullptr;
  }
  const int nqb = (p.n + kQBlock - 1) / kQBlock;
  if (p.scale_log2 > 0.0f)
    return launch_kernel_events(prefill_attn_kernel<true>, dim3(nqb, p.heads, p.batch), dim3(256), stream, e0, e1, p);
  return launch_kernel_events(prefill_attn_kernel<false>, dim3(nqb, p.heads, p.batch), dim3(256), stream, e0, e1, p);
}

}  // namespace mla
