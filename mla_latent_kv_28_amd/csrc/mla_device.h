// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4).
//
// MFMA operand layouts used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16: A is 32x16, B is 16x32, C is 32x32.
//     lane l = 32*hh + r holds A[r][8*hh + 0..7] and B[8*hh + 0..7][r];
//     accumulator i of lane l is C[8*(i/4) + 4*hh + (i%4)][r].
//   v_mfma_f32_32x32x64_f8f6f4 (e4m3 operands): lane l holds bytes
//     A[r][32*hh + 0..31] and B[32*hh + 0..31][r] in order; the same C layout.
//   v_mfma_f32_32x32x2_f32: lane l holds A[r][hh], B[hh][r]; the same C layout.
//     Eight of them in a row, the e-th fed with element e of an 8-element lane
//     vector, contract a 16-wide k block where lane half hh owns k = 8*hh + e,
//     the same k placement as one bf16 32x32x16.
// Only the pairing of A and B over k matters for a product, so every k block
// may place its k indices as convenient as long as A and B agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2v __attribute__((vector_size(4)));   // operand type of the fp8 conversions

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight fp32 32x32x2 products contracting one 16-wide k block (see above).
__device__ __forceinline__ f32x16 mfma32x32x16_f32(const float (&a)[8], const float (&b)[8], f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two floats to a pair of bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
  typedef float f32x2_ __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_){lo, hi}, bf16x2_));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Byte permutes: low (or high) 16-bit halves of x and y packed as (x_half | y_half << 16).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// 16-byte global load into registers.
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Direct global -> LDS 16-byte load: lane i's 16 bytes land at lds_base + 16*i.
__device__ __forceinline__ void load16_to_lds(const void* gptr, MLA_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3;
// reads past the end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Direct buffer -> LDS loads (the MUBUF form of the direct-to-LDS load): lane
// i's SIZE bytes from base + soff + voff land at lds_base + SIZE * i. The
// compiler counts these on the vector-memory counter only, so LDS reads issued
// after them keep their own in-order waits; with the global (FLAT-encoded)
// form in flight it waits for every outstanding LDS read at each use.
__device__ __forceinline__ void buf_load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                  MLA_LDS void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_load4_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                 MLA_LDS void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read: within each 16-lane group, lane 4*a + x receives
// element x of the 8 bytes addressed by source lanes a, a+4, a+8, a+12.
__device__ __forceinline__ bf16x4 lds_read_tr16(const MLA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p);
}

// Transposing LDS read of bytes: within each 16-lane group, lane 8*a + x
// receives, as byte k (k = 0..7), byte x of the 8 bytes addressed by source
// lane 2*k + a (measured on gfx950).
__device__ __forceinline__ i32x2 lds_read_tr8(const MLA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)p);
}

// 32x32x64 product of e4m3 operands, B scaled by 2^(SCALE_B - 127) (E8M0).
// Always the scaled instruction: in a chain of dependent products on gfx950
// the unscaled form (what zero scales select) issued far slower.
template <int SCALE_B>
__device__ __forceinline__ f32x16 mfma32x32x64_e4m3(const i32x8& a, const i32x8& b, const f32x16& c) {
  static_assert(SCALE_B > 0 && SCALE_B < 255, "an E8M0 scale");
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, SCALE_B);
}

// Two fp8 e4m3 codes (bytes 0,1 or 2,3 of `w`) to two bf16 values (exact).
template <bool HIGH_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HIGH_WORD);
  return __builtin_bit_cast(uint32_t, v);
}

// Eight e4m3 codes (byte k of `w` = element k) to eight bf16 values (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(const i32x2& w) {
  const uint32_t a = e4m3x2_to_bf16x2<false>((uint32_t)w[0]), b = e4m3x2_to_bf16x2<true>((uint32_t)w[0]);
  const uint32_t c = e4m3x2_to_bf16x2<false>((uint32_t)w[1]), d = e4m3x2_to_bf16x2<true>((uint32_t)w[1]);
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

__device__ __forceinline__ float wave_max32(float x) {   // max with the lane 32 away
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace mla
