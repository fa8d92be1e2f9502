// Device-side helpers shared by the pnattn kernels (gfx950 / CDNA4 only).
//
// Register layouts used throughout (measured on gfx950 with an in-bounds
// lane-layout check of each builtin):
//  * 32x32 MFMA accumulator (bf16, i8 and f32 inputs alike): lane l, register
//    r holds C[8*(r/4) + 4*(l/32) + r%4][l%32].
//  * v_mfma_f32_32x32x16_bf16: A lane l holds A[l%32][8*(l/32) + e], e=0..7;
//    B lane l holds B[8*(l/32) + e][l%32].
//  * v_mfma_i32_32x32x32_i8: the same with 16 int8 per lane, k = 16*(l/32)+e.
//  * v_mfma_f32_32x32x2f32: one float per lane, k = l/32.
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives
//    element i%4 of the 4-element rows addressed by lanes 4e + i/4, e=0..3.
//  * permlane32_swap(x, x) returns {x[l%32], x[32 + l%32]} in every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_approx(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(0) == 1 exactly
}

// max / sum of a value over the lane pair (l, l ^ 32); both lanes get the
// bitwise-same result (low-half operand first).
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int pair32_isum(int x) {
  auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(r[0] + r[1]);
}

// bf16 bit pattern <-> float (exact widening; RNE narrowing)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float round_to_bf16(float x) {
  return bf16_to_f32(f32_to_bf16(x));
}

// Transposed 64-bit LDS read (ds_read_b64_tr_b16) from a generic pointer
// into LDS.
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) char*)(p)));
}
__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 lo, i16x4 hi) {
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// Two E4M3 (OCP fp8, bias 7 on gfx950) products of 32x32x16 over the 16
// bytes of an int8-style operand chunk: the low eight bytes of every lane
// form one 16-deep product and the high eight the other, a consistent
// split of the 32 k-values of the chunk between the A and B operands.
// The hardware sums each product's 16 terms with less than fp32 precision
// (about 7e-5 of the largest partial sum, measured on random operands).
__device__ __forceinline__ f32x16 mfma_fp8x2(i32x4 a, i32x4 b, f32x16 c) {
  const long alo = (long)(((uint64_t)(uint32_t)a[1] << 32) | (uint32_t)a[0]);
  const long ahi = (long)(((uint64_t)(uint32_t)a[3] << 32) | (uint32_t)a[2]);
  const long blo = (long)(((uint64_t)(uint32_t)b[1] << 32) | (uint32_t)b[0]);
  const long bhi = (long)(((uint64_t)(uint32_t)b[3] << 32) | (uint32_t)b[2]);
  c = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(alo, blo, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(ahi, bhi, c, 0, 0, 0);
}

// The same E4M3 products as two mfma_fp8x2 calls, in one 32x32x64 product
// of gfx950 (the block-scaled form with unit scales, E8M0 code 127 = 2^0):
// lane by lane the 32 bytes of chunks a0, a1 (A) and b0, b1 (B) are the
// k-values the two operands share, in the same order.  It runs at the fp8
// rate, twice that of the 32x32x16 fp8 product: 64 cycles for 64 k-values
// instead of 128.
__device__ __forceinline__ f32x16 mfma_fp8x4(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, f32x16 c) {
  const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> E4M3 code, round to nearest with ties to even; magnitudes at or
// above 448 saturate to 448, NaN gives 0x7f, the sign bit is the input's.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7f;
  if (a >= 448.0f) return (uint8_t)(sign | 0x7eu);
  uint32_t mag;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code = multiple)
    mag = (uint32_t)rintf(a * 512.0f);
  } else {  // round the fp32 significand to 3 bits, ties to even
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20;  // exponent:mantissa
    mag = r - ((127u - 7u) << 3);
    if (mag > 0x7eu) mag = 0x7eu;
  }
  return (uint8_t)(sign | mag);
}

// Compile-time constants as types, for loops whose index must be a constant.
template <int I> struct IntC { static constexpr int value = I; };
template <bool B> struct BoolC { static constexpr bool value = B; };

// f(IntC<0>{}), ..., f(IntC<N-1>{}): a loop whose index is a constant
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

// Row order of a 32-row MFMA A operand that makes the 32x32 accumulator
// land in the order of the next product's operand: when row m of the A
// operand carries element perm_row(m) of its 32-element subtile, accumulator
// register r of lane group g (lanes 32g..32g+31) holds element
// elem_of_reg(r, g) = 16(r/8) + 8g + r%8, so a lane's sixteen results of a
// subtile are, in register order, the sixteen consecutive pairs of eight
// elements that lane feeds as the B operand of a 32x32x16 product.
__device__ __forceinline__ int perm_row(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
__device__ __forceinline__ int elem_of_reg(int r, int g) { return 16 * (r >> 3) + 8 * g + (r & 7); }

}  // namespace pn
