// Device helpers for the gfx950 MLA kernels: storage conversions, MFMA
// operand types, LDS address-space pointers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))
typedef MLA_LDS char lds_char;

// bfloat16 is the upper half of a binary32.
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// binary32 -> bfloat16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// two binary32 -> packed bfloat16 pair (one v_cvt_pk_bf16_f32, round to
// nearest even); lo in bits 15:0.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const b2_t v = __builtin_convertvector((f2_t){lo, hi}, b2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// D = A(16x32) * B(32x16) + C on bf16 inputs with fp32 accumulation.
// Lane l holds row/column l%16 and K elements 8*(l/16)..+7 of A/B; the
// result holds column l%16 and rows 4*(l/16)..+3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed 64-bit LDS read: in each group of 16 lanes, lane i receives
// column i of the 4x16 block of 16-bit values whose rows the group's lanes
// read four at a time (lane i reads row i/4, elements 4*(i%4)..+3).
__device__ __forceinline__ bf16x4_t lds_read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4_t*)p);
}

__device__ __forceinline__ bf16x8_t lds_read_b128(const lds_char* p) {
  return *(const MLA_LDS bf16x8_t*)p;
}

__device__ __forceinline__ bf16x8_t concat(const bf16x4_t& lo, const bf16x4_t& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return *(const bf16x8_t*)p;
}

// 2^x on the hardware transcendental unit (results below 2^-126 flush to 0,
// which is immaterial for softmax weights next to the row maximum's 2^0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) on the VALU: v_permlane16_swap exchanges odd rows of its first operand
// with even rows of its second, v_permlane32_swap the upper half of the first
// with the lower half of the second; with both operands equal, the pair
// {result0, result1} holds {v[l], v[l^16]} (resp. {v[l], v[l^32]}) up to order.
// Every lane ends with the same bits: (r0 op r1) op (r2 op r3).
__device__ __forceinline__ float wave_max16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace mla
