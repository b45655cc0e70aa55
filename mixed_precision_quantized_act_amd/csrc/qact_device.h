// Device helpers shared by the gfx950 kernels of libqact: bfloat16 bit
// handling and the E2M1 / E4M3 encoders and decoders of the NVFP4 format
// (E2M1 elements, one E4M3 scale per 16, one float32 tensor scale), rounding
// to nearest with ties to the even code and saturating.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qact_internal.h"

namespace qact {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs; overflow
// rounds to infinity as round-to-nearest prescribes).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two float32 -> packed bfloat16 (a in the low half), round to nearest
// even, one v_cvt_pk_bf16_f32: equal to round-to-nearest-even on every
// finite float32 (tests/test_gpu_convert.py runs it on all of them through
// qa_test_convert).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t bf16_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// 1/y, and 0 for y == 0 (correctly rounded float32 division).
__device__ __forceinline__ float recip0(float y) { return y == 0.0f ? 0.0f : 1.0f / y; }

// E4M3FN code (0..0x7E) of a finite float32 scale s >= 0: nearest value,
// ties to the even code, saturating at 448 (0x7E).
//   normal range (s >= 2^-6): round the float32 encoding to 3 mantissa
//   bits (a carry moves into the exponent), then rebias 127 -> 7;
//   below 2^-6 the E4M3 step is 2^-9: code = rint(s * 512), up to 8 = 0x08.
// Both ranges are computed and one is selected (no branch: lanes of a
// wave take different ranges).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  const uint32_t sub = (uint32_t)rintf(s * 512.0f);
  const uint32_t u = __float_as_uint(s);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // exp8:mant3
  r -= (127u - 7u) << 3;                                   // (wraps below 2^-6: not selected)
  r = r > 0x7Eu ? 0x7Eu : r;
  return s < 0.015625f ? sub : r;
}

// Value of a non-negative E4M3FN code 0..0x7E (both forms computed, one
// selected).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  const float sub = (float)m * 0.001953125f;                  // m * 2^-9
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// E2M1 codes of two float32 values, packed into byte `sel` of `old` (the
// first value in the low nibble): nearest of 0,.5,1,1.5,2,3,4,6 with ties
// to the even code, saturating at 6, bit 3 = the sign bit of the input.
// gfx950's v_cvt_scalef32_pk_fp4_f32 with a unit scale rounds exactly so
// on every finite float32 (tests/test_gpu_convert.py, through
// qa_test_convert; e4m3_encode likewise on every non-negative one).
#define QACT_E2M1_PK(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// E2M1 codes of the 8 bf16 values of a 16-byte vector times `inv`, as 8
// nibbles (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t e2m1_pack8(u32x4 w, float inv) {
  uint32_t r = 0;
  r = QACT_E2M1_PK(r, bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, 0);
  r = QACT_E2M1_PK(r, bf16_lo(w[1]) * inv, bf16_hi(w[1]) * inv, 1);
  r = QACT_E2M1_PK(r, bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, 2);
  r = QACT_E2M1_PK(r, bf16_lo(w[3]) * inv, bf16_hi(w[3]) * inv, 3);
  return r;
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

// Max of the |bf16| bit patterns of the 8 values in a 16-byte vector,
// folded into mx (the patterns of non-negative floats sort as integers);
// two values per packed 16-bit max.
__device__ __forceinline__ u16x2 abs_max8_pk(u32x4 a, u16x2 mx) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, a[i] & 0x7FFF7FFFu));
  return mx;
}
__device__ __forceinline__ uint32_t fold_max(u16x2 m) { return max((uint32_t)m[0], (uint32_t)m[1]); }

// E2M1 value times 2 (an integer in -12..12) of a 4-bit code.
__device__ __forceinline__ int e2m1_twice(uint32_t c) {
  const int mag = (int)((0xC8643210u >> ((c & 7u) * 4u)) & 0xFu);   // 0,1,2,3,4,6,8,12
  return (c & 8u) ? -mag : mag;
}

// True when the call's gate is closed: its kernels then return at once.
// (One uniform byte load; every kernel of a gated call checks it first.)
__device__ __forceinline__ bool gated_off(Gate g) {
  if (!g.flags) return false;
  const uint32_t v = *g.flags;
  if ((v & g.bits) == 0u || (v & g.veto) != 0u) return true;
  return g.flags2 && (*g.flags2 & g.bits2) == 0u;
}

// Wave-level (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace qact
