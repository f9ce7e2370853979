// Device-side helpers shared by the qmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// ---------------------------------------------------------------------------
// int4, interleaved word layout: word j of a row holds inputs 8j..8j+7 with
// input 8j+2k in bits [4k,4k+4) and 8j+2k+1 in bits [16+4k,16+4k+4).
// Pair k of a word, moved so that each 4-bit code u lands in the top mantissa
// bits of a 16-bit float whose exponent encodes 1.0, reads as 1 + u/16
// exactly.  A group sum of such values times x is then
//   sum (u-8) x = 16 * sum (1+u/16) x - 24 * sum x.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t int4_pair_bf16(uint32_t w, int k) {
  // bf16: 7 mantissa bits, code goes to bits [3,7) of each half
  const uint32_t m = 0x00780078u, one = 0x3F803F80u;
  uint32_t s = (k == 0) ? (w << 3) : (w >> (4 * k - 3));
  return (s & m) | one;
}
__device__ __forceinline__ uint32_t int4_pair_f16(uint32_t w, int k) {
  // fp16: 10 mantissa bits, code goes to bits [6,10) of each half
  const uint32_t m = 0x03C003C0u, one = 0x3C003C00u;
  uint32_t s = (k == 0) ? (w << 6) : (k == 1) ? (w << 2) : (w >> (4 * k - 6));
  return (s & m) | one;
}

// ---------------------------------------------------------------------------
// NVFP4: byte j holds inputs (2j, 2j+1) as E2M1 codes (low nibble first).
// gfx950's scaled conversions apply only the exponent of their fp32 scale, so
// they are called with 1.0 and the E4M3 block scale is applied separately.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t w, int j) {
  bf16x2 v;
  switch (j) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t fp4_pair_f16(uint32_t w, int j) {
  f16x2 v;
  switch (j) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, v);
}
// E4M3 ("fn") byte j of w -> float, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t w, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_scalef32_f32_fp8(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_f32_fp8(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_f32_fp8(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_f32_fp8(w, 1.0f, 3);
  }
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ---------------------------------------------------------------------------
// Wave reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace qmoe
