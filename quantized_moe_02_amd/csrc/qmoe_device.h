// Device-side helpers shared by the qmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
// (x & mask) | one in a single v_and_or_b32.  gfx9 VOP3 encodings cannot hold
// 32-bit literals, so left alone the compiler splits this into v_and + v_or;
// here the mask comes from an SGPR and `one` from a VGPR (one constant-bus read).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t one) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(one));
  return r;
}
// A VGPR holding `c`, opaque to the optimiser so it stays a register operand.
__device__ __forceinline__ uint32_t vreg(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}
// One-constants for the two 16-bit float flavours (1.0 in both halves).
struct Int4Consts {
  uint32_t one_bf16, one_f16;
};
__device__ __forceinline__ Int4Consts int4_consts() { return {vreg(0x3F803F80u), vreg(0x3C003C00u)}; }

__device__ __forceinline__ uint32_t int4_pair_bf16(uint32_t w, int k, uint32_t one) {
  // bf16: 7 mantissa bits, code goes to bits [3,7) of each half
  const uint32_t s = (k == 0) ? (w << 3) : (w >> (4 * k - 3));
  return and_or(s, 0x00780078u, one);
}
__device__ __forceinline__ uint32_t int4_pair_f16(uint32_t w, int k, uint32_t one) {
  // fp16: 10 mantissa bits, code goes to bits [6,10) of each half
  const uint32_t s = (k == 0) ? (w << 6) : (k == 1) ? (w << 2) : (w >> (4 * k - 6));
  return and_or(s, 0x03C003C0u, one);
}
// int2 codes (word layout of MOE_WFMT_INT2_ROW_F32: pair k = inputs 2k, 2k+1
// of the word's 16 in bits [2k, 2k+2) and [16+2k, 16+2k+2)) into the top two
// mantissa bits of a 16-bit float of exponent 1.0: 1 + u/4 exactly.
__device__ __forceinline__ uint32_t int2_pair_bf16(uint32_t w, int k, uint32_t one) {
  // bf16: code goes to bits [5,7) of each half
  const uint32_t s = (k <= 2) ? (w << (5 - 2 * k)) : (w >> (2 * k - 5));
  return and_or(s, 0x00600060u, one);
}
__device__ __forceinline__ uint32_t int2_pair_f16(uint32_t w, int k, uint32_t one) {
  // fp16: code goes to bits [8,10) of each half
  const uint32_t s = (k <= 4) ? (w << (8 - 2 * k)) : (w >> (2 * k - 8));
  return and_or(s, 0x03000300u, one);
}
// int8 bytes b0, b1 (selector 0x04010400) or b2, b3 (0x04030402) of a word
// whose sign bits were flipped (u = q + 128) into the mantissa of fp16 1024:
// 1024 + u exactly.
__device__ __forceinline__ uint32_t int8_pair_f16(uint32_t wflip, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, wflip, sel);
}
__device__ __forceinline__ uint32_t int4_pair_bf16(uint32_t w, int k) {
  return int4_pair_bf16(w, k, 0x3F803F80u);
}
__device__ __forceinline__ uint32_t int4_pair_f16(uint32_t w, int k) {
  return int4_pair_f16(w, k, 0x3C003C00u);
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

// ---------------------------------------------------------------------------
// Buffer loads: a 128-bit resource descriptor in SGPRs (base, size in bytes;
// word 3 = 0x00020000 for the gfx9 family), a per-lane 32-bit VGPR offset and
// a wave-uniform SGPR offset.  Rows of one matrix then share a single VGPR
// offset, and reads past `bytes` return zero.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bload16(uint32_t (&d)[4], rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  d[0] = v[0];
  d[1] = v[1];
  d[2] = v[2];
  d[3] = v[3];
}
// The same 16-byte load at device scope (sc1): it reads what other
// workgroups' device-scope stores wrote during this launch.
__device__ __forceinline__ uint4 bload16_device(rsrc_t r, uint32_t voff, uint32_t soff) {
  constexpr int kSc1 = 16;   // cache-policy bit of device (agent) scope
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kSc1);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void bload8(uint32_t* d, rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  d[0] = v[0];
  d[1] = v[1];
}
__device__ __forceinline__ uint32_t bload_u16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Hides a loaded value from the optimiser, so that a later select on it is
// not turned back into a predicated (branching) load.
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ---------------------------------------------------------------------------
// Wave-wide reductions on the VALU cross-lane paths (no LDS round trip):
// DPP quad_perm xor1 / xor2, row_half_mirror (i <-> 7-i in 8) and row_mirror
// (i <-> 15-i in 16) combine lanes within a row of 16; v_permlane16_swap and
// v_permlane32_swap then exchange rows.  Called with (v, v), the swaps return
// {v[i & ~16], v[i | 16]} and {v[i & 31], v[i | 32]}, so combining the two
// halves symmetrically gives every lane the same result.  Every step pairs
// lanes symmetrically, so all 64 lanes end with bit-identical values.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ float swap16_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<kDppXor1>(v);
  v += dppf<kDppXor2>(v);
  v += dppf<kDppHalfMirror>(v);
  v += dppf<kDppMirror>(v);
  v = swap16_sum(v);
  return swap32_sum(v);
}

template <int CTRL>
__device__ __forceinline__ double dppd(double v) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = dpp<CTRL>((uint32_t)b), hi = dpp<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
// {value at lane i & ~M, value at lane i | M} for M = 16 or 32
template <int M>
__device__ __forceinline__ void swap_pair(double v, double& a, double& b) {
  const uint64_t x = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  uint32_t alo, ahi, blo, bhi;
  if constexpr (M == 16) {
    auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    alo = rl[0]; blo = rl[1]; ahi = rh[0]; bhi = rh[1];
  } else {
    auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    alo = rl[0]; blo = rl[1]; ahi = rh[0]; bhi = rh[1];
  }
  a = __longlong_as_double(((uint64_t)ahi << 32) | alo);
  b = __longlong_as_double(((uint64_t)bhi << 32) | blo);
}
template <int M>
__device__ __forceinline__ void swap_pair(int v, int& a, int& b) {
  if constexpr (M == 16) {
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    a = (int)r[0]; b = (int)r[1];
  } else {
    auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    a = (int)r[0]; b = (int)r[1];
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dppd<kDppXor1>(v);
  v += dppd<kDppXor2>(v);
  v += dppd<kDppHalfMirror>(v);
  v += dppd<kDppMirror>(v);
  double a, b;
  swap_pair<16>(v, a, b);
  v = a + b;
  swap_pair<32>(v, a, b);
  return a + b;
}

// (value, index) arg-max across the wave: larger value wins, equal values go
// to the lower index.  Symmetric, so all lanes agree.
__device__ __forceinline__ void better_of(double& v, int& i, double ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(double& v, int& i) {
  better_of(v, i, dppd<CTRL>(v), (int)dpp<CTRL>((uint32_t)i));
}
template <int M>
__device__ __forceinline__ void argmax_swap(double& v, int& i) {
  double a, b;
  int ia, ib;
  swap_pair<M>(v, a, b);
  swap_pair<M>(i, ia, ib);
  v = a;
  i = ia;
  better_of(v, i, b, ib);
}
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  argmax_dpp<kDppXor1>(v, i);
  argmax_dpp<kDppXor2>(v, i);
  argmax_dpp<kDppHalfMirror>(v, i);
  argmax_dpp<kDppMirror>(v, i);
  argmax_swap<16>(v, i);
  argmax_swap<32>(v, i);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, j>) for j = 0 .. N-1
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace qmoe
