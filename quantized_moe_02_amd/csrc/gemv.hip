// Grouped GEMV for decode-shaped calls: the SwiGLU expert FFN over 4-bit
// weights dequantised in registers (page "Show HN: Menjalankan GLM 5.2 di
// komputer lambat", sections "Cara kerja eksekusi MoE" and "Fitur utama";
// NVFP4 per page "NVIDIA stellt neues GLM-5.2 NVFP4 Modell vor", section
// "Technische Details").
//
// The work is HBM-bound: every selected expert's packed weights are streamed
// once per call.  A lane owns whole 32-input groups (16 bytes of codes, one
// 128-bit load, plus the group's scale), turns each pair of codes into a pair
// of 16-bit floats with two integer ops, and accumulates with the packed dot
// products v_dot2_f32_{bf16,f16}; the partial sums are reduced across the
// wave at the end.
//   gate/up  x (bf16) . deq(Wg), deq(Wu), then h = silu(g) * u, stored fp16.
//   down     h (fp16) . deq(Wd), fp32 out per pick.
// A slot's tokens go through the weights two per pass, an odd last one
// alone (most decode slots hold one token, whose pass then does no extra
// arithmetic).
// Grid: (row blocks, expert slots); slot s < max_slots is the s-th active
// expert of the permutation (blocks past n_active exit), the last slot is the
// expert applied to every token (shared expert or dense mode).
#include "qmoe_device.h"

namespace qmoe {
namespace {


struct Slot {
  bool ok;
  bool routed;
  int e;          // expert index inside its weight set
  int tok_begin;  // first sorted slot (routed) or 0
  int M;          // tokens
};

__device__ __forceinline__ Slot resolve_slot(const FfnArgs& a, int slot) {
  Slot r;
  const int routed_slots = a.has_routed ? a.max_slots : 0;
  if (slot < routed_slots) {
    r.routed = true;
    r.ok = slot < *a.n_active;
    if (!r.ok) return r;
    r.e = a.active[slot];
    r.tok_begin = a.offsets[r.e];
    r.M = a.offsets[r.e + 1] - r.tok_begin;
  } else {
    r.routed = false;
    r.ok = a.has_dense;
    r.e = 0;
    r.tok_begin = 0;
    r.M = a.T;
  }
  return r;
}

__device__ __forceinline__ int token_of(const FfnArgs& a, const Slot& s, int m) {
  return s.routed ? a.sorted_token[s.tok_begin + m] : m;
}

__device__ __forceinline__ void load16(uint32_t* dst, const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  dst[0] = v.x;
  dst[1] = v.y;
  dst[2] = v.z;
  dst[3] = v.w;
}

// One 32-input group of one weight row against TB activation groups.
// acc[tb] += sum_k w_k * act_k for the group.
template <int FMT, bool F16ACT, int TB>
__device__ __forceinline__ void group_dot(const uint32_t (&wq)[4], uint32_t sc,
                                          const uint32_t (&act)[TB][16], const float (&asum)[TB],
                                          float gs, float (&acc)[TB]) {
  if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
    uint32_t p[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        p[4 * j + k] = F16ACT ? int4_pair_f16(wq[j], k) : int4_pair_bf16(wq[j], k);
    const float s16 = 16.0f * half_bits_to_f32(sc & 0xffffu);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) d = F16ACT ? dot2_f16(p[i], act[tb][i], d) : dot2_bf16(p[i], act[tb][i], d);
      acc[tb] = fmaf(s16, fmaf(-1.5f, asum[tb], d), acc[tb]);
    }
  } else {
    uint32_t p[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) p[4 * j + k] = F16ACT ? fp4_pair_f16(wq[j], k) : fp4_pair_bf16(wq[j], k);
    const float s0 = e4m3_to_f32(sc, 0) * gs;
    const float s1 = e4m3_to_f32(sc, 1) * gs;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d0 = F16ACT ? dot2_f16(p[i], act[tb][i], d0) : dot2_bf16(p[i], act[tb][i], d0);
#pragma unroll
      for (int i = 8; i < 16; ++i) d1 = F16ACT ? dot2_f16(p[i], act[tb][i], d1) : dot2_bf16(p[i], act[tb][i], d1);
      acc[tb] = fmaf(s0, d0, fmaf(s1, d1, acc[tb]));
    }
  }
}

// Scale word of group c of a row: int4 -> the fp16 bits; nvfp4 -> two E4M3 bytes.
template <int FMT>
__device__ __forceinline__ uint32_t load_scale(const void* s, size_t row, int nG, int c) {
  if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
    return reinterpret_cast<const uint16_t*>(s)[row * nG + c];
  } else {
    return reinterpret_cast<const uint16_t*>(s)[row * nG + c];  // bytes 2c, 2c+1 of the row
  }
}

// Per-row-scale formats: one 32-input group of one row (BITS 32-bit code
// words) against TB activation groups, without the row scale (applied once
// per row after the reduction).  acc[tb] += sum_k q_k * act_k.
//   int4: 1 + u/16 pairs, sum (u-8) a = 16 (d - 1.5 A)
//   int2: 1 + u/4 pairs,  sum (u-2) a = 4 (d - 1.5 A)
//   int8: u = q + 128; bf16 activations: fp32 products, sum q a = d - 128 A;
//         fp16 activations: 1024 + u pairs, sum q a = d - 1152 A
// with d the dot product of the formed values and A the activation sum.
template <int FMT, bool F16ACT, int TB>
__device__ __forceinline__ void group_dot_row(const uint32_t* wq, const uint32_t (&act)[TB][16],
                                              const float (&asum)[TB], float (&acc)[TB]) {
  if constexpr (FMT == MOE_WFMT_INT8_ROW_F32 && !F16ACT) {
    float d[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) d[tb] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = wq[j] ^ 0x80808080u;
      float u[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) u[b] = (float)((w >> (8 * b)) & 0xffu);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint32_t x01 = act[tb][2 * j], x23 = act[tb][2 * j + 1];
        d[tb] = fmaf(u[0], __uint_as_float(x01 << 16), d[tb]);
        d[tb] = fmaf(u[1], __uint_as_float(x01 & 0xffff0000u), d[tb]);
        d[tb] = fmaf(u[2], __uint_as_float(x23 << 16), d[tb]);
        d[tb] = fmaf(u[3], __uint_as_float(x23 & 0xffff0000u), d[tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] += fmaf(-128.0f, asum[tb], d[tb]);
  } else {
    uint32_t p[16];
    float mul, off;
    if constexpr (FMT == MOE_WFMT_INT8_ROW_F32) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = wq[j] ^ 0x80808080u;
        p[2 * j] = int8_pair_f16(w, 0x04010400u);
        p[2 * j + 1] = int8_pair_f16(w, 0x04030402u);
      }
      mul = 1.0f;
      off = -1152.0f;
    } else if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          p[8 * j + k] = F16ACT ? int2_pair_f16(wq[j], k, 0x3C003C00u) : int2_pair_bf16(wq[j], k, 0x3F803F80u);
      mul = 4.0f;
      off = -1.5f;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          p[4 * j + k] = F16ACT ? int4_pair_f16(wq[j], k) : int4_pair_bf16(wq[j], k);
      mul = 16.0f;
      off = -1.5f;
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) d = F16ACT ? dot2_f16(p[i], act[tb][i], d) : dot2_bf16(p[i], act[tb][i], d);
      acc[tb] = fmaf(mul, fmaf(off, asum[tb], d), acc[tb]);
    }
  }
}

// The code words of one 32-input group: 32 * bits / 8 bytes at p.
template <int FMT>
__device__ __forceinline__ void load_codes(uint32_t* dst, const uint8_t* p) {
  constexpr int BITS = wfmt_bits(FMT);
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) load16(dst + 4 * i, p + 16 * i);
  }
}

template <int FMT>
__device__ __forceinline__ float row_scale(const void* s, size_t row) {
  return wfmt_row(FMT) ? reinterpret_cast<const float*>(s)[row] : 1.0f;
}

#ifndef QMOE_GU_RPW
#define QMOE_GU_RPW 4
#endif
#ifndef QMOE_GU_RPW8
#define QMOE_GU_RPW8 1
#endif
#ifndef QMOE_DN_RPW
#define QMOE_DN_RPW 4
#endif
#ifndef QMOE_DN_RPW8
#define QMOE_DN_RPW8 4
#endif
// Rows (gate/up: row pairs) per wave.  int8's 32-byte groups take one row
// pair in gate/up: more waves in flight (45 us at one token against 48 with
// two row pairs and 58 with four); two rows per wave elsewhere measured no
// better.
template <int FMT>
constexpr int gu_rpw() {
  return wfmt_bits(FMT) == 8 ? QMOE_GU_RPW8 : QMOE_GU_RPW;
}
template <int FMT>
constexpr int dn_rpw() {
  return wfmt_bits(FMT) == 8 ? QMOE_DN_RPW8 : QMOE_DN_RPW;
}

// The registers of one group step of a pass: codes (and group scale words) of
// the wave's RPW rows in NP projections, and the TB tokens' 32 inputs.
template <int FMT, int TB, int NP, int RPW>
struct GemvStep {
  uint32_t q[NP][RPW][wfmt_bits(FMT)];
  uint32_t sc[NP][RPW];
  uint32_t act[TB][16];
};

// The group steps c = lane, lane + 64, ... < nG of a pass.  (Issuing step
// i + 1's loads before step i is reduced measured slower: 90.4 against 88.9
// us per int8 single-token call, at half the waves per SIMD.)
template <class Step, class Load, class Compute>
__device__ __forceinline__ void group_steps(int nG, Load load, Compute compute) {
  for (int c = threadIdx.x & 63; c < nG; c += 64) {
    Step st;
    load(st, c);
    compute(st, c);
  }
}

// Gate/up of tokens m0 .. m0 + TB - 1 of a slot (TB = 2 while two remain,
// then 1): each pass streams the wave's rows once.
template <int FMT, int TB>
__device__ __forceinline__ void gateup_pass(const FfnArgs& a, const Slot& sl, const ExpertSet& X,
                                            int row0, int m0) {
  constexpr int RPW = gu_rpw<FMT>();
  const int lane = threadIdx.x & 63;
  const int inter = X.inter;
  const int H = a.H;
  const int nG = H / 32;
  constexpr int BITS = wfmt_bits(FMT);
  constexpr bool ROW = wfmt_row(FMT);
  const size_t rowBytes = (size_t)H * BITS / 8;
  const size_t rbase = (size_t)sl.e * inter;
  const float gg = (FMT == MOE_WFMT_NVFP4) ? X.gate.g[sl.e] : 1.0f;
  const float gu = (FMT == MOE_WFMT_NVFP4) ? X.up.g[sl.e] : 1.0f;
  uint16_t* hbase = sl.routed ? a.h_routed + (size_t)sl.tok_begin * a.ldh : a.h_dense;
  int tok[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) tok[tb] = token_of(a, sl, m0 + tb);
  float ag[RPW][TB], au[RPW][TB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) ag[r][tb] = au[r][tb] = 0.0f;

  using Step = GemvStep<FMT, TB, 2, RPW>;
  auto load = [&](Step& st, int c) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const size_t row = rbase + row0 + r;
      load_codes<FMT>(st.q[0][r], X.gate.q + row * rowBytes + (size_t)c * (4 * BITS));
      load_codes<FMT>(st.q[1][r], X.up.q + row * rowBytes + (size_t)c * (4 * BITS));
      if constexpr (!ROW) {
        st.sc[0][r] = load_scale<FMT>(X.gate.s, row, nG, c);
        st.sc[1][r] = load_scale<FMT>(X.up.s, row, nG, c);
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const uint16_t* xp = a.x + (size_t)tok[tb] * H + (size_t)c * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) load16(&st.act[tb][4 * q], xp + 8 * q);
    }
  };
  auto compute = [&](const Step& st, int) {
    float xs[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float s = 0.0f;
      if constexpr (FMT != MOE_WFMT_NVFP4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s = dot2_bf16(st.act[tb][i], 0x3F803F80u, s);
      }
      xs[tb] = s;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if constexpr (ROW) {
        group_dot_row<FMT, false, TB>(st.q[0][r], st.act, xs, ag[r]);
        group_dot_row<FMT, false, TB>(st.q[1][r], st.act, xs, au[r]);
      } else {
        group_dot<FMT, false, TB>(st.q[0][r], st.sc[0][r], st.act, xs, gg, ag[r]);
        group_dot<FMT, false, TB>(st.q[1][r], st.sc[1][r], st.act, xs, gu, au[r]);
      }
    }
  };
  group_steps<Step>(nG, load, compute);
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const size_t row = rbase + row0 + r;
      const float g = wave_sum(ag[r][tb]) * row_scale<FMT>(X.gate.s, row);
      const float u = wave_sum(au[r][tb]) * row_scale<FMT>(X.up.s, row);
      if (lane == r * TB + tb) {
        const _Float16 hv = (_Float16)silu_mul(g, u);
        hbase[(size_t)(m0 + tb) * a.ldh + row0 + r] = __builtin_bit_cast(uint16_t, hv);
      }
    }
}

template <int FMT>
__global__ void __launch_bounds__(256) gateup_gemv_kernel(FfnArgs a) {
  const int wv = threadIdx.x >> 6;
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.ok) return;
  const ExpertSet& X = sl.routed ? a.routed : a.dense;
  const int row0 = (blockIdx.x * 4 + wv) * gu_rpw<FMT>();
  if (row0 >= X.inter) return;
  int m0 = 0;
  for (; m0 + 2 <= sl.M; m0 += 2) gateup_pass<FMT, 2>(a, sl, X, row0, m0);
  if (m0 < sl.M) gateup_pass<FMT, 1>(a, sl, X, row0, m0);
}

// Down of tokens m0 .. m0 + TB - 1 of a slot, as gateup_pass.
template <int FMT, int TB>
__device__ __forceinline__ void down_pass(const FfnArgs& a, const Slot& sl, const ExpertSet& X,
                                          int row0, int m0) {
  constexpr int RPW = dn_rpw<FMT>();
  const int lane = threadIdx.x & 63;
  const int inter = X.inter;
  const int H = a.H;
  const int nG = inter / 32;
  constexpr int BITS = wfmt_bits(FMT);
  constexpr bool ROW = wfmt_row(FMT);
  const size_t rowBytes = (size_t)inter * BITS / 8;
  const size_t rbase = (size_t)sl.e * H;
  const float gd = (FMT == MOE_WFMT_NVFP4) ? X.down.g[sl.e] : 1.0f;
  const uint16_t* hbase = sl.routed ? a.h_routed + (size_t)sl.tok_begin * a.ldh : a.h_dense;
  float* obase = sl.routed ? a.o_routed + (size_t)sl.tok_begin * H : a.o_dense;
  float acc[RPW][TB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[r][tb] = 0.0f;

  using Step = GemvStep<FMT, TB, 1, RPW>;
  auto load = [&](Step& st, int c) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const size_t row = rbase + row0 + r;
      load_codes<FMT>(st.q[0][r], X.down.q + row * rowBytes + (size_t)c * (4 * BITS));
      if constexpr (!ROW) st.sc[0][r] = load_scale<FMT>(X.down.s, row, nG, c);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const uint16_t* hp = hbase + (size_t)(m0 + tb) * a.ldh + (size_t)c * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) load16(&st.act[tb][4 * q], hp + 8 * q);
    }
  };
  auto compute = [&](const Step& st, int) {
    float hs[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float s = 0.0f;
      if constexpr (FMT != MOE_WFMT_NVFP4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s = dot2_f16(st.act[tb][i], 0x3C003C00u, s);
      }
      hs[tb] = s;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if constexpr (ROW)
        group_dot_row<FMT, true, TB>(st.q[0][r], st.act, hs, acc[r]);
      else
        group_dot<FMT, true, TB>(st.q[0][r], st.sc[0][r], st.act, hs, gd, acc[r]);
    }
  };
  group_steps<Step>(nG, load, compute);
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float v = wave_sum(acc[r][tb]) * row_scale<FMT>(X.down.s, rbase + row0 + r);
      if (lane == r * TB + tb) obase[(size_t)(m0 + tb) * H + row0 + r] = v;
    }
}

template <int FMT>
__global__ void __launch_bounds__(256) down_gemv_kernel(FfnArgs a) {
  const int wv = threadIdx.x >> 6;
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.ok) return;
  const ExpertSet& X = sl.routed ? a.routed : a.dense;
  const int row0 = (blockIdx.x * 4 + wv) * dn_rpw<FMT>();
  if (row0 >= a.H) return;
  int m0 = 0;
  for (; m0 + 2 <= sl.M; m0 += 2) down_pass<FMT, 2>(a, sl, X, row0, m0);
  if (m0 < sl.M) down_pass<FMT, 1>(a, sl, X, row0, m0);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// One block per (token, 1024 columns): each thread's k + 1 row loads are all
// in flight together (a block per token leaves most of the chip idle at small
// T and serialises the rows).  Per element the sum runs in pick order, then
// the shared expert, as before.
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int H = a.H, K = a.K;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < K; ++i) {
    // inv_perm -1: a pick the adaptive top-p dropped (weight 0, no row)
    const int p = a.inv_perm[(size_t)t * K + i];
    const float w = a.tw[(size_t)t * K + i];
    float4 o = *reinterpret_cast<const float4*>(a.expert_out + (size_t)(p < 0 ? 0 : p) * H + n);
    if (p < 0) o = make_float4(0.f, 0.f, 0.f, 0.f);
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
  }
  if (a.shared_out) {
    const float4 o = *reinterpret_cast<const float4*>(a.shared_out + (size_t)t * H + n);
    acc.x += o.x;
    acc.y += o.y;
    acc.z += o.z;
    acc.w += o.w;
  }
  if (a.out_bf16) {
    uint2 v;
    v.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    v.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + (size_t)t * H + n) = v;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + (size_t)t * H + n) = acc;
  }
}

}  // namespace

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  const int slots = (a.has_routed ? a.max_slots : 0) + (a.has_dense ? 1 : 0);
  if (slots == 0) return hipSuccess;
  int max_inter = 0;
  if (a.has_routed) max_inter = a.routed.inter;
  if (a.has_dense && a.dense.inter > max_inter) max_inter = a.dense.inter;
  hipError_t e;
  auto launch = [&](auto F) {
    constexpr int fmt = decltype(F)::value;
    constexpr int rows_per_block = 4 * gu_rpw<fmt>();
    dim3 g1((max_inter + rows_per_block - 1) / rows_per_block, slots);
    hipLaunchKernelGGL(gateup_gemv_kernel<fmt>, g1, dim3(256), 0, s, a);
    return hipGetLastError();
  };
  auto launch_down = [&](auto F) {
    constexpr int fmt = decltype(F)::value;
    constexpr int rows_per_block = 4 * dn_rpw<fmt>();
    dim3 g2((a.H + rows_per_block - 1) / rows_per_block, slots);
    hipLaunchKernelGGL(down_gemv_kernel<fmt>, g2, dim3(256), 0, s, a);
    return hipGetLastError();
  };
  if ((e = dispatch_wfmt(a.wfmt, launch)) != hipSuccess) return e;
  if (tr && (e = tr->mark("gateup_gemv")) != hipSuccess) return e;
  if ((e = dispatch_wfmt(a.wfmt, launch_down)) != hipSuccess) return e;
  if (tr && (e = tr->mark("down_gemv")) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.T, (a.H + 1023) / 1024), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && tr) e = tr->mark("combine");
  return e;
}

}  // namespace qmoe
