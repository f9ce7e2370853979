// Small-batch path of the quantized MoE layer (T <= 4 tokens per call):
// decode and short speculative-verify batches.  Every byte of the selected
// experts' packed weights is streamed from HBM once; the work is memory
// bound, so the kernels are built around keeping many independent 128-bit
// loads in flight and doing as little else as possible.
//
//   K1 dec_router          router scores (float64 logits through the
//                          sigmoid, one block per expert)
//   one token, when the device's resident grid is known: dec_fused_t1 --
//                          every workgroup selects the experts itself, then
//                          the shared and routed gate/up GEMVs, a grid
//                          barrier, and the down GEMV with the combine
//   2..4 tokens: dec_select_gateup -- K2 and K3 below in one launch, the
//                          gate/up workgroups waiting for the selecting one
//   otherwise (or under MOE_OPT_NO_GRID_WAIT):
//   K2 dec_select_permute  one workgroup: per-token selection (one wave per
//                          token) and the grouping of the <= 64 picks by
//                          expert (batch union); the shared expert's gate/up
//                          GEMV of every token in the other workgroups
//   K3 dec_gateup          gate/up GEMV of every pick's expert with SwiGLU
//   K4                     down GEMV of every selected expert and the shared
//                          expert with the weighted combine in registers:
//                          dec_down_t1 (one token), dec_down_multi (2..4
//                          tokens, SwiGLU outputs staged in LDS) or
//                          dec_down_combine (other shapes)
//
// Pages: "Show HN: Menjalankan GLM 5.2 di komputer lambat" (sections "Cara
// kerja eksekusi MoE" -- routed experts vs resident shared expert -- and
// "Fitur utama" -- DeepSeek-V3 router, batch-union MoE, int4
// dequant-on-use); "NVIDIA stellt neues GLM-5.2 NVFP4 Modell vor" (section
// "Technische Details": NVFP4 expert weights).
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "select_token.h"

namespace qmoe {
namespace {

#ifndef QMOE_DEC_RPW
#define QMOE_DEC_RPW 1
#endif
#ifndef QMOE_DEC_ITEMS
#define QMOE_DEC_ITEMS 4
#endif
#ifndef QMOE_DEC_DOWN_ROWS
#define QMOE_DEC_DOWN_ROWS 4
#endif
constexpr int kRPW = QMOE_DEC_RPW;           // gate/up row pairs per pipeline item
constexpr int kItems = QMOE_DEC_ITEMS;       // pipeline items per wave (even)
constexpr int kPairsPerWave = kRPW * kItems;
constexpr int kPairsPerBlock = 4 * kPairsPerWave;
#ifndef QMOE_K2_ITEMS
#define QMOE_K2_ITEMS 4
#endif
constexpr int kSharedRP = 1;                              // K2 shared gate/up: row pairs per item
constexpr int kSharedItems = QMOE_K2_ITEMS;               // K2 shared gate/up: items per wave
constexpr int kSharedPairsPerBlock = 4 * kSharedItems * kSharedRP;
static_assert(kItems % 2 == 0, "items are double-buffered in pairs");
static_assert(32 % kPairsPerWave == 0 && 32 % (2 * kRPW) == 0, "a wave never straddles inter (a multiple of 32)");
constexpr int kDownRows = QMOE_DEC_DOWN_ROWS; // down/combine output rows per block
constexpr int kMaxT = kDecodeMaxTokens;
constexpr int kRouterUnroll = 6;             // 16-byte router-weight loads per lane per pass

__device__ __forceinline__ void load16(uint32_t (&d)[4], const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  d[0] = v.x;
  d[1] = v.y;
  d[2] = v.z;
  d[3] = v.w;
}

// sum_k w_k * a_k over one 32-input group.  wq: the group's 16 code bytes;
// sc: its scale word (int4: fp16 bits; nvfp4: two E4M3 bytes); act: 16 pairs
// of 16-bit activations; asum: sum of the 32 activations (int4 only).
// Per-row formats (scale applied per row after the reduction): int4 as
// above with no group scale; int2 (two code words per group) as 1 + u/4
// pairs, sum (u - 2) a = 4 (d - 1.5 A).
template <int FMT, bool F16ACT>
__device__ __forceinline__ float group_dot(const uint32_t (&wq)[4], uint32_t sc,
                                           const uint32_t (&act)[16], float asum, float gs) {
  if constexpr (FMT == MOE_WFMT_INT4_ROW_F32) {
    float d = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d = F16ACT ? dot2_f16(int4_pair_f16(wq[j], k), act[4 * j + k], d)
                   : dot2_bf16(int4_pair_bf16(wq[j], k), act[4 * j + k], d);
    return 16.0f * fmaf(-1.5f, asum, d);
  } else if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) {
    float d = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        d = F16ACT ? dot2_f16(int2_pair_f16(wq[j], k, 0x3C003C00u), act[8 * j + k], d)
                   : dot2_bf16(int2_pair_bf16(wq[j], k, 0x3F803F80u), act[8 * j + k], d);
    return 4.0f * fmaf(-1.5f, asum, d);
  } else if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
    float d = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d = F16ACT ? dot2_f16(int4_pair_f16(wq[j], k), act[4 * j + k], d)
                   : dot2_bf16(int4_pair_bf16(wq[j], k), act[4 * j + k], d);
    return 16.0f * half_bits_to_f32(sc & 0xffffu) * fmaf(-1.5f, asum, d);
  } else {
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d0 = F16ACT ? dot2_f16(fp4_pair_f16(wq[j], k), act[4 * j + k], d0)
                    : dot2_bf16(fp4_pair_bf16(wq[j], k), act[4 * j + k], d0);
#pragma unroll
    for (int j = 2; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d1 = F16ACT ? dot2_f16(fp4_pair_f16(wq[j], k), act[4 * j + k], d1)
                    : dot2_bf16(fp4_pair_bf16(wq[j], k), act[4 * j + k], d1);
    return fmaf(e4m3_to_f32(sc, 0), d0, e4m3_to_f32(sc, 1) * d1) * gs;
  }
}

// Sum of the 32 activations of a group, for the int4 offset correction.
template <bool F16ACT>
__device__ __forceinline__ float act_sum(const uint32_t (&act)[16]) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s = F16ACT ? dot2_f16(act[i], 0x3C003C00u, s) : dot2_bf16(act[i], 0x3F803F80u, s);
  return s;
}

// int4 codes against fp16 activations (the SwiGLU outputs h): or-ing a code u
// into the mantissa of fp16 1024 gives 1024 + u (nibble at bits 0-3 of a
// half) or 1024 + 16 u (bits 4-7), so pairs 0 and 1 of a word take one
// v_and_or_b32 each and pairs 2 and 3 share one shift by 8.  Over a group,
//   sum (u - 8) a = d_even + d_odd / 16 - (1032 A_even + 72 A_odd)
// with d_even / d_odd the dot products over the even / odd pairs and A_even /
// A_odd the activation sums over them; the last term depends on the
// activations only (int4_offset) and is computed once per group of h.
__device__ __forceinline__ void int4_f16_1024(const uint32_t (&wq)[4], uint32_t (&wf)[16]) {
  const uint32_t one = 0x64006400u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = wq[j], w8 = w >> 8;
    wf[4 * j + 0] = and_or(w, 0x000F000Fu, one);
    wf[4 * j + 1] = and_or(w, 0x00F000F0u, one);
    wf[4 * j + 2] = and_or(w8, 0x000F000Fu, one);
    wf[4 * j + 3] = and_or(w8, 0x00F000F0u, one);
  }
}
__device__ __forceinline__ float int4_dot_1024(const uint32_t (&wf)[16], const uint32_t (&act)[16]) {
  float de = 0.0f, dd = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    de = dot2_f16(wf[i], act[i], de);
    dd = dot2_f16(wf[i + 1], act[i + 1], dd);
  }
  return fmaf(0.0625f, dd, de);
}
__device__ __forceinline__ float int4_offset(const uint32_t (&act)[16]) {
  float se = 0.0f, so = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; m += 2) {
    se = dot2_f16(act[m], 0x3C003C00u, se);
    so = dot2_f16(act[m + 1], 0x3C003C00u, so);
  }
  return fmaf(1032.0f, se, 72.0f * so);
}
// One group against fp16 activations.  int4: `off` = int4_offset(act);
// nvfp4: `off` unused, gs the per-tensor scale.
template <int FMT>
__device__ __forceinline__ float group_dot_h(const uint32_t (&wq)[4], uint32_t sc,
                                             const uint32_t (&act)[16], float off, float gs) {
  if constexpr (FMT == MOE_WFMT_INT4_G32_F16 || FMT == MOE_WFMT_INT4_ROW_F32) {
    uint32_t wf[16];
    int4_f16_1024(wq, wf);
    const float d = int4_dot_1024(wf, act) - off;
    return FMT == MOE_WFMT_INT4_G32_F16 ? half_bits_to_f32(sc & 0xffffu) * d : d;
  } else if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) {
    return group_dot<FMT, true>(wq, sc, act, off, gs);   // off: the sum of h
  } else {
    return group_dot<FMT, true>(wq, sc, act, 0.0f, gs);
  }
}
template <int FMT>
__device__ __forceinline__ float offset_h(const uint32_t (&act)[16]) {
  if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) return act_sum<true>(act);
  return (FMT == MOE_WFMT_INT4_G32_F16 || FMT == MOE_WFMT_INT4_ROW_F32) ? int4_offset(act) : 0.0f;
}
// Bytes of codes per 32-input group; scale bytes per row (per-row formats) or
// per group.
template <int FMT>
__host__ __device__ constexpr uint32_t group_code_bytes() { return 4u * (uint32_t)wfmt_bits(FMT); }
__device__ __forceinline__ uint32_t bload_u32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// The code words of one group: 16 bytes, or 8 for int2 (words 2, 3 unused).
template <int FMT>
__device__ __forceinline__ void load_group(uint32_t (&d)[4], rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (wfmt_bits(FMT) == 2)
    bload8(d, r, voff, soff);
  else
    bload16(d, r, voff, soff);
}

// ---------------------------------------------------------------------------
// Double-buffered gate/up GEMV of one wave.  The wave owns kPairsPerWave
// consecutive row pairs (gate row i, up row i), processed as kItems items of
// kRPW pairs; item i+1's loads are in flight while item i is dequantised and
// reduced, so the memory pipe stays busy.  Lane l owns the 32-input groups
// l, l+64, ... (GPL of them); x (one token) lives in registers.
// ---------------------------------------------------------------------------
template <int GPL, int RP>
struct GateUpItem {
  uint32_t wg[RP][GPL][4], wu[RP][GPL][4], sg[RP][GPL], su[RP][GPL];
};

// Buffers of one expert's gate and up projections (codes and scales).
struct GateUpBufs {
  rsrc_t qg, qu, sg, su;
  uint32_t rowBytes, scaleRowBytes;
};

// Per-row formats: sg[r][0] / su[r][0] hold the rows' fp32 scales (the same
// address in every lane).
template <int FMT, int GPL, int RP>
__device__ __forceinline__ void gu_load(GateUpItem<GPL, RP>& it, const GateUpBufs& b,
                                        const uint32_t (&off)[GPL], int pair0) {
  constexpr uint32_t CB = group_code_bytes<FMT>();
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const uint32_t row = (uint32_t)(pair0 + r);
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      load_group<FMT>(it.wg[r][j], b.qg, off[j] * CB, row * b.rowBytes);
      load_group<FMT>(it.wu[r][j], b.qu, off[j] * CB, row * b.rowBytes);
      if constexpr (!wfmt_row(FMT)) {
        it.sg[r][j] = bload_u16(b.sg, off[j] * 2u, row * b.scaleRowBytes);
        it.su[r][j] = bload_u16(b.su, off[j] * 2u, row * b.scaleRowBytes);
      }
    }
    if constexpr (wfmt_row(FMT)) {
      it.sg[r][0] = bload_u32(b.sg, 0u, row * 4u);
      it.su[r][0] = bload_u32(b.su, 0u, row * 4u);
    }
  }
}

template <int FMT, int GPL, int RP>
__device__ __forceinline__ void gu_compute(const GateUpItem<GPL, RP>& it,
                                           const uint32_t (&xw)[GPL][16], const float (&xs)[GPL],
                                           const bool (&ok)[GPL], float gg, float gu, int pair0,
                                           uint16_t* __restrict__ hrow) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const float vg = group_dot<FMT, false>(it.wg[r][j], it.sg[r][j], xw[j], xs[j], gg);
      const float vu = group_dot<FMT, false>(it.wu[r][j], it.su[r][j], xw[j], xs[j], gu);
      g += ok[j] ? vg : 0.0f;
      u += ok[j] ? vu : 0.0f;
      // bound the number of dequantised pairs the scheduler keeps live
      __builtin_amdgcn_sched_barrier(0);
    }
    g = wave_sum(g);
    u = wave_sum(u);
    if constexpr (wfmt_row(FMT)) {
      g *= __uint_as_float(it.sg[r][0]);
      u *= __uint_as_float(it.su[r][0]);
    }
    if (lane == r) {
      // a device-scope store: dec_fused_t1 reads h in the same launch
      const _Float16 hv = (_Float16)silu_mul(g, u);
      __hip_atomic_store(hrow + pair0 + r, __builtin_bit_cast(uint16_t, hv), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Gate/up for row pairs [pair_begin, pair_begin + kPairsPerWave) of one
// expert (rows [row_base, row_base + inter) of the projections) and one token
// x; h written to hrow.
template <int FMT, int GPL, int ITEMS = kItems, int RP = kRPW>
__device__ __forceinline__ void gateup_wave(const uint16_t* __restrict__ x, int H,
                                            const ProjPtr& Pg, const ProjPtr& Pu, size_t row_base,
                                            int inter, int pair_begin, float gg, float gu,
                                            uint16_t* __restrict__ hrow) {
  const int lane = threadIdx.x & 63;
  const int nG = H / 32;
  GateUpBufs b;
  b.rowBytes = (uint32_t)H * wfmt_bits(FMT) / 8;
  b.scaleRowBytes = wfmt_row(FMT) ? 4u : (uint32_t)nG * 2;
  b.qg = make_rsrc(Pg.q + row_base * b.rowBytes, (uint32_t)inter * b.rowBytes);
  b.qu = make_rsrc(Pu.q + row_base * b.rowBytes, (uint32_t)inter * b.rowBytes);
  b.sg = make_rsrc(reinterpret_cast<const uint8_t*>(Pg.s) + row_base * b.scaleRowBytes,
                   (uint32_t)inter * b.scaleRowBytes);
  b.su = make_rsrc(reinterpret_cast<const uint8_t*>(Pu.s) + row_base * b.scaleRowBytes,
                   (uint32_t)inter * b.scaleRowBytes);
  const rsrc_t xr = make_rsrc(x, (uint32_t)H * 2u);
  uint32_t cc[GPL];
  bool ok[GPL];
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int c = lane + 64 * j;
    ok[j] = c < nG;
    cc[j] = ok[j] ? c : nG - 1;
  }
  GateUpItem<GPL, RP> A, B;
  gu_load<FMT, GPL, RP>(A, b, cc, pair_begin);
  gu_load<FMT, GPL, RP>(B, b, cc, pair_begin + RP);
  uint32_t xw[GPL][16];
  float xs[GPL];
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t t4[4];
      bload16(t4, xr, cc[j] * 64u + 16u * q, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) xw[j][4 * q + i] = t4[i];
    }
  }
#pragma unroll
  for (int j = 0; j < GPL; ++j)
    xs[j] = (FMT != MOE_WFMT_NVFP4) ? act_sum<false>(xw[j]) : 0.0f;
#pragma unroll
  for (int i = 0; i < ITEMS; i += 2) {
    const int p = pair_begin + i * RP;
    gu_compute<FMT, GPL, RP>(A, xw, xs, ok, gg, gu, p, hrow);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < ITEMS) gu_load<FMT, GPL, RP>(A, b, cc, p + 2 * RP);
    __builtin_amdgcn_sched_barrier(0);
    gu_compute<FMT, GPL, RP>(B, xw, xs, ok, gg, gu, p + RP, hrow);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 3 < ITEMS) gu_load<FMT, GPL, RP>(B, b, cc, p + 3 * RP);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// K1: router scores sigmoid(logit) in float64, one block per expert
// ---------------------------------------------------------------------------
// scores[t][e] for expert e = blockIdx.x and the T <= kMaxT tokens of x (one
// block of 256 threads: the four waves take quarters of the hidden dimension,
// then their partial sums are added in wave order).
__device__ __forceinline__ void router_scores_block(const uint16_t* __restrict__ x,
                                                    const float* __restrict__ router_w,
                                                    double* __restrict__ scores, int T, int H, int E) {
  __shared__ double rpart[4][kMaxT];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.x;
  const int q0 = wv * (H / 4), q1 = q0 + H / 4;
  const float* wrow = router_w + (size_t)e * H;
  double acc[kMaxT];
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) acc[t] = 0.0;
  for (int h0 = q0; h0 < q1; h0 += 256 * kRouterUnroll) {
    float4 w4[kRouterUnroll];
    uint2 xv[kRouterUnroll][kMaxT];
    bool ok[kRouterUnroll];
#pragma unroll
    for (int i = 0; i < kRouterUnroll; ++i) {
      const int h_raw = h0 + 256 * i + lane * 4;
      ok[i] = h_raw < q1;
      const int h = ok[i] ? h_raw : q0;
      w4[i] = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
      for (int t = 0; t < kMaxT; ++t)
        xv[i][t] = *reinterpret_cast<const uint2*>(x + (size_t)(t < T ? t : 0) * H + h);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kRouterUnroll; ++i) {
      if (!ok[i]) continue;
#pragma unroll
      for (int t = 0; t < kMaxT; ++t) {
        double s2 = acc[t];
        s2 = fma((double)bf16_lo(xv[i][t].x), (double)w4[i].x, s2);
        s2 = fma((double)bf16_hi(xv[i][t].x), (double)w4[i].y, s2);
        s2 = fma((double)bf16_lo(xv[i][t].y), (double)w4[i].z, s2);
        s2 = fma((double)bf16_hi(xv[i][t].y), (double)w4[i].w, s2);
        acc[t] = s2;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) {
    const double v = wave_sum(acc[t]);
    if (lane == 0) rpart[wv][t] = v;
  }
  __syncthreads();
  // the sigmoid score: the selection reads scores, not logits
  if (threadIdx.x < T) {
    const double l = ((rpart[0][threadIdx.x] + rpart[1][threadIdx.x]) + rpart[2][threadIdx.x]) +
                     rpart[3][threadIdx.x];
    scores[(size_t)threadIdx.x * E + e] = 1.0 / (1.0 + exp(-l));
  }
}

// The first workgroups also zero dec_fused_t1's barrier count and flags.
__global__ void __launch_bounds__(256) dec_router_kernel(DecodeArgs a) {
  for (int i = (int)blockIdx.x * 256 + (int)threadIdx.x; i <= kDecFusedMaxGrid; i += (int)gridDim.x * 256)
    a.bar[kDecFlagStride * i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.flags[0] = 0u;
  router_scores_block(a.x, a.router_w, a.logits, a.T, a.H, a.E);
}

// The same scores for moe_route and the split path of moe_layer at T <= kMaxT.
__global__ void __launch_bounds__(256) route_scores_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ router_w,
                                                           double* __restrict__ scores, int T, int H,
                                                           int E) {
  router_scores_block(x, router_w, scores, T, H, E);
}

// Selection of 2..4 tokens (one wave per token) and the grouping of the
// P <= 64 picks by expert (wave 0): the layer's ids and weights, one record
// per selected expert, their count, and each sorted pick's (expert, token)
// word.  The caller's other waves (wv >= T) only pass the barrier.
template <bool DEV>
__device__ __forceinline__ void select_group_multi(const DecodeArgs& a, SelectScratch (&sc)[4],
                                                   int (&pid)[64], float (&pw)[64]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.K, P = a.T * a.K;
  if (wv < a.T) {
    int id, rank, n_kept;
    float w;
    select_token<true>(a.logits + (size_t)wv * a.E, a.bias, a.E, a.G, a.TG, K, a.rsf, a.top_p,
                       sc[wv], id, w, rank, n_kept);
    if (lane < K) {
      a.ids[wv * K + rank] = id;
      a.tw[wv * K + rank] = w;
      pid[wv * K + rank] = id;
      pw[wv * K + rank] = w;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  // One pick per lane (P <= 64), p = t*k + i.  Sorted order: expert id, then
  // pick index.  Lanes holding the same expert, and those holding a smaller
  // one, are found with one ballot per id bit, from the top bit down: `eq`
  // keeps the lanes that agree with this one on the bits so far, and a lane
  // that agrees so far but has 0 where this one has 1 is smaller.
  // picks the adaptive top-p dropped (id -1) take no slot; sorted picks run
  // to the number of kept ones, and K3's blocks past them exit
  const int pe = lane < P ? pid[lane] : -1;
  const bool have = pe >= 0;
  const int e = have ? pe : 0;
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  uint64_t eq = __ballot(have), lt = 0;
  for (int bit = nbits - 1; bit >= 0; --bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t b = __ballot(have && set);
    lt |= set ? (eq & ~b) : 0ull;
    eq &= set ? b : ~b;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const int pos = __popcll(lt) + __popcll(eq & below);
  const bool first = have && (eq & below) == 0;
  const uint64_t firsts = __ballot(first);
  // DEV: device-scope stores, read by other workgroups of the same launch
  auto put_et = [&](int i, int v) {
    if constexpr (DEV)
      __hip_atomic_store(a.sorted_et + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      a.sorted_et[i] = v;
  };
  if (have) put_et(pos, e | ((lane / K) << 16));
  if (lane < P && lane >= __popcll(__ballot(have))) put_et(lane, -1);
  if (first) {
    // the expert's record: its picks (the lanes in eq) in pick order, at most
    // one per token, so at most four
    DecSlot sl;
    sl.e = e;
    sl.p0 = pos;
    sl.M = __popcll(eq);
    sl.pad = 0;
    uint64_t rem = eq;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int l = rem ? (int)__builtin_ctzll(rem) : lane;
      rem &= rem - 1ull;
      sl.t[m] = m < sl.M ? l / K : 0;
      sl.w[m] = m < sl.M ? pw[l] : 0.0f;
    }
    a.slots[__popcll(lt & firsts)] = sl;
  }
  if (lane == 0) a.n_active[0] = __popcll(firsts);
}

// ---------------------------------------------------------------------------
// K2: selection of every token, then the permutation of the P <= 64 picks
// ---------------------------------------------------------------------------
// Selection and grouping.  What the later kernels read: the per-token ids
// and weights (outputs of the layer), the selected experts' records (slots,
// in ascending expert order, each with its picks in pick order), their count,
// and for each sorted pick p (grouped by expert) its expert and token; the h
// rows follow the sorted pick order.
// The other workgroups run the shared expert's gate/up GEMV, one per (token,
// row block): it does not depend on the routing, so it streams while block 0
// selects.  (For 2..4 tokens this measured 2 us per call faster than extra
// blocks of K3: 141.5 against 143.7 us at four tokens.)
template <int FMT, int GPL>
__global__ void __launch_bounds__(256) dec_select_permute_kernel(DecodeArgs a) {
  if (blockIdx.x > 0) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const ExpertSet& S = a.shared;
    const int nsb = (S.inter + kSharedPairsPerBlock - 1) / kSharedPairsPerBlock;   // row blocks
    const int t = ((int)blockIdx.x - 1) / nsb, rb = ((int)blockIdx.x - 1) - t * nsb;
    const int pair0 = rb * kSharedPairsPerBlock + wv * (kSharedItems * kSharedRP);
    if (pair0 >= S.inter) return;
    const float gg = (FMT == MOE_WFMT_NVFP4) ? S.gate.g[0] : 1.0f;
    const float gu = (FMT == MOE_WFMT_NVFP4) ? S.up.g[0] : 1.0f;
    gateup_wave<FMT, GPL, kSharedItems, kSharedRP>(a.x + (size_t)t * a.H, a.H, S.gate, S.up, 0, S.inter, pair0, gg,
                                        gu, a.h_shared + (size_t)t * a.ldh);
    return;
  }
  __shared__ SelectScratch sc[4];
  __shared__ int pid[64];
  __shared__ float pw[64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.K;
  if (a.T == 1) {
    // One token: its k picks are distinct experts, so the sorted order is the
    // ascending-id order select_token ranks them in, and every record follows
    // from (id, weight, rank) in the picking lanes.
    if (wv != 0) return;
    int id, rank, n_kept;
    float w;
    select_token<true>(a.logits, a.bias, a.E, a.G, a.TG, K, a.rsf, a.top_p, sc[0], id, w, rank,
                       n_kept);
    if (lane < K) {
      a.ids[rank] = id;
      a.tw[rank] = w;
      // picks the adaptive top-p dropped (ranks from n_kept on) have no h row
      a.sorted_et[rank] = id;
    }
    if (lane < K && rank < n_kept) {
      DecSlot sl;
      sl.e = id;
      sl.p0 = rank;
      sl.M = 1;
      sl.pad = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sl.t[i] = 0;
        sl.w[i] = i == 0 ? w : 0.0f;
      }
      a.slots[rank] = sl;
    }
    if (lane == 0) a.n_active[0] = n_kept;
    return;
  }
  select_group_multi<false>(a, sc, pid, pw);
}

// ---------------------------------------------------------------------------
// K3: gate/up of the selected experts.  Block = (row block, sorted pick p):
// the double-buffered GEMV of the pick's expert over the block's row pairs
// for the pick's token, written to h row p.  Picks of one expert sit next to
// each other, so the blocks that share its weights run together on one XCD
// and the later ones read them from L2.
// ---------------------------------------------------------------------------
template <int FMT, int GPL>
__global__ void __launch_bounds__(256) dec_gateup_kernel(DecodeArgs a) {
  const int p = (int)blockIdx.y;
  const int et = __builtin_amdgcn_readfirstlane(a.sorted_et[p]);
  if (et < 0) return;   // a pick the adaptive top-p dropped
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const ExpertSet& R = a.routed;
  const int pair0 = blockIdx.x * kPairsPerBlock + wv * kPairsPerWave;
  if (pair0 >= R.inter) return;
  const int e = et & 0xffff, t = et >> 16;
  const float gg = (FMT == MOE_WFMT_NVFP4) ? R.gate.g[e] : 1.0f;
  const float gu = (FMT == MOE_WFMT_NVFP4) ? R.up.g[e] : 1.0f;
  gateup_wave<FMT, GPL>(a.x + (size_t)t * a.H, a.H, R.gate, R.up, (size_t)e * R.inter, R.inter,
                        pair0, gg, gu, a.h_routed + (size_t)p * a.ldh);
}

// ---------------------------------------------------------------------------
// K2 and K3 in one launch for 2..4 tokens (dec_select_gateup).  Grid (row
// blocks, 1 + T + P): block (0, 0) selects and groups the picks as K2 does,
// then raises kSelFlags flags; blocks (x, 1..T) run the shared expert's
// gate/up for token y - 1, which does not depend on the routing and streams
// while the selection runs; blocks (x, 1 + T + p) wait for a flag and then run
// K3's GEMV for sorted pick p.  Block (0, 0) is dispatched first, so it runs
// whatever the waiting blocks occupy.  The pick words that the waiting
// blocks read are device-scope stores, complete (vmcnt(0), then the
// workgroup barrier) before the flags are stored at device scope; the
// waiters read them with device-scope loads issued after their flag has
// returned.  The other records (ids, weights, expert records) are read by
// K4, after the launch.  K1 zeroes the flags.  A wait is bounded
// (barrier_spins polls); a block that gives up writes NaN to its h rows and
// raises the layer's flag.
// ---------------------------------------------------------------------------
constexpr int kSelFlags = 64;
static_assert(kSelFlags <= kDecFusedMaxGrid, "the flags sit in the barrier words K1 zeroes");

template <int FMT, int GPL>
__global__ void __launch_bounds__(256) dec_select_gateup_kernel(DecodeArgs a) {
  const int y = (int)blockIdx.y;
  const int T = a.T;
  if (y == 0) {
    if (blockIdx.x != 0) return;
    __shared__ SelectScratch sc[4];
    __shared__ int pid[64];
    __shared__ float pw[64];
    select_group_multi<true>(a, sc, pid, pw);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the pick words are stored
    __syncthreads();
    if (threadIdx.x < kSelFlags)
      __hip_atomic_store(a.bar + kDecFlagStride * (1 + threadIdx.x), 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair0 = blockIdx.x * kPairsPerBlock + wv * kPairsPerWave;
  if (y <= T) {
    const ExpertSet& S = a.shared;
    if (!a.has_shared || pair0 >= S.inter) return;
    const float gg = (FMT == MOE_WFMT_NVFP4) ? S.gate.g[0] : 1.0f;
    const float gu = (FMT == MOE_WFMT_NVFP4) ? S.up.g[0] : 1.0f;
    gateup_wave<FMT, GPL>(a.x + (size_t)(y - 1) * a.H, a.H, S.gate, S.up, 0, S.inter, pair0, gg, gu,
                          a.h_shared + (size_t)(y - 1) * a.ldh);
    return;
  }
  const int p = y - 1 - T;
  const ExpertSet& R = a.routed;
  __shared__ int ready;
  if (threadIdx.x == 0) {
    const uint32_t* flag = a.bar + kDecFlagStride * (1 + ((int)blockIdx.x + p) % kSelFlags);
    int ok = 0;
    for (uint32_t spin = 0; spin < a.barrier_spins; ++spin) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    ready = ok;
  }
  __syncthreads();
  if (!ready) {
    // the pick is unknown: its h rows of this block become NaN
    if (threadIdx.x == 0) a.flags[0] = MOE_FLAG_GRID_WAIT_TIMEOUT;
    const int r = blockIdx.x * kPairsPerBlock + (int)threadIdx.x;
    if ((int)threadIdx.x < kPairsPerBlock && r < R.inter) a.h_routed[(size_t)p * a.ldh + r] = 0x7E00u;
    return;
  }
  const int et = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(a.sorted_et + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (et < 0 || pair0 >= R.inter) return;   // et < 0: a pick the adaptive top-p dropped
  const int e = et & 0xffff, t = et >> 16;
  const float gg = (FMT == MOE_WFMT_NVFP4) ? R.gate.g[e] : 1.0f;
  const float gu = (FMT == MOE_WFMT_NVFP4) ? R.up.g[e] : 1.0f;
  gateup_wave<FMT, GPL>(a.x + (size_t)t * a.H, a.H, R.gate, R.up, (size_t)e * R.inter, R.inter,
                        pair0, gg, gu, a.h_routed + (size_t)p * a.ldh);
}

// ---------------------------------------------------------------------------
// K4: down projection of every selected expert and the shared expert for
// kDownRows output rows, combined into y in registers.  The four waves of a
// block take expert slots round-robin; each wave keeps the next slot's rows
// in flight while it dequantises the current one.  Partial sums meet in LDS
// in wave order, so the result does not depend on timing.
// ---------------------------------------------------------------------------
struct DownItem {
  uint32_t w[kDownRows][4];
  uint32_t sc[kDownRows];
  uint32_t h[16];
};

struct SlotInfo {
  rsrc_t q, s, h;
  int p0, M, nG;
  uint32_t tpk;   // token of pick i in byte i
  float w[4];
  float g;
  bool routed;
};

// Slot s of the down projection: routed slot s < n_routed from its record
// `ent`, else the shared expert (all T tokens, weight 1).
template <int FMT>
__device__ __forceinline__ SlotInfo slot_info(const DecodeArgs& a, int s, int n_routed, int row0,
                                              const DecSlot& ent) {
  SlotInfo d;
  d.routed = s < n_routed;
  const ExpertSet& X = d.routed ? a.routed : a.shared;
  const int e = d.routed ? __builtin_amdgcn_readfirstlane(ent.e) : 0;
  d.p0 = d.routed ? __builtin_amdgcn_readfirstlane(ent.p0) : 0;
  d.M = d.routed ? __builtin_amdgcn_readfirstlane(ent.M) : a.T;
  d.tpk = d.routed ? (uint32_t)__builtin_amdgcn_readfirstlane(ent.t[0] | (ent.t[1] << 8) |
                                                               (ent.t[2] << 16) | (ent.t[3] << 24))
                   : 0x03020100u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.w[i] = d.routed ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                            __builtin_bit_cast(int, ent.w[i])))
                      : 1.0f;
  d.nG = X.inter / 32;
  const uint32_t rowBytes = (uint32_t)X.inter / 2;
  const size_t rb = (size_t)e * a.H + row0;
  d.q = make_rsrc(X.down.q + rb * rowBytes, kDownRows * rowBytes);
  d.s = make_rsrc(reinterpret_cast<const uint16_t*>(X.down.s) + rb * d.nG, kDownRows * d.nG * 2u);
  const uint16_t* hp = d.routed ? a.h_routed + (size_t)d.p0 * a.ldh : a.h_shared;
  d.h = make_rsrc(hp, (uint32_t)d.M * a.ldh * 2u);
  d.g = (FMT == MOE_WFMT_NVFP4) ? X.down.g[e] : 1.0f;
  return d;
}

// Buffer loads range-check only the per-lane offset, so lanes past the row's
// last group (small inter) load group 0 instead and are masked in compute.
__device__ __forceinline__ void down_load(DownItem& it, const SlotInfo& d, uint32_t c_raw) {
  const uint32_t c = (int)c_raw < d.nG ? c_raw : 0u;
  const uint32_t rowBytes = (uint32_t)d.nG * 16u;
#pragma unroll
  for (int r = 0; r < kDownRows; ++r) {
    bload16(it.w[r], d.q, c * 16u, r * rowBytes);
    it.sc[r] = bload_u16(d.s, c * 2u, r * (uint32_t)d.nG * 2u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t t4[4];
    bload16(t4, d.h, c * 64u + 16u * q, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) it.h[4 * q + i] = t4[i];
  }
}

template <int FMT, int MT>
__device__ __forceinline__ void down_compute(const DownItem& it, const SlotInfo& d, uint32_t c,
                                             bool valid, const DecodeArgs& a,
                                             float (&acc)[MT][kDownRows]) {
  const bool ok = valid && (int)c < d.nG;
  for (int m = 0; m < d.M; ++m) {
    uint32_t hm[16];
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) hm[i] = it.h[i];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t t4[4];
        bload16(t4, d.h, (ok ? c : 0u) * 64u + 16u * q, (uint32_t)m * a.ldh * 2u);
#pragma unroll
        for (int i = 0; i < 4; ++i) hm[4 * q + i] = t4[i];
      }
    }
    const float hs = offset_h<FMT>(hm);
    const int t = (int)((d.tpk >> (8 * m)) & 0xffu);
    const float wm = m == 0 ? d.w[0] : m == 1 ? d.w[1] : m == 2 ? d.w[2] : d.w[3];
    const float wpick = ok ? wm : 0.0f;
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) {
      const float v = wpick * group_dot_h<FMT>(it.w[r], it.sc[r], hm, hs, d.g);
#pragma unroll
      for (int tt = 0; tt < MT; ++tt)
        if (tt == t) acc[tt][r] += v;
    }
  }
}

template <int FMT, int MT>
__global__ void __launch_bounds__(256) dec_down_combine_kernel(DecodeArgs a) {
  __shared__ float part[4][MT][kDownRows];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H, T = a.T;
  const int row0 = blockIdx.x * kDownRows;
  // the count and this wave's first record are fetched together
  const int n_routed = __builtin_amdgcn_readfirstlane(*a.n_active);
  const DecSlot ent0 = a.slots[wv];
  const int nslots = n_routed + (a.has_shared ? 1 : 0);
  const int nG_max = max(a.routed.inter, a.has_shared ? a.shared.inter : 0) / 32;
  float acc[MT][kDownRows];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) acc[t][r] = 0.0f;

  if (wv < nslots) {
    const int last = nslots - 1;
    for (int c0 = 0; c0 < nG_max; c0 += 64) {
      const uint32_t c = (uint32_t)(c0 + lane);
      // slots wv, wv+4, ... with two in flight: A holds slot sa, B slot sb.  A
      // prefetch past the last slot reads the last slot again (in bounds) and
      // is never computed.
      int sa = wv, sb = wv + 4;
      SlotInfo da = slot_info<FMT>(a, sa, n_routed, row0, ent0);
      SlotInfo db = slot_info<FMT>(a, min(sb, last), n_routed, row0, a.slots[min(sb, last)]);
      DownItem A, B;
      down_load(A, da, c);
      down_load(B, db, c);
      while (true) {
        __builtin_amdgcn_sched_barrier(0);
        down_compute<FMT, MT>(A, da, c, true, a, acc);  // sa <= last here
        __builtin_amdgcn_sched_barrier(0);
        if (sb > last) break;
        sa = sb + 4;
        da = slot_info<FMT>(a, min(sa, last), n_routed, row0, a.slots[min(sa, last)]);
        down_load(A, da, c);
        __builtin_amdgcn_sched_barrier(0);
        down_compute<FMT, MT>(B, db, c, true, a, acc);  // sb <= last here
        __builtin_amdgcn_sched_barrier(0);
        if (sa > last) break;
        sb = sa + 4;
        db = slot_info<FMT>(a, min(sb, last), n_routed, row0, a.slots[min(sb, last)]);
        down_load(B, db, c);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t < T) {
#pragma unroll
      for (int r = 0; r < kDownRows; ++r) {
        const float v = wave_sum(acc[t][r]);
        if (lane == 0) part[wv][t][r] = v;
      }
    }
  }
  __syncthreads();
  const int t = threadIdx.x / kDownRows, r = threadIdx.x % kDownRows;
  if (t < T) {
    const float v = ((part[0][t][r] + part[1][t][r]) + part[2][t][r]) + part[3][t][r];
    if (a.out_bf16) {
      uint32_t u = __float_as_uint(v);
      if ((u & 0x7fffffffu) > 0x7f800000u) {
        u = (u >> 16) | 0x40u;
      } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        u >>= 16;
      }
      reinterpret_cast<uint16_t*>(a.y)[(size_t)t * H + row0 + r] = (uint16_t)u;
    } else {
      reinterpret_cast<float*>(a.y)[(size_t)t * H + row0 + r] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// K4 for a single token (the decode shape): down projection of the k <= 8
// selected experts and the shared expert, combined into y.
//
// One resident round of workgroups; each wave streams whole output rows.
// For row r it issues, for every slot, the 16-byte code chunk and the scale of
// group `lane` (inter <= 2048, so one pass of 64 lanes covers a row) -- all
// slots of row r + stride are in flight while row r is reduced.  The SwiGLU
// outputs h of all slots sit in LDS, staged once per workgroup in the order
// the lanes read them: quarter q of group c of slot s at 16-byte slot
// (s * 4 + q) * nG + c, so each read of 64 lanes is 1 KB contiguous.  The sum
// over slots runs in slot order within each lane, then across the lanes.
// ---------------------------------------------------------------------------
constexpr int kD1MaxRouted = 8;  // top_k <= 8 routed experts, plus the shared expert

__device__ __forceinline__ void store_y(const DecodeArgs& a, int t, int row, float v) {
  if (a.out_bf16) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      u = (u >> 16) | 0x40u;
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
      u >>= 16;
    }
    reinterpret_cast<uint16_t*>(a.y)[(size_t)t * a.H + row] = (uint16_t)u;
  } else {
    reinterpret_cast<float*>(a.y)[(size_t)t * a.H + row] = v;
  }
}

// Rows gw, gw + nw, ... of y for one token; hl: (k + 1) * inter * 2 bytes of
// LDS.  FUSED (dec_fused_t1): the weights of the first row are requested
// before `before_h` (the grid barrier) is called, h and then the second row's
// weights after it (more rows requested early measured slower: they compete with the
// last gate/up waves, which the barrier waits for); a false return writes NaN
// to the rows.  Otherwise h is requested first, and each row's weights while
// the row before it is reduced.
template <int FMT, bool FUSED, int NT, class BeforeH>
__device__ __forceinline__ void down_t1_rows(const DecodeArgs& a, uint4* hl, int gw, int nw,
                                             BeforeH before_h, const int* sel_e = nullptr,
                                             const float* sel_w = nullptr, int sel_n = 0) {
  const int lane = threadIdx.x & 63;
  const int H = a.H;
  // one token: its distinct selected experts (k, or fewer after the adaptive
  // top-p)
  const int nr = FUSED ? sel_n : __builtin_amdgcn_readfirstlane(*a.n_active);
  const bool shared = a.has_shared;
  const int ns = nr + (shared ? 1 : 0);
  const int inter = a.routed.inter;         // routed and shared inter are equal here
  const int nG = inter / 32;
  constexpr bool ROW = wfmt_row(FMT);
  constexpr uint32_t CB = group_code_bytes<FMT>();
  const uint32_t rowBytes = (uint32_t)inter * wfmt_bits(FMT) / 8;

  // slots in ascending expert order (expert, weight; nvfp4: the expert's
  // tensor scale), FUSED: from the workgroup's own selection (sel_e, sel_w in
  // LDS), else from K2's records: lane s reads slot s, then every lane takes
  // them from there -- one round trip
  int es[kD1MaxRouted];
  float wsl[kD1MaxRouted], gsl[kD1MaxRouted];
  {
    const int sl = lane < nr ? lane : 0;
    const int e_l = FUSED ? sel_e[sl] : a.slots[sl].e;
    const float w_l = FUSED ? sel_w[sl] : a.slots[sl].w[0];
    const float g_l = FMT == MOE_WFMT_NVFP4 ? a.routed.down.g[e_l] : 1.0f;
#pragma unroll
    for (int s = 0; s < kD1MaxRouted; ++s) {
      es[s] = s < nr ? __builtin_amdgcn_readlane(e_l, s) : 0;
      wsl[s] = s < nr ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), s))
                      : 0.0f;
      gsl[s] = s < nr ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g_l), s))
                      : 1.0f;
    }
  }
  const float gsh = (FMT == MOE_WFMT_NVFP4 && shared) ? a.shared.down.g[0] : 1.0f;
  const rsrc_t rq = make_rsrc(a.routed.down.q, 0xFFFFFFFFu);
  const rsrc_t rs = make_rsrc(a.routed.down.s, 0xFFFFFFFFu);
  const rsrc_t sq = make_rsrc(a.shared.down.q, shared ? 0xFFFFFFFFu : 0u);
  const rsrc_t ss = make_rsrc(a.shared.down.s, shared ? 0xFFFFFFFFu : 0u);
  // h of all slots (rows 0..k-1 routed in slot order, row k shared): every
  // load is issued here, the LDS writes wait until the weights of the first
  // row are requested as well
  constexpr int kHPerThread = ((kD1MaxRouted + 1) * 256 + NT - 1) / NT;   // 16-byte chunks per thread
  const int hper = nG * 4;                  // 16-byte chunks per row
  // h rows 0..k (the shared expert's row follows the k routed ones); FUSED:
  // device-scope loads, as the rows were written in this launch
  uint4 hv[kHPerThread];
  // the shared expert's h row is row k (its place after all k picks), also
  // when the adaptive top-p kept fewer: slot s < nr reads row s, slot nr row k
  const rsrc_t hr = make_rsrc(a.h_routed, (uint32_t)((a.K + 1) * a.ldh * 2));
  auto load_h = [&] {
#pragma unroll
    for (int j = 0; j < kHPerThread; ++j) {
      const int i = threadIdx.x + NT * j;
      const int sl = i / hper, rem = i - sl * hper;
      const int hrow = sl < nr ? sl : a.K;
      const uint32_t off = (uint32_t)(hrow * a.ldh + rem * 8) * 2u;
      if constexpr (FUSED)
        hv[j] = i < ns * hper ? bload16_device(hr, off, 0) : make_uint4(0, 0, 0, 0);
      else
        hv[j] = i < ns * hper ? *reinterpret_cast<const uint4*>(a.h_routed + (size_t)hrow * a.ldh + rem * 8)
                              : make_uint4(0, 0, 0, 0);
    }
  };
  if constexpr (!FUSED) load_h();
  const bool ok = lane < nG;
  const uint32_t c = ok ? (uint32_t)lane : 0u;
  const uint32_t srow = ROW ? 4u : (uint32_t)nG * 2u;

  // B: buffer; routed slots 0..7 and the shared slot
  constexpr int NB = 2;                     // row buffers
  uint32_t wq[NB][kD1MaxRouted][4], wsc[NB][kD1MaxRouted], wqs[NB][4], wscs[NB];
  auto load_row = [&](auto B, int r) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int s = 0; s < kD1MaxRouted; ++s) {
      if (s < nr) {
        const uint32_t row = (uint32_t)(es[s] * H + r);
        load_group<FMT>(wq[b][s], rq, c * CB, row * rowBytes);
        // per-row formats: the row's fp32 scale (the same word in every lane)
        wsc[b][s] = ROW ? bload_u32(rs, 0u, row * 4u) : bload_u16(rs, c * 2u, row * srow);
      }
    }
    if (shared) {
      load_group<FMT>(wqs[b], sq, c * CB, (uint32_t)r * rowBytes);
      wscs[b] = ROW ? bload_u32(ss, 0u, (uint32_t)r * 4u) : bload_u16(ss, c * 2u, (uint32_t)r * srow);
    }
  };
  if (gw < H) load_row(std::integral_constant<int, 0>{}, gw);
  const bool fine = before_h();
  // a workgroup that gave up raises the layer's flag (plain vector store: any
  // number of workgroups may write the same value)
  if (FUSED && !fine && threadIdx.x == 0) a.flags[0] = MOE_FLAG_GRID_WAIT_TIMEOUT;
  if constexpr (FUSED) load_h();   // first, so that it does not queue behind the second row
  if (FUSED && gw + nw < H) load_row(std::integral_constant<int, 1>{}, gw + nw);
#pragma unroll
  for (int j = 0; j < kHPerThread; ++j) {
    const int i = threadIdx.x + NT * j;
    const int sl = i / hper, rem = i - sl * hper;
    if (i < ns * hper) hl[(sl * 4 + (rem & 3)) * nG + (rem >> 2)] = hv[j];
  }
  __syncthreads();
  auto h_of = [&](int s, uint32_t (&hm)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = hl[(s * 4 + q) * nG + c];
      hm[4 * q] = v.x; hm[4 * q + 1] = v.y; hm[4 * q + 2] = v.z; hm[4 * q + 3] = v.w;
    }
  };
  // per-slot activation sums (int4 offset correction), the same for every row
  float hsum[kD1MaxRouted], hsums = 0.0f;
#pragma unroll
  for (int s = 0; s < kD1MaxRouted; ++s) {
    hsum[s] = 0.0f;
    if (FMT != MOE_WFMT_NVFP4 && s < nr) {
      uint32_t hm[16];
      h_of(s, hm);
      hsum[s] = offset_h<FMT>(hm);
    }
  }
  if (FMT != MOE_WFMT_NVFP4 && shared) {
    uint32_t hm[16];
    h_of(nr, hm);
    hsums = offset_h<FMT>(hm);
  }
  // row r from buffer B; row r + nw requested into the other buffer first, or
  // (FUSED, both buffers filled before the first row) row r + 2 nw into this
  // one after
  auto row_step = [&](auto B, int r) {
    constexpr int b = decltype(B)::value;
    if (!FUSED && r + nw < H) load_row(std::integral_constant<int, (b + 1) % NB>{}, r + nw);
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < kD1MaxRouted; ++s) {
      if (s < nr) {
        uint32_t hm[16];
        h_of(s, hm);
        const float d = group_dot_h<FMT>(wq[b][s], wsc[b][s], hm, hsum[s], gsl[s]);
        const float ws = ROW ? wsl[s] * __uint_as_float(wsc[b][s]) : wsl[s];
        acc += ok ? ws * d : 0.0f;
      }
    }
    if (shared) {
      uint32_t hm[16];
      h_of(nr, hm);
      const float d = group_dot_h<FMT>(wqs[b], wscs[b], hm, hsums, gsh);
      acc += ok ? (ROW ? __uint_as_float(wscs[b]) * d : d) : 0.0f;
    }
    if (FUSED && r + NB * nw < H) load_row(B, r + NB * nw);
    const float v = wave_sum(acc);
    if (lane == 0) store_y(a, 0, r, fine ? v : __builtin_nanf(""));
  };
  for (int r = gw; r < H; r += NB * nw) {
    static_for<NB>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (r + i * nw < H) row_step(I, r + i * nw);
    });
  }
}

template <int FMT>
__global__ void __launch_bounds__(256, 2) dec_down_t1_kernel(DecodeArgs a) {
  extern __shared__ uint4 hl[];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  down_t1_rows<FMT, false, 256>(a, hl, blockIdx.x * 4 + wv, gridDim.x * 4, [] { return true; });
}

// Whether the single-token down kernel covers this shape; its LDS bytes.
__host__ __device__ inline bool down_t1_fits(const DecodeArgs& a) {
  const long long nG = a.routed.inter / 32;
  return a.T == 1 && a.K <= kD1MaxRouted && nG <= 64 &&
         (!a.has_shared || a.shared.inter == a.routed.inter) &&
         (long long)(a.K + 1) * a.routed.inter * 2 <= 65536 &&
         (long long)a.E * a.H * (a.routed.inter / 2) < 0xFFFFFFFFll &&
         (long long)a.E * a.H * nG * 2 < 0xFFFFFFFFll;
}

// ---------------------------------------------------------------------------
// One token after K1 in one launch (dec_fused_t1): every workgroup selects
// the experts itself from K1's scores (wave 0; the same result everywhere, so
// no workgroup waits for another to publish it) while its other waves run the
// shared expert's gate/up; then the gate/up GEMVs of the k picks, a barrier
// across the grid, and the rows of dec_down_t1.  The down weights do not
// depend on h, so every wave requests its first row as soon as its workgroup
// has arrived at the barrier: the down stream starts while the last gate/up
// waves finish, and neither K2 nor K4 ramps up a launch of its own.
//
// One workgroup of kFusedWaves waves per CU: each workgroup stages all of h
// in LDS after the barrier, so fewer, larger workgroups read less of it.  The
// barrier needs every workgroup resident at once, so the grid is at most what
// the device holds (hipOccupancyMaxActiveBlocksPerMultiprocessor x CUs, and
// kDecFusedMaxGrid), and the kernel is launched after K1 on the same stream,
// with the whole GPU free to it.  h is written and read with device-scope
// (sc1) accesses, so no cache-wide write-back or invalidate is needed: a
// workgroup arrives once its waves' stores have completed, by adding one to
// bar[0]; the last to arrive sets every workgroup's flag (bar[kDecFlagStride *
// (1 + b)], one per 256 bytes, so that the waiting workgroups do not all poll
// one address).  K1 zeroes the count and the flags.  The wait is bounded
// (kBarrierSpins polls); a workgroup that gives up writes NaN to its rows of y
// rather than a sum over an incomplete h.
// ---------------------------------------------------------------------------
constexpr int kFusedPairs = 8;            // gate/up row pairs per wave item
constexpr int kFusedWaves = 8;           // waves per workgroup, one workgroup per CU
constexpr int kFusedBlocksPerCU = 1;
constexpr uint32_t kBarrierSpins = 1u << 16;
static_assert(32 % kFusedPairs == 0, "an item never straddles an expert (inter is a multiple of 32)");

__device__ __forceinline__ void grid_arrive(uint32_t* bar, uint32_t n) {
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's h stores are done
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(old) == n - 1)
      for (uint32_t b = lane; b < n; b += 64)
        __hip_atomic_store(bar + kDecFlagStride * (1 + b), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Whether this workgroup's flag was set within `spins` polls.
__device__ __forceinline__ bool grid_wait(const uint32_t* bar, uint32_t spins) {
  __shared__ int arrived;
  if (threadIdx.x == 0) {
    const uint32_t* flag = bar + kDecFlagStride * (1 + blockIdx.x);
    int ok = 0;
    for (uint32_t spin = 0; spin < spins; ++spin) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    arrived = ok;
  }
  __syncthreads();
  return arrived != 0;
}

template <int FMT, int GPL>
__global__ void __launch_bounds__(64 * kFusedWaves, kFusedBlocksPerCU) dec_fused_t1_kernel(DecodeArgs a) {
  extern __shared__ uint4 hl[];
  __shared__ SelectScratch sc;
  __shared__ int sel_e[kD1MaxRouted];
  __shared__ float sel_w[kD1MaxRouted];
  __shared__ int sel_n;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kFusedWaves + wv, nw = gridDim.x * kFusedWaves;
  if (wv == 0) {
    // every workgroup selects the token's experts itself (the same result
    // everywhere), so no workgroup waits for another to publish them;
    // workgroup 0 writes the layer's ids and weights
    int id, rank, n_kept;
    float w;
    select_token<true>(a.logits, a.bias, a.E, a.G, a.TG, a.K, a.rsf, a.top_p, sc, id, w, rank,
                       n_kept);
    if (lane == 0) sel_n = n_kept;
    if (lane < a.K) {
      sel_e[rank] = id;
      sel_w[rank] = w;
      if (blockIdx.x == 0) {
        a.ids[rank] = id;
        a.tw[rank] = w;
      }
    }
  } else if (a.has_shared) {
    // meanwhile the other waves run the shared expert's gate/up, two row
    // pairs at a time
    const ExpertSet& S = a.shared;
    const float gg = (FMT == MOE_WFMT_NVFP4) ? S.gate.g[0] : 1.0f;
    const float gu = (FMT == MOE_WFMT_NVFP4) ? S.up.g[0] : 1.0f;
    constexpr int kW = kFusedWaves - 1;
    for (int pair0 = 2 * ((int)blockIdx.x * kW + wv - 1); pair0 < S.inter; pair0 += 2 * kW * (int)gridDim.x)
      gateup_wave<FMT, GPL, 2, 1>(a.x, a.H, S.gate, S.up, 0, S.inter, pair0, gg, gu, a.h_shared);
  }
  __syncthreads();
  const ExpertSet& R = a.routed;
  // wave item it: pick p = it / per_pick (rank p of the k distinct experts),
  // row pairs [8 m, 8 m + 8) with m = it % per_pick
  const int per_pick = R.inter / kFusedPairs;
  for (int it = gw; it < sel_n * per_pick; it += nw) {
    const int p = it / per_pick;
    const int e = sel_e[p];
    const float gg = (FMT == MOE_WFMT_NVFP4) ? R.gate.g[e] : 1.0f;
    const float gu = (FMT == MOE_WFMT_NVFP4) ? R.up.g[e] : 1.0f;
    gateup_wave<FMT, GPL, kFusedPairs, 1>(a.x, a.H, R.gate, R.up, (size_t)e * R.inter, R.inter,
                                          (it - p * per_pick) * kFusedPairs, gg, gu,
                                          a.h_routed + (size_t)p * a.ldh);
  }
  grid_arrive(a.bar, gridDim.x);
  down_t1_rows<FMT, true, 64 * kFusedWaves>(a, hl, gw, nw, [&] { return grid_wait(a.bar, a.barrier_spins); },
                                            sel_e, sel_w, sel_n);
}

// ---------------------------------------------------------------------------
// K4 for 2..4 tokens (short verify batches): down projection of the selected
// experts and the shared expert, combined into y.
//
// One workgroup per CU.  The SwiGLU outputs of all P = T*k picks (rows
// 0..P-1, sorted pick order) and of the shared expert (rows P..P+T-1) are
// staged in LDS once: quarter q of group c of row j at 16-byte slot
// (j * 4 + q) * 64 + c, groups past the row's last one zero, so 64 lanes read
// 1 KB contiguous at offsets that are compile-time constants.  Next to them,
// the int4 code-offset term of every (row, group).  Each wave then streams whole
// output rows: for row r and slot s, lane c loads group c of expert s's row r
// (inter <= 2048) and applies it to every token routed to s.  The (row, slot)
// items of a wave form one sequence with kDMDepth items in flight; the sum
// runs in slot order within a lane, then across the lanes, independent of
// timing.  The work is bound by the dequantisation and dot products, so each
// item's codes are dequantised once for all its tokens.
// ---------------------------------------------------------------------------
#ifndef QMOE_DM_WAVES
#define QMOE_DM_WAVES 8
#endif
#ifndef QMOE_DM_DEPTH
#define QMOE_DM_DEPTH 12
#endif
constexpr int kDMWaves = QMOE_DM_WAVES;   // waves per workgroup
// up to 36 h rows (4 tokens x 8 picks and the shared expert's 4 rows); one
// workgroup per CU.  (Used for one token as well -- 16 rows, every item of a
// wave in flight -- it measured slower than dec_down_t1.)
constexpr int kDMRows = 36, kDMDepth = QMOE_DM_DEPTH, kDMBlocks = 256;

// ROWS: h rows the LDS holds; D: (row, slot) items in flight per wave
template <int FMT, int ROWS, int D>
__global__ void __launch_bounds__(64 * kDMWaves) dec_down_multi_kernel(DecodeArgs a) {
  constexpr int kDMChunks = ROWS * 256;   // 16-byte chunks: 4 quarters x 64 groups per row
  constexpr int kDMDepth = D;
  static_assert(kDMChunks % (64 * kDMWaves) == 0, "h chunks split evenly over the threads");
  __shared__ uint4 hl[kDMChunks];
  __shared__ float hsl[ROWS * 64];
  constexpr int NT = 64 * kDMWaves;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H, T = a.T, P = a.T * a.K;
  // the count and the records are fetched together; lanes at or past the
  // count hold stale records that are never read
  const DecSlot rec = a.slots[lane];
  const int nr = __builtin_amdgcn_readfirstlane(*a.n_active);
  const bool shared = a.has_shared;
  const int ns = nr + (shared ? 1 : 0);
  const int nG = a.routed.inter / 32;
  const int nrows = P + (shared ? T : 0);
  constexpr bool ROW = wfmt_row(FMT);
  constexpr uint32_t CB = group_code_bytes<FMT>();
  const uint32_t rowBytes = (uint32_t)nG * CB, srow = (uint32_t)nG * 2u;

  // slot `lane`'s record: weight row base, tokens, weights, first h row
  const bool sh_lane = shared && lane == nr;
  const bool rt_lane = lane < nr;
  const uint32_t m_row = rt_lane ? (uint32_t)rec.e * (uint32_t)H : 0u;
  // tokens as a bit mask, weights by token (zero where absent); the slot's
  // h rows are p0 + (rank of the token in the mask)
  const int m_p0 = sh_lane ? P : rec.p0;
  int m_mask = sh_lane ? (1 << T) - 1 : 0;
  float m_wt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) m_wt[t] = sh_lane && t < T ? 1.0f : 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bool has = !sh_lane && m < rec.M;
    m_mask |= has ? 1 << (rec.t[m] & 3) : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) m_wt[t] = has && rec.t[m] == t ? rec.w[m] : m_wt[t];
  }
  float m_g = 1.0f;
  if (FMT == MOE_WFMT_NVFP4) {
    if (rt_lane) m_g = a.routed.down.g[rec.e];
    if (sh_lane) m_g = a.shared.down.g[0];
  }
  const rsrc_t rq = make_rsrc(a.routed.down.q, 0xFFFFFFFFu);
  const rsrc_t rs = make_rsrc(a.routed.down.s, 0xFFFFFFFFu);
  const rsrc_t sq = make_rsrc(a.shared.down.q, shared ? 0xFFFFFFFFu : 0u);
  const rsrc_t ss = make_rsrc(a.shared.down.s, shared ? 0xFFFFFFFFu : 0u);
  // lanes past the row's last group load group 0 and meet zero h
  const uint32_t c = lane < nG ? (uint32_t)lane : 0u;

  // this wave's items: rows gw, gw + nw, ...; slots 0 .. ns-1 within a row
  const int gw = blockIdx.x * kDMWaves + wv, nw = gridDim.x * kDMWaves;
  const int nrw = gw < H ? (H - gw + nw - 1) / nw : 0;
  const int N = nrw * ns;

  // h of every row, in LDS order: all of this thread's loads are issued
  // before the first weight items', so they do not queue behind them
  constexpr int kStPer = kDMChunks / NT;   // 16-byte chunks per thread
  uint32_t hv[kStPer][4];
  static_for<kStPer>([&](auto U) {   // fully unrolled, so hv stays in registers
    constexpr int u = decltype(U)::value;
    const int L = (int)threadIdx.x + u * NT;          // LDS chunk
    const int g = L & 63, jq = L >> 6, j = jq >> 2, q = jq & 3;
    // chunks outside the staged rows or past the last group reload a valid
    // one and are stored as zero
    const bool in = j < nrows && g < nG;
    const int jj = in ? j : 0, gg = in ? g : 0;
    const uint16_t* src = jj < P ? a.h_routed + (size_t)jj * a.ldh : a.h_shared + (size_t)(jj - P) * a.ldh;
    load16(hv[u], src + gg * 32 + q * 8);
  });
  __builtin_amdgcn_sched_barrier(0);   // keep the h loads ahead of the weight loads

  uint32_t wq[kDMDepth][4], wsc[kDMDepth];
  int is = 0, ir = gw < H ? gw : 0, iss = 0;   // next item to issue: slot, row, index
  // Items past the last one reload the last one (in bounds) and are never
  // computed, so every step issues the same loads; a wave without rows loads
  // row 0 of slot 0.  (Issuing the first items under a condition would leave
  // the compiler unsure of the load order and make every wait a full one.)
  auto issue = [&](auto B) {
    constexpr int b = decltype(B)::value;
    const int sl = __builtin_amdgcn_readfirstlane(is);
    const bool sh = shared && sl == nr;
    const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)m_row, sl) + (uint32_t)ir;
    load_group<FMT>(wq[b], sh ? sq : rq, c * CB, row * rowBytes);
    // per-row formats: the row's fp32 scale (the same word in every lane)
    wsc[b] = ROW ? bload_u32(sh ? ss : rs, 0u, row * 4u) : bload_u16(sh ? ss : rs, c * 2u, row * srow);
    if (iss < N - 1) {
      ++iss;
      if (++is == ns) {
        is = 0;
        ir += nw;
      }
    }
  };
  static_for<kDMDepth>([&](auto B) { issue(B); });
  __builtin_amdgcn_sched_barrier(0);

  static_for<kStPer>([&](auto U) {
    constexpr int u = decltype(U)::value;
    const int L = (int)threadIdx.x + u * NT;
    const int g = L & 63, j = L >> 8;
    const bool in = j < nrows && g < nG;
    hl[L] = in ? make_uint4(hv[u][0], hv[u][1], hv[u][2], hv[u][3]) : make_uint4(0, 0, 0, 0);
  });
  __syncthreads();
  if (FMT != MOE_WFMT_NVFP4) {
    // each (row, group)'s offset term: int4's, or (int2) the sum of h
    for (int i = threadIdx.x; i < ROWS * 64; i += NT) {
      const int j = i >> 6, g = i & 63;
      uint32_t hm[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = hl[(j * 4 + q) * 64 + g];
        hm[4 * q] = v.x; hm[4 * q + 1] = v.y; hm[4 * q + 2] = v.z; hm[4 * q + 3] = v.w;
      }
      hsl[i] = offset_h<FMT>(hm);
    }
    __syncthreads();
  }
  if (N == 0) return;

  int cs = 0, cr = 0;    // next item to compute: slot, row index within the wave
  float y0 = 0.0f, y1 = 0.0f, y2 = 0.0f, y3 = 0.0f;
  // one accumulator per token
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint4* hlane = hl + lane;
  const float* hslane = hsl + lane;
  auto compute = [&](auto B) {
    constexpr int b = decltype(B)::value;
    const int sl = __builtin_amdgcn_readfirstlane(cs);
    const uint32_t mask = (uint32_t)__builtin_amdgcn_readlane(m_mask, sl);
    const int p0 = __builtin_amdgcn_readlane(m_p0, sl);
    // the codes as 16-bit float pairs, once for all tokens of the slot
    uint32_t wf[16];
    float sc0, sc1 = 0.0f;
    if constexpr (FMT == MOE_WFMT_INT4_G32_F16 || FMT == MOE_WFMT_INT4_ROW_F32) {
      int4_f16_1024(wq[b], wf);
      sc0 = ROW ? __uint_as_float(wsc[b]) : half_bits_to_f32(wsc[b] & 0xffffu);
    } else if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) wf[8 * j + k] = int2_pair_f16(wq[b][j], k, 0x3C003C00u);
      sc0 = 4.0f * __uint_as_float(wsc[b]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) wf[4 * j + k] = fp4_pair_f16(wq[b][j], k);
      const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_g), sl));
      sc0 = e4m3_to_f32(wsc[b], 0) * g;
      sc1 = e4m3_to_f32(wsc[b], 1) * g;
    }
    // token t (a compile-time index, so its accumulator is a fixed register)
    // under a uniform branch on the slot's mask
    static_for<4>([&](auto TT) {
      constexpr int t = decltype(TT)::value;
      if (mask & (1u << t)) {
        const int j = p0 + __builtin_popcount(mask & ((1u << t) - 1u));
        uint32_t hm[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = hlane[(j * 4 + q) * 64];
          hm[4 * q] = v.x; hm[4 * q + 1] = v.y; hm[4 * q + 2] = v.z; hm[4 * q + 3] = v.w;
        }
        float v;
        if constexpr (FMT == MOE_WFMT_INT4_G32_F16 || FMT == MOE_WFMT_INT4_ROW_F32) {
          v = sc0 * (int4_dot_1024(wf, hm) - hslane[j * 64]);   // offset staged with h
        } else if constexpr (FMT == MOE_WFMT_INT2_ROW_F32) {
          float d = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) d = dot2_f16(wf[i], hm[i], d);
          v = sc0 * fmaf(-1.5f, hslane[j * 64], d);   // 4 s (d - 1.5 sum h)
        } else {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) d0 = dot2_f16(wf[i], hm[i], d0);
#pragma unroll
          for (int i = 8; i < 16; ++i) d1 = dot2_f16(wf[i], hm[i], d1);
          v = fmaf(sc0, d0, sc1 * d1);
        }
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_wt[t]), sl));
        acc[t] = fmaf(w, v, acc[t]);
      }
    });
    if (++cs == ns) {
      // row k's sums go to lane k; y is written after the loop, so no store
      // sits between the loads and their use
      const float v0 = wave_sum(acc[0]), v1 = wave_sum(acc[1]);
      const float v2 = wave_sum(acc[2]), v3 = wave_sum(acc[3]);
      const bool mine = lane == cr;
      y0 = mine ? v0 : y0;
      y1 = mine ? v1 : y1;
      y2 = mine ? v2 : y2;
      y3 = mine ? v3 : y3;
      acc[0] = acc[1] = acc[2] = acc[3] = 0.0f;
      cs = 0;
      ++cr;
    }
  };
  for (int i0 = 0; i0 < N; i0 += kDMDepth) {
    static_for<kDMDepth>([&](auto B) {
      if (i0 + decltype(B)::value < N) compute(B);
      issue(B);
    });
  }
  if (lane < nrw) {
    const int r = gw + lane * nw;
    store_y(a, 0, r, y0);
    if (T > 1) store_y(a, 1, r, y1);
    if (T > 2) store_y(a, 2, r, y2);
    if (T > 3) store_y(a, 3, r, y3);
  }
}

// Whether dec_down_multi with ROWS h rows in LDS covers this shape.
template <int ROWS>
__host__ __device__ inline bool down_multi_fits(const DecodeArgs& a) {
  const long long nG = a.routed.inter / 32;
  const long long P = (long long)a.T * a.K;
  const bool sh4 = a.has_shared;
  return a.T >= 1 && a.T <= kMaxT && nG <= 64 && P + (sh4 ? 1 : 0) <= 64 &&
         (!sh4 || a.shared.inter == a.routed.inter) && P + (sh4 ? a.T : 0) <= ROWS &&
         (a.H + 256 * kDMWaves - 1) / (256 * kDMWaves) <= 64 &&
         (long long)a.E * a.H * (a.routed.inter / 2) < 0xFFFFFFFFll &&
         (long long)a.E * a.H * nG * 2 < 0xFFFFFFFFll;
}

// The formats the small-batch kernels take: f(integral_constant<fmt>).  The
// per-row int4 and int2 formats run the single-token kernels only (the
// caller routes other shapes and int8 to the grouped GEMV).
template <class F>
auto dec_fmt(int wfmt, F&& f) {
  switch (wfmt) {
    case MOE_WFMT_NVFP4: return f(std::integral_constant<int, MOE_WFMT_NVFP4>{});
    case MOE_WFMT_INT4_ROW_F32: return f(std::integral_constant<int, MOE_WFMT_INT4_ROW_F32>{});
    case MOE_WFMT_INT2_ROW_F32: return f(std::integral_constant<int, MOE_WFMT_INT2_ROW_F32>{});
    default: return f(std::integral_constant<int, MOE_WFMT_INT4_G32_F16>{});
  }
}

template <int GPL>
hipError_t launch_k2(const DecodeArgs& a, hipStream_t s, int blocks) {
  dec_fmt(a.wfmt, [&](auto F) {
    hipLaunchKernelGGL((dec_select_permute_kernel<decltype(F)::value, GPL>), dim3(blocks), dim3(256), 0, s, a);
    return 0;
  });
  return hipGetLastError();
}

template <int GPL>
hipError_t launch_k23(const DecodeArgs& a, hipStream_t s, dim3 grid) {
  dec_fmt(a.wfmt, [&](auto F) {
    hipLaunchKernelGGL((dec_select_gateup_kernel<decltype(F)::value, GPL>), grid, dim3(256), 0, s, a);
    return 0;
  });
  return hipGetLastError();
}

template <int GPL>
hipError_t launch_k3(const DecodeArgs& a, hipStream_t s, dim3 grid) {
  dec_fmt(a.wfmt, [&](auto F) {
    hipLaunchKernelGGL((dec_gateup_kernel<decltype(F)::value, GPL>), grid, dim3(256), 0, s, a);
    return 0;
  });
  return hipGetLastError();
}

// Grid of dec_fused_t1<FMT, GPL> on the current device: the workgroups it
// holds at once (at most kFusedBlocksPerCU per CU) for the largest LDS size
// down_t1_fits allows; 0 if that cannot be determined.  Cached per device.
template <int FMT, int GPL>
int fused_grid_of() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];   // 0: not known yet, -1: none
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v != 0) return v < 0 ? 0 : v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dec_fused_t1_kernel<FMT, GPL>,
                                                   64 * kFusedWaves, 65536) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    per_cu = cus = 0;
  v = std::min(std::min(per_cu, kFusedBlocksPerCU) * cus, kDecFusedMaxGrid);
  (void)hipGetLastError();
  cache[dev].store(v > 0 ? v : -1, std::memory_order_relaxed);
  return v > 0 ? v : 0;
}
template <int GPL>
int fused_grid(int wfmt) {
  return dec_fmt(wfmt, [&](auto F) { return fused_grid_of<decltype(F)::value, GPL>(); });
}

template <int GPL>
hipError_t launch_fused(const DecodeArgs& a, hipStream_t s, size_t lds, int grid) {
  dec_fmt(a.wfmt, [&](auto F) {
    hipLaunchKernelGGL((dec_fused_t1_kernel<decltype(F)::value, GPL>), dim3(grid), dim3(64 * kFusedWaves),
                       lds, s, a);
    return 0;
  });
  return hipGetLastError();
}


}  // namespace

hipError_t launch_route_scores(const uint16_t* x, const float* router_w, double* scores, int T, int H,
                               int E, hipStream_t s) {
  if (T < 1 || T > kMaxT || H % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_scores_kernel, dim3(E), dim3(256), 0, s, x, router_w, scores, T, H, E);
  return hipGetLastError();
}

bool decode_supported(int H) { return H / 32 <= 64 * kDecodeMaxGPL; }

bool decode_row_format_ok(const moe_config& c, int T) {
  if (c.wfmt != MOE_WFMT_INT4_ROW_F32 && c.wfmt != MOE_WFMT_INT2_ROW_F32) return false;
  if (T < 1 || T > kDecodeMaxTokens || !decode_supported(c.hidden)) return false;
  DecodeArgs a{};
  a.T = T;
  a.K = c.top_k;
  a.E = c.n_routed_experts;
  a.H = c.hidden;
  a.routed.inter = c.moe_inter;
  a.has_shared = c.n_shared_experts == 1;
  a.shared.inter = c.shared_inter;
  return T == 1 ? down_t1_fits(a) : down_multi_fits<kDMRows>(a);
}

// K4: the down projection with the combine, for the shapes each kernel takes.
static hipError_t launch_k4(const DecodeArgs& a, hipStream_t s, Tracer* tr, size_t lds1) {
  hipError_t e;
  const bool f4 = a.wfmt == MOE_WFMT_NVFP4;
  dim3 g4(a.H / kDownRows);
  if (down_t1_fits(a)) {
    const int blocks = std::min((a.H + 3) / 4, 512);
    dec_fmt(a.wfmt, [&](auto F) {
      hipLaunchKernelGGL((dec_down_t1_kernel<decltype(F)::value>), dim3(blocks), dim3(256), lds1, s, a);
      return 0;
    });
  } else if (a.T > 1 && down_multi_fits<kDMRows>(a)) {
    const int blocks = std::min((a.H + kDMWaves - 1) / kDMWaves, kDMBlocks);
    dec_fmt(a.wfmt, [&](auto F) {
      hipLaunchKernelGGL((dec_down_multi_kernel<decltype(F)::value, kDMRows, kDMDepth>), dim3(blocks),
                         dim3(64 * kDMWaves), 0, s, a);
      return 0;
    });
  } else if (a.T == 1) {
    if (f4)
      hipLaunchKernelGGL((dec_down_combine_kernel<MOE_WFMT_NVFP4, 1>), g4, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((dec_down_combine_kernel<MOE_WFMT_INT4_G32_F16, 1>), g4, dim3(256), 0, s, a);
  } else {
    if (f4)
      hipLaunchKernelGGL((dec_down_combine_kernel<MOE_WFMT_NVFP4, kMaxT>), g4, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((dec_down_combine_kernel<MOE_WFMT_INT4_G32_F16, kMaxT>), g4, dim3(256), 0, s,
                         a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("dec_down_combine")) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  hipError_t e;
  const int gpl = (a.H / 32 + 63) / 64;
  // per-row formats: shapes whose down rows fit dec_down_t1 (one token) or
  // dec_down_multi (2-4 tokens) only
  if (wfmt_row(a.wfmt) && (a.wfmt == MOE_WFMT_INT8_ROW_F32 ||
                           !(a.T == 1 ? down_t1_fits(a) : down_multi_fits<kDMRows>(a))))
    return hipErrorInvalidValue;
  // one token: selection, the shared expert's gate/up and K3/K4 in
  // dec_fused_t1 when the device's resident grid is known
  int fgrid = 0;
  // MOE_OPT_NO_GRID_WAIT turns dec_fused_t1 off (one token then takes K2, K3
  // and dec_down_t1)
  if (down_t1_fits(a) && !(a.options & MOE_OPT_NO_GRID_WAIT)) {
    switch (gpl) {
      case 1: fgrid = fused_grid<1>(a.wfmt); break;
      case 2: fgrid = fused_grid<2>(a.wfmt); break;
      case 3: fgrid = fused_grid<3>(a.wfmt); break;
      default: fgrid = fused_grid<4>(a.wfmt); break;
    }
  }
  hipLaunchKernelGGL(dec_router_kernel, dim3(a.E), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("dec_router")) != hipSuccess) return e;
  const size_t lds1 = (size_t)(a.K + (a.has_shared ? 1 : 0)) * a.routed.inter * 2;
  if (fgrid > 0) {
    DecodeArgs af = a;
    // MOE_OPT_GRID_WAIT_NONE: no poll at all, to exercise the give-up path
    af.barrier_spins = (a.options & MOE_OPT_GRID_WAIT_NONE) ? 0u : kBarrierSpins;
    switch (gpl) {
      case 1: e = launch_fused<1>(af, s, lds1, fgrid); break;
      case 2: e = launch_fused<2>(af, s, lds1, fgrid); break;
      case 3: e = launch_fused<3>(af, s, lds1, fgrid); break;
      default: e = launch_fused<4>(af, s, lds1, fgrid); break;
    }
    if (e != hipSuccess) return e;
    return tr ? tr->mark("dec_fused_t1") : hipSuccess;
  }

#ifndef QMOE_MERGED_K23
#define QMOE_MERGED_K23 1
#endif
  // 2..4 tokens: the selection and gate/up in one launch, unless the caller
  // asked for kernels whose workgroups never wait for each other
  if (QMOE_MERGED_K23 && a.T >= 2 && !(a.options & MOE_OPT_NO_GRID_WAIT)) {
    DecodeArgs am = a;
    am.barrier_spins = (a.options & MOE_OPT_GRID_WAIT_NONE) ? 0u : kBarrierSpins;
    const int imax = std::max(a.routed.inter, a.has_shared ? a.shared.inter : 0);
    dim3 g23((imax + kPairsPerBlock - 1) / kPairsPerBlock, 1 + a.T + a.T * a.K);
    switch (gpl) {
      case 1: e = launch_k23<1>(am, s, g23); break;
      case 2: e = launch_k23<2>(am, s, g23); break;
      case 3: e = launch_k23<3>(am, s, g23); break;
      default: e = launch_k23<4>(am, s, g23); break;
    }
    if (e != hipSuccess) return e;
    if (tr && (e = tr->mark("dec_select_gateup")) != hipSuccess) return e;
    return launch_k4(a, s, tr, lds1);
  }
  // the shared expert's gate/up in K2, beside the selection
  const int k2_blocks =
      1 + (a.has_shared ? a.T * ((a.shared.inter + kSharedPairsPerBlock - 1) / kSharedPairsPerBlock) : 0);
  switch (gpl) {
    case 1: e = launch_k2<1>(a, s, k2_blocks); break;
    case 2: e = launch_k2<2>(a, s, k2_blocks); break;
    case 3: e = launch_k2<3>(a, s, k2_blocks); break;
    default: e = launch_k2<4>(a, s, k2_blocks); break;
  }
  if (e != hipSuccess) return e;
  if (tr && (e = tr->mark("dec_select_permute")) != hipSuccess) return e;

  dim3 g3((a.routed.inter + kPairsPerBlock - 1) / kPairsPerBlock, a.T * a.K);
  switch (gpl) {
    case 1: e = launch_k3<1>(a, s, g3); break;
    case 2: e = launch_k3<2>(a, s, g3); break;
    case 3: e = launch_k3<3>(a, s, g3); break;
    default: e = launch_k3<4>(a, s, g3); break;
  }
  if (e != hipSuccess) return e;
  if (tr && (e = tr->mark("dec_gateup")) != hipSuccess) return e;

  return launch_k4(a, s, tr, lds1);
}

}  // namespace qmoe
