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
// Grid: (row blocks, expert slots); slot s < max_slots is the s-th active
// expert of the permutation (blocks past n_active exit), the last slot is the
// expert applied to every token (shared expert or dense mode).
#include "qmoe_device.h"

namespace qmoe {
namespace {

constexpr int kRPW = 4;                  // output rows per wave (gate/up: row pairs)
constexpr int kRowsPerBlock = 4 * kRPW;  // 4 waves per block
constexpr int kTB = 2;                   // tokens per pass over the weights

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

// One 32-input group of one weight row against kTB activation groups.
// acc[tb] += sum_k w_k * act_k for the group.
template <int FMT, bool F16ACT>
__device__ __forceinline__ void group_dot(const uint32_t (&wq)[4], uint32_t sc,
                                          const uint32_t (&act)[kTB][16], const float (&asum)[kTB],
                                          float gs, float (&acc)[kTB]) {
  if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
    uint32_t p[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        p[4 * j + k] = F16ACT ? int4_pair_f16(wq[j], k) : int4_pair_bf16(wq[j], k);
    const float s16 = 16.0f * half_bits_to_f32(sc & 0xffffu);
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
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
    for (int tb = 0; tb < kTB; ++tb) {
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

template <int FMT>
__global__ void __launch_bounds__(256) gateup_gemv_kernel(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.ok) return;
  const ExpertSet& X = sl.routed ? a.routed : a.dense;
  const int inter = X.inter;
  const int row0 = blockIdx.x * kRowsPerBlock + wv * kRPW;
  if (row0 >= inter) return;
  const int H = a.H;
  const int nG = H / 32;
  const size_t rowBytes = (size_t)H / 2;
  const size_t rbase = (size_t)sl.e * inter;
  const float gg = (FMT == MOE_WFMT_NVFP4) ? X.gate.g[sl.e] : 1.0f;
  const float gu = (FMT == MOE_WFMT_NVFP4) ? X.up.g[sl.e] : 1.0f;
  uint16_t* hbase = sl.routed ? a.h_routed + (size_t)sl.tok_begin * a.ldh : a.h_dense;

  for (int m0 = 0; m0 < sl.M; m0 += kTB) {
    int tok[kTB];
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) tok[tb] = token_of(a, sl, min(m0 + tb, sl.M - 1));
    float ag[kRPW][kTB], au[kRPW][kTB];
#pragma unroll
    for (int r = 0; r < kRPW; ++r)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) ag[r][tb] = au[r][tb] = 0.0f;

    for (int c = lane; c < nG; c += 64) {
      uint32_t xw[kTB][16];
      float xs[kTB];
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const uint16_t* xp = a.x + (size_t)tok[tb] * H + (size_t)c * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) load16(&xw[tb][4 * q], xp + 8 * q);
        float s = 0.0f;
        if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s = dot2_bf16(xw[tb][i], 0x3F803F80u, s);
        }
        xs[tb] = s;
      }
#pragma unroll
      for (int r = 0; r < kRPW; ++r) {
        const size_t row = rbase + row0 + r;
        uint32_t wq[4];
        load16(wq, X.gate.q + row * rowBytes + (size_t)c * 16);
        group_dot<FMT, false>(wq, load_scale<FMT>(X.gate.s, row, nG, c), xw, xs, gg, ag[r]);
        load16(wq, X.up.q + row * rowBytes + (size_t)c * 16);
        group_dot<FMT, false>(wq, load_scale<FMT>(X.up.s, row, nG, c), xw, xs, gu, au[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRPW; ++r)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const float g = wave_sum(ag[r][tb]);
        const float u = wave_sum(au[r][tb]);
        if (lane == r * kTB + tb && m0 + tb < sl.M) {
          const _Float16 hv = (_Float16)silu_mul(g, u);
          hbase[(size_t)(m0 + tb) * a.ldh + row0 + r] = __builtin_bit_cast(uint16_t, hv);
        }
      }
  }
}

template <int FMT>
__global__ void __launch_bounds__(256) down_gemv_kernel(FfnArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.ok) return;
  const ExpertSet& X = sl.routed ? a.routed : a.dense;
  const int inter = X.inter;
  const int H = a.H;
  const int row0 = blockIdx.x * kRowsPerBlock + wv * kRPW;
  if (row0 >= H) return;
  const int nG = inter / 32;
  const size_t rowBytes = (size_t)inter / 2;
  const size_t rbase = (size_t)sl.e * H;
  const float gd = (FMT == MOE_WFMT_NVFP4) ? X.down.g[sl.e] : 1.0f;
  const uint16_t* hbase = sl.routed ? a.h_routed + (size_t)sl.tok_begin * a.ldh : a.h_dense;
  float* obase = sl.routed ? a.o_routed + (size_t)sl.tok_begin * H : a.o_dense;

  for (int m0 = 0; m0 < sl.M; m0 += kTB) {
    int mm[kTB];
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) mm[tb] = min(m0 + tb, sl.M - 1);
    float acc[kRPW][kTB];
#pragma unroll
    for (int r = 0; r < kRPW; ++r)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) acc[r][tb] = 0.0f;
    for (int c = lane; c < nG; c += 64) {
      uint32_t hw[kTB][16];
      float hs[kTB];
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const uint16_t* hp = hbase + (size_t)mm[tb] * a.ldh + (size_t)c * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) load16(&hw[tb][4 * q], hp + 8 * q);
        float s = 0.0f;
        if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s = dot2_f16(hw[tb][i], 0x3C003C00u, s);
        }
        hs[tb] = s;
      }
#pragma unroll
      for (int r = 0; r < kRPW; ++r) {
        const size_t row = rbase + row0 + r;
        uint32_t wq[4];
        load16(wq, X.down.q + row * rowBytes + (size_t)c * 16);
        group_dot<FMT, true>(wq, load_scale<FMT>(X.down.s, row, nG, c), hw, hs, gd, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRPW; ++r)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const float v = wave_sum(acc[r][tb]);
        if (lane == r * kTB + tb && m0 + tb < sl.M) obase[(size_t)(m0 + tb) * H + row0 + r] = v;
      }
  }
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
    const int p = a.inv_perm[(size_t)t * K + i];
    const float w = a.tw[(size_t)t * K + i];
    const float4 o = *reinterpret_cast<const float4*>(a.expert_out + (size_t)p * H + n);
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
  dim3 g1((max_inter + kRowsPerBlock - 1) / kRowsPerBlock, slots);
  dim3 g2((a.H + kRowsPerBlock - 1) / kRowsPerBlock, slots);
  hipError_t e;
  if (a.wfmt == MOE_WFMT_INT4_G32_F16)
    hipLaunchKernelGGL(gateup_gemv_kernel<MOE_WFMT_INT4_G32_F16>, g1, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gateup_gemv_kernel<MOE_WFMT_NVFP4>, g1, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("gateup_gemv")) != hipSuccess) return e;
  if (a.wfmt == MOE_WFMT_INT4_G32_F16)
    hipLaunchKernelGGL(down_gemv_kernel<MOE_WFMT_INT4_G32_F16>, g2, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(down_gemv_kernel<MOE_WFMT_NVFP4>, g2, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
