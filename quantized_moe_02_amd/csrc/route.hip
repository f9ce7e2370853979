// Router: DeepSeek-V3-style sigmoid scores, bias-corrected group-limited top-k
// ("noaux_tc"), renormalised weights times routed_scaling_factor
// (page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section "Fitur utama").
//
// Two kernels:
//   route_logits  l[t][e] = sum_h x[t][h] * Wr[e][h] in float64.  A bf16 times
//                 an fp32 is exact in float64, so the only rounding is the
//                 float64 sum.  One wave per (expert, block of TT tokens); the
//                 lanes stride the hidden dimension with 16-byte loads of Wr.
//   route_select  one wave per token (select_token.h).
#include "select_token.h"

namespace qmoe {
namespace {

constexpr int kLogitTokens = 8;  // tokens per wave in route_logits

__global__ void __launch_bounds__(256) route_logits_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ Wr,
                                                           double* __restrict__ logits, int T,
                                                           int H, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kLogitTokens;
  if (e >= E) return;
  const int nt = min(kLogitTokens, T - t0);
  double acc[kLogitTokens];
#pragma unroll
  for (int i = 0; i < kLogitTokens; ++i) acc[i] = 0.0;
  const float* wrow = Wr + (size_t)e * H;
  for (int h = lane * 4; h < H; h += 256) {
    const float4 w4 = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int i = 0; i < kLogitTokens; ++i) {
      if (i < nt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + i) * H + h);
        double a = acc[i];
        a = fma((double)bf16_lo(xv.x), (double)w4.x, a);
        a = fma((double)bf16_hi(xv.x), (double)w4.y, a);
        a = fma((double)bf16_lo(xv.y), (double)w4.z, a);
        a = fma((double)bf16_hi(xv.y), (double)w4.w, a);
        acc[i] = a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kLogitTokens; ++i) {
    const double v = wave_sum(acc[i]);
    if (lane == 0 && i < nt) logits[(size_t)(t0 + i) * E + e] = v;
  }
}

__global__ void __launch_bounds__(256) route_select_kernel(const double* __restrict__ logits,
                                                           const float* __restrict__ bias,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ tw, int T, int E,
                                                           int G, int TG, int K, float rsf) {
  __shared__ SelectScratch sc[4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  int id, rank;
  float w;
  select_token(logits + (size_t)t * E, bias, E, G, TG, K, rsf, sc[wv], id, w, rank);
  if (lane < K) {
    ids[(size_t)t * K + rank] = id;
    tw[(size_t)t * K + rank] = w;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  hipError_t e;
  dim3 g1((a.E + 3) / 4, (a.T + kLogitTokens - 1) / kLogitTokens);
  hipLaunchKernelGGL(route_logits_kernel, g1, dim3(256), 0, s, a.x, a.router_w, a.logits, a.T,
                     a.H, a.E);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_logits")) != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.bias,
                     a.ids, a.tw, a.T, a.E, a.G, a.TG, a.K, a.rsf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_select")) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace qmoe
