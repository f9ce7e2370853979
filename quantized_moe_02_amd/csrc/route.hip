// Router: DeepSeek-V3-style sigmoid scores, bias-corrected group-limited top-k
// ("noaux_tc"), renormalised weights times routed_scaling_factor
// (page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section "Fitur utama").
//
// Two kernels:
//   route_logits  l[t][e] = sum_h x[t][h] * Wr[e][h] in float64.  A bf16 times
//                 an fp32 is exact in float64, so the only rounding is the
//                 float64 sum.  One wave per (expert, block of TT tokens); the
//                 lanes stride the hidden dimension with 16-byte loads of Wr.
//   route_select  one wave per token: sigmoid, bias, group scores, group and
//                 expert selection by wave-wide arg-max, ascending ids, weights.
#include "qmoe_device.h"

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

// (value, index) arg-max across the wave; ties go to the lower index.
__device__ __forceinline__ void wave_argmax(double& v, int& idx) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(v, off, kWave);
    const int oi = __shfl_xor(idx, off, kWave);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
}

constexpr int kMaxE = 256;
constexpr int kMaxG = 64;

__global__ void __launch_bounds__(256) route_select_kernel(const double* __restrict__ logits,
                                                           const float* __restrict__ bias,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ tw, int T, int E,
                                                           int G, int TG, int K, float rsf) {
  __shared__ double s_lds[4][kMaxE];
  __shared__ double sb_lds[4][kMaxE];
  __shared__ double gs_lds[4][kMaxG];
  __shared__ int keep_lds[4][kMaxG];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const bool valid = t < T;
  const int per = E / G;

  if (valid) {
    for (int e = lane; e < E; e += 64) {
      const double l = logits[(size_t)t * E + e];
      const double s = 1.0 / (1.0 + exp(-l));
      s_lds[w][e] = s;
      sb_lds[w][e] = s + (bias ? (double)bias[e] : 0.0);
    }
  }
  __syncthreads();
  if (valid && lane < G) {
    // group score: sum of the two largest biased scores of the group
    double m1 = -INFINITY, m2 = -INFINITY;
    for (int i = 0; i < per; ++i) {
      const double v = sb_lds[w][lane * per + i];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    gs_lds[w][lane] = per >= 2 ? m1 + m2 : m1;
  }
  __syncthreads();
  if (valid && lane < G) {
    const double mine = gs_lds[w][lane];
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const double o = gs_lds[w][g];
      rank += (o > mine || (o == mine && g < lane)) ? 1 : 0;
    }
    keep_lds[w][lane] = rank < TG;
  }
  __syncthreads();
  if (!valid) return;

  // candidates held by this lane: experts lane, lane+64, lane+128, lane+192
  double v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = (e < E && keep_lds[w][e / per]) ? sb_lds[w][e] : -INFINITY;
  }
  int my_id = 0x7fffffff;
  for (int r = 0; r < K; ++r) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (lane == r) my_id = bi;
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == bi) v[j] = -INFINITY;
    }
  }
  // Only NaN scores can leave a round without a winner; keep the id in range
  // so that later kernels never index outside the expert arrays.
  if (lane < K && (my_id < 0 || my_id >= E)) my_id = lane;
  // ascending order and renormalised weights
  int rank = 0;
  for (int j = 0; j < K; ++j) {
    const int o = __shfl(my_id, j, kWave);
    rank += (o < my_id) ? 1 : 0;
  }
  const double s_mine = lane < K ? s_lds[w][my_id] : 0.0;
  const double total = wave_sum(s_mine);
  if (lane < K) {
    ids[(size_t)t * K + rank] = my_id;
    tw[(size_t)t * K + rank] = (float)(s_mine / total * (double)rsf);
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  dim3 g1((a.E + 3) / 4, (a.T + kLogitTokens - 1) / kLogitTokens);
  hipLaunchKernelGGL(route_logits_kernel, g1, dim3(256), 0, s, a.x, a.router_w, a.logits, a.T,
                     a.H, a.E);
  hipLaunchKernelGGL(route_select_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.bias,
                     a.ids, a.tw, a.T, a.E, a.G, a.TG, a.K, a.rsf);
  return hipGetLastError();
}

}  // namespace qmoe
