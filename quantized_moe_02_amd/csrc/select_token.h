// One token's expert selection by one wave (page "Show HN: Menjalankan GLM 5.2
// di komputer lambat", section "Fitur utama": DeepSeek-V3-style sigmoid
// router, noaux_tc, routed_scaling_factor).
//
//   s = sigmoid(logit), s' = s + bias;  group score = sum of the two largest
//   s' of the group (the single one for one-expert groups);  keep the
//   topk_group best groups (ties: lower group);  choose the top_k largest s'
//   among experts of kept groups (ties: lower id);  weights
//   s / sum(s over chosen) * routed_scaling_factor.
// Everything in float64.
#pragma once

#include "qmoe_device.h"

namespace qmoe {

constexpr int kSelMaxE = 256;
constexpr int kSelMaxG = 64;

// Per-wave LDS scratch of select_token.
struct SelectScratch {
  double s[kSelMaxE];
  double sb[kSelMaxE];
  double gs[kSelMaxG];
  int keep[kSelMaxG];
  int ids[32];
};

// Orders LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lanes < K return their chosen expert in `id`, its weight in `w` and its
// position in ascending id order in `rank`.  `logits` points at the token's E
// float64 logits.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ void select_token(const double* __restrict__ logits,
                                             const float* __restrict__ bias, int E, int G, int TG,
                                             int K, float rsf, SelectScratch& sc, int& id, float& w,
                                             int& rank) {
  const int lane = threadIdx.x & 63;
  const int per = E / G;
  wave_lds_sync();  // a previous call's reads of `sc` come first
  double sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    sb[j] = -INFINITY;
    if (e < E) {
      const double l = logits[e];
      const double s = 1.0 / (1.0 + exp(-l));
      sb[j] = s + (bias ? (double)bias[e] : 0.0);
      sc.s[e] = s;
      sc.sb[e] = sb[j];
    }
  }
  wave_lds_sync();
  if (lane < G) {
    double m1 = -INFINITY, m2 = -INFINITY;
    for (int i = 0; i < per; ++i) {
      const double v = sc.sb[lane * per + i];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    sc.gs[lane] = per >= 2 ? m1 + m2 : m1;
  }
  wave_lds_sync();
  if (lane < G) {
    const double mine = sc.gs[lane];
    int r = 0;
    for (int g = 0; g < G; ++g) {
      const double o = sc.gs[g];
      r += (o > mine || (o == mine && g < lane)) ? 1 : 0;
    }
    sc.keep[lane] = r < TG;
  }
  wave_lds_sync();
  double v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = (e < E && sc.keep[e / per]) ? sb[j] : -INFINITY;
  }
  int my_id = 0x7fffffff;
  for (int r = 0; r < K; ++r) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E) better_of(bv, bi, v[j], e);
    }
    wave_argmax(bv, bi);
    if (lane == r) my_id = bi;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) v[j] = -INFINITY;
  }
  // Only NaN scores can leave a round without a winner; keep ids in range so
  // that later kernels never index outside the expert arrays.
  if (lane < K && (my_id < 0 || my_id >= E)) my_id = lane;
  if (lane < K) sc.ids[lane] = my_id;
  wave_lds_sync();
  rank = 0;
  for (int j = 0; j < K; ++j) rank += (sc.ids[j] < my_id) ? 1 : 0;
  const double s_mine = lane < K ? sc.s[my_id] : 0.0;
  const double total = wave_sum(s_mine);
  id = my_id;
  w = (float)(s_mine / total * (double)rsf);
}

}  // namespace qmoe
