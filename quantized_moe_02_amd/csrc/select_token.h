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
//
// Lane l holds experts 4l .. 4l+3.  When a group is a power-of-two number of
// whole lanes, the group top-2 is merged across its lanes with DPP; other
// group shapes go through LDS.  Each top-k round takes the wave maximum of the
// lanes' best remaining candidates with v_max_f64 over DPP / permlane steps;
// the lowest lane holding the maximum wins, which is also the lowest expert id
// because lanes hold ascending id ranges and a lane orders its own candidates
// by (value desc, id asc).
#pragma once

#include "qmoe_device.h"

namespace qmoe {

constexpr int kSelMaxE = 256;
constexpr int kSelMaxG = 64;

// Per-wave LDS scratch of select_token (used only for irregular group shapes).
struct SelectScratch {
  double sb[kSelMaxE];
  double gs[kSelMaxG];
};

// Orders LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// top-2 pair (a1 >= a2) merged with (b1 >= b2)
__device__ __forceinline__ void merge_top2(double& a1, double& a2, double b1, double b2) {
  const double hi = fmax(a1, b1);
  const double lo = fmax(fmin(a1, b1), fmax(a2, b2));
  a1 = hi;
  a2 = lo;
}
template <int CTRL>
__device__ __forceinline__ void top2_dpp(double& m1, double& m2) {
  merge_top2(m1, m2, dppd<CTRL>(m1), dppd<CTRL>(m2));
}
template <int M>
__device__ __forceinline__ void top2_swap(double& m1, double& m2) {
  double a1, b1, a2, b2;
  swap_pair<M>(m1, a1, b1);
  swap_pair<M>(m2, a2, b2);
  m1 = a1;
  m2 = a2;
  merge_top2(m1, m2, b1, b2);
}

template <int CTRL>
__device__ __forceinline__ double max_dpp(double v) {
  return fmax(v, dppd<CTRL>(v));
}
template <int M>
__device__ __forceinline__ double max_swap(double v) {
  double a, b;
  swap_pair<M>(v, a, b);
  return fmax(a, b);
}
__device__ __forceinline__ double wave_max(double v) {
  v = max_dpp<kDppXor1>(v);
  v = max_dpp<kDppXor2>(v);
  v = max_dpp<kDppHalfMirror>(v);
  v = max_dpp<kDppMirror>(v);
  v = max_swap<16>(v);
  return max_swap<32>(v);
}

// Lanes < K return their chosen expert in `id`, its weight in `w` and its
// position in ascending id order in `rank`.  `logits` points at the token's E
// float64 logits, given as `nsplit` partial sums `split_stride` apart (added
// in order).  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ void select_token(const double* __restrict__ logits,
                                             const float* __restrict__ bias, int E, int G, int TG,
                                             int K, float rsf, SelectScratch& sc, int& id, float& w,
                                             int& rank, int nsplit = 1, size_t split_stride = 0) {
  const int lane = threadIdx.x & 63;
  const int per = E / G;
  const int e0 = 4 * lane;
  double s[4], sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + j;
    const bool in = e < E;
    double l = logits[in ? e : 0];
    for (int sp = 1; sp < nsplit; ++sp) l += logits[sp * split_stride + (in ? e : 0)];
    s[j] = 1.0 / (1.0 + exp(-l));
    sb[j] = in ? s[j] + (bias ? (double)bias[e] : 0.0) : -INFINITY;
  }
  // ---- group scores and kept groups ------------------------------------
  const int L = per / 4;  // lanes per group when groups are whole lanes
  const bool lane_groups = (per % 4 == 0) && L >= 1 && L <= 64 && (L & (L - 1)) == 0;
  bool keep_j[4];
  if (lane_groups) {
    // local top-2 of four, then merge across the group's lanes
    double m1 = fmax(sb[0], sb[1]), m2 = fmin(sb[0], sb[1]);
    merge_top2(m1, m2, fmax(sb[2], sb[3]), fmin(sb[2], sb[3]));
    if (L >= 2) top2_dpp<kDppXor1>(m1, m2);
    if (L >= 4) top2_dpp<kDppXor2>(m1, m2);
    if (L >= 8) top2_dpp<kDppHalfMirror>(m1, m2);
    if (L >= 16) top2_dpp<kDppMirror>(m1, m2);
    if (L >= 32) top2_swap<16>(m1, m2);
    if (L >= 64) top2_swap<32>(m1, m2);
    const double gmine = m1 + m2;
    const int gidx = lane / L;
    int r = 0;
    for (int g = 0; g < G; ++g) {
      const double o = readlane_d(gmine, g * L);
      r += (o > gmine || (o == gmine && g < gidx)) ? 1 : 0;
    }
    const bool keep = r < TG;
#pragma unroll
    for (int j = 0; j < 4; ++j) keep_j[j] = keep;
  } else {
    wave_lds_sync();  // a previous call's reads of `sc` come first
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + j < E) sc.sb[e0 + j] = sb[j];
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
    double gmine[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gmine[j] = sc.gs[(e0 + j < E ? e0 + j : 0) / per];
    int r[4] = {0, 0, 0, 0};
    for (int g = 0; g < G; ++g) {
      const double o = sc.gs[g];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gj = (e0 + j < E ? e0 + j : 0) / per;
        r[j] += (o > gmine[j] || (o == gmine[j] && g < gj)) ? 1 : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) keep_j[j] = r[j] < TG;
  }
  // ---- candidates sorted within the lane: value desc, id asc -------------
  double cv[4];
  int cj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cv[j] = keep_j[j] ? sb[j] : -INFINITY;
    cj[j] = j;
  }
  auto cswap = [&](int a, int b) {
    // keep (cv[a], cj[a]) ahead of (cv[b], cj[b])
    const bool sw = cv[b] > cv[a] || (cv[b] == cv[a] && cj[b] < cj[a]);
    const double tv = sw ? cv[b] : cv[a];
    const int tj = sw ? cj[b] : cj[a];
    cv[b] = sw ? cv[a] : cv[b];
    cj[b] = sw ? cj[a] : cj[b];
    cv[a] = tv;
    cj[a] = tj;
  };
  cswap(0, 1);
  cswap(2, 3);
  cswap(0, 2);
  cswap(1, 3);
  cswap(1, 2);
  // ---- top_k rounds -------------------------------------------------------
  int head = 0;
  int my_id = 0;
  double my_s = 0.0;
  for (int rr = 0; rr < K; ++rr) {
    const double hv = head == 0 ? cv[0] : head == 1 ? cv[1] : head == 2 ? cv[2] : head == 3 ? cv[3] : -INFINITY;
    const int hj = head == 0 ? cj[0] : head == 1 ? cj[1] : head == 2 ? cj[2] : cj[3];
    const double mx = wave_max(hv);
    const uint64_t hit = __ballot(hv == mx && head < 4);
    // hit is never empty for finite scores; an empty mask (NaN scores) picks lane 0
    const int wl = hit ? (int)__builtin_ctzll(hit) : 0;
    const int wid = __builtin_amdgcn_readlane(e0 + hj, wl);
    const double hs = (hj == 0 ? s[0] : hj == 1 ? s[1] : hj == 2 ? s[2] : s[3]);
    const double ws = readlane_d(hs, wl);
    if (lane == rr) {
      my_id = wid < E ? wid : 0;
      my_s = ws;
    }
    if (lane == wl) ++head;
  }
  // ---- ascending order and weights ---------------------------------------
  rank = 0;
  for (int j = 0; j < K; ++j) {
    const int o = __builtin_amdgcn_readlane(my_id, j);
    rank += (o < my_id || (o == my_id && j < lane)) ? 1 : 0;
  }
  const double total = wave_sum(lane < K ? my_s : 0.0);
  id = my_id;
  w = (float)(my_s / total * (double)rsf);
}

}  // namespace qmoe
