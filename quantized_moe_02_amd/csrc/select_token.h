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

// Per-wave LDS scratch of select_token.
struct alignas(16) SelectScratch {
  double sb[kSelMaxE];   // irregular group shapes only
  double gs[kSelMaxG];   // group scores (more than 16 groups)
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

// max / min by compare and select: the scores are never NaN, so the IEEE
// maxNum quieting that fmax compiles to is not needed
__device__ __forceinline__ double dmax(double a, double b) { return a > b ? a : b; }
__device__ __forceinline__ double dmin(double a, double b) { return a < b ? a : b; }

// top-2 pair (a1 >= a2) merged with (b1 >= b2)
__device__ __forceinline__ void merge_top2(double& a1, double& a2, double b1, double b2) {
  const double hi = dmax(a1, b1);
  const double lo = dmax(dmin(a1, b1), dmax(a2, b2));
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
  return dmax(v, dppd<CTRL>(v));
}
template <int M>
__device__ __forceinline__ double max_swap(double v) {
  double a, b;
  swap_pair<M>(v, a, b);
  return dmax(a, b);
}
__device__ __forceinline__ double wave_max(double v) {
  v = max_dpp<kDppXor1>(v);
  v = max_dpp<kDppXor2>(v);
  v = max_dpp<kDppHalfMirror>(v);
  v = max_dpp<kDppMirror>(v);
  v = max_swap<16>(v);
  return max_swap<32>(v);
}

// Order-preserving map of a (non-NaN) float64 to an unsigned 64-bit key.
__device__ __forceinline__ uint64_t okey(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
  const uint32_t o = dpp<CTRL>(v);
  return v > o ? v : o;
}
template <int M>
__device__ __forceinline__ uint32_t umax_swap(uint32_t v) {
  int a, b;
  swap_pair<M>((int)v, a, b);
  return (uint32_t)a > (uint32_t)b ? (uint32_t)a : (uint32_t)b;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax_dpp<kDppXor1>(v);
  v = umax_dpp<kDppXor2>(v);
  v = umax_dpp<kDppHalfMirror>(v);
  v = umax_dpp<kDppMirror>(v);
  v = umax_swap<16>(v);
  return umax_swap<32>(v);
}

// Lanes < K return their chosen expert in `id`, its weight in `w` and its
// position in ascending id order in `rank`; every lane returns in `n_kept`
// how many of the K stay after the adaptive expert top-p (page "Show HN:
// Menjalankan GLM 5.2 ...", section "Mengunduh model dan menjalankannya",
// --topp): with 0 < top_p < 1 only the shortest prefix of the chosen experts,
// ordered by share s / sum(s) (descending; equal shares: lower id first),
// whose shares reach top_p stays -- at least one; the weights are
// renormalised over the kept experts, and a dropped expert returns id -1,
// weight 0 and a rank >= n_kept.  Otherwise n_kept = K.  `logits` points at the token's E
// float64 logits, given as `nsplit` partial sums `split_stride` apart (added
// in order); SCORES: at the E sigmoid scores instead (nsplit 1), computed
// where the logits were, off this wave's critical path.  Must be called by
// all 64 lanes of the wave.
template <bool SCORES = false>
__device__ __forceinline__ void select_token(const double* __restrict__ logits,
                                             const float* __restrict__ bias, int E, int G, int TG,
                                             int K, float rsf, float top_p, SelectScratch& sc,
                                             int& id, float& w, int& rank, int& n_kept,
                                             int nsplit = 1, size_t split_stride = 0) {
  const int lane = threadIdx.x & 63;
  const int per = E / G;
  const int e0 = 4 * lane;
  double s[4], sb[4], l[4];
  float bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    l[j] = logits[e0 + j < E ? e0 + j : 0];
    bv[j] = bias ? bias[e0 + j < E ? e0 + j : 0] : 0.0f;
  }
  // partial sums added in split order; each batch's loads are issued together
  constexpr int kBatch = 8;
  for (int sp = 1; sp < nsplit; sp += kBatch) {
    double v[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[u][j] = logits[(size_t)min(sp + u, nsplit - 1) * split_stride + (e0 + j < E ? e0 + j : 0)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (sp + u < nsplit) l[j] += v[u][j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + j;
    const bool in = e < E;
    s[j] = SCORES ? l[j] : 1.0 / (1.0 + exp(-l[j]));
    sb[j] = in ? s[j] + (double)bv[j] : -INFINITY;
  }
  // ---- group scores and kept groups ------------------------------------
  const int L = per / 4;  // lanes per group when groups are whole lanes
  const bool lane_groups = (per % 4 == 0) && L >= 1 && L <= 64 && (L & (L - 1)) == 0;
  bool keep_j[4];
  if (lane_groups) {
    // local top-2 of four, then merge across the group's lanes
    double m1 = dmax(sb[0], sb[1]), m2 = dmin(sb[0], sb[1]);
    merge_top2(m1, m2, dmax(sb[2], sb[3]), dmin(sb[2], sb[3]));
    if (L >= 2) top2_dpp<kDppXor1>(m1, m2);
    if (L >= 4) top2_dpp<kDppXor2>(m1, m2);
    if (L >= 8) top2_dpp<kDppHalfMirror>(m1, m2);
    if (L >= 16) top2_dpp<kDppMirror>(m1, m2);
    if (L >= 32) top2_swap<16>(m1, m2);
    if (L >= 64) top2_swap<32>(m1, m2);
    const double gmine = m1 + m2;
    const int gidx = lane / L;
    // every lane ranks its own group against the G group scores: up to 16
    // read straight from the groups' first lanes, more through LDS
    int r = 0;
    if (G <= 16) {
      for (int g = 0; g < G; ++g) {
        const double o = readlane_d(gmine, g * L);
        r += (o > gmine || (o == gmine && g < gidx)) ? 1 : 0;
      }
    } else {
      wave_lds_sync();  // a previous call's reads of `sc` come first
      if (lane % L == 0) sc.gs[gidx] = gmine;
      wave_lds_sync();
      for (int g = 0; g < G; g += 2) {
        const double2 o2 = *reinterpret_cast<const double2*>(&sc.gs[g]);
        r += (o2.x > gmine || (o2.x == gmine && g < gidx)) ? 1 : 0;
        r += (g + 1 < G && (o2.y > gmine || (o2.y == gmine && g + 1 < gidx))) ? 1 : 0;
      }
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
  // Keys are the order-preserving integer images of s'; experts outside the
  // kept groups get key 0, below every score.
  uint64_t ck[4];
  double cs[4];
  int cj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ck[j] = (keep_j[j] && e0 + j < E) ? okey(sb[j]) : 0ull;
    cs[j] = s[j];
    cj[j] = e0 + j;
  }
  auto cswap = [&](int a, int b) {
    // keep (ck[a], cj[a]) ahead of (ck[b], cj[b]): key descending, id
    // ascending (a sorting network is not stable, so the id decides ties)
    const bool sw = ck[b] > ck[a] || (ck[b] == ck[a] && cj[b] < cj[a]);
    const uint64_t tk = sw ? ck[b] : ck[a];
    const double ts = sw ? cs[b] : cs[a];
    const int tj = sw ? cj[b] : cj[a];
    ck[b] = sw ? ck[a] : ck[b];
    cs[b] = sw ? cs[a] : cs[b];
    cj[b] = sw ? cj[a] : cj[b];
    ck[a] = tk;
    cs[a] = ts;
    cj[a] = tj;
  };
  cswap(0, 1);
  cswap(2, 3);
  cswap(0, 2);
  cswap(1, 3);
  cswap(1, 2);
  // ---- top_k rounds -------------------------------------------------------
  // Each round takes the wave maximum of the lanes' head keys, first on their
  // high 32 bits; lanes tied there are settled on the low 32 bits (rare).  The
  // lowest lane holding the maximum wins, which is also the lowest expert id.
  // The winning lane shifts its list.  No lane branches: every step is a
  // select.
  int my_id = 0;
  double my_s = 0.0;
  for (int rr = 0; rr < K; ++rr) {
    const uint32_t hi = (uint32_t)(ck[0] >> 32), lo = (uint32_t)ck[0];
    const uint32_t mhi = wave_max_u32(hi);
    uint64_t hit = __ballot(hi == mhi);
    if (__popcll(hit) > 1) {
      const uint32_t mlo = wave_max_u32(hi == mhi ? lo : 0u);
      hit = __ballot(hi == mhi && lo == mlo);
    }
    const int wl = hit ? (int)__builtin_ctzll(hit) : 0;
    const int wid = __builtin_amdgcn_readlane(cj[0], wl);
    const double ws = readlane_d(cs[0], wl);
    my_id = lane == rr ? wid : my_id;
    my_s = lane == rr ? ws : my_s;
    const bool take = lane == wl;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      ck[j] = take ? ck[j + 1] : ck[j];
      cs[j] = take ? cs[j + 1] : cs[j];
      cj[j] = take ? cj[j + 1] : cj[j];
    }
    ck[3] = take ? 0ull : ck[3];
  }
  my_id = my_id < E ? my_id : 0;
  // ---- ascending order and weights ---------------------------------------
  // pick j's id sits in lane j (K <= 16)
  rank = 0;
  for (int j = 0; j < K; ++j) {
    const int o = __builtin_amdgcn_readlane(my_id, j);
    rank += (o < my_id || (o == my_id && j < lane)) ? 1 : 0;
  }
  const double total = wave_sum(lane < K ? my_s : 0.0);
  id = my_id;
  n_kept = K;
  if (top_p > 0.0f && top_p < 1.0f) {
    // share order: picks with a larger score, or an equal one and a lower id,
    // come first; the running sum of shares in that order, one pick at a
    // time, decides how many stay
    int pos = 0;
    for (int j = 0; j < K; ++j) {
      const double o = readlane_d(my_s, j);
      const int oid = __builtin_amdgcn_readlane(my_id, j);
      pos += (j != lane && (o > my_s || (o == my_s && oid < my_id))) ? 1 : 0;
    }
    const double share = my_s / total;
    double csum = 0.0;
    int keep = K;
    for (int q = 0; q < K; ++q) {
      const uint64_t at = __ballot(lane < K && pos == q);
      csum += readlane_d(share, at ? (int)__builtin_ctzll(at) : 0);
      if (keep == K && csum >= (double)top_p) keep = q + 1;
    }
    const bool kept = lane < K && pos < keep;
    const double total_kept = wave_sum(kept ? my_s : 0.0);
    // ascending id order among the kept picks; the dropped ones after them
    // (in lane order)
    const uint64_t kept_mask = __ballot(kept);
    int nr = 0;
    for (int j = 0; j < K; ++j) {
      const int oid = __builtin_amdgcn_readlane(my_id, j);
      const bool ok = (kept_mask >> j) & 1ull;
      nr += kept ? ((ok && oid < my_id) ? 1 : 0) : ((!ok && j < lane) ? 1 : 0);
    }
    rank = kept ? nr : keep + nr;
    id = kept ? my_id : -1;
    w = kept ? (float)(my_s / total_kept * (double)rsf) : 0.0f;
    n_kept = keep;
    return;
  }
  w = (float)(my_s / total * (double)rsf);
}

}  // namespace qmoe
