// Router: DeepSeek-V3-style sigmoid scores, bias-corrected group-limited top-k
// ("noaux_tc"), renormalised weights times routed_scaling_factor
// (page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section "Fitur utama").
//
// Two kernels:
//   route_logits  l[t][e] = sum_h x[t][h] * Wr[e][h] in float64 on the matrix
//                 cores (v_mfma_f64_16x16x4_f64).  A bf16 times an fp32 is
//                 exact in float64, so the only rounding is the float64 sum.
//                 One wave per 32 tokens x 64 experts x slice of the hidden
//                 dimension; with several slices (few tokens) each writes its
//                 partial sums and route_select adds them in slice order.
//                 For at most four tokens the small-batch router kernel
//                 (one block per expert, float64 FMAs, the sigmoid applied)
//                 takes its place: the matrix-core tiles hold 32 tokens, and
//                 the slices' partial sums cost the selection a long read.
//   route_select  one wave per token (select_token.h).
#include <algorithm>

#include "select_token.h"

namespace qmoe {
namespace {

typedef double double4v __attribute__((ext_vector_type(4)));

constexpr int kLogitTok = 32;   // tokens per wave (two 16-row tiles)
constexpr int kLogitExp = 64;   // experts per wave (four 16-column tiles)

// v_mfma_f64_16x16x4_f64: A lane l holds row l%16, k = l/16; B lane l holds
// column l%16, k = l/16; D lane l holds rows l/16 + 4i (i = 0..3) of column
// l%16.  Rows are tokens and columns experts, so that the 16 lanes of a row
// group store 16 consecutive logits.  Within a 32-input block, lane group q
// supplies inputs 8q..8q+7 over the block's 8 MFMA steps (K order is free).
__global__ void __launch_bounds__(256) route_logits_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ Wr,
                                                           double* __restrict__ logits, int T,
                                                           int H, int E, int kb_per_split) {
  const int lane = threadIdx.x & 63;
  const int tg = blockIdx.x * 4 + (threadIdx.x >> 6);
  logits += (size_t)blockIdx.z * T * E;
  const int kb0 = blockIdx.z * kb_per_split;
  const int kb1 = min(H / 32, kb0 + kb_per_split);
  if (tg * kLogitTok >= T) return;
  const int t0 = tg * kLogitTok, e0 = blockIdx.y * kLogitExp;
  const int r = lane & 15, q = lane >> 4;
  // rows and columns past the end are clamped (their results are not stored)
  const uint16_t* xp[2];
  const float* wp[4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) xp[rt] = x + (size_t)min(t0 + 16 * rt + r, T - 1) * H + q * 8;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wp[ct] = Wr + (size_t)min(e0 + 16 * ct + r, E - 1) * H + q * 8;

  double4v acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = double4v{0.0, 0.0, 0.0, 0.0};

  uint4 xa[2], xn[2];
  float4 wa[4][2], wn[4][2];
  auto load = [&](int kb, uint4 (&xv)[2], float4 (&wv)[4][2]) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) xv[rt] = *reinterpret_cast<const uint4*>(xp[rt] + kb * 32);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      wv[ct][0] = *reinterpret_cast<const float4*>(wp[ct] + kb * 32);
      wv[ct][1] = *reinterpret_cast<const float4*>(wp[ct] + kb * 32 + 4);
    }
  };
  load(kb0, xa, wa);
  for (int kb = kb0; kb < kb1; ++kb) {
    if (kb + 1 < kb1) load(kb + 1, xn, wn);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double xd[2], wd[4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const uint32_t w = (&xa[rt].x)[j >> 1];
        xd[rt] = (double)((j & 1) ? bf16_hi(w) : bf16_lo(w));
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) wd[ct] = (double)(&wa[ct][j >> 2].x)[j & 3];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[rt], wd[ct], acc[rt][ct], 0, 0, 0);
    }
    if (kb + 1 < kb1) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) xa[rt] = xn[rt];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        wa[ct][0] = wn[ct][0];
        wa[ct][1] = wn[ct][1];
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int e = e0 + 16 * ct + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * rt + q + 4 * i;
        if (t < T && e < E) logits[(size_t)t * E + e] = acc[rt][ct][i];
      }
    }
}

// SCORES: the input holds sigmoid scores (one slice), else logits in nsplit
// slices.
template <bool SCORES>
__global__ void __launch_bounds__(256) route_select_kernel(const double* __restrict__ logits,
                                                           const float* __restrict__ bias,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ tw, int T, int E,
                                                           int G, int TG, int K, float rsf,
                                                           int nsplit, uint32_t* __restrict__ flags,
                                                           float top_p) {
  __shared__ SelectScratch sc[4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  // moe_layer's flags word: nothing on this path raises one
  if (flags && blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0u;
  if (t >= T) return;
  int id, rank, n_kept;
  float w;
  select_token<SCORES>(logits + (size_t)t * E, bias, E, G, TG, K, rsf, top_p, sc[wv], id, w, rank,
                       n_kept, nsplit, (size_t)T * E);
  if (lane < K) {
    ids[(size_t)t * K + rank] = id;
    tw[(size_t)t * K + rank] = w;
  }
}

// At most four tokens (P = T*k <= 64 picks): the selection and the
// permutation in one workgroup, from the scores of route_scores.  Wave t
// selects token t; every thread then counts, for its experts e (and E), the
// kept picks with a smaller id (offsets[e]); wave 0 sorts the picks, one per
// lane: a ballot per id bit, from the top bit down, leaves each lane the
// lanes holding its expert (eq) and those holding a smaller one (lt), so its
// slot is |lt| plus the equal picks on lower lanes -- by expert, then pick
// order, as the permutation kernels order them.  The outputs are theirs
// (offsets, sorted tokens, inverse permutation, active experts and count).
__global__ void __launch_bounds__(256) route_select_permute_kernel(
    const double* __restrict__ scores, const float* __restrict__ bias, int32_t* __restrict__ ids,
    float* __restrict__ tw, int T, int E, int G, int TG, int K, float rsf, uint32_t* __restrict__ flags,
    float top_p, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ SelectScratch sc[4];
  __shared__ int pid[64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int P = T * K;
  if (flags && threadIdx.x == 0) flags[0] = 0u;
  if (wv < T) {
    int id, rank, n_kept;
    float w;
    select_token<true>(scores + (size_t)wv * E, bias, E, G, TG, K, rsf, top_p, sc[wv], id, w, rank,
                       n_kept);
    if (lane < K) {
      ids[wv * K + rank] = id;   // -1: a pick the adaptive top-p dropped
      tw[wv * K + rank] = w;
      pid[wv * K + rank] = id;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += 256) {
    int c = 0;
    for (int p = 0; p < P; ++p) {
      const int v = pid[p];
      c += (v >= 0 && v < e) ? 1 : 0;
    }
    offsets[e] = c;
  }
  if (wv != 0) return;
  const int pe = lane < P ? pid[lane] : -1;
  const bool have = pe >= 0;
  const int e = have ? pe : 0;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  uint64_t eq = __ballot(have), lt = 0;
  for (int bit = nbits - 1; bit >= 0; --bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t b = __ballot(have && set);
    lt |= set ? (eq & ~b) : 0ull;
    eq &= set ? b : ~b;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const int pos = __popcll(lt) + __popcll(eq & below);
  if (lane < P) inv_perm[lane] = have ? pos : -1;
  if (have) sorted_token[pos] = lane / K;
  const bool first = have && (eq & below) == 0;
  const uint64_t firsts = __ballot(first);
  if (first) active[__popcll(lt & firsts)] = e;
  if (lane == 0) n_active[0] = __popcll(firsts);
}

}  // namespace

bool route_permute_small_ok(int T, int K) { return T >= 1 && T <= kDecodeMaxTokens && T * K <= 64; }

hipError_t launch_route_permute_small(const RouteArgs& a, const PermuteArgs& pa, hipStream_t s,
                                      Tracer* tr) {
  if (!route_permute_small_ok(a.T, a.K)) return hipErrorInvalidValue;
  hipError_t e;
  if ((e = launch_route_scores(a.x, a.router_w, a.logits, a.T, a.H, a.E, s)) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_logits")) != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_permute_kernel, dim3(1), dim3(256), 0, s, a.logits, a.bias, a.ids, a.tw,
                     a.T, a.E, a.G, a.TG, a.K, a.rsf, a.flags, a.top_p, pa.offsets, pa.sorted_token,
                     pa.inv_perm, pa.active, pa.n_active);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_select")) != hipSuccess) return e;
  return hipSuccess;
}

int route_splits(int T, int H, int E) {
  // enough waves to fill the chip, at least 4 K blocks of 32 inputs per wave
  const int waves = ((T + kLogitTok - 1) / kLogitTok) * ((E + kLogitExp - 1) / kLogitExp);
  const int by_waves = (2048 + waves - 1) / waves;
  const int by_k = H / 32 / 4;
  return std::max(1, std::min(by_waves, by_k));
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  hipError_t e;
  if (a.T <= kDecodeMaxTokens) {
    if ((e = launch_route_scores(a.x, a.router_w, a.logits, a.T, a.H, a.E, s)) != hipSuccess) return e;
    if (tr && (e = tr->mark("route_logits")) != hipSuccess) return e;
    hipLaunchKernelGGL(route_select_kernel<true>, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.bias,
                       a.ids, a.tw, a.T, a.E, a.G, a.TG, a.K, a.rsf, 1, a.flags, a.top_p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (tr && (e = tr->mark("route_select")) != hipSuccess) return e;
    return hipSuccess;
  }
  const int groups = (a.T + kLogitTok - 1) / kLogitTok;
  const int S = route_splits(a.T, a.H, a.E);
  const int nkb = a.H / 32;
  const int per = (nkb + S - 1) / S;
  const int S_used = (nkb + per - 1) / per;
  dim3 g1((groups + 3) / 4, (a.E + kLogitExp - 1) / kLogitExp, S_used);
  hipLaunchKernelGGL(route_logits_kernel, g1, dim3(256), 0, s, a.x, a.router_w, a.logits, a.T,
                     a.H, a.E, per);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_logits")) != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel<false>, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.bias,
                     a.ids, a.tw, a.T, a.E, a.G, a.TG, a.K, a.rsf, S_used, a.flags, a.top_p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tr && (e = tr->mark("route_select")) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace qmoe
