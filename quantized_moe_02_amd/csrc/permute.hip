// Batch-union permutation (page "Show HN: Menjalankan GLM 5.2 di komputer
// lambat", section "Fitur utama": the unique experts of a batch are read once
// and applied to every position routed to them).
//
// Stable counting sort of the P = T*k picks by expert id, order within an
// expert by pick index p = t*k + i.  The tokens are cut into B <= 128 chunks:
//   perm_hist     one workgroup per chunk: the chunk's count of each expert
//   perm_scan     one workgroup: per expert, the exclusive prefix of the chunk
//                 counts (the chunk's first slot in that expert's run), the
//                 expert offsets, and the active experts in ascending order
//   perm_scatter  one wave per chunk walks its picks in order, 64 at a time; a
//                 pick's slot is its expert's cursor plus its rank among the
//                 equal picks of the step, after which the cursor advances
// Counts are integers, so the LDS atomics leave nothing order-dependent.
// Up to 8192 picks, perm_small does all three steps in one workgroup.
#include "qmoe_device.h"

namespace qmoe {
namespace {

constexpr int kMaxE = 256;
constexpr int kMaxChunks = 128;

__global__ void __launch_bounds__(256) perm_hist_kernel(const int32_t* __restrict__ ids,
                                                        int32_t* __restrict__ hist, int T, int K,
                                                        int E, int chunk) {
  __shared__ int h[kMaxE];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < kMaxE; e += 256) h[e] = 0;
  __syncthreads();
  const int p0 = b * chunk * K, p1 = min(T, (b + 1) * chunk) * K;
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const int e = ids[p];
    if (e >= 0) atomicAdd(&h[e], 1);   // -1: a pick the adaptive top-p dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)b * E + e] = h[e];
}

constexpr int kScanGroups = 4;                         // chunk ranges scanned side by side
constexpr int kScanPer = kMaxChunks / kScanGroups;     // chunks per range

// 1024 threads: thread (g, e) holds the counts of expert e in chunk range g
// in registers (all loads in flight at once), so hist is read and written
// once each.
__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ n_active, int E,
                                                         int nb) {
  __shared__ int gtot[kScanGroups][kMaxE];
  __shared__ int cnt[kMaxE], act[kMaxE];
  const int e = threadIdx.x % kMaxE;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kMaxE);   // one range per wave
  const int per = (nb + kScanGroups - 1) / kScanGroups;
  const int b0 = g * per, nloc = max(0, min(nb, b0 + per) - b0);
  // one VGPR offset per lane, the chunk row in the scalar offset
  const rsrc_t rh = make_rsrc(hist, (uint32_t)(nb * E * 4));
  const uint32_t voff = (uint32_t)min(e, E - 1) * 4;
  int v[kScanPer];
#pragma unroll
  for (int j = 0; j < kScanPer; ++j)
    if (j < per)
      v[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rh, voff, (uint32_t)(min(b0 + j, nb - 1) * E * 4), 0);
  int run = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (j < per) {
      const int c = (j < nloc && e < E) ? v[j] : 0;
      v[j] = run;   // exclusive prefix within the range
      run += c;
    }
  }
  gtot[g][e] = run;
  __syncthreads();
  int gpre = 0, tot = 0;
#pragma unroll
  for (int r = 0; r < kScanGroups; ++r) {
    const int t = gtot[r][e];
    gpre += r < g ? t : 0;
    tot += t;
  }
  if (g == 0) {
    cnt[e] = tot;
    act[e] = tot > 0 ? 1 : 0;
  }
  __syncthreads();
  // inclusive scans over the 256 buckets (Hillis-Steele in LDS)
  for (int d = 1; d < kMaxE; d <<= 1) {
    int c = 0, a = 0;
    if (g == 0 && e >= d) {
      c = cnt[e - d];
      a = act[e - d];
    }
    __syncthreads();
    if (g == 0) {
      cnt[e] += c;
      act[e] += a;
    }
    __syncthreads();
  }
  const int excl = cnt[e] - tot;
  if (e < E) {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
      if (j < nloc)
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(excl + gpre + v[j]), rh, voff,
                                              (uint32_t)((b0 + j) * E * 4), 0);
    if (g == 0) {
      offsets[e] = excl;
      if (tot > 0) active[act[e] - 1] = e;
    }
  }
  if (threadIdx.x == kMaxE - 1) {
    offsets[E] = cnt[kMaxE - 1];
    n_active[0] = act[kMaxE - 1];
  }
}

// One wave per chunk, 64 consecutive picks per step.  Lanes holding the same
// expert find each other with one ballot per bit of the id; a pick's slot is
// its expert's cursor plus the number of equal picks on lower lanes, and the
// highest of them advances the cursor.
__global__ void __launch_bounds__(64) perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ sorted_token,
                                                          int32_t* __restrict__ inv_perm, int T,
                                                          int K, int E, int chunk) {
  __shared__ int cur[kMaxE];
  const int b = blockIdx.x, lane = threadIdx.x;
  {
    int v[kMaxE / 64];
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) v[j] = hist[(size_t)b * E + min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) cur[lane + 64 * j] = v[j];
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (1ull << lane) - 1;
  const int p0 = b * chunk * K, p1 = min(T, (b + 1) * chunk) * K;
  for (int q0 = p0; q0 < p1; q0 += 64 * 8) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ids[min(q0 + 64 * j + lane, p1 - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (q0 + 64 * j >= p1) break;
      const int p = q0 + 64 * j + lane;
      const bool in = p < p1;
      const bool valid = in && v[j] >= 0;   // -1: dropped pick, no slot
      const int e = valid ? v[j] : 0;
      if (in && !valid) inv_perm[p] = -1;
      uint64_t m = __builtin_amdgcn_ballot_w64(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t bb = __builtin_amdgcn_ballot_w64(set);
        m &= set ? bb : ~bb;
      }
      const int rank = __popcll(m & below), cnt = __popcll(m);
      const int base = cur[e];
      if (valid) {
        inv_perm[p] = base + rank;
        sorted_token[base + rank] = p / K;
        if (rank == cnt - 1) cur[e] = base + cnt;
      }
    }
  }
}

// Small batches (P <= kSmallP picks): the same stable counting sort in one
// workgroup of 16 waves, wave w taking the w-th chunk of picks, so that the
// three launches above become one.  Counts per (chunk, expert) in LDS; each
// chunk's first slot per expert is the expert's offset plus the counts of
// the earlier chunks; the scatter is perm_scatter's, one wave per chunk.
constexpr int kSmallWaves = 16;
constexpr int kSmallP = 8192;

__global__ void __launch_bounds__(64 * kSmallWaves) perm_small_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ active, int32_t* __restrict__ n_active, int P,
    int K, int E) {
  __shared__ int cnt[kSmallWaves][kMaxE];
  __shared__ int tot[kMaxE], act[kMaxE];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = (P + kSmallWaves - 1) / kSmallWaves;
  const int p0 = min(P, w * chunk), p1 = min(P, p0 + chunk);
  for (int i = threadIdx.x; i < kSmallWaves * kMaxE; i += 64 * kSmallWaves) (&cnt[0][0])[i] = 0;
  __syncthreads();
  for (int p = p0 + lane; p < p1; p += 64) {
    const int e = ids[p];
    if (e >= 0) atomicAdd(&cnt[w][e], 1);   // -1: a pick the adaptive top-p dropped
  }
  __syncthreads();
  // per expert: exclusive prefix over the chunks, and the total
  if (threadIdx.x < kMaxE) {
    const int e = threadIdx.x;
    int run = 0;
#pragma unroll
    for (int c = 0; c < kSmallWaves; ++c) {
      const int v = cnt[c][e];
      cnt[c][e] = run;
      run += v;
    }
    tot[e] = e < E ? run : 0;
    act[e] = e < E && run > 0 ? 1 : 0;
  }
  __syncthreads();
  // inclusive scans of the totals and of the active flags over the experts
  for (int d = 1; d < kMaxE; d <<= 1) {
    int c = 0, a = 0;
    if (threadIdx.x < kMaxE && (int)threadIdx.x >= d) {
      c = tot[threadIdx.x - d];
      a = act[threadIdx.x - d];
    }
    __syncthreads();
    if (threadIdx.x < kMaxE) {
      tot[threadIdx.x] += c;
      act[threadIdx.x] += a;
    }
    __syncthreads();
  }
  if (threadIdx.x < kMaxE) {
    const int e = threadIdx.x;
    const int incl = tot[e];
    const int excl = e > 0 ? tot[e - 1] : 0;
#pragma unroll
    for (int c = 0; c < kSmallWaves; ++c) cnt[c][e] += excl;
    if (e < E) {
      offsets[e] = excl;
      if (incl > excl) active[act[e] - 1] = e;
    }
    if (e == kMaxE - 1) {
      offsets[E] = incl;
      n_active[0] = act[e];
    }
  }
  __syncthreads();
  // scatter: chunk w in pick order, 64 picks at a time
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (1ull << lane) - 1;
  for (int q = p0; q < p1; q += 64) {
    const int p = q + lane;
    const int ev = p < p1 ? ids[p] : 0;
    const bool valid = p < p1 && ev >= 0;   // -1: dropped pick, no slot
    const int e = valid ? ev : 0;
    if (p < p1 && !valid) inv_perm[p] = -1;
    uint64_t m = __builtin_amdgcn_ballot_w64(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t bb = __builtin_amdgcn_ballot_w64(set);
      m &= set ? bb : ~bb;
    }
    const int rank = __popcll(m & below), n = __popcll(m);
    const int base = cnt[w][e];
    if (valid) {
      inv_perm[p] = base + rank;
      sorted_token[base + rank] = p / K;
      if (rank == n - 1) cnt[w][e] = base + n;
    }
  }
}

// Expert id -> cache slot of every pick (the map travels as a kernel argument).
__global__ void __launch_bounds__(256) remap_ids_kernel(const int32_t* __restrict__ ids,
                                                        int32_t* __restrict__ out, int P, SlotMap map) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= P) return;
  const int e = ids[i];
  out[i] = e < 0 ? -1 : map.slot[e];
}

}  // namespace

hipError_t launch_remap_ids(const int32_t* ids, int32_t* out, int P, const SlotMap& map,
                            hipStream_t s) {
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(remap_ids_kernel, dim3((P + 255) / 256), dim3(256), 0, s, ids, out, P, map);
  return hipGetLastError();
}

int permute_chunk(int T) { return std::max(64, (T + kMaxChunks - 1) / kMaxChunks); }
size_t permute_hist_ints(int T, int E) {
  const int c = permute_chunk(T);
  return (size_t)((T + c - 1) / c) * E;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  if ((long)a.T * a.K <= kSmallP) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(64 * kSmallWaves), 0, s, a.ids, a.offsets,
                       a.sorted_token, a.inv_perm, a.active, a.n_active, a.T * a.K, a.K, a.E);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && tr) e = tr->mark("permute");
    return e;
  }
  const int chunk = permute_chunk(a.T);
  const int nb = (a.T + chunk - 1) / chunk;
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), 0, s, a.ids, a.hist, a.T, a.K, a.E, chunk);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanGroups * kMaxE), 0, s, a.hist, a.offsets, a.active,
                     a.n_active, a.E, nb);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(64), 0, s, a.ids, a.hist, a.sorted_token,
                     a.inv_perm, a.T, a.K, a.E, chunk);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && tr) e = tr->mark("permute");
  return e;
}

}  // namespace qmoe
