// Batch-union permutation (page "Show HN: Menjalankan GLM 5.2 di komputer
// lambat", section "Fitur utama": the unique experts of a batch are read once
// and applied to every position routed to them).
//
// Stable counting sort of the P = T*k picks by expert id.  One workgroup of
// 1024 threads: an LDS histogram, an exclusive scan over the E <= 256 buckets,
// then the picks in chunks of 1024 in pick order.  Inside a chunk a pick's
// rank among equal keys is (equal keys in earlier waves of the chunk) + (equal
// keys in lower lanes of its own wave); the latter comes from eight ballots
// over the bits of the key.
#include "qmoe_device.h"

namespace qmoe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kMaxE = 256;

__global__ void __launch_bounds__(kPermThreads) permute_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int P, int K, int E) {
  __shared__ int count[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int wcount[kPermWaves][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;

  for (int e = tid; e < kMaxE; e += kPermThreads) count[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) atomicAdd(&count[ids[p]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      cursor[e] = run;
      if (count[e] > 0) active[na++] = e;
      run += count[e];
    }
    offsets[E] = run;
    n_active[0] = na;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kPermThreads) {
    for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&wcount[0][0])[i] = 0;
    __syncthreads();
    const int p = base + tid;
    const bool has = p < P;
    const int e = has ? ids[p] : 0;
    // lanes of this wave holding the same key
    uint64_t peers = __ballot(has);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t ones = __ballot(has && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt_mask);
    if (has && rank == 0) wcount[wv][e] = __popcll(peers);
    __syncthreads();
    if (has) {
      int before = 0;
      for (int w2 = 0; w2 < wv; ++w2) before += wcount[w2][e];
      const int pos = cursor[e] + before + rank;
      sorted_token[pos] = p / K;
      inv_perm[p] = pos;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kPermThreads) {
      int tot = 0;
      for (int w2 = 0; w2 < kPermWaves; ++w2) tot += wcount[w2][e2];
      cursor[e2] += tot;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s, Tracer* tr) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, a.ids, a.offsets,
                     a.sorted_token, a.inv_perm, a.active, a.n_active, a.T * a.K, a.K, a.E);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && tr) e = tr->mark("permute");
  return e;
}

}  // namespace qmoe
