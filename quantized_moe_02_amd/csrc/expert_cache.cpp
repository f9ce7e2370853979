// Expert streaming from host memory into HBM slots (moe_cache_* and
// moe_layer_cached in include/qmoe.h).
//
// Page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section "Cara kerja
// eksekusi MoE berbasis streaming disk": the routed experts stay in a slow
// tier and are brought in through a per-layer LRU cache with an optional
// pinned hot store; section "Fitur utama yang diimplementasikan": readahead of
// the next expert block while the current one is multiplied, and a router
// lookahead that prefetches.  The slow tier here is page-locked host RAM, the
// fast one the device's HBM; copies are DMA (hipMemcpyAsync) on the caller's
// streams.
//
// A layer call routes on the device, waits for the routing on the host (the
// only synchronisation), lets the slot policy place the missing experts,
// enqueues their copies, then maps each pick's expert id to its slot and runs
// the permutation, the expert FFNs over the slot arrays, the shared expert and
// the combine -- the split path of moe_layer with E replaced by the slots.
//
// Ordering.  Every slot write must follow the kernels that read the slot
// before.  A layer call first makes its stream wait for the latest layer call
// and the latest prefetch (events), then synchronises after routing: from
// there on nothing else in flight touches a slot, so its own copies go on its
// stream.  A prefetch may run beside the latest layer call's kernels (that is
// its purpose), so it never evicts that call's experts (a stamp bound); every
// older call has finished, since the latest one synchronised after waiting for
// them.  A prefetch waits for the previous prefetch, and the next layer call
// waits for it.
#include <algorithm>
#include <cstdint>
#include <limits>
#include <new>
#include <vector>

#include "expert_cache_policy.h"
#include "qmoe_internal.h"

using namespace qmoe;

struct moe_expert_cache {
  moe_config cfg;
  int n_slots;
  moe_qexperts host;    // E experts, host pointers
  moe_qexperts slots;   // n_slots experts, device pointers
  SlotPolicy policy;
  moe_cache_stats stats{};
  uint64_t last_call_stamp = 0;   // policy clock of the latest layer call (0: none)
  bool have_events = false;
  bool call_recorded = false, prefetch_recorded = false;
  int device = -1;
  hipEvent_t ev_call = nullptr;       // after the latest layer call's kernels
  hipEvent_t ev_prefetch = nullptr;   // after the latest prefetch's copies
  std::vector<int32_t> ids_host;

  moe_expert_cache(const moe_config& c, int s, const moe_qexperts& h, const moe_qexperts& d)
      : cfg(c), n_slots(s), host(h), slots(d), policy(c.n_routed_experts, s) {}
};

namespace {

// Bytes of one expert's codes, scales and tensor scale in one projection.
struct ProjBytes {
  size_t q, s, g;
};

ProjBytes proj_bytes(int wfmt, int N, int K) {
  ProjBytes b;
  b.q = (size_t)N * K * wfmt_bits(wfmt) / 8;
  if (wfmt_row(wfmt))
    b.s = (size_t)N * sizeof(float);
  else
    b.s = wfmt == MOE_WFMT_NVFP4 ? (size_t)N * K / 16 : (size_t)N * (K / 32) * 2;
  b.g = wfmt == MOE_WFMT_NVFP4 ? sizeof(float) : 0;
  return b;
}

size_t expert_bytes(const moe_config& c) {
  const ProjBytes gu = proj_bytes(c.wfmt, c.moe_inter, c.hidden);
  const ProjBytes d = proj_bytes(c.wfmt, c.hidden, c.moe_inter);
  return 2 * (gu.q + gu.s + gu.g) + d.q + d.s + d.g;
}

hipError_t copy_proj(const moe_qproj& from, const moe_qproj& to, int e, int slot, ProjBytes b,
                     hipStream_t s) {
  hipError_t r;
  if ((r = hipMemcpyAsync(const_cast<uint8_t*>(to.q) + slot * b.q, from.q + e * b.q, b.q,
                          hipMemcpyHostToDevice, s)) != hipSuccess)
    return r;
  if ((r = hipMemcpyAsync(static_cast<uint8_t*>(const_cast<void*>(to.scale)) + slot * b.s,
                          static_cast<const uint8_t*>(from.scale) + e * b.s, b.s,
                          hipMemcpyHostToDevice, s)) != hipSuccess)
    return r;
  if (b.g)
    r = hipMemcpyAsync(const_cast<float*>(to.gscale) + slot, from.gscale + e, b.g,
                       hipMemcpyHostToDevice, s);
  return r;
}

// Copies expert e from the host store into slot `slot` on stream s.
hipError_t load_expert(moe_expert_cache* c, int e, int slot, hipStream_t s) {
  const ProjBytes gu = proj_bytes(c->cfg.wfmt, c->cfg.moe_inter, c->cfg.hidden);
  const ProjBytes d = proj_bytes(c->cfg.wfmt, c->cfg.hidden, c->cfg.moe_inter);
  hipError_t r;
  if ((r = copy_proj(c->host.gate, c->slots.gate, e, slot, gu, s)) != hipSuccess) return r;
  if ((r = copy_proj(c->host.up, c->slots.up, e, slot, gu, s)) != hipSuccess) return r;
  return copy_proj(c->host.down, c->slots.down, e, slot, d, s);
}

// Creates the events on the first HIP-using call; later calls must run on
// the same device.
moe_status ensure_events(moe_expert_cache* c) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (c->have_events) return dev == c->device ? MOE_OK : MOE_ERR_INVALID_ARG;
  if (hipEventCreateWithFlags(&c->ev_call, hipEventDisableTiming) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreateWithFlags(&c->ev_prefetch, hipEventDisableTiming) != hipSuccess) {
    (void)hipEventDestroy(c->ev_call);
    c->ev_call = nullptr;
    return MOE_ERR_HIP;
  }
  c->device = dev;
  c->have_events = true;
  return MOE_OK;
}

// Makes `s` wait for the latest prefetch's copies (if any were recorded).
hipError_t wait_prefetch(const moe_expert_cache* c, hipStream_t s) {
  return c->prefetch_recorded ? hipStreamWaitEvent(s, c->ev_prefetch, 0) : hipSuccess;
}

// The policy's stamp bound for loads beside the latest layer call's kernels.
uint64_t protect_latest_call(const moe_expert_cache* c) {
  return c->last_call_stamp ? c->last_call_stamp : std::numeric_limits<uint64_t>::max();
}

moe_status check_expert_list(const moe_expert_cache* c, const int32_t* experts, int32_t n) {
  if (n < 0 || (n > 0 && !experts)) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= c->cfg.n_routed_experts) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_cache_create(const moe_config* cfg, int32_t n_slots,
                            const moe_qexperts* host_store, const moe_qexperts* slots,
                            moe_expert_cache** cache) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  *cache = nullptr;
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if (n_slots < 1 || n_slots > cfg->n_routed_experts) return MOE_ERR_INVALID_ARG;
  if ((s = check_experts(host_store, cfg->wfmt)) != MOE_OK) return s;
  if ((s = check_experts(slots, cfg->wfmt)) != MOE_OK) return s;
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache(*cfg, n_slots, *host_store, *slots);
  if (!c) return MOE_ERR_UNSUPPORTED;
  *cache = c;
  return MOE_OK;
}

moe_status moe_cache_destroy(moe_expert_cache* cache) {
  if (!cache) return MOE_OK;
  if (cache->have_events) {
    (void)hipEventDestroy(cache->ev_call);
    (void)hipEventDestroy(cache->ev_prefetch);
  }
  delete cache;
  return MOE_OK;
}

moe_status moe_cache_get_stats(const moe_expert_cache* cache, moe_cache_stats* stats) {
  if (!cache || !stats) return MOE_ERR_INVALID_ARG;
  *stats = cache->stats;
  stats->evictions = cache->policy.evictions();
  return MOE_OK;
}

moe_status moe_cache_slot_of(const moe_expert_cache* cache, int32_t expert, int32_t* slot) {
  if (!cache || !slot) return MOE_ERR_INVALID_ARG;
  if (expert < 0 || expert >= cache->cfg.n_routed_experts) return MOE_ERR_INVALID_ARG;
  *slot = cache->policy.slot_of(expert);
  return MOE_OK;
}

moe_status moe_cache_unpin_all(moe_expert_cache* cache) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  cache->policy.unpin_all();
  return MOE_OK;
}

moe_status moe_cache_prefetch(moe_expert_cache* cache, const int32_t* experts, int32_t n,
                              int32_t* n_loaded, hipStream_t stream) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  moe_status s;
  if ((s = check_expert_list(cache, experts, n)) != MOE_OK) return s;
  if (n_loaded) *n_loaded = 0;
  if (n == 0) return MOE_OK;
  if ((s = ensure_events(cache)) != MOE_OK) return s;
  if (wait_prefetch(cache, stream) != hipSuccess) return MOE_ERR_HIP;
  // one expert at a time, in the caller's priority order: those that find no
  // slot are skipped
  int32_t loaded = 0;
  std::vector<std::pair<int, int>> loads;
  for (int32_t i = 0; i < n; ++i) {
    int hits = 0;
    if (!cache->policy.acquire({experts[i]}, protect_latest_call(cache), loads, hits)) continue;
    for (const auto& l : loads) {
      if (load_expert(cache, l.first, l.second, stream) != hipSuccess) return MOE_ERR_HIP;
      ++loaded;
      ++cache->stats.prefetched;
      cache->stats.bytes_loaded += expert_bytes(cache->cfg);
    }
  }
  if (hipEventRecord(cache->ev_prefetch, stream) != hipSuccess) return MOE_ERR_HIP;
  cache->prefetch_recorded = true;
  if (n_loaded) *n_loaded = loaded;
  return MOE_OK;
}

moe_status moe_cache_pin(moe_expert_cache* cache, const int32_t* experts, int32_t n,
                         hipStream_t stream) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  moe_status s;
  if ((s = check_expert_list(cache, experts, n)) != MOE_OK) return s;
  if (n == 0) return MOE_OK;
  std::vector<int> need(experts, experts + n);
  // all or nothing: the policy changes nothing if they do not all fit
  {
    SlotPolicy probe = cache->policy;
    std::vector<std::pair<int, int>> loads;
    int hits = 0;
    if (!probe.acquire(need, protect_latest_call(cache), loads, hits)) return MOE_ERR_UNSUPPORTED;
  }
  if ((s = ensure_events(cache)) != MOE_OK) return s;
  if (wait_prefetch(cache, stream) != hipSuccess) return MOE_ERR_HIP;
  std::vector<std::pair<int, int>> loads;
  int hits = 0;
  cache->policy.acquire(need, protect_latest_call(cache), loads, hits);
  for (const auto& l : loads) {
    if (load_expert(cache, l.first, l.second, stream) != hipSuccess) return MOE_ERR_HIP;
    ++cache->stats.prefetched;
    cache->stats.bytes_loaded += expert_bytes(cache->cfg);
  }
  cache->policy.pin(need);
  if (hipEventRecord(cache->ev_prefetch, stream) != hipSuccess) return MOE_ERR_HIP;
  cache->prefetch_recorded = true;
  return MOE_OK;
}

moe_status moe_layer_cached(moe_expert_cache* cache, int32_t T, const uint16_t* x,
                            const float* router_w, const float* bias, const moe_qexperts* shared,
                            void* y, int32_t out_dtype, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  const moe_config& cfg = cache->cfg;
  moe_status s;
  if ((s = check_layer_args(&cfg, T, x, router_w, &cache->slots, shared, y, out_dtype)) != MOE_OK)
    return s;
  if ((s = check_ws(cfg, T, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const bool has_shared = cfg.n_shared_experts == 1;
  const int ldh = pad_k(std::max(cfg.moe_inter, has_shared ? cfg.shared_inter : 0));
  const int K = cfg.top_k, S = cache->n_slots;
  const int P = T * K;
  const bool small = T <= kDecodeMaxTokens;
  if (!small && !gemm_fits(T, (int64_t)P + (has_shared ? T : 0), pad_k(cfg.hidden), ldh))
    return MOE_ERR_UNSUPPORTED;
  if ((s = ensure_events(cache)) != MOE_OK) return s;

  const Workspace w = carve_workspace(cfg, T, ws);
  int32_t* ids = topk_ids_out ? topk_ids_out : w.ids;
  float* tw = topk_w_out ? topk_w_out : w.tw;
  // slots may still be read by the previous call or written by a prefetch
  if ((cache->call_recorded && hipStreamWaitEvent(stream, cache->ev_call, 0) != hipSuccess) ||
      wait_prefetch(cache, stream) != hipSuccess)
    return MOE_ERR_HIP;
  RouteArgs ra{x, router_w, bias, ids, tw, w.logits, T, cfg.hidden, cfg.n_routed_experts,
               cfg.n_group, cfg.topk_group, K, cfg.routed_scaling_factor, w.flags,
               cfg.expert_top_p};
  if (launch_route(ra, stream) != hipSuccess) return MOE_ERR_HIP;
  cache->ids_host.resize(P);
  if (hipMemcpyAsync(cache->ids_host.data(), ids, (size_t)P * sizeof(int32_t),
                     hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_ERR_HIP;

  std::vector<int> need;
  need.reserve(P);
  for (int32_t e : cache->ids_host) {
    if (e >= cfg.n_routed_experts) return MOE_ERR_HIP;   // cannot come from the router
    if (e >= 0) need.push_back(e);
  }
  std::vector<std::pair<int, int>> loads;
  int hits = 0;
  if (!cache->policy.acquire(need, std::numeric_limits<uint64_t>::max(), loads, hits))
    return MOE_ERR_UNSUPPORTED;
  for (const auto& l : loads)
    if (load_expert(cache, l.first, l.second, stream) != hipSuccess) return MOE_ERR_HIP;
  ++cache->stats.calls;
  cache->stats.hits += hits;
  cache->stats.misses += loads.size();
  cache->stats.bytes_loaded += loads.size() * expert_bytes(cfg);
  cache->last_call_stamp = cache->policy.clock();

  SlotMap map;
  for (int e = 0; e < cfg.n_routed_experts; ++e) map.slot[e] = cache->policy.slot_of(e);
  if (launch_remap_ids(ids, w.cache_ids, P, map, stream) != hipSuccess) return MOE_ERR_HIP;
  const ExpertSet rset = expert_set(cache->slots, cfg.moe_inter);
  const ExpertSet sset = has_shared ? expert_set(*shared, cfg.shared_inter) : ExpertSet{};
  if (run_ffn_combine(cfg, T, x, w, w.cache_ids, S, rset, has_shared, sset, tw, y,
                      out_dtype == MOE_OUT_BF16, small, stream, nullptr) != hipSuccess)
    return MOE_ERR_HIP;
  if (hipEventRecord(cache->ev_call, stream) != hipSuccess) return MOE_ERR_HIP;
  cache->call_recorded = true;
  return MOE_OK;
}

}  // extern "C"
