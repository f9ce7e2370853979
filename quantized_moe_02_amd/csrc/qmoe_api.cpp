// C-ABI entry points of libqmoe (declared in include/qmoe.h): argument
// validation, workspace layout and kernel dispatch.  Every check runs before
// the first HIP call, so invalid calls leave the device untouched.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->hidden % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (c->moe_inter <= 0 || c->moe_inter % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (c->n_shared_experts != 0 && c->n_shared_experts != 1) return MOE_ERR_INVALID_ARG;
  if (c->n_shared_experts == 1 && (c->shared_inter <= 0 || c->shared_inter % 32 != 0))
    return MOE_ERR_INVALID_ARG;
  if (c->n_routed_experts <= 0 || c->n_group <= 0) return MOE_ERR_INVALID_ARG;
  if (c->n_routed_experts % c->n_group != 0) return MOE_ERR_INVALID_ARG;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_INVALID_ARG;
  const int64_t allowed =
      (int64_t)c->topk_group * (c->n_routed_experts / c->n_group);
  if (c->top_k < 1 || c->top_k > allowed) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->routed_scaling_factor) || !(c->routed_scaling_factor > 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (c->wfmt != MOE_WFMT_INT4_G32_F16 && c->wfmt != MOE_WFMT_NVFP4 && !wfmt_row(c->wfmt))
    return MOE_ERR_INVALID_ARG;
  if (c->options & ~(MOE_OPT_NO_GRID_WAIT | MOE_OPT_GRID_WAIT_NONE | MOE_OPT_INT8_ACTIVATIONS))
    return MOE_ERR_INVALID_ARG;
  if ((c->options & MOE_OPT_INT8_ACTIVATIONS) && c->wfmt != MOE_WFMT_INT4_ROW_F32)
    return MOE_ERR_INVALID_ARG;
  if (!(c->expert_top_p >= 0.0f && c->expert_top_p <= 1.0f)) return MOE_ERR_INVALID_ARG;   // NaN too
  // kernel limits
  if (c->n_routed_experts > 256 || c->n_group > 64 || c->top_k > 16) return MOE_ERR_UNSUPPORTED;
  if (c->hidden > 65536 || c->moe_inter > 65536) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared_experts == 1 && c->shared_inter > 65536) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_T(int32_t T) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_proj(const moe_qproj& p, int wfmt) {
  if (!p.q || !p.scale) return MOE_ERR_INVALID_ARG;
  if (!aligned(p.q, 16) || !aligned(p.scale, 16)) return MOE_ERR_INVALID_ARG;
  if (wfmt == MOE_WFMT_NVFP4) {
    if (!p.gscale || !aligned(p.gscale, 4)) return MOE_ERR_INVALID_ARG;
  } else if (p.gscale) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status check_experts(const moe_qexperts* w, int wfmt) {
  if (!w) return MOE_ERR_INVALID_ARG;
  moe_status s;
  if ((s = check_proj(w->gate, wfmt)) != MOE_OK) return s;
  if ((s = check_proj(w->up, wfmt)) != MOE_OK) return s;
  return check_proj(w->down, wfmt);
}

moe_status check_ws(const moe_config& c, int T, const void* ws, size_t ws_bytes) {
  const size_t need = carve_workspace(c, T, nullptr).total;
  if (need == 0) return MOE_OK;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

ExpertSet expert_set(const moe_qexperts& w, int inter) {
  ExpertSet s;
  s.gate = {w.gate.q, w.gate.scale, w.gate.gscale};
  s.up = {w.up.q, w.up.scale, w.up.gscale};
  s.down = {w.down.q, w.down.scale, w.down.gscale};
  s.inter = inter;
  return s;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Expert FFNs on the grouped MFMA GEMM: work units from the permutation (or
// the shared / dense expert alone), fp16 activations, gate/up, down.
hipError_t run_gemm_ffn(const moe_config& c, int T, const uint16_t* x, const Workspace& w,
                        bool has_routed, const ExpertSet& routed, const int32_t* offsets,
                        const int32_t* active, const int32_t* n_active,
                        const int32_t* sorted_token, bool has_shared, const ExpertSet& shared,
                        int P, int ldh, uint16_t* h, float* o, hipStream_t stream, Tracer* tr) {
  hipError_t e;
  const int K = has_routed ? c.top_k : 0, E = has_routed ? c.n_routed_experts : 0;
  const bool a8 = (c.options & MOE_OPT_INT8_ACTIVATIONS) != 0;
  const int bmf = a8 ? kGemmUnitTokensQ : kGemmUnitTokensF;
  if ((e = launch_build_units(offsets, has_routed ? active : nullptr,
                              has_routed ? n_active : nullptr, w.tiles, w.n_tiles, T, P, K, E,
                              has_shared, stream, bmf)) != hipSuccess)
    return e;
  if (a8) {
    // W4A8: x -> int8 rows, gate/up (fp16 h), h -> int8 rows, down
    GemmQArgs q{};
    q.tiles = w.tiles;
    q.n_tiles = w.n_tiles;
    q.thin_off = gemm_thin_offset(T, K, E, has_shared, bmf);
    q.xq = reinterpret_cast<const int8_t*>(w.x16);
    q.ldxq = pad_k(c.hidden);
    q.xs = w.xs;
    q.xsum = w.xsum;
    q.sorted_token = sorted_token;
    q.hq = w.hq;
    q.ldhq = ldh;
    q.hs = w.hs;
    q.hsum = w.hsum;
    q.routed = routed;
    q.has_shared = has_shared;
    q.shared = shared;
    q.h_out = h;
    q.ldh = ldh;
    q.o_out = o;
    q.T = T;
    q.H = c.hidden;
    q.P = P;
    if ((e = launch_quant_rows(x, c.hidden, true, T, T, c.hidden, c.hidden,
                               reinterpret_cast<int8_t*>(w.x16), q.ldxq, w.xs, w.xsum, stream)) !=
        hipSuccess)
      return e;
    if (tr && (e = tr->mark("gemm_prep")) != hipSuccess) return e;
    if ((e = launch_gemm_q(q, 0, K, E, stream)) != hipSuccess) return e;
    if (tr && (e = tr->mark("gemm_gateup")) != hipSuccess) return e;
    if ((e = launch_quant_rows(h, ldh, false, P + (has_shared ? T : 0), P, routed.inter,
                               has_shared ? shared.inter : routed.inter, w.hq, ldh, w.hs, w.hsum,
                               stream)) != hipSuccess)
      return e;
    if (tr && (e = tr->mark("quant_h")) != hipSuccess) return e;
    if ((e = launch_gemm_q(q, 1, K, E, stream)) != hipSuccess) return e;
    if (tr && (e = tr->mark("gemm_down")) != hipSuccess) return e;
    return hipSuccess;
  }
  if ((e = launch_x_to_f16(x, w.x16, T, c.hidden, pad_k(c.hidden), stream)) != hipSuccess) return e;
  if (tr && (e = tr->mark("gemm_prep")) != hipSuccess) return e;
  GemmArgs g{};
  g.tiles = w.tiles;
  g.n_tiles = w.n_tiles;
  g.thin_off = gemm_thin_offset(T, K, E, has_shared, bmf);
  g.x16 = w.x16;
  g.ldx = pad_k(c.hidden);
  g.sorted_token = sorted_token;
  g.hin = h;
  g.ldh = ldh;
  g.routed = routed;
  g.has_shared = has_shared;
  g.shared = shared;
  g.h_out = h;
  g.o_out = o;
  g.T = T;
  g.H = c.hidden;
  g.P = P;
  g.wfmt = c.wfmt;
  return launch_gemm(g, K, E, stream, tr);
}

hipError_t run_ffn_combine(const moe_config& c, int T, const uint16_t* x, const Workspace& w,
                           const int32_t* picks, int n_experts, const ExpertSet& routed,
                           bool has_shared, const ExpertSet& shared, const float* tw, void* y,
                           bool out_bf16, bool gemv, hipStream_t stream, Tracer* tr, bool permuted) {
  hipError_t e;
  const int K = c.top_k, P = T * K;
  const int ldh = pad_k(std::max(c.moe_inter, has_shared ? c.shared_inter : 0));
  PermuteArgs pa{picks, w.offsets, w.sorted_token, w.inv_perm, w.active, w.n_active,
                 T, K, n_experts, w.phist};
  if (!permuted && (e = launch_permute(pa, stream, tr)) != hipSuccess) return e;
  float* o_shared = has_shared ? w.O + (size_t)P * c.hidden : nullptr;
  if (gemv) {
    FfnArgs a{};
    a.x = x;
    a.T = T;
    a.H = c.hidden;
    a.K = K;
    a.wfmt = c.wfmt;
    a.ldh = ldh;
    a.has_routed = true;
    a.routed = routed;
    a.max_slots = std::min(n_experts, P);
    a.offsets = w.offsets;
    a.sorted_token = w.sorted_token;
    a.active = w.active;
    a.n_active = w.n_active;
    a.h_routed = w.h;
    a.o_routed = w.O;
    a.has_dense = has_shared;
    a.dense = shared;
    a.h_dense = w.h + (size_t)P * ldh;
    a.o_dense = o_shared;
    if ((e = launch_ffn(a, stream, tr)) != hipSuccess) return e;
  } else {
    moe_config ce = c;
    ce.n_routed_experts = n_experts;
    if ((e = run_gemm_ffn(ce, T, x, w, true, routed, w.offsets, w.active, w.n_active,
                          w.sorted_token, has_shared, shared, P, ldh, w.h, w.O, stream, tr)) !=
        hipSuccess)
      return e;
  }
  CombineArgs ca{w.O, w.inv_perm, tw, o_shared, y, out_bf16, T, c.hidden, K};
  return launch_combine(ca, stream, tr);
}

Workspace carve_workspace(const moe_config& c, int T, void* base) {
  Workspace w{};
  if (T == 0) return w;
  const size_t E = c.n_routed_experts, K = c.top_k, H = c.hidden;
  const size_t P = (size_t)T * K;
  const size_t imax = (size_t)pad_k(std::max(c.moe_inter, c.n_shared_experts ? c.shared_inter : 0));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  const size_t o_flags = take(sizeof(uint32_t));   // offset 0, as moe_layer_flags documents
  const size_t o_logits =
      take((size_t)route_splits(T, c.hidden, (int)E) * T * E * sizeof(double));
  const size_t o_ids = take(P * sizeof(int32_t));
  const size_t o_tw = take(P * sizeof(float));
  const size_t o_off = take((E + 1) * sizeof(int32_t));
  const size_t o_act = take(E * sizeof(int32_t));
  const size_t o_na = take(4 * sizeof(int32_t));
  const size_t o_st = take(P * sizeof(int32_t));
  const size_t o_inv = take(P * sizeof(int32_t));
  const size_t o_sw = take(P * sizeof(float));
  const size_t o_h = take((P + T) * imax * sizeof(uint16_t));
  const size_t o_O = take((P + T) * H * sizeof(float));
  const size_t o_x16 = take((size_t)T * pad_k((int)H) * sizeof(uint16_t));
  const size_t o_tiles =
      take((size_t)gemm_max_units(T, (int)K, (int)E, c.n_shared_experts == 1) * 4 * sizeof(int32_t));
  const size_t o_ntiles = take(4 * sizeof(int32_t));
  const size_t o_dslots = take(kDecMaxSlots * sizeof(DecSlot));
  const size_t o_dpick = take(kDecMaxSlots * sizeof(int32_t));
  const size_t o_dbar = take(kDecBarrierWords * sizeof(uint32_t));
  const size_t o_phist = take(permute_hist_ints(T, (int)E) * sizeof(int32_t));
  const size_t o_cids = take(P * sizeof(int32_t));
  const bool a8 = (c.options & MOE_OPT_INT8_ACTIVATIONS) != 0;
  const size_t o_xs = take(a8 ? (size_t)T * sizeof(float) : 0);
  const size_t o_xsum = take(a8 ? (size_t)T * sizeof(int32_t) : 0);
  const size_t o_hq = take(a8 ? (P + T) * imax : 0);
  const size_t o_hs = take(a8 ? (P + T) * sizeof(float) : 0);
  const size_t o_hsum = take(a8 ? (P + T) * sizeof(int32_t) : 0);
  w.total = off;
  if (base) {
    char* b = static_cast<char*>(base);
    w.flags = reinterpret_cast<uint32_t*>(b + o_flags);
    w.logits = reinterpret_cast<double*>(b + o_logits);
    w.ids = reinterpret_cast<int32_t*>(b + o_ids);
    w.tw = reinterpret_cast<float*>(b + o_tw);
    w.offsets = reinterpret_cast<int32_t*>(b + o_off);
    w.active = reinterpret_cast<int32_t*>(b + o_act);
    w.n_active = reinterpret_cast<int32_t*>(b + o_na);
    w.sorted_token = reinterpret_cast<int32_t*>(b + o_st);
    w.inv_perm = reinterpret_cast<int32_t*>(b + o_inv);
    w.sorted_w = reinterpret_cast<float*>(b + o_sw);
    w.h = reinterpret_cast<uint16_t*>(b + o_h);
    w.O = reinterpret_cast<float*>(b + o_O);
    w.x16 = reinterpret_cast<uint16_t*>(b + o_x16);
    w.tiles = reinterpret_cast<int4*>(b + o_tiles);
    w.n_tiles = reinterpret_cast<int32_t*>(b + o_ntiles);
    w.dslots = reinterpret_cast<DecSlot*>(b + o_dslots);
    w.dpick = reinterpret_cast<int32_t*>(b + o_dpick);
    w.dbar = reinterpret_cast<uint32_t*>(b + o_dbar);
    w.phist = reinterpret_cast<int32_t*>(b + o_phist);
    w.cache_ids = reinterpret_cast<int32_t*>(b + o_cids);
    if (a8) {
      w.xs = reinterpret_cast<float*>(b + o_xs);
      w.xsum = reinterpret_cast<int32_t*>(b + o_xsum);
      w.hq = reinterpret_cast<int8_t*>(b + o_hq);
      w.hs = reinterpret_cast<float*>(b + o_hs);
      w.hsum = reinterpret_cast<int32_t*>(b + o_hsum);
    }
  }
  return w;
}

moe_status check_layer_args(const moe_config* cfg, int32_t T, const uint16_t* x,
                            const float* router_w, const moe_qexperts* routed,
                            const moe_qexperts* shared, const void* y, int32_t out_dtype) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!x || !router_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16) return MOE_ERR_INVALID_ARG;
  if ((s = check_experts(routed, cfg->wfmt)) != MOE_OK) return s;
  if (cfg->n_shared_experts == 1) {
    if ((s = check_experts(shared, cfg->wfmt)) != MOE_OK) return s;
  } else if (shared) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, int32_t T, size_t* bytes) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = carve_workspace(*cfg, T, nullptr).total;
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  // callers may pass any int (the header's other codes, or none of them):
  // read it as an int, since a value outside the enumerators is not a valid
  // moe_status in C++
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_layer_flags(const void* ws, uint32_t* flags, hipStream_t stream) {
  if (!flags) return MOE_ERR_INVALID_ARG;
  if (ws && !aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  if (!ws && !(ws = noalloc_workspace())) return MOE_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_ERR_HIP;
  *flags = v;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, int32_t T, const uint16_t* x, const float* router_w,
                     const float* bias, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!x || !router_w || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16)) return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(*cfg, T, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const Workspace w = carve_workspace(*cfg, T, ws);
  RouteArgs a{x, router_w, bias, topk_ids, topk_w, w.logits, T, cfg->hidden,
              cfg->n_routed_experts, cfg->n_group, cfg->topk_group, cfg->top_k,
              cfg->routed_scaling_factor, nullptr, cfg->expert_top_p};
  return hip_status(launch_route(a, stream));
}

moe_status moe_permute(const moe_config* cfg, int32_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_perm,
                       int32_t* active_experts, int32_t* n_active, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!topk_ids || !expert_offsets || !sorted_token || !inv_perm || !active_experts || !n_active)
    return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(*cfg, T, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const Workspace w = carve_workspace(*cfg, T, ws);
  PermuteArgs a{topk_ids, expert_offsets, sorted_token, inv_perm, active_experts, n_active,
                T, cfg->top_k, cfg->n_routed_experts, w.phist};
  return hip_status(launch_permute(a, stream));
}

moe_status moe_expert_ffn_q4(const moe_config* cfg, int32_t T, const uint16_t* x,
                             const moe_qexperts* w, const int32_t* expert_offsets,
                             const int32_t* sorted_token, const int32_t* active_experts,
                             const int32_t* n_active, float* out, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  if ((s = check_experts(w, cfg->wfmt)) != MOE_OK) return s;
  const bool routed = expert_offsets != nullptr;
  if (routed) {
    if (!sorted_token || !active_experts || !n_active) return MOE_ERR_INVALID_ARG;
  } else {
    if (sorted_token || active_experts || n_active) return MOE_ERR_INVALID_ARG;
    if (cfg->n_shared_experts == 0) return MOE_ERR_INVALID_ARG;  // no shared_inter to use
  }
  if ((s = check_ws(*cfg, T, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const Workspace ws_ = carve_workspace(*cfg, T, ws);
  const int ldh = pad_k(std::max(cfg->moe_inter, cfg->n_shared_experts ? cfg->shared_inter : 0));
  FfnArgs a{};
  a.x = x;
  a.T = T;
  a.H = cfg->hidden;
  a.K = cfg->top_k;
  a.wfmt = cfg->wfmt;
  a.ldh = ldh;
  if (T > kDecodeMaxTokens) {
    const int64_t rows = routed ? (int64_t)T * cfg->top_k : T;
    if (!gemm_fits(T, rows, pad_k(cfg->hidden), ldh)) return MOE_ERR_UNSUPPORTED;
    const ExpertSet es = expert_set(*w, routed ? cfg->moe_inter : cfg->shared_inter);
    const int P = routed ? T * cfg->top_k : 0;
    return hip_status(run_gemm_ffn(*cfg, T, x, ws_, routed, es, expert_offsets, active_experts,
                                   n_active, sorted_token, !routed, es, P, ldh, ws_.h, out,
                                   stream, nullptr));
  }
  if (routed) {
    a.has_routed = true;
    a.routed = expert_set(*w, cfg->moe_inter);
    a.max_slots = std::min<int64_t>(cfg->n_routed_experts, (int64_t)T * cfg->top_k);
    a.offsets = expert_offsets;
    a.sorted_token = sorted_token;
    a.active = active_experts;
    a.n_active = n_active;
    a.h_routed = ws_.h;
    a.o_routed = out;
  } else {
    a.has_dense = true;
    a.dense = expert_set(*w, cfg->shared_inter);
    a.h_dense = ws_.h;
    a.o_dense = out;
  }
  return hip_status(launch_ffn(a, stream));
}

moe_status moe_combine(const moe_config* cfg, int32_t T, const float* expert_out,
                       const int32_t* inv_perm, const float* topk_w, const float* shared_out,
                       void* y, int32_t out_dtype, hipStream_t stream) {
  moe_status s;
  if ((s = check_cfg(cfg)) != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (!expert_out || !inv_perm || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16) return MOE_ERR_INVALID_ARG;
  if (!aligned(expert_out, 16) || !aligned(y, 16) || (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  CombineArgs a{expert_out, inv_perm, topk_w, shared_out, y, out_dtype == MOE_OUT_BF16,
                T, cfg->hidden, cfg->top_k};
  return hip_status(launch_combine(a, stream));
}

}  // extern "C"

namespace {

moe_status layer_impl(const moe_config* cfg, int32_t T, const uint16_t* x, const float* router_w,
                      const float* bias, const moe_qexperts* routed, const moe_qexperts* shared,
                      void* y, int32_t out_dtype, int32_t* topk_ids_out, float* topk_w_out,
                      void* ws, size_t ws_bytes, hipStream_t stream, moe_trace* trace) {
  moe_status s;
  if ((s = check_layer_args(cfg, T, x, router_w, routed, shared, y, out_dtype)) != MOE_OK) return s;
  if ((s = check_ws(*cfg, T, ws, ws_bytes)) != MOE_OK) return s;
  if (trace) {
    for (int i = 0; i <= MOE_TRACE_MAX; ++i)
      if (!trace->events[i]) return MOE_ERR_INVALID_ARG;
  }
  if (T == 0) {
    if (trace) trace->n_kernels = 0;
    return MOE_OK;
  }

  const bool has_shared = cfg->n_shared_experts == 1;
  const int ldh = pad_k(std::max(cfg->moe_inter, has_shared ? cfg->shared_inter : 0));
  const size_t P = (size_t)T * cfg->top_k;
  // the single-token and small-batch kernels take the group-scaled formats;
  // small batches in the per-row formats take the grouped GEMV
  const bool small = T <= kDecodeMaxTokens && decode_supported(cfg->hidden) &&
                     (!wfmt_row(cfg->wfmt) || decode_row_format_ok(*cfg, T));
  const bool gemv = T <= kDecodeMaxTokens && wfmt_row(cfg->wfmt) && !small;
  if (!small && !gemv && !gemm_fits(T, (int64_t)P + (has_shared ? T : 0), pad_k(cfg->hidden), ldh))
    return MOE_ERR_UNSUPPORTED;

  const Workspace w = carve_workspace(*cfg, T, ws);
  Tracer tracer;
  tracer.t = trace;
  tracer.s = stream;
  Tracer* tr = trace ? &tracer : nullptr;
  if (tr && tr->begin() != hipSuccess) return MOE_ERR_HIP;
  int32_t* ids = topk_ids_out ? topk_ids_out : w.ids;
  float* tw = topk_w_out ? topk_w_out : w.tw;
  hipError_t e;
  if (small) {
    DecodeArgs d{};
    d.x = x;
    d.T = T;
    d.H = cfg->hidden;
    d.E = cfg->n_routed_experts;
    d.G = cfg->n_group;
    d.TG = cfg->topk_group;
    d.K = cfg->top_k;
    d.rsf = cfg->routed_scaling_factor;
    d.top_p = cfg->expert_top_p;
    d.router_w = router_w;
    d.bias = bias;
    d.logits = w.logits;
    d.ids = ids;
    d.tw = tw;
    d.offsets = w.offsets;
    d.sorted_token = w.sorted_token;
    d.inv_perm = w.inv_perm;
    d.active = w.active;
    d.n_active = w.n_active;
    d.sorted_w = w.sorted_w;
    d.slots = w.dslots;
    d.sorted_et = w.dpick;
    d.bar = w.dbar;
    d.options = cfg->options;
    d.flags = w.flags;
    d.routed = expert_set(*routed, cfg->moe_inter);
    d.has_shared = has_shared;
    if (has_shared) d.shared = expert_set(*shared, cfg->shared_inter);
    d.h_routed = w.h;
    d.h_shared = w.h + P * ldh;
    d.ldh = ldh;
    d.y = y;
    d.out_bf16 = out_dtype == MOE_OUT_BF16;
    d.wfmt = cfg->wfmt;
    return hip_status(launch_decode(d, stream, tr));
  }
  RouteArgs ra{x, router_w, bias, ids, tw, w.logits, T, cfg->hidden, cfg->n_routed_experts,
               cfg->n_group, cfg->topk_group, cfg->top_k, cfg->routed_scaling_factor, w.flags,
               cfg->expert_top_p};
  // up to four tokens: the selection also sorts the picks (no permutation
  // launch)
  const bool fused_perm = route_permute_small_ok(T, cfg->top_k);
  if (fused_perm) {
    PermuteArgs pa{ids, w.offsets, w.sorted_token, w.inv_perm, w.active, w.n_active,
                   T, cfg->top_k, cfg->n_routed_experts, w.phist};
    e = launch_route_permute_small(ra, pa, stream, tr);
  } else {
    e = launch_route(ra, stream, tr);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  const ExpertSet rset = expert_set(*routed, cfg->moe_inter);
  const ExpertSet sset = has_shared ? expert_set(*shared, cfg->shared_inter) : ExpertSet{};
  return hip_status(run_ffn_combine(*cfg, T, x, w, ids, cfg->n_routed_experts, rset, has_shared,
                                    sset, tw, y, out_dtype == MOE_OUT_BF16, gemv, stream, tr,
                                    fused_perm));
}

}  // namespace

extern "C" {

moe_status moe_layer(const moe_config* cfg, int32_t T, const uint16_t* x, const float* router_w,
                     const float* bias, const moe_qexperts* routed, const moe_qexperts* shared,
                     void* y, int32_t out_dtype, int32_t* topk_ids_out, float* topk_w_out,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_impl(cfg, T, x, router_w, bias, routed, shared, y, out_dtype, topk_ids_out,
                    topk_w_out, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_trace(const moe_config* cfg, int32_t T, const uint16_t* x,
                           const float* router_w, const float* bias, const moe_qexperts* routed,
                           const moe_qexperts* shared, void* y, int32_t out_dtype,
                           int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                           hipStream_t stream, moe_trace* trace) {
  if (!trace) return MOE_ERR_INVALID_ARG;
  return layer_impl(cfg, T, x, router_w, bias, routed, shared, y, out_dtype, topk_ids_out,
                    topk_w_out, ws, ws_bytes, stream, trace);
}

}  // extern "C"
