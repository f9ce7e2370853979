// Internal interfaces between the C-ABI layer (qmoe_api.cpp) and the kernel
// launchers (*.hip).  Not installed; the public interface is include/qmoe.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include <type_traits>

#include "../../include/qmoe.h"

namespace qmoe {

// Per-row-scale weight formats: code bits, and whether a format is one.
__host__ __device__ constexpr bool wfmt_row(int f) {
  return f == MOE_WFMT_INT4_ROW_F32 || f == MOE_WFMT_INT8_ROW_F32 || f == MOE_WFMT_INT2_ROW_F32;
}
__host__ __device__ constexpr int wfmt_bits(int f) {
  return f == MOE_WFMT_INT8_ROW_F32 ? 8 : f == MOE_WFMT_INT2_ROW_F32 ? 2 : 4;
}

// Calls f(std::integral_constant<int, fmt>{}) for the runtime format.
template <class F>
inline auto dispatch_wfmt(int wfmt, F&& f) {
  switch (wfmt) {
    case MOE_WFMT_NVFP4: return f(std::integral_constant<int, MOE_WFMT_NVFP4>{});
    case MOE_WFMT_INT4_ROW_F32: return f(std::integral_constant<int, MOE_WFMT_INT4_ROW_F32>{});
    case MOE_WFMT_INT8_ROW_F32: return f(std::integral_constant<int, MOE_WFMT_INT8_ROW_F32>{});
    case MOE_WFMT_INT2_ROW_F32: return f(std::integral_constant<int, MOE_WFMT_INT2_ROW_F32>{});
    default: return f(std::integral_constant<int, MOE_WFMT_INT4_G32_F16>{});
  }
}

struct ProjPtr {
  const uint8_t* q;
  const void* s;
  const float* g;
};

struct ExpertSet {
  ProjPtr gate, up, down;
  int inter;
};

// Pieces of the caller's workspace.  Every piece starts on a 256-byte boundary.
// One selected expert of a small batch (decode path), written by the
// selection kernel and read by the FFN kernels in three 16-byte loads:
// expert e, its first sorted slot p0, its M <= 4 tokens and their weights in
// pick order.
struct alignas(16) DecSlot {
  int32_t e, p0, M, pad;
  int32_t t[4];
  float w[4];
};
static_assert(sizeof(DecSlot) == 48, "three 16-byte loads");
constexpr int kDecMaxSlots = 64;

struct Workspace {
  uint32_t* flags;        // [1] at offset 0: MOE_FLAG_* of the last moe_layer call
  double* logits;         // [T][E]   router logits (fp64)
  int32_t* ids;           // [T][k]   routing when the caller keeps none
  float* tw;              // [T][k]
  int32_t* offsets;       // [E+1]
  int32_t* active;        // [E]
  int32_t* n_active;      // [4]
  int32_t* sorted_token;  // [P]
  int32_t* inv_perm;      // [P]
  float* sorted_w;        // [P]     routing weight of the pick at each sorted slot
  uint16_t* h;            // [P+T][Imax] fp16 SwiGLU outputs
  float* O;               // [P+T][H]   per-pick expert outputs (fp32)
  uint16_t* x16;          // [T][H]     fp16 activations (GEMM path)
  int4* tiles;            // [max units] GEMM work units
  DecSlot* dslots;        // [kDecMaxSlots] decode path: selected experts
  int32_t* dpick;         // [kDecMaxSlots] decode path: expert | token << 16 of each sorted pick
  uint32_t* dbar;         // [kDecBarrierWords] decode path: grid-barrier count and flags
  int32_t* n_tiles;       // [4]
  int32_t* phist;         // [permute_hist_ints] permutation scratch
  int32_t* cache_ids;     // [P] moe_layer_cached: the picks' slot ids
  // int8 activations (MOE_OPT_INT8_ACTIVATIONS only; x codes reuse x16)
  float* xs;              // [T]
  int32_t* xsum;          // [T]
  int8_t* hq;             // [P+T][Imax]
  float* hs;              // [P+T]
  int32_t* hsum;          // [P+T]
  size_t total;
};

// Records caller-owned events at kernel boundaries (moe_layer_trace).
struct Tracer {
  moe_trace* t = nullptr;
  hipStream_t s = nullptr;
  int n = 0;
  hipError_t begin() {
    if (!t) return hipSuccess;
    t->n_kernels = 0;
    return hipEventRecord(t->events[0], s);
  }
  // Call right after launching a kernel on the traced stream.
  hipError_t mark(const char* name) {
    if (!t || n >= MOE_TRACE_MAX) return hipSuccess;
    t->names[n] = name;
    ++n;
    t->n_kernels = n;
    return hipEventRecord(t->events[n], s);
  }
};

// Lays the workspace out from `base` (nullptr: only sizes it).
Workspace carve_workspace(const moe_config& c, int T, void* base);
// moe_layer's argument checks other than the workspace's (no HIP call).
moe_status check_layer_args(const moe_config* cfg, int32_t T, const uint16_t* x,
                            const float* router_w, const moe_qexperts* routed,
                            const moe_qexperts* shared, const void* y, int32_t out_dtype);
// Argument checks shared by the entry points (no HIP call).
bool aligned(const void* p, size_t a);
moe_status check_cfg(const moe_config* c);
moe_status check_T(int32_t T);
moe_status check_experts(const moe_qexperts* w, int wfmt);
moe_status check_ws(const moe_config& c, int T, const void* ws, size_t ws_bytes);
ExpertSet expert_set(const moe_qexperts& w, int inter);
moe_status hip_status(hipError_t e);
// moe_layer_noalloc's workspace on the current device (its device address,
// looked up on the first call on that device); nullptr if the lookup failed.
void* noalloc_workspace();

struct RouteArgs {
  const uint16_t* x;
  const float* router_w;
  const float* bias;  // nullable
  int32_t* ids;
  float* tw;
  double* logits;
  int T, H, E, G, TG, K;
  float rsf;
  uint32_t* flags;    // nullable: moe_layer's flags word, cleared by the selection kernel
  float top_p;        // adaptive expert top-p (0: keep all top_k)
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s, Tracer* tr = nullptr);
// Number of hidden-dimension slices route_logits uses (its logits buffer
// holds that many T x E partial sums).
int route_splits(int T, int H, int E);

struct PermuteArgs {
  const int32_t* ids;
  int32_t* offsets;
  int32_t* sorted_token;
  int32_t* inv_perm;
  int32_t* active;
  int32_t* n_active;
  int T, K, E;
  int32_t* hist;   // [permute_hist_ints] per-chunk expert counts (scratch)
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s, Tracer* tr = nullptr);
// Routing and permutation of 1 <= T <= kDecodeMaxTokens tokens with T*k <=
// 64 picks (route_permute_small_ok) in two launches: the scores, then one
// workgroup that selects and sorts; the outputs of launch_route followed by
// launch_permute (pa.ids is not read: the picks go from the selection to the
// sort in LDS).
bool route_permute_small_ok(int T, int K);
hipError_t launch_route_permute_small(const RouteArgs& a, const PermuteArgs& pa, hipStream_t s,
                                      Tracer* tr = nullptr);
// Tokens per chunk of the permutation and the size of its scratch.
int permute_chunk(int T);
size_t permute_hist_ints(int T, int E);

struct FfnArgs {
  const uint16_t* x;
  int T, H, K, wfmt;
  // routed experts (grouped by the permutation)
  bool has_routed;
  ExpertSet routed;
  int max_slots;  // upper bound on the number of active experts
  const int32_t* offsets;
  const int32_t* sorted_token;
  const int32_t* active;
  const int32_t* n_active;
  uint16_t* h_routed;  // [P][ldh]
  float* o_routed;     // [P][H]
  // one expert applied to all T tokens (the shared expert, or dense mode)
  bool has_dense;
  ExpertSet dense;
  uint16_t* h_dense;   // [T][ldh]
  float* o_dense;      // [T][H]
  int ldh;
};
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, Tracer* tr = nullptr);

struct CombineArgs {
  const float* expert_out;  // [P][H]
  const int32_t* inv_perm;
  const float* tw;
  const float* shared_out;  // nullable, [T][H]
  void* y;
  int out_bf16;
  int T, H, K;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s, Tracer* tr = nullptr);

// Small-batch path of moe_layer (T <= kDecodeMaxTokens): router scores,
// selection + grouping of the picks, gate/up, down with the weighted combine
// (one token: the last three in one launch; 2..4 tokens: the middle two).
constexpr int kDecodeMaxTokens = 4;
constexpr int kDecodeMaxGPL = 4;   // hidden <= 64 lanes * 4 groups * 32 = 8192
// Grid barrier of the fused single-token kernel: an arrival count and one
// flag per workgroup (at most kDecFusedMaxGrid), kDecFlagStride words apart.
constexpr int kDecFlagStride = 64;
constexpr int kDecFusedMaxGrid = 1024;
constexpr size_t kDecBarrierWords = (size_t)kDecFlagStride * (kDecFusedMaxGrid + 1);
bool decode_supported(int hidden);
// Router scores sigmoid(x . Wr[e]) in float64 for 1 <= T <= kDecodeMaxTokens
// tokens (one block per expert) into scores[T][E]; launch_route takes it for
// such T.  hipErrorInvalidValue for other T or H % 16 != 0.
hipError_t launch_route_scores(const uint16_t* x, const float* router_w, double* scores, int T, int H,
                               int E, hipStream_t s);
// Whether a per-row format call of T tokens takes the single-token kernels
// (per-row int4 and int2, one token, down rows within dec_down_t1's limits).
bool decode_row_format_ok(const moe_config& c, int T);

struct DecodeArgs {
  const uint16_t* x;
  int T, H, E, G, TG, K;
  float rsf;
  float top_p;            // adaptive expert top-p (0: keep all top_k)
  const float* router_w;
  const float* bias;
  double* logits;         // [T][E] router scores (sigmoid of the float64 logits)
  int32_t* ids;
  float* tw;
  int32_t* offsets;
  int32_t* sorted_token;
  int32_t* inv_perm;
  int32_t* active;
  int32_t* n_active;
  float* sorted_w;
  DecSlot* slots;
  int32_t* sorted_et;     // [P] expert (low 16 bits) and token (high 16 bits) of sorted pick p
  uint32_t* bar;          // grid-barrier count and flags of the fused single-token kernel
  uint32_t barrier_spins; // polls before a workgroup of that kernel gives up on the barrier
  uint32_t options;       // moe_config.options
  uint32_t* flags;        // moe_layer's flags word: cleared by K1, raised on a barrier give-up
  ExpertSet routed;
  bool has_shared;
  ExpertSet shared;
  uint16_t* h_routed;  // [P][ldh]
  uint16_t* h_shared;  // [T][ldh]
  int ldh;
  void* y;
  int out_bf16;
  int wfmt;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr = nullptr);

// Grouped MFMA GEMM path (prefill-shaped calls).
struct GemmArgs {
  const int4* tiles;          // work units (see build_units): fat units, then thin ones
  const int32_t* n_tiles;     // [0]: fat units, [1]: thin units
  int thin_off;               // index of the first thin unit in tiles
  const uint16_t* x16;        // fp16 activations [T][ldx], zero past H
  int ldx;
  const int32_t* sorted_token;
  const uint16_t* hin;        // fp16 h [P+T][ldh] (down input), zero past inter
  int ldh;
  ExpertSet routed;
  bool has_shared;
  ExpertSet shared;
  uint16_t* h_out;            // fp16 h [P+T][ldh] (gate/up output)
  float* o_out;               // fp32 [P+T][H] (down output)
  int T, H, P, wfmt;
};
// W4A8 grouped GEMM (csrc/gemm_i8.hip): per-row int4 weights, int8
// activations with one fp32 scale and one code sum per row.
struct GemmQArgs {
  const int4* tiles;
  const int32_t* n_tiles;
  int thin_off;
  const int8_t* xq;           // int8 x [T][ldxq] (bytes), chunk order of the kernel
  int ldxq;
  const float* xs;            // [T] scales
  const int32_t* xsum;        // [T] code sums
  const int32_t* sorted_token;
  const int8_t* hq;           // int8 h [P+T][ldhq]
  int ldhq;
  const float* hs;            // [P+T]
  const int32_t* hsum;        // [P+T]
  ExpertSet routed;
  bool has_shared;
  ExpertSet shared;
  uint16_t* h_out;            // fp16 h [P+T][ldh] (gate/up output)
  int ldh;
  float* o_out;               // fp32 [P+T][H] (down output)
  int T, H, P;
};
// Row quantiser: rows of bf16 (x) or fp16 (h; width n below row `split`, n2
// from there) -> int8 codes [rows][ld_dst] in the W4A8 GEMM's chunk order,
// scale and code sum per row.
hipError_t launch_quant_rows(const uint16_t* src, int ld_src, bool bf16, int rows, int split, int n,
                             int n2, int8_t* dst, int ld_dst, float* scale, int32_t* sum, hipStream_t s);
// proj 0: gate/up (+SwiGLU into h_out); 1: down (into o_out).
hipError_t launch_gemm_q(const GemmQArgs& g, int proj, int K, int E, hipStream_t s);

// Tokens per fat work unit of the W4A8 GEMM and of the fp16 GEMM.
#ifndef QMOE_Q_BM
#define QMOE_Q_BM 192
#endif
#ifndef QMOE_F16_BM
#define QMOE_F16_BM 192
#endif
constexpr int kGemmUnitTokensQ = QMOE_Q_BM;
constexpr int kGemmUnitTokensF = QMOE_F16_BM;
int gemm_max_units(int T, int K, int E, bool has_shared);
// Row strides (elements) of the fp16 activation and intermediate buffers: a
// multiple of the GEMM's K block, the padding held at zero.
__host__ __device__ inline int pad_k(int n) { return (n + 127) & ~127; }
// Whether the GEMM path's activation buffers (T x ldx fp16 activations, rows x
// ldh fp16 intermediates) fit its buffer descriptors (2 GiB each).
bool gemm_fits(int64_t T, int64_t rows, int64_t ldx, int64_t ldh);
// bmf: tokens per fat unit (kGemmUnitTokensF, or kGemmUnitTokensQ for the W4A8 GEMM).
int gemm_thin_offset(int T, int K, int E, bool has_shared, int bmf);
hipError_t launch_build_units(const int32_t* offsets, const int32_t* active,
                              const int32_t* n_active, int4* tiles, int32_t* n_tiles, int T, int P,
                              int K, int E, bool has_shared, hipStream_t s, int bmf);
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, int T, int H, int ldx, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, int K, int E, hipStream_t s, Tracer* tr = nullptr);
// Expert FFNs of a T > kDecodeMaxTokens call on the grouped GEMM: work units
// from the permutation (E = c.n_routed_experts experts) and/or the shared
// expert, fp16 activations, gate/up, down into o.
hipError_t run_gemm_ffn(const moe_config& c, int T, const uint16_t* x, const Workspace& w,
                        bool has_routed, const ExpertSet& routed, const int32_t* offsets,
                        const int32_t* active, const int32_t* n_active,
                        const int32_t* sorted_token, bool has_shared, const ExpertSet& shared,
                        int P, int ldh, uint16_t* h, float* o, hipStream_t stream, Tracer* tr);

// The layer after routing: permutation of `picks` (ids in [0, n_experts) or
// -1) over n_experts experts whose weights are `routed` (skipped when
// `permuted`: w's permutation arrays already hold it), the expert FFNs
// (grouped GEMV if `gemv`, else the grouped GEMM) with the shared expert, and
// the weighted combine into y.
hipError_t run_ffn_combine(const moe_config& c, int T, const uint16_t* x, const Workspace& w,
                           const int32_t* picks, int n_experts, const ExpertSet& routed,
                           bool has_shared, const ExpertSet& shared, const float* tw, void* y,
                           bool out_bf16, bool gemv, hipStream_t stream, Tracer* tr,
                           bool permuted = false);

// Replaces each pick's expert id by its cache slot (map[id]); -1 stays -1.
struct SlotMap {
  int32_t slot[256];
};
hipError_t launch_remap_ids(const int32_t* ids, int32_t* out, int P, const SlotMap& map,
                            hipStream_t s);

}  // namespace qmoe
