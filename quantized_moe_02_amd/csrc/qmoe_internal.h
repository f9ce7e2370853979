// Internal interfaces between the C-ABI layer (qmoe_api.cpp) and the kernel
// launchers (*.hip).  Not installed; the public interface is include/qmoe.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/qmoe.h"

namespace qmoe {

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

struct RouteArgs {
  const uint16_t* x;
  const float* router_w;
  const float* bias;  // nullable
  int32_t* ids;
  float* tw;
  double* logits;
  int T, H, E, G, TG, K;
  float rsf;
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

// Small-batch path of moe_layer (T <= kDecodeMaxTokens): four kernels --
// router logits, selection + grouping of the picks, gate/up, down with the
// weighted combine.
constexpr int kDecodeMaxTokens = 4;
constexpr int kDecodeMaxGPL = 4;   // hidden <= 64 lanes * 4 groups * 32 = 8192
// Grid barrier of the fused single-token kernel: an arrival count and one
// flag per workgroup (at most kDecFusedMaxGrid), kDecFlagStride words apart.
constexpr int kDecFlagStride = 64;
constexpr int kDecFusedMaxGrid = 1024;
constexpr size_t kDecBarrierWords = (size_t)kDecFlagStride * (kDecFusedMaxGrid + 1);
bool decode_supported(int hidden);

struct DecodeArgs {
  const uint16_t* x;
  int T, H, E, G, TG, K;
  float rsf;
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
int gemm_max_units(int T, int K, int E, bool has_shared);
// Row strides (elements) of the fp16 activation and intermediate buffers: a
// multiple of the GEMM's K block, the padding held at zero.
__host__ __device__ inline int pad_k(int n) { return (n + 127) & ~127; }
// Whether the GEMM path's activation buffers (T x ldx fp16 activations, rows x
// ldh fp16 intermediates) fit its buffer descriptors (2 GiB each).
bool gemm_fits(int64_t T, int64_t rows, int64_t ldx, int64_t ldh);
int gemm_thin_offset(int T, int K, int E, bool has_shared);
hipError_t launch_build_units(const int32_t* offsets, const int32_t* active,
                              const int32_t* n_active, int4* tiles, int32_t* n_tiles, int T, int P,
                              int K, int E, bool has_shared, hipStream_t s);
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, int T, int H, int ldx, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, int K, int E, hipStream_t s, Tracer* tr = nullptr);

}  // namespace qmoe
