/*
 * qmoe.h -- C ABI of libqmoe: one quantized Mixture-of-Experts layer on an
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The layer (page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section
 * "Fitur utama yang diimplementasikan"; page "NVIDIA stellt neues GLM-5.2
 * NVFP4 Modell vor", section "Technische Details und Quantisierungsansatz"):
 *
 *   route    DeepSeek-V3-style sigmoid router with the score-correction bias
 *            used for selection only ("noaux_tc"), group-limited top-k,
 *            renormalised weights times routed_scaling_factor;
 *   permute  "batch-union": the T*k (token, expert) picks grouped by expert so
 *            that each selected expert's weights are read once per call;
 *   ffn      SwiGLU experts, FFN(x) = Wd (silu(Wg x) * (Wu x)), over 4-bit
 *            weights dequantised on use (int4 with fp16 group scales, or NVFP4);
 *   combine  y_t = sum_i w_{t,i} FFN_{e_{t,i}}(x_t) + FFN_shared(x_t).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  All array arguments are DEVICE pointers on the current HIP device,
 *   except `cfg`, the moe_qexperts structs, and the `bytes` output of
 *   moe_workspace_size, which are HOST pointers read or written during the
 *   call only.  The caller owns every buffer, including the workspace.  The
 *   library never allocates or frees memory and keeps no mutable global state,
 *   so calls on different streams are independent as long as their workspaces
 *   and outputs do not overlap.
 * Alignment.  Packed weight arrays (`q`), scale arrays and `x` must be 16-byte
 *   aligned; the workspace 256-byte aligned.  Otherwise MOE_ERR_INVALID_ARG.
 * Asynchrony.  Every call only enqueues kernels on `stream` and returns
 *   without synchronising.  A launch failure returns MOE_ERR_HIP; a fault
 *   inside a kernel surfaces at the caller's next synchronisation.
 * Validation.  All argument checks run before any HIP call, so an invalid call
 *   has no effect on the device and can be made without one.
 * Determinism.  No kernel uses floating-point atomics: identical inputs give
 *   bit-identical outputs, ids and permutations on the same device.
 * Empty input.  T == 0 is valid and enqueues nothing.
 *
 * Weight formats (one projection of E experts, N output rows, K inputs)
 * ---------------------------------------------------------------------
 * MOE_WFMT_INT4_G32_F16  symmetric int4, one fp16 scale per 32 inputs.
 *   q     uint8 [E][N][K/2]: per row K/8 little-endian 32-bit words; word j
 *         holds inputs 8j..8j+7, input 8j+2i (i = 0..3) in bits [4i, 4i+4) and
 *         input 8j+2i+1 in bits [16+4i, 16+4i+4).  A code u in 0..15 means
 *         q = u - 8.
 *   scale fp16 [E][N][K/32]; weight = (u - 8) * scale.
 *   gscale must be NULL.
 * MOE_WFMT_NVFP4  E2M1 elements, one FP8 E4M3 scale per 16 inputs, one fp32
 *   scale per (expert, projection).
 *   q      uint8 [E][N][K/2]: byte j holds input 2j in the low nibble and input
 *          2j+1 in the high nibble; a nibble is an E2M1 code (bit 3 sign).
 *   scale  uint8 [E][N][K/16] E4M3 "fn" codes (bias 7, no infinities).
 *   gscale float32 [E]; weight = e2m1 * e4m3 * gscale[e].
 * Gate and up have N = inter, K = hidden; down has N = hidden, K = inter.
 *
 * Activations are bfloat16 [T][hidden], row-major.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,         /* null/misaligned pointer, inconsistent config */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but outside what the kernels handle */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < moe_workspace_size(cfg, T) */
  MOE_ERR_HIP = 4                  /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_WFMT_INT4_G32_F16 = 0, MOE_WFMT_NVFP4 = 1 } moe_wfmt;
typedef enum { MOE_OUT_F32 = 0, MOE_OUT_BF16 = 1 } moe_out_dtype;

/* Layer geometry.  Limits (else MOE_ERR_INVALID_ARG): hidden, moe_inter and
 * shared_inter positive multiples of 32; n_group >= 1 divides
 * n_routed_experts; 1 <= topk_group <= n_group;
 * 1 <= top_k <= topk_group * n_routed_experts / n_group;
 * n_shared_experts in {0, 1}; routed_scaling_factor finite and > 0.
 * Kernel limits (else MOE_ERR_UNSUPPORTED): n_routed_experts <= 256,
 * top_k <= 16, hidden, moe_inter, shared_inter <= 65536. */
typedef struct {
  int32_t hidden;                  /* H */
  int32_t moe_inter;               /* I: inter size of each routed expert */
  int32_t n_routed_experts;        /* E */
  int32_t n_group;                 /* G: experts [j*E/G, (j+1)*E/G) form group j */
  int32_t topk_group;              /* TG: groups kept per token */
  int32_t top_k;                   /* k: experts per token */
  int32_t n_shared_experts;        /* 0 or 1 */
  int32_t shared_inter;            /* Is: inter size of the shared expert */
  float routed_scaling_factor;     /* rsf: multiplies the renormalised routed weights */
  int32_t wfmt;                    /* moe_wfmt of routed and shared experts */
} moe_config;

/* One projection of E experts (device pointers; see the formats above). */
typedef struct {
  const uint8_t* q;
  const void* scale;
  const float* gscale;
} moe_qproj;

typedef struct {
  moe_qproj gate; /* N = inter, K = hidden */
  moe_qproj up;   /* N = inter, K = hidden */
  moe_qproj down; /* N = hidden, K = inter */
} moe_qexperts;

/* Largest T the library accepts (else MOE_ERR_UNSUPPORTED). */
#define MOE_MAX_TOKENS 262144

/* Bytes of workspace any entry point below needs for `T` tokens under `cfg`
 * (one size covers all of them).  `bytes` is a host pointer. */
moe_status moe_workspace_size(const moe_config* cfg, int32_t T, size_t* bytes);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status s);

/* Router (page "Show HN: Menjalankan GLM 5.2 ...", section "Fitur utama":
 * DeepSeek-V3-style sigmoid router, noaux_tc, routed_scaling_factor).
 *   x        bf16 [T][H]
 *   router_w fp32 [E][H]
 *   bias     fp32 [E] score-correction bias (selection only); NULL = zeros
 *   topk_ids int32 [T][k] out: chosen experts, ascending id per token
 *   topk_w   fp32 [T][k] out: s_e / sum(s over chosen) * rsf, same order
 * Logits, sigmoid and every comparison are evaluated in float64 (products of
 * the bf16 and fp32 operands are exact there), so the selection agrees with a
 * float64 evaluation except where two candidates are within about 1e-12.
 * Selection: group score = sum of the two largest s+b in the group (the
 * single one if a group has one expert); the topk_group best groups are kept
 * (equal scores: lower index); the top_k experts by s+b within kept groups
 * are chosen (equal: lower id). */
moe_status moe_route(const moe_config* cfg, int32_t T, const uint16_t* x,
                     const float* router_w, const float* bias, int32_t* topk_ids,
                     float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* Batch-union permutation (same page, section "Fitur utama": each unique expert
 * of the batch is read once and applied to every position routed to it).
 * Stable counting sort of the P = T*k picks by expert id, keeping pick order
 * p = t*k + i inside each expert.
 *   topk_ids       int32 [T][k] in: values in [0, E) (else results undefined)
 *   expert_offsets int32 [E+1] out: exclusive prefix sum of per-expert counts
 *   sorted_token   int32 [P]   out: token index of the pick at each sorted slot
 *   inv_perm       int32 [P]   out: sorted slot of pick p
 *   active_experts int32 [E]   out: experts with >= 1 pick, ascending; the tail
 *                                   beyond n_active is left unspecified
 *   n_active       int32 [1]   out */
moe_status moe_permute(const moe_config* cfg, int32_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_perm,
                       int32_t* active_experts, int32_t* n_active, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Expert SwiGLU FFNs over 4-bit weights, dequantised on use (same page,
 * sections "Cara kerja" and "Fitur utama"; NVFP4 per the NVIDIA page).
 * Routed mode (expert_offsets != NULL): `w` holds the E routed experts
 *   (inter = cfg->moe_inter); the permutation arrays are moe_permute's
 *   outputs; out fp32 [T*k][H] receives FFN_e(x_t) at each sorted slot.
 * Dense mode (expert_offsets == NULL; the three other permutation pointers
 *   must be NULL too): `w` holds one expert (inter = cfg->shared_inter, e.g.
 *   the shared expert); out fp32 [T][H] receives FFN(x_t).
 * Products are accumulated in fp32; the SwiGLU output h is rounded to fp16
 * before the down projection. */
moe_status moe_expert_ffn_q4(const moe_config* cfg, int32_t T, const uint16_t* x,
                             const moe_qexperts* w, const int32_t* expert_offsets,
                             const int32_t* sorted_token, const int32_t* active_experts,
                             const int32_t* n_active, float* out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Weighted combine: y_t = sum_i topk_w[t][i] * expert_out[inv_perm[t*k+i]]
 *                         + shared_out[t]   (shared_out may be NULL).
 *   expert_out fp32 [T*k][H] (sorted order); y [T][H] fp32 or bf16 (RNE). */
moe_status moe_combine(const moe_config* cfg, int32_t T, const float* expert_out,
                       const int32_t* inv_perm, const float* topk_w,
                       const float* shared_out, void* y, int32_t out_dtype,
                       hipStream_t stream);

/* The whole layer: route, permute, routed and shared expert FFNs, combine,
 * enqueued on one stream.
 *   routed   E experts (inter = moe_inter)
 *   shared   one expert (inter = shared_inter); NULL iff n_shared_experts == 0
 *   y        [T][H] fp32 or bf16
 *   topk_ids_out, topk_w_out  optional copies of the routing ([T][k]), or NULL
 * For one token in the usual decode shapes (top_k <= 8, moe_inter <= 2048,
 * shared_inter equal to moe_inter if there is a shared expert), one of the
 * kernels sizes its grid to what the device holds at once and has its
 * workgroups wait for each other; it expects the device to itself while it
 * runs.  If other work keeps some of its workgroups from starting, the wait
 * gives up after a bounded time and the rows of y it could not finish are
 * NaN.  Setting QMOE_DECODE_FUSED=0 in the environment selects kernels that
 * do not wait for each other (same results, bit for bit); QMOE_BARRIER_SPINS
 * (at most 65536, the default) lowers the number of polls before giving up,
 * which tests use to reach that path. */
moe_status moe_layer(const moe_config* cfg, int32_t T, const uint16_t* x,
                     const float* router_w, const float* bias, const moe_qexperts* routed,
                     const moe_qexperts* shared, void* y, int32_t out_dtype,
                     int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Kernel-boundary timing of moe_layer, for profiling and benchmarks.
 * events[0..MOE_TRACE_MAX] are caller-created HIP events (hipEventCreate,
 * timing enabled), all non-NULL; the library records events[0] on `stream`
 * before its first kernel and events[i] right after its i-th kernel, sets
 * n_kernels to the number of kernels it launched (<= MOE_TRACE_MAX) and
 * names[i-1] to a static name of kernel i.  The interval between events[i-1]
 * and events[i] is then kernel i's time on the stream.  Events beyond
 * n_kernels are not touched. */
#define MOE_TRACE_MAX 16
typedef struct {
  hipEvent_t events[MOE_TRACE_MAX + 1];
  int32_t n_kernels;
  const char* names[MOE_TRACE_MAX];
} moe_trace;

/* moe_layer, recording kernel-boundary events into `trace` (non-NULL; a
 * NULL event returns MOE_ERR_INVALID_ARG).  Same results as moe_layer. */
moe_status moe_layer_trace(const moe_config* cfg, int32_t T, const uint16_t* x,
                           const float* router_w, const float* bias,
                           const moe_qexperts* routed, const moe_qexperts* shared, void* y,
                           int32_t out_dtype, int32_t* topk_ids_out, float* topk_w_out,
                           void* ws, size_t ws_bytes, hipStream_t stream, moe_trace* trace);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
