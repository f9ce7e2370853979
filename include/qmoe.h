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
 *   call only (the expert cache's host store and id lists are HOST memory
 *   too, as stated there).  The caller owns every buffer, including the
 *   workspace.  The library never allocates or frees device memory; host
 *   memory only for a moe_expert_cache's bookkeeping.  Its only global state
 *   is a per-device record of how many workgroups of the single-token kernel
 *   fit on the device (computed once, read-only after) and the device buffer
 *   of moe_layer_noalloc.  Calls on different streams are independent as long
 *   as their workspaces and outputs do not overlap.
 * Alignment.  Packed weight arrays (`q`), scale arrays and `x` must be 16-byte
 *   aligned; the workspace 256-byte aligned.  Otherwise MOE_ERR_INVALID_ARG.
 * Asynchrony.  Every call only enqueues work on `stream` and returns without
 *   synchronising, except moe_layer_flags and moe_layer_cached, which wait as
 *   they state.  A launch failure returns MOE_ERR_HIP; a fault
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
 *         q = u - 8.  This is not the natural order (input 2j in the low
 *         nibble of byte j): such data must be repacked once, a fixed
 *         permutation of the eight nibbles of each word (the Python helper
 *         synth.repack_int4_natural does it); unrepacked, it decodes to
 *         wrong values without any error.
 *   scale fp16 [E][N][K/32]; weight = (u - 8) * scale.
 *   gscale must be NULL.
 * MOE_WFMT_NVFP4  E2M1 elements, one FP8 E4M3 scale per 16 inputs, one fp32
 *   scale per (expert, projection).
 *   q      uint8 [E][N][K/2]: byte j holds input 2j in the low nibble and input
 *          2j+1 in the high nibble; a nibble is an E2M1 code (bit 3 sign).
 *   scale  uint8 [E][N][K/16] E4M3 "fn" codes (bias 7, no infinities).
 *   gscale float32 [E]; weight = e2m1 * e4m3 * gscale[e].
 * Per-row-scale formats (page "Show HN: Menjalankan GLM 5.2 ...", section
 * "Fitur utama": the quantisation kernels take int8, packed int4 and packed
 * int2 with one scale per row, dequantised on use; the pages give no layout,
 * so these are the library's): symmetric integer codes and one float32 scale
 * per output row, weight = q * scale[e][n]; gscale must be NULL.
 *   MOE_WFMT_INT4_ROW_F32  q as MOE_WFMT_INT4_G32_F16 (q = u - 8);
 *                          scale float32 [E][N].
 *   MOE_WFMT_INT8_ROW_F32  q int8 [E][N][K], two's complement, input order;
 *                          scale float32 [E][N].
 *   MOE_WFMT_INT2_ROW_F32  q uint8 [E][N][K/4]: per row K/16 little-endian
 *                          32-bit words; word j holds inputs 16j..16j+15,
 *                          input 16j+2i (i = 0..7) in bits [2i, 2i+2) and
 *                          input 16j+2i+1 in bits [16+2i, 16+2i+2); a code u
 *                          in 0..3 means q = u - 2 (natural order, four inputs
 *                          per byte from bit 0 up, must be repacked:
 *                          synth.repack_int2_natural); scale float32 [E][N].
 *   In moe_layer, per-row int4 and int2 take the small-batch kernels for
 *   T <= 4 (as the group-scaled formats do), int8 the grouped GEMV
 *   (moe_expert_ffn_q4 uses the GEMV for all three); the grouped GEMM takes
 *   all of them for larger T.
 * Gate and up have N = inter, K = hidden; down has N = hidden, K = inter.
 *
 * Activations are bfloat16 [T][hidden], row-major.  For T > 4 the grouped
 * GEMM multiplies them as fp16: magnitudes of 65520 and above (beyond the
 * fp16 range) become infinities there; T <= 4 reads the bf16 values
 * directly.
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

typedef enum {
  MOE_WFMT_INT4_G32_F16 = 0,
  MOE_WFMT_NVFP4 = 1,
  MOE_WFMT_INT4_ROW_F32 = 2,
  MOE_WFMT_INT8_ROW_F32 = 3,
  MOE_WFMT_INT2_ROW_F32 = 4
} moe_wfmt;
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
  uint32_t options;                /* MOE_OPT_* bits; 0 for the defaults */
  float expert_top_p;              /* adaptive expert top-p p in [0, 1]; 0 (or 1): off */
} moe_config;

/* Adaptive expert top-p (page "Show HN: Menjalankan GLM 5.2 ...", section
 * "Mengunduh model dan menjalankannya": the --topp option; the pages name it
 * without a definition, and the reading taken here is the following).  With
 * 0 < expert_top_p < 1, after the top_k selection each token keeps only the
 * shortest prefix of its chosen experts, ordered by share s / sum(s over the
 * chosen) (descending; equal shares: lower id first), whose shares add up to
 * at least expert_top_p -- at least one expert; the kept weights are
 * renormalised (s / sum(s over the kept) * rsf).  topk_ids then hold the kept
 * ids in ascending order followed by -1, topk_w the weights followed by 0;
 * moe_permute gives dropped picks no slot (inv_perm -1), moe_combine skips
 * them, and their experts' weights are not read.  The decision is taken in
 * float64 on the float32 value of expert_top_p.  NaN or values outside
 * [0, 1] are MOE_ERR_INVALID_ARG. */

/* moe_config.options.  Unknown bits are MOE_ERR_INVALID_ARG.
 * MOE_OPT_NO_GRID_WAIT   moe_layer never runs the small-batch kernels whose
 *                        workgroups wait for each other (see moe_layer); one
 *                        to four tokens then take kernels that do not, with
 *                        results identical bit for bit.  For callers that
 *                        share the device with other work while the layer
 *                        runs.
 * MOE_OPT_GRID_WAIT_NONE those kernels' workgroups give up on the wait at
 *                        once (no poll): every row of y is NaN and the
 *                        workspace flag MOE_FLAG_GRID_WAIT_TIMEOUT is raised.
 *                        Exists to exercise the give-up path; never needed
 *                        otherwise. */
#define MOE_OPT_NO_GRID_WAIT 1u
#define MOE_OPT_GRID_WAIT_NONE 2u
/* MOE_OPT_INT8_ACTIVATIONS  W4A8 integer-dot path (page "Show HN: ...", section
 *   "Fitur utama": int8 activations in the Q8_0 manner against int4 weights,
 *   faster on batches; single rows stay in float).  Requires
 *   wfmt == MOE_WFMT_INT4_ROW_F32 (else MOE_ERR_INVALID_ARG).  For T > 4 the
 *   expert FFNs quantise their inputs to int8 with one fp32 scale per row --
 *   x per token, the fp16 SwiGLU output per (token, expert) row: scale =
 *   amax / 127, q = rint(a * (127 / amax)) clamped to +-127, in fp32 -- and
 *   multiply on the int8 matrix cores with exact int32 sums; the results
 *   then carry the activations' int8 rounding (the layer's bar is measured
 *   against a reference that rounds the same way).  T <= 4 is unaffected. */
#define MOE_OPT_INT8_ACTIVATIONS 4u

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

/* Flags raised by the last moe_layer call that used workspace `ws` (host
 * output `flags`); the first 4 bytes of every workspace hold them, and
 * moe_layer clears them before it does anything else.  The call enqueues a
 * copy on `stream` and waits for it, so it returns after all work queued on
 * `stream` before it has finished.  ws == NULL reads the flags of
 * moe_layer_noalloc's workspace on the current device.
 * MOE_FLAG_GRID_WAIT_TIMEOUT  a small-batch kernel's workgroups waited for
 *   each other in vain (other work on the device kept some from starting);
 *   the rows of y that depend on them are NaN.  Rerun with
 *   MOE_OPT_NO_GRID_WAIT. */
#define MOE_FLAG_GRID_WAIT_TIMEOUT 1u
moe_status moe_layer_flags(const void* ws, uint32_t* flags, hipStream_t stream);

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
 *   topk_ids       int32 [T][k] in: values in [0, E), or -1 for a pick the
 *                                   adaptive top-p dropped (else results
 *                                   undefined)
 *   expert_offsets int32 [E+1] out: exclusive prefix sum of per-expert counts;
 *                                   offsets[E] is the number of kept picks
 *   sorted_token   int32 [P]   out: token index of the pick at each sorted slot
 *                                   (slots past offsets[E] unspecified)
 *   inv_perm       int32 [P]   out: sorted slot of pick p, -1 if dropped
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
 *                         + shared_out[t]   (shared_out may be NULL);
 * picks with inv_perm -1 (dropped by the adaptive top-p) are skipped.
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
 * gives up after a bounded time (2^16 polls), the rows of y it could not
 * finish are NaN, and MOE_FLAG_GRID_WAIT_TIMEOUT is raised in the workspace
 * (moe_layer_flags).  For 2-4 tokens in those shapes, the gate/up workgroups
 * wait for the one that selects the experts (the first dispatched), with the
 * same bound, NaN rows and flag.  cfg->options MOE_OPT_NO_GRID_WAIT selects
 * kernels that do not wait for each other (same results, bit for bit). */
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

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  The workspace is a buffer inside the library's
 * device code, MOE_NOALLOC_WS_BYTES on every GPU the library runs on, held
 * until the process ends; the call allocates nothing (no hipMalloc, no
 * allocating library routine).  The caller still passes inputs and outputs.
 * Calls whose moe_workspace_size(cfg, T) exceeds MOE_NOALLOC_WS_BYTES return
 * MOE_ERR_UNSUPPORTED before any HIP call (the GLM-5.2 layer shape, int4
 * group-32 weights, fits up to 90 tokens).  All calls on one device share its buffer: calls that overlap
 * on one device (other streams, other threads) race and give wrong results.
 * Each call writes every workspace word it reads, so a call's results do not
 * depend on the previous call.  Otherwise as moe_layer (same kernels, same
 * results); moe_layer_flags(NULL, ...) reads its flags. */
#define MOE_NOALLOC_WS_BYTES (32u << 20)
moe_status moe_layer_noalloc(const moe_config* cfg, int32_t T, const uint16_t* x,
                             const float* router_w, const float* bias,
                             const moe_qexperts* routed, const moe_qexperts* shared, void* y,
                             int32_t out_dtype, int32_t* topk_ids_out, float* topk_w_out,
                             hipStream_t stream);

/* Expert streaming from host memory (page "Show HN: Menjalankan GLM 5.2 ...",
 * section "Cara kerja eksekusi MoE berbasis streaming disk": the routed experts
 * stay in a slow tier and come in through a least-recently-used cache per
 * layer, with an optional pinned hot store; section "Fitur utama": readahead
 * while an expert is multiplied, a router lookahead that prefetches).  The
 * slow tier here is host RAM and the fast one HBM: for layers, or models,
 * whose experts do not all fit on the device.
 *
 * A moe_expert_cache serves ONE layer on one device and owns no device memory:
 *   host_store  the E routed experts in the formats above, HOST pointers; they
 *               should be page-locked (hipHostMalloc) so that the copies are
 *               asynchronous DMA (pageable memory works, copied synchronously);
 *   slots       DEVICE arrays in the same layout for n_slots experts:
 *               q [n_slots][N][K/2], scale [n_slots][N][...], gscale [n_slots].
 * Both stay the caller's and must outlive the cache.  The cache itself is
 * host bookkeeping plus two HIP events, created by its first call that makes
 * HIP calls, on the device then current (later calls on another device:
 * MOE_ERR_INVALID_ARG).  Not thread-safe: one thread at a time per cache.
 * After a call returns MOE_ERR_HIP the slots may not hold what the cache
 * records: destroy the cache and create a new one.
 *
 * Slot policy.  A call needs the distinct experts its tokens picked (or the
 * experts a prefetch lists); resident ones are hits.  The misses are placed
 * in ascending expert order into the free slot of lowest index, else into the
 * least recently used slot that is neither pinned nor needed by the same call
 * (equal age: lowest slot).  Every slot a call or prefetch uses becomes the
 * most recently used. */
typedef struct moe_expert_cache moe_expert_cache;

typedef struct {
  uint64_t calls;        /* moe_layer_cached calls that ran their experts */
  uint64_t hits;         /* experts those calls needed and found resident */
  uint64_t misses;       /* experts those calls loaded */
  uint64_t prefetched;   /* experts loaded by moe_cache_prefetch and moe_cache_pin */
  uint64_t evictions;    /* loads that replaced a resident expert */
  uint64_t bytes_loaded; /* host-to-device bytes of all loads */
} moe_cache_stats;

/* 1 <= n_slots <= n_routed_experts; host_store and slots as above (checked
 * like moe_layer's experts: non-NULL, aligned, gscale iff NVFP4).  *cache
 * (host) receives the new cache, NULL on error.  Makes no HIP call. */
moe_status moe_cache_create(const moe_config* cfg, int32_t n_slots,
                            const moe_qexperts* host_store, const moe_qexperts* slots,
                            moe_expert_cache** cache);

/* Frees the cache (NULL: nothing).  Waits for nothing: work already queued
 * keeps reading the caller's slots. */
moe_status moe_cache_destroy(moe_expert_cache* cache);

/* The layer, as moe_layer, with the routed experts read from the cache's
 * slots.  It routes on the device, waits on the host for the routing (the call
 * synchronises `stream`), places the missing experts and enqueues their copies
 * on `stream`, then enqueues the permutation, the expert FFNs over the slots,
 * the shared expert and the combine, and returns without waiting for them.
 * The routing (topk ids and weights) equals moe_layer's; y agrees with it
 * within the layer's tolerance (these are the kernels moe_layer runs for T > 4
 * and those of moe_expert_ffn_q4 for T <= 4).  If the call needs more
 * distinct experts than the slots that are not pinned, it returns
 * MOE_ERR_UNSUPPORTED after writing the routing, and loads nothing. */
moe_status moe_layer_cached(moe_expert_cache* cache, int32_t T, const uint16_t* x,
                            const float* router_w, const float* bias,
                            const moe_qexperts* shared, void* y, int32_t out_dtype,
                            int32_t* topk_ids_out, float* topk_w_out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Readahead / router lookahead: loads the listed experts now (HOST array of
 * n ids in priority order; resident ones and repeats cost nothing), with the
 * copies on `stream`, which may be another stream than the layer's so that
 * they overlap its kernels.  It never evicts an expert of the latest
 * moe_layer_cached call (whose kernels may still run; every earlier call has
 * finished), its copies wait for the previous prefetch, and the next
 * moe_layer_cached waits for them.  Experts that find no slot are skipped;
 * *n_loaded (host, may be NULL) receives the number of experts loaded. */
moe_status moe_cache_prefetch(moe_expert_cache* cache, const int32_t* experts, int32_t n,
                              int32_t* n_loaded, hipStream_t stream);

/* Pinned hot store: loads the listed experts as moe_cache_prefetch does and
 * pins their slots, which are then never evicted (until moe_cache_unpin_all).
 * All or nothing: MOE_ERR_UNSUPPORTED, with nothing loaded or pinned, if they
 * do not all find slots. */
moe_status moe_cache_pin(moe_expert_cache* cache, const int32_t* experts, int32_t n,
                         hipStream_t stream);
moe_status moe_cache_unpin_all(moe_expert_cache* cache);

/* Counters since creation (host output). */
moe_status moe_cache_get_stats(const moe_expert_cache* cache, moe_cache_stats* stats);

/* Slot holding `expert` (host output), or -1 if it is not resident. */
moe_status moe_cache_slot_of(const moe_expert_cache* cache, int32_t expert, int32_t* slot);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
