// Grouped GEMM for prefill-shaped calls: the SwiGLU expert FFN over 4-bit
// weights on the matrix cores (page "Show HN: Menjalankan GLM 5.2 di komputer
// lambat", sections "Cara kerja eksekusi MoE" and "Fitur utama": int4
// dequant-on-use, batch-union MoE; NVFP4 per page "NVIDIA stellt neues
// GLM-5.2 NVFP4 Modell vor", section "Technische Details").
//
// Work unit = (m tile of up to 192 tokens of one expert (32 in the thin
// launch), n tile of weight rows).  Each wave dequantises its own weight rows
// straight from HBM into fp16 A operands (scale folded in, one rounding) and
// multiplies them against the unit's activations, staged in LDS as fp16, with
// v_mfma_f32_16x16x32_f16 (fp32 accumulate).
//   gate/up: 128 row pairs per unit; each wave holds 32 gate rows and the 32
//            matching up rows, so the SwiGLU epilogue pairs them in registers
//            and writes h (fp16).
//   down:    256 output rows per unit over K = inter; writes fp32 per pick.
//
// Operand layouts of v_mfma_f32_16x16x32_f16 (wave64): A lane l holds row
// l%16, K 8*(l/16)..+7; B lane l holds column l%16, the same K; D lane l holds
// rows 4*(l/16)..+3 of column l%16.  K is summed, so any K order shared by A
// and B is valid: within a 128-input block a lane loads one 16-byte chunk of
// its row (a whole 32-input group, one scale) and feeds its four 32-bit words
// to four consecutive MFMA K steps; the B reads from LDS use the same order.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "gemm_common.h"

namespace qmoe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;          // inputs per K block
constexpr int kChunks = kBK / 8;  // 16-byte chunks per activation row of a K block
// Thin units: up to kBMThin tokens of an expert with few tokens, run by the
// thin kernel, whose LDS stages hold kBMThin rows.  With few token columns a K
// block carries little MFMA work, so the thin kernel keeps more K blocks in
// flight to cover the memory latency.
#ifndef QMOE_THIN_NS
#define QMOE_THIN_NS 4
#endif
constexpr int kNSThin = QMOE_THIN_NS;

__device__ __forceinline__ uint32_t pk_fma_f16(uint32_t a, uint32_t b, uint32_t c) {
  const half2v r = __builtin_bit_cast(half2v, a) * __builtin_bit_cast(half2v, b) +
                   __builtin_bit_cast(half2v, c);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
  const half2v r = __builtin_bit_cast(half2v, a) + __builtin_bit_cast(half2v, b);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  const half2v r = __builtin_bit_cast(half2v, a) * __builtin_bit_cast(half2v, b);
  return __builtin_bit_cast(uint32_t, r);
}
// both halves of a times s (the splat is an operand modifier, not an
// instruction of its own)
__device__ __forceinline__ uint32_t pk_mul_f16_splat(uint32_t a, _Float16 s) {
  const half2v r = __builtin_bit_cast(half2v, a) * half2v{s, s};
  return __builtin_bit_cast(uint32_t, r);
}

// One 32-bit word (8 consecutive inputs of one row) -> fp16 A operand.
//   int4:  (u - 8) * scale, exact integer first, then one rounding.  The word
//          holds pair k = (u_2k, u_2k+1) in bits 4k..4k+3 of its two halves;
//          or-ing a nibble into the mantissa of fp16 1024 gives 1024 + u (bits
//          0-3) or 1024 + 16 u (bits 4-7), so pairs 0 and 1 take one
//          v_and_or each and pairs 2 and 3 share one shift by 8.
//   nvfp4: e2m1 * e4m3 (exact in fp16); the per-tensor fp32 scale is applied
//          to the accumulator in the epilogue.
template <int FMT>
__device__ __forceinline__ half8 dequant_word(uint32_t w, _Float16 scale) {
  uint32_t p[4];
  if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
    const uint32_t w8 = w >> 8;
    const uint32_t v0 = and_or(w, 0x000F000Fu, 0x64006400u);    // 1024 + u
    const uint32_t v1 = and_or(w, 0x00F000F0u, 0x64006400u);    // 1024 + 16 u
    const uint32_t v2 = and_or(w8, 0x000F000Fu, 0x64006400u);
    const uint32_t v3 = and_or(w8, 0x00F000F0u, 0x64006400u);
    // u - 8, exactly: v - 1032, or v / 16 - 72
    p[0] = pk_add_f16(v0, 0xE408E408u);
    p[1] = pk_fma_f16(v1, 0x2C002C00u, 0xD480D480u);
    p[2] = pk_add_f16(v2, 0xE408E408u);
    p[3] = pk_fma_f16(v3, 0x2C002C00u, 0xD480D480u);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = pk_mul_f16_splat(p[k], scale);
  } else {
    // natural nibble order: byte k holds inputs 2k, 2k+1
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = pk_mul_f16_splat(fp4_pair_f16(w, k), scale);
  }
  half8 r;
  __builtin_memcpy(&r, p, 16);
  return r;
}

// Per-row-scale formats: the 8 inputs of one K step of one row -> fp16 A
// operand, exact integers q (the row scale multiplies the accumulator in the
// epilogue).  w: the lane's code words of the K block; ks: the K step.
//   int4: word ks, 1024 + u (or 1024 + 16 u), then u - 8 as for int4 g32;
//   int8: words 2 ks, 2 ks + 1, sign bits flipped (u = q + 128), bytes into
//         the mantissa of fp16 1024 (1024 + u), minus 1152;
//   int2: half (ks & 1) of word ks / 2, pairs into the mantissa of fp16 1024
//         (1024 + u), minus 1026.
template <int FMT>
__device__ __forceinline__ half8 dequant_row(const uint32_t* w, int ks) {
  uint32_t p[4];
  if constexpr (FMT == MOE_WFMT_INT4_ROW_F32) {
    const uint32_t x = w[ks], x8 = x >> 8;
    p[0] = pk_add_f16(and_or(x, 0x000F000Fu, 0x64006400u), 0xE408E408u);
    p[1] = pk_fma_f16(and_or(x, 0x00F000F0u, 0x64006400u), 0x2C002C00u, 0xD480D480u);
    p[2] = pk_add_f16(and_or(x8, 0x000F000Fu, 0x64006400u), 0xE408E408u);
    p[3] = pk_fma_f16(and_or(x8, 0x00F000F0u, 0x64006400u), 0x2C002C00u, 0xD480D480u);
  } else if constexpr (FMT == MOE_WFMT_INT8_ROW_F32) {
    const uint32_t a = w[2 * ks] ^ 0x80808080u, b = w[2 * ks + 1] ^ 0x80808080u;
    p[0] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u), 0xE480E480u);
    p[1] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, a, 0x04030402u), 0xE480E480u);
    p[2] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u), 0xE480E480u);
    p[3] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u), 0xE480E480u);
  } else {
    const uint32_t x = w[ks >> 1] >> (8 * (ks & 1));
    p[0] = pk_add_f16(and_or(x, 0x00030003u, 0x64006400u), 0xE402E402u);
    p[1] = pk_add_f16(and_or(x >> 2, 0x00030003u, 0x64006400u), 0xE402E402u);
    p[2] = pk_add_f16(and_or(x >> 4, 0x00030003u, 0x64006400u), 0xE402E402u);
    p[3] = pk_add_f16(and_or(x >> 6, 0x00030003u, 0x64006400u), 0xE402E402u);
  }
  half8 r;
  __builtin_memcpy(&r, p, 16);
  return r;
}


// Activations go from HBM straight into LDS (buffer_load ... lds: lane l of a
// load writes 16 bytes at base + 16 l).  Stage layout: BM token rows of 16
// chunks of 16 bytes, chunk c of row r at slot r * 16 + (c ^ (r & 15)); the
// XOR spreads the 16 rows that one B-operand read touches over all banks.
// Load i of wave w covers slots (8 w + i) * 64 .. +63, i.e. rows 4 (8 w + i)
// + lane / 16, slot lane % 16.  Rows are padded with zeros to a multiple of
// the K block, so a partial last K block reads zeros past K.
template <int BM>
__host__ __device__ constexpr int act_loads() { return BM * kChunks / 256; }   // loads per thread per K block

// Byte offset of each of this thread's loads at K block 0 (K block kb adds
// kb * 256).
template <int PROJ, int NA>
__device__ __forceinline__ void act_rows(const GemmArgs& g, const Unit& u, int wv, int lane,
                                         uint32_t (&abase)[NA]) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = (wv * NA + i) * 4 + (lane >> 4);
    const uint32_t chunk = (uint32_t)((lane & 15) ^ (m & 15));
    uint32_t off = kOOBRow;
    if (m < u.M) {
      if constexpr (PROJ == 0) {
        const int t = u.routed ? g.sorted_token[u.tok0 + m] : u.tok0 + m;
        off = (uint32_t)t * (uint32_t)g.ldx * 2u;
      } else {
        off = (uint32_t)(u.p0 + m) * (uint32_t)g.ldh * 2u;
      }
    }
    abase[i] = off + chunk * 16u;
  }
}

template <int NA>
__device__ __forceinline__ void issue_act(const rsrc_t& ar, const uint32_t* abase, int kb,
                                          int wv, uint16_t* stage) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ar, (__attribute__((address_space(3))) void*)(stage + (wv * NA + i) * 64 * 8), 16,
        abase[i] + (uint32_t)kb * (kBK * 2), 0, 0, 0);
}

// 16 bytes per lane from buffer offset voff into LDS at dst + 16 * lane.
__device__ __forceinline__ void lds_copy16(const rsrc_t& r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 0);
}


// s_waitcnt immediate that waits for all but the n most recent vector memory
// ops (gfx9 encoding: vmcnt in bits 3-0 and 15-14, expcnt and lgkmcnt at their
// no-wait values).  Issued through the builtin, so the compiler's own wait
// insertion knows the older loads have landed and adds no waits of its own.
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}
// The same with lgkmcnt(0): this wave's LDS reads have returned as well.
__host__ __device__ constexpr int waitcnt_vm_lds(int n) { return waitcnt_vm(n) & ~(15 << 8); }

// K-block hand-over between the waves of a workgroup: this wave's loads of
// the next block have landed (LDS-DMA included: vmcnt counts them until their
// data is in LDS) and its reads of the stage about to be refilled have
// returned; then the workgroup barrier.
//   EXACT (thin units): the wait through the builtin, so the compiler's own
//   wait insertion knows the older loads have landed; no memory fence (a fence
//   makes the compiler wait for every LDS-DMA write in flight, the blocks
//   requested ahead included); the empty asm keeps memory accesses on their
//   side of the barrier and the sched_barrier keeps later work from being
//   scheduled above it.  At 64 tokens: 1.098 -> 1.083 ms per layer.
//   Otherwise (fat units) the wait as inline asm and a fenced barrier: the
//   compiler then adds waits of its own (partial drains of the blocks in
//   flight), but its schedule, which overlaps the next block's first dequant
//   and LDS reads with the current block's last MFMAs, measured faster
//   (4096 tokens: 3.8-3.9 against 4.0-4.1 ms per layer).
template <int WAITN, bool EXACT>
__device__ __forceinline__ void kblock_handover() {
  if constexpr (EXACT) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(WAITN));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WAITN) : "memory");
    __syncthreads();
  }
}

constexpr int kNS = 4;            // K blocks in flight (LDS stages, weight register ring)
constexpr int kRT = 4;            // 16-row weight tiles per wave
constexpr int kLdsBytes = 160 * 1024;
// K blocks in flight for units of BM tokens: four LDS stages where they fit
// (128 tokens: 128 KB), else three (192 tokens: 144 KB)
template <int BM>
constexpr int gemm_stages() { return 4 * BM * kBK * 2 <= kLdsBytes - 4096 ? 4 : 3; }
constexpr int kNSF = gemm_stages<kBMF>();
static_assert(3 * kBMF * kBK * 2 <= kLdsBytes - 4096, "a fat unit's LDS stages fit");


// PROJ 0: gate/up (+SwiGLU), PROJ 1: down.
//
// One workgroup of 4 waves per CU (one wave per SIMD, all 512 registers per
// lane).  BM: token rows of a unit; NS: K blocks in flight.  K loop: NS-stage
// pipeline.  K block kb + NS - 1 is requested (weights into the register
// ring, activations straight into an LDS stage) while block kb is
// multiplied; within a block, the next K step's B operands (LDS) and A
// operands (dequantised weights) are produced while the current step's MFMAs
// run.  Every K block issues the same number of vector memory ops per thread
// (blocks past K are requested too and never read), so "block kb + 1 has
// landed" is vmcnt <= WAITN, the ops of the NS - 2 blocks after it, once
// block kb + NS - 1 is requested.  One barrier per K block, before its last
// K step.
#ifndef QMOE_THIN_WGS
#define QMOE_THIN_WGS 2
#endif
//
// Scales.  Each lane needs one 2-byte scale per K block, scattered over 16
// rows per load; loaded per block, these requests cost as much as the codes.
// SL (thin units, K % 512 == 0): each wave instead copies the scales of its 64 rows for
// four K blocks at a time (a "super-block", 32 bytes per row) straight into
// LDS with two 16-byte-per-lane loads, three super-blocks deep, and reads its
// 2 bytes from there.  The copy for super-block S + 1 rides on the even K
// blocks of super-block S, so every two K blocks carry one extra load.
// Otherwise (ragged K) each lane loads its own 2 bytes per block.
constexpr int kSclBytesPerWave = 3 * 2 * 1024;   // three super-blocks x two 1 KB copies

// int8 codes take twice the ring registers: its thin units run one
// workgroup per CU, which leaves them the registers they need unspilled.
template <int FMT, int BM>
constexpr int gemm_wgs_per_cu() {
  return BM == kBMThin && FMT != MOE_WFMT_INT8_ROW_F32 ? QMOE_THIN_WGS : 1;
}

template <int FMT, int PROJ, int BM, int NS, bool SL>
__global__ void __launch_bounds__(256, (gemm_wgs_per_cu<FMT, BM>())) moe_gemm_kernel(GemmArgs g) {
  constexpr int RT = kRT;
  constexpr int NA = act_loads<BM>();
  constexpr bool ROW = wfmt_row(FMT);
  constexpr int BITS = wfmt_bits(FMT);
  constexpr int WPL = BITS;                  // code words per lane per K block (32 inputs)
  constexpr int CL = BITS == 8 ? 2 : 1;      // code loads per row tile per K block
  static_assert(!SL || NS == 4, "the scale copies ride on K blocks 0 and 2 of each group of four");
  static_assert(NS * BM * kBK * 2 + (SL ? 4 * kSclBytesPerWave : 16) <= kLdsBytes, "LDS stages fit");
  static_assert(!(ROW && SL), "per-row scales are read in the epilogue");
  // vector memory ops per thread issued for K blocks kb + 2 .. kb + NS - 1:
  // all that may still be in flight once block kb + 1 has landed
  constexpr int WAITN = (NS - 2) * (NA + RT * CL + (SL || ROW ? 0 : RT)) + (SL ? 1 : 0);
  static_assert(WAITN < 64, "vmcnt holds 6 bits");
  __shared__ __attribute__((aligned(16))) uint16_t xs[NS][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t scl[SL ? 4 * kSclBytesPerWave : 16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int max_inter = max(g.routed.inter, g.has_shared ? g.shared.inter : 0);
  const int NT = PROJ == 0 ? (max_inter + kGateUpPairs - 1) / kGateUpPairs
                           : (g.H + kDownRows - 1) / kDownRows;
  constexpr bool thin = BM == kBMThin;
  const int total = __builtin_amdgcn_readfirstlane(g.n_tiles[thin ? 1 : 0]) * NT;
  if ((int)blockIdx.x >= total) return;
  const int w = xcd_item(blockIdx.x, total);
  const int uidx = w / NT;
  const int nt = w - uidx * NT;
  const Unit u = load_unit(thin ? g.tiles + g.thin_off : g.tiles, uidx);
  const ExpertSet& X = u.routed ? g.routed : g.shared;
  const int inter = X.inter;
  const int K = PROJ == 0 ? g.H : inter;
  const int nrow_out = PROJ == 0 ? inter : g.H;
  // first output row of this wave (gate/up: row pairs)
  const int wrow = PROJ == 0 ? nt * kGateUpPairs + wv * 32 : nt * kDownRows + wv * 64;
  if (nt * (PROJ == 0 ? kGateUpPairs : kDownRows) >= nrow_out) return;
  const uint32_t rowBytes = (uint32_t)K * BITS / 8;
  const int sgpr = FMT == MOE_WFMT_INT4_G32_F16 ? 32 : 16;   // inputs per scale
  const uint32_t scaleRowBytes = ROW ? 4u : (uint32_t)(K / sgpr) * (FMT == MOE_WFMT_INT4_G32_F16 ? 2 : 1);

  // One buffer per projection over this expert's whole matrix (codes and
  // scales); rows past the end read as zero through the range check.
  constexpr int NPJ = PROJ == 0 ? 2 : 1;
  rsrc_t qb[NPJ], sb[NPJ];
  float gsc[NPJ];
#pragma unroll
  for (int j = 0; j < NPJ; ++j) {
    const ProjPtr& P = PROJ == 0 ? (j == 0 ? X.gate : X.up) : X.down;
    const size_t row0 = (size_t)u.e * nrow_out;
    qb[j] = make_rsrc(P.q + row0 * rowBytes, (uint32_t)nrow_out * rowBytes);
    sb[j] = make_rsrc(reinterpret_cast<const uint8_t*>(P.s) + row0 * scaleRowBytes,
                      (uint32_t)nrow_out * scaleRowBytes);
    gsc[j] = FMT == MOE_WFMT_NVFP4 ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                         __builtin_bit_cast(int, P.g[u.e])))
                                   : 1.0f;
  }
  // row tiles of this wave: gate/up rt 0,1 gate rows, rt 2,3 the matching up
  // rows; down rt 0..3 consecutive rows
  int rbase[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) rbase[rt] = PROJ == 0 ? wrow + 16 * (rt & 1) : wrow + 16 * rt;
  const int lrow = lane & 15, lq = lane >> 4;
  const int nkb = (K + kBK - 1) / kBK;
  const int nct = (u.M + 15) >> 4;

  // weights of one K block: lane (lrow, lq) loads group 4 kb + lq of its row.
  // Groups past the row (a partial last K block) meet zero activations; rows
  // past the matrix read zeros through the range check.
  uint32_t qoff[RT], soff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    qoff[rt] = (uint32_t)(rbase[rt] + lrow) * rowBytes + (uint32_t)lq * (4u * WPL);
    soff[rt] = (uint32_t)(rbase[rt] + lrow) * scaleRowBytes + (uint32_t)lq * 2u;   // !SL
  }
  // SL: copy q (0, 1) of a super-block holds 32 rows x 32 bytes; lane l
  // copies half l & 1 of row l >> 1 (gate/up: copy 0 the gate rows, copy 1
  // the up rows; down: copy q rows 32 q ..).  Lane (lrow, lq) reads row
  // 16 (rt & 1) + lrow of copy rt >> 1, byte 8 (kb & 3) + 2 lq.
  uint8_t* const sclw = scl + (SL ? wv * kSclBytesPerWave : 0);
  uint32_t scopy[2], sread[RT];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    scopy[q] = (uint32_t)(wrow + (PROJ == 0 ? 0 : 32 * q) + (lane >> 1)) * scaleRowBytes +
               16u * (uint32_t)(lane & 1);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    sread[rt] = (uint32_t)((rt >> 1) * 1024 + 32 * (16 * (rt & 1) + lrow) + 2 * lq);
  // copy q of super-block sbk into its LDS slot (sbk % 3)
  auto copy_scales = [&](int q, int sbk) {
    const int j = PROJ == 0 ? q : 0;
    lds_copy16(sb[j], sclw + (sbk % 3) * 2048 + q * 1024, scopy[q] + (uint32_t)sbk * 32u);
  };
  uint32_t wcode[NS][RT][WPL], wsc[NS][RT];
  const rsrc_t ar = PROJ == 0 ? make_rsrc(g.x16, (uint32_t)g.T * (uint32_t)g.ldx * 2u)
                              : make_rsrc(g.hin, (uint32_t)(g.P + g.T) * (uint32_t)g.ldh * 2u);
  uint32_t arow[NA];
  act_rows<PROJ, NA>(g, u, wv, lane, arow);

  // request K block kb into stage S (LDS) and ring slot S (registers); kb is
  // congruent to S modulo NS, so (kb & 3) is known here
  auto issue = [&](auto S, int kb) {
    constexpr int st = decltype(S)::value;
    issue_act<NA>(ar, arow, kb, wv, xs[st]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int j = PROJ == 0 ? rt >> 1 : 0;
      const uint32_t kq = qoff[rt] + (uint32_t)kb * (16u * WPL);
      if constexpr (BITS == 2) {
        bload8(wcode[st][rt], qb[j], kq, 0);
      } else {
#pragma unroll
        for (int h = 0; h < CL; ++h)
          bload16(*reinterpret_cast<uint32_t(*)[4]>(&wcode[st][rt][4 * h]), qb[j], kq + 16u * h, 0);
      }
      if constexpr (!SL && !ROW) wsc[st][rt] = bload_u16(sb[j], soff[rt] + (uint32_t)kb * 8u, 0);
    }
    if constexpr (SL && (st & 1) == 0) copy_scales(st >> 1, (kb >> 2) + 1);
  };
  // SL: this lane's scales of K block kb (congruent to S) into ring slot S
  auto read_scales = [&](auto S, int kb) {
    constexpr int st = decltype(S)::value;
    if constexpr (SL) {
      const uint8_t* base = sclw + ((kb >> 2) % 3) * 2048 + 8 * st;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        wsc[st][rt] = *reinterpret_cast<const uint16_t*>(base + sread[rt]);
    }
  };
  // A operands (dequantised weights) of K step ks from ring slot S
  auto dequant_ks = [&](auto S, int ks, half8 (&A)[RT]) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (ROW) {
        A[rt] = dequant_row<FMT>(wcode[st][rt], ks);
        continue;
      }
      _Float16 sh;
      const uint32_t sw = wsc[st][rt];
      if constexpr (FMT == MOE_WFMT_INT4_G32_F16) {
        sh = __builtin_bit_cast(_Float16, (uint16_t)sw);
      } else {
        // inputs 0-15 of the group use scale byte 0, 16-31 byte 1
        sh = (_Float16)e4m3_to_f32(sw, ks >> 1);
      }
      A[rt] = dequant_word<FMT == MOE_WFMT_NVFP4 ? FMT : MOE_WFMT_INT4_G32_F16>(wcode[st][rt][ks], sh);
    }
  };

  auto run = [&](auto CTC) {
    constexpr int CT = decltype(CTC)::value;   // column tiles computed (>= nct)
    float4v acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[rt][c] = float4v{0.f, 0.f, 0.f, 0.f};
    half8 A[2][RT], B[2][CT];
    auto read_b = [&](const uint16_t* xb, int ks, half8 (&Bv)[CT]) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
        Bv[c] = *reinterpret_cast<const half8*>(xb + (16 * c + lrow) * kBK +
                                                 (((lq * 4 + ks) ^ lrow) * 8));
    };
    auto mfmas = [&](const half8 (&Av)[RT], const half8 (&Bv)[CT]) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av[rt], Bv[c], acc[rt][c], 0, 0, 0);
    };
    // interleave: each MFMA followed by its share of the next step's VALU and
    // LDS reads
    auto interleave = [&]() {
      constexpr int NM = RT * CT;
      constexpr int VPM = (16 * RT + NM - 1) / NM;   // dequant VALU per MFMA
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        if (i % RT == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };

    if constexpr (SL) {   // super-block 0's scales, ahead of every K block
      copy_scales(0, 0);
      copy_scales(1, 0);
    }
    static_for<NS - 1>([&](auto J) { issue(J, J); });
    kblock_handover<WAITN, thin>();
    read_scales(ic<0>{}, 0);
    read_b(xs[0], 0, B[0]);
    dequant_ks(ic<0>{}, 0, A[0]);

    auto kblock = [&](auto S, int kb) {
      constexpr int st = decltype(S)::value;
      constexpr int sn = (st + 1) % NS;
      constexpr int s3 = (st + NS - 1) % NS;
      // stage s3 held block kb - 1, whose last reads every wave finished
      // before the barrier of block kb - 1
      issue(ic<s3>{}, kb + NS - 1);
      // block kb + 1's scales: their copy rode on block kb - 1 or earlier,
      // which has landed
      read_scales(ic<sn>{}, kb + 1);
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        read_b(xs[st], ks + 1, B[(ks + 1) & 1]);
        dequant_ks(ic<st>{}, ks + 1, A[(ks + 1) & 1]);
        mfmas(A[ks & 1], B[ks & 1]);
        interleave();
      }
      // block kb + 1 landed in every wave (blocks up to kb + NS - 1 may be in flight)
      kblock_handover<WAITN, thin>();
      read_b(xs[sn], 0, B[0]);
      dequant_ks(ic<sn>{}, 0, A[0]);
      mfmas(A[1], B[1]);
      interleave();
    };
    if constexpr (thin) {
      // whole groups of NS blocks without branches (a block skipped on one
      // path would leave the compiler's wait counts merged from the shallower
      // pipeline, and it would drain the loads in flight), then the rest
      int kb = 0;
      for (; kb + NS <= nkb; kb += NS) static_for<NS>([&](auto J) { kblock(J, kb + J); });
      static_for<NS - 1>([&](auto J) {
        if (kb + J < nkb) kblock(J, kb + J);
      });
    } else {
      for (int kb = 0; kb < nkb; kb += NS)
        static_for<NS>([&](auto J) {
          if (kb + J < nkb) kblock(J, kb + J);
        });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // per-row formats: the scales of this lane's four rows of each tile
    // (rows past the matrix read zeros through the range check)
    float rsc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (ROW) {
        uint32_t v[4];
        bload16(v, sb[PROJ == 0 ? rt >> 1 : 0], (uint32_t)(rbase[rt] + 4 * lq) * 4u, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) rsc[rt][i] = __uint_as_float(v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) rsc[rt][i] = gsc[PROJ == 0 ? rt >> 1 : 0];
      }
    }

    // epilogue
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int m = 16 * c + lrow;
      if (m >= u.M) continue;
      const int orow = u.p0 + m;
      if constexpr (PROJ == 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          uint32_t packed[2];
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float h0 = silu_mul(acc[rt][c][i] * rsc[rt][i], acc[rt + 2][c][i] * rsc[rt + 2][i]);
            const float h1 = silu_mul(acc[rt][c][i + 1] * rsc[rt][i + 1],
                                      acc[rt + 2][c][i + 1] * rsc[rt + 2][i + 1]);
            const _Float16 a0 = (_Float16)h0, a1 = (_Float16)h1;
            packed[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          }
          // columns from inter up to the padded stride hold zeros (the
          // down projection's last K block reads them)
          const int col = rbase[rt] + 4 * lq;
          if (col < inter)
            *reinterpret_cast<uint2*>(g.h_out + (size_t)orow * g.ldh + col) =
                make_uint2(packed[0], packed[1]);
          else if (col < pad_k(inter))
            *reinterpret_cast<uint2*>(g.h_out + (size_t)orow * g.ldh + col) = make_uint2(0u, 0u);
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int col = rbase[rt] + 4 * lq;
          if (col < g.H) {
            float4 o;
            o.x = acc[rt][c][0] * rsc[rt][0];
            o.y = acc[rt][c][1] * rsc[rt][1];
            o.z = acc[rt][c][2] * rsc[rt][2];
            o.w = acc[rt][c][3] * rsc[rt][3];
            *reinterpret_cast<float4*>(g.o_out + (size_t)orow * g.H + col) = o;
          }
        }
      }
    }
  };
  if constexpr (thin) {
    // units of at most 16 tokens (most of them at small batch) need one
    // column tile: half the B reads and MFMAs
    if (nct > 1)
      run(ic<kBMThin / 16>{});
    else
      run(ic<1>{});
  } else {
    // 129-160 tokens (common at ~128 tokens per expert) take ten column tiles
    if constexpr (BM / 16 > 10) {
      if (nct > 10) {
        run(ic<BM / 16>{});
        return;
      }
    }
    if constexpr (BM / 16 > 8) {
      if (nct > 8) {
        run(ic<(BM / 16 > 10 ? 10 : BM / 16)>{});
        return;
      }
    }
    if (nct > 4)
      run(ic<8>{});
    else if (nct > 2)
      run(ic<4>{});
    else
      run(ic<2>{});
  }
}

// bf16 -> fp16 copy of the activations (exact for |x| in the fp16 normal
// range) into rows of ldx elements, zero past H.  One thread per 8 elements.
__global__ void __launch_bounds__(256) x_to_f16_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ y, int T, int H,
                                                       int ldx) {
  const int c8 = ldx / 8;
  const size_t n8 = (size_t)T * c8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const int t = (int)(i / c8), c = (int)(i % c8);
    uint4 o = make_uint4(0, 0, 0, 0);
    if (c * 8 < H) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)t * H + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 lo = (_Float16)bf16_lo(w[j]), hi = (_Float16)bf16_hi(w[j]);
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      o = make_uint4(r[0], r[1], r[2], r[3]);
    }
    *reinterpret_cast<uint4*>(y + (size_t)t * ldx + c * 8) = o;
  }
}

// Work units: for each active expert (ascending) its sorted slots in slices of
// bm, then the shared expert's tokens in slices of bm (bm = BMF, or kBMNarrow
// when units of BMF would be few).
// tiles[i] = {expert or -1, first h/O row, tokens, first sorted slot or token}.
template <int BMF>
__global__ void __launch_bounds__(64) build_units_kernel(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ active,
                                                         const int32_t* __restrict__ n_active,
                                                         int4* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles, int T, int P,
                                                         int has_shared, int thin_off) {
  const int lane = threadIdx.x;
  const int na = n_active ? *n_active : 0;
  int4* thin = tiles + thin_off;
  // fat units if every expert with more than kBMThin tokens took units of bm
  auto count_fat = [&](int bm) {
    int n = 0;
    for (int a = lane; a < na; a += 64) {
      const int e = active[a];
      const int M = offsets[e + 1] - offsets[e];
      n += M > kBMThin ? (M + bm - 1) / bm : 0;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d, 64);
    if (has_shared && T > kBMThin) n += (T + bm - 1) / bm;
    return n;
  };
  // Units of BMF tokens when there are enough of them to fill the chip for a
  // few rounds; else units of kBMNarrow, which spread the same experts over
  // more workgroups.
  int bm = BMF, nfat = count_fat(BMF);
  if (BMF > kBMNarrow && nfat < kFewWide) {
    bm = kBMNarrow;
    nfat = count_fat(bm);
  }
  // when there are fewer than kFewFat fat units, their launch would leave
  // most of the chip idle, so every expert is cut into thin units instead
  const int thin_max = nfat < kFewFat ? 0x7fffffff : kBMThin;   // most tokens of a thin-cut expert
  int base = 0, tbase = 0;   // fat units, thin units so far
  for (int a0 = 0; a0 < na; a0 += 64) {
    const int a = a0 + lane;
    int e = 0, o = 0, M = 0, nm = 0, nt = 0;
    if (a < na) {
      e = active[a];
      o = offsets[e];
      M = offsets[e + 1] - o;
      nt = M <= thin_max ? (M + kBMThin - 1) / kBMThin : 0;
      nm = nt ? 0 : (M + bm - 1) / bm;
    }
    // exclusive prefixes of the fat and thin unit counts across the wave
    int pre = nm, tpre = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(pre, d, 64), tv = __shfl_up(tpre, d, 64);
      if (lane >= d) {
        pre += v;
        tpre += tv;
      }
    }
    const int excl = base + pre - nm;
    for (int i = 0; i < nm; ++i) {
      const int m0 = i * bm;
      tiles[excl + i] = make_int4(e, o + m0, min(bm, M - m0), o + m0);
    }
    for (int i = 0; i < nt; ++i) {
      const int m0 = i * kBMThin;
      thin[tbase + tpre - nt + i] = make_int4(e, o + m0, min(kBMThin, M - m0), o + m0);
    }
    base += __shfl(pre, 63, 64);
    tbase += __shfl(tpre, 63, 64);
  }
  if (has_shared) {
    if (T <= thin_max) {
      const int ns = (T + kBMThin - 1) / kBMThin;
      for (int i = lane; i < ns; i += 64)
        thin[tbase + i] = make_int4(-1, P + i * kBMThin, min(kBMThin, T - i * kBMThin), i * kBMThin);
      tbase += ns;
    } else {
      const int ns = (T + bm - 1) / bm;
      for (int i = lane; i < ns; i += 64) {
        const int t0 = i * bm;
        tiles[base + i] = make_int4(-1, P + t0, min(bm, T - t0), t0);
      }
      base += ns;
    }
  }
  if (lane == 0) {
    n_tiles[0] = base;
    n_tiles[1] = tbase;
  }
}

}  // namespace

// Most work units of each kind: fat units hold up to bmf tokens of an expert
// with more than kBMThin of them, thin units up to kBMThin tokens of an
// expert (or the shared expert) with at most kBMThin, or of any expert when
// there would be fewer than kFewFat fat units.
long fat_units_max(int T, int K, int E, bool has_shared, int bmf) {
  bmf = std::min(bmf, kBMNarrow);   // build_units may fall back to narrow units
  const long P = (long)T * K;
  const long fat_experts = std::min<long>(E, P / (kBMThin + 1));
  const long routed = (P + bmf - 1) / bmf + fat_experts;
  const long shared = has_shared && T > kBMThin ? (T + bmf - 1) / bmf : 0;
  return routed + shared;
}
long thin_units_max(int T, int K, int E, bool has_shared, int bmf) {
  const long P = (long)T * K;
  // one per expert with at most kBMThin tokens (and the shared expert's one);
  // when fewer than kFewFat fat units are cut up, each gives at most
  // bmf / kBMThin thin units
  return std::min<long>(E, P) + (has_shared ? 1 : 0) + (long)(kFewFat - 1) * (bmf / kBMThin);
}

hipError_t launch_build_units(const int32_t* offsets, const int32_t* active,
                              const int32_t* n_active, int4* tiles, int32_t* n_tiles, int T, int P,
                              int K, int E, bool has_shared, hipStream_t s, int bmf) {
  const int thin_off = (int)fat_units_max(T, K, E, has_shared, bmf);
  if (bmf == kBMQ)
    hipLaunchKernelGGL(build_units_kernel<kBMQ>, dim3(1), dim3(64), 0, s, offsets, active, n_active, tiles,
                       n_tiles, T, P, has_shared ? 1 : 0, thin_off);
  else if (bmf == kBMF)
    hipLaunchKernelGGL(build_units_kernel<kBMF>, dim3(1), dim3(64), 0, s, offsets, active, n_active, tiles,
                       n_tiles, T, P, has_shared ? 1 : 0, thin_off);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Work units: for each active expert (ascending) its sorted slots, in thin
// units of kBMThin or fat units of kBMF (kBMQ); then the shared expert's tokens
// likewise.
// tiles[i] = {expert or -1, first h/O row, tokens, first sorted slot or
// token}; the thin units start at tiles[thin_off].
int gemm_max_units(int T, int K, int E, bool has_shared) {
  // the larger of the two unit tables (fat units of kBMF or kBMQ tokens)
  return (int)std::max(fat_units_max(T, K, E, has_shared, kBMF) + thin_units_max(T, K, E, has_shared, kBMF),
                       fat_units_max(T, K, E, has_shared, kBMQ) + thin_units_max(T, K, E, has_shared, kBMQ));
}
int gemm_thin_offset(int T, int K, int E, bool has_shared, int bmf) {
  return (int)fat_units_max(T, K, E, has_shared, bmf);
}
bool gemm_fits(int64_t T, int64_t rows, int64_t ldx, int64_t ldh) {
  return T * ldx * 2 <= (int64_t)kOOBRow && rows * ldh * 2 <= (int64_t)kOOBRow;
}

hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, int T, int H, int ldx, hipStream_t s) {
  const size_t n8 = (size_t)T * (ldx / 8);
  const int blocks = (int)std::min<size_t>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(x_to_f16_kernel, dim3(blocks), dim3(256), 0, s, x, y, T, H, ldx);
  return hipGetLastError();
}

template <int PROJ, int BM, int NS>
hipError_t launch_gemm_kernel(const GemmArgs& g, long units, int nt, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)(units * nt));
  // scales through LDS: thin units (for the MFMA-bound fat units the copies
  // cost more than they save), every K of this projection (hidden; routed
  // and shared inter) a multiple of 512
  bool sdw;
  if (PROJ == 0)
    sdw = g.H % 512 == 0;
  else
    sdw = g.routed.inter % 512 == 0 && (!g.has_shared || g.shared.inter % 512 == 0);
  sdw = sdw && BM == kBMThin;
  dispatch_wfmt(g.wfmt, [&](auto F) {
    constexpr int fmt = decltype(F)::value;
    // per-row formats have no per-block scales to copy; fat units load them
    // per block
    if constexpr (wfmt_row(fmt) || BM != kBMThin) {
      hipLaunchKernelGGL((moe_gemm_kernel<fmt, PROJ, BM, NS, false>), grid, dim3(256), 0, s, g);
    } else {
      if (sdw)
        hipLaunchKernelGGL((moe_gemm_kernel<fmt, PROJ, BM, NS, true>), grid, dim3(256), 0, s, g);
      else
        hipLaunchKernelGGL((moe_gemm_kernel<fmt, PROJ, BM, NS, false>), grid, dim3(256), 0, s, g);
    }
    return 0;
  });
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int K, int E, hipStream_t s, Tracer* tr) {
  hipError_t e;
  int max_inter = g.routed.inter;
  if (g.has_shared && g.shared.inter > max_inter) max_inter = g.shared.inter;
  const long fat = fat_units_max(g.T, K, E, g.has_shared, kBMF);
  const long thin = thin_units_max(g.T, K, E, g.has_shared, kBMF);
  // one workgroup per work item (unit, n tile); items past the actual number
  // of units exit at once
  const int ntg = (max_inter + kGateUpPairs - 1) / kGateUpPairs;
  const int ntd = (g.H + kDownRows - 1) / kDownRows;
  if ((e = launch_gemm_kernel<0, kBMF, kNSF>(g, fat, ntg, s)) != hipSuccess) return e;
  if ((e = launch_gemm_kernel<0, kBMThin, kNSThin>(g, thin, ntg, s)) != hipSuccess) return e;
  if (tr && (e = tr->mark("gemm_gateup")) != hipSuccess) return e;
  if ((e = launch_gemm_kernel<1, kBMF, kNSF>(g, fat, ntd, s)) != hipSuccess) return e;
  if ((e = launch_gemm_kernel<1, kBMThin, kNSThin>(g, thin, ntd, s)) != hipSuccess) return e;
  if (tr && (e = tr->mark("gemm_down")) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace qmoe
