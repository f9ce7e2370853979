// W4A8 grouped GEMM: the SwiGLU expert FFN as integer dot products on the
// int8 matrix cores (page "Show HN: Menjalankan GLM 5.2 di komputer lambat",
// section "Fitur utama yang diimplementasikan": an integer-dot kernel with int8
// activations in the Q8_0 manner, int4 weights faster on batches).
//
// Weights: per-row int4 (MOE_WFMT_INT4_ROW_F32), codes u = q + 8 in the int4
// word layout, one fp32 scale per row.  Activations: int8 with one fp32 scale
// per row -- x per token, the fp16 SwiGLU output h per (token, expert) row --
// quantised by quant_rows_kernel (amax, q = rint(a * 127/amax) in fp32, the
// decisions the oracle takes too).  Both scales factor out of a row's dot
// product, so a unit accumulates sum_k u_k q_k exactly in int32 and the
// epilogue applies (acc - 8 sum_k q_k) * s_w * s_a once.
//
// v_mfma_i32_16x16x64_i8: A lane l holds 16 int8 K values of row l%16, B lane
// l the same 16 K values of column l%16, D lane l rows 4*(l/16)..+3 of column
// l%16; any K order shared by A and B is valid.  A lane (lrow, lq) owns
// inputs 32 lq .. 32 lq + 31 of each 128-input K block (one 16-byte load of
// codes) and feeds them to two K steps.  The codes need no arithmetic beyond
// two masks: (w & 0x0f0f0f0f) holds the codes of inputs 0, 4, 1, 5 of the
// word's eight and ((w >> 4) & 0x0f0f0f0f) those of 2, 6, 3, 7, so the
// quantiser stores each eight int8 activations in that order and the B bytes
// line up with no shuffle.
#include <algorithm>

#include "gemm_common.h"

namespace qmoe {
namespace {

typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kBKq = 128;            // inputs (= int8 bytes) per K block
constexpr int kChq = kBKq / 16;      // 16-byte chunks per activation row of a K block
constexpr int kNSq = 4;              // K blocks in flight
constexpr int kRTq = 4;              // 16-row weight tiles per wave

// Position of input w (0..7) of an 8-input chunk in the stored int8 order
// 0, 4, 1, 5, 2, 6, 3, 7.
__host__ __device__ constexpr int q_pos(int w) { return (w & 3) * 2 + (w >> 2); }

// ---------------------------------------------------------------------------
// Row quantiser.  One block per row: amax, then codes in the chunk order
// above (zeros past the row's n inputs up to ld), their sum and the scale.
// SRC_BF16: rows of bf16 x; else rows of fp16 h whose width is `n` for rows
// below `split` and `n2` from there on (routed picks, then the shared expert).
// ---------------------------------------------------------------------------
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ src, int ld_src,
                                                         int split, int n, int n2, int8_t* __restrict__ dst,
                                                         int ld_dst, float* __restrict__ scale,
                                                         int32_t* __restrict__ sum) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  const int r = blockIdx.x;
  const int cols = r < split ? n : n2;
  const uint16_t* row = src + (size_t)r * ld_src;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  auto val = [&](uint16_t b) -> float {
    if constexpr (SRC_BF16) return __uint_as_float((uint32_t)b << 16);
    return (float)__builtin_bit_cast(_Float16, b);
  };
  float amax = 0.0f;
  for (int c = threadIdx.x; c * 8 < cols; c += 256) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(val((uint16_t)(w[j] & 0xffffu))));
      amax = fmaxf(amax, fabsf(val((uint16_t)(w[j] >> 16))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) red_f[wv] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  int acc = 0;
  for (int c = threadIdx.x; c * 8 < ld_dst; c += 256) {
    uint32_t lo = 0, hi = 0;
    if (c * 8 < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t b = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
        const int q = (int)fminf(fmaxf(rintf(val(b) * inv), -127.0f), 127.0f);
        acc += q;
        const int p = q_pos(i);
        const uint32_t byte = (uint32_t)(q & 0xff) << (8 * (p & 3));
        if (p < 4) lo |= byte; else hi |= byte;
      }
    }
    *reinterpret_cast<uint2*>(dst + (size_t)r * ld_dst + c * 8) = make_uint2(lo, hi);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) red_i[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    scale[r] = amax / 127.0f;
    sum[r] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
  }
}

// ---------------------------------------------------------------------------
// The GEMM.  Same work items, XCD mapping and K pipeline as the fp16 grouped
// GEMM (csrc/gemm.hip): four waves, each 64 weight rows x BM tokens; NS K
// blocks in flight, codes into a register ring, activations straight into
// LDS.  Its fat units hold kBMQ = 192 tokens instead of 128 (the int8 path
// has the registers, its dequantisation being two masks): at 4096 tokens an
// expert's weights are then read once instead of twice for most experts
// (2.95 -> 2.61 ms per layer; 256-token units spill and ran 2.79).  Stage layout: BM rows of 8 chunks of 16 bytes, chunk c of row r
// at slot r * 8 + (c ^ ((r >> 1) & 7)), so the 16 rows of one B read (two
// rows per 256-byte bank row) fall on distinct banks.  Load i of wave w covers
// slots (w NA + i) * 64 .. +63: rows 8 (w NA + i) + lane / 8, slot lane % 8.
// ---------------------------------------------------------------------------
template <int BM>
__host__ __device__ constexpr int act_loads_q() { return BM * kChq / 256; }

template <int PROJ, int NA>
__device__ __forceinline__ void act_rows_q(const GemmQArgs& g, const Unit& u, int wv, int lane,
                                           uint32_t (&abase)[NA]) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = (wv * NA + i) * 8 + (lane >> 3);
    const uint32_t chunk = (uint32_t)((lane & 7) ^ ((m >> 1) & 7));
    uint32_t off = kOOBRow;
    if (m < u.M) {
      if constexpr (PROJ == 0) {
        const int t = u.routed ? g.sorted_token[u.tok0 + m] : u.tok0 + m;
        off = (uint32_t)t * (uint32_t)g.ldxq;
      } else {
        off = (uint32_t)(u.p0 + m) * (uint32_t)g.ldhq;
      }
    }
    abase[i] = off + chunk * 16u;
  }
}

// 16 bytes per lane from buffer offset voff into LDS at dst + 16 * lane.
__device__ __forceinline__ void lds_dma16(const rsrc_t& r, int8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 0);
}

template <int PROJ, int BM, int NS>
__global__ void __launch_bounds__(256, BM == kBMThin ? 2 : 1) moe_gemm_q_kernel(GemmQArgs g) {
  constexpr int RT = kRTq;
  constexpr int NA = act_loads_q<BM>();
  // vector memory ops per thread for K blocks kb + 2 and kb + 3: all that may
  // still be in flight once block kb + 1 has landed
  constexpr int WAITN = 2 * (NA + RT);
  __shared__ __attribute__((aligned(16))) int8_t xs[NS][BM * kBKq];
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
  const int wrow = PROJ == 0 ? nt * kGateUpPairs + wv * 32 : nt * kDownRows + wv * 64;
  if (nt * (PROJ == 0 ? kGateUpPairs : kDownRows) >= nrow_out) return;
  const uint32_t rowBytes = (uint32_t)K / 2;

  constexpr int NPJ = PROJ == 0 ? 2 : 1;
  rsrc_t qb[NPJ], sb[NPJ];
#pragma unroll
  for (int j = 0; j < NPJ; ++j) {
    const ProjPtr& P = PROJ == 0 ? (j == 0 ? X.gate : X.up) : X.down;
    const size_t row0 = (size_t)u.e * nrow_out;
    qb[j] = make_rsrc(P.q + row0 * rowBytes, (uint32_t)nrow_out * rowBytes);
    sb[j] = make_rsrc(reinterpret_cast<const float*>(P.s) + row0, (uint32_t)nrow_out * 4u);
  }
  int rbase[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) rbase[rt] = PROJ == 0 ? wrow + 16 * (rt & 1) : wrow + 16 * rt;
  const int lrow = lane & 15, lq = lane >> 4;
  const int nkb = (K + kBKq - 1) / kBKq;
  const int nct = (u.M + 15) >> 4;
  uint32_t qoff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) qoff[rt] = (uint32_t)(rbase[rt] + lrow) * rowBytes + (uint32_t)lq * 16u;

  uint32_t wcode[NS][RT][4];
  const rsrc_t ar = PROJ == 0 ? make_rsrc(g.xq, (uint32_t)g.T * (uint32_t)g.ldxq)
                              : make_rsrc(g.hq, (uint32_t)(g.P + g.T) * (uint32_t)g.ldhq);
  uint32_t arow[NA];
  act_rows_q<PROJ, NA>(g, u, wv, lane, arow);

  auto issue = [&](auto S, int kb) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_dma16(ar, xs[st] + (wv * NA + i) * 64 * 16, arow[i] + (uint32_t)kb * kBKq);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      bload16(wcode[st][rt], qb[PROJ == 0 ? rt >> 1 : 0], qoff[rt] + (uint32_t)kb * 64u, 0);
  };
  // A of K step ks (inputs 16 ks .. 16 ks + 15 of the lane's 32): codes of
  // words 2 ks and 2 ks + 1, each as (w & m, (w >> 4) & m)
  auto codes_ks = [&](auto S, int ks, int4v (&A)[RT]) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t w0 = wcode[st][rt][2 * ks], w1 = wcode[st][rt][2 * ks + 1];
      A[rt] = int4v{(int)(w0 & 0x0f0f0f0fu), (int)((w0 >> 4) & 0x0f0f0f0fu), (int)(w1 & 0x0f0f0f0fu),
                    (int)((w1 >> 4) & 0x0f0f0f0fu)};
    }
  };

  auto run = [&](auto CTC) {
    constexpr int CT = decltype(CTC)::value;   // column tiles computed (>= nct)
    int4v acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[rt][c] = int4v{0, 0, 0, 0};
    int4v A[2][RT], B[2][CT];
    auto read_b = [&](const int8_t* stage, int ks, int4v (&Bv)[CT]) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int slot = (16 * c + lrow) * kChq + ((2 * lq + ks) ^ (lrow >> 1));
        Bv[c] = *reinterpret_cast<const int4v*>(stage + slot * 16);
      }
    };
    auto mfmas = [&](const int4v (&Av)[RT], const int4v (&Bv)[CT]) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Av[rt], Bv[c], acc[rt][c], 0, 0, 0);
    };

    static_for<NS - 1>([&](auto J) { issue(J, J); });
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WAITN) : "memory");
    __syncthreads();
    read_b(xs[0], 0, B[0]);
    codes_ks(ic<0>{}, 0, A[0]);

    auto kblock = [&](auto S, int kb) {
      constexpr int st = decltype(S)::value;
      constexpr int sn = (st + 1) % NS;
      constexpr int s3 = (st + NS - 1) % NS;
      // stage s3 held block kb - 1, whose reads every wave finished before
      // the barrier of block kb - 1
      issue(ic<s3>{}, kb + NS - 1);
      read_b(xs[st], 1, B[1]);
      codes_ks(ic<st>{}, 1, A[1]);
      mfmas(A[0], B[0]);
      // block kb + 1 landed in every wave (blocks kb + 2, kb + 3 may be in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WAITN) : "memory");
      __syncthreads();
      read_b(xs[sn], 0, B[0]);
      codes_ks(ic<sn>{}, 0, A[0]);
      mfmas(A[1], B[1]);
    };
    for (int kb = 0; kb < nkb; kb += NS)
      static_for<NS>([&](auto J) {
        if (kb + J < nkb) kblock(J, kb + J);
      });
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // row scales of this lane's four rows of each tile (zeros past the matrix)
    float rsc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t v[4];
      bload16(v, sb[PROJ == 0 ? rt >> 1 : 0], (uint32_t)(rbase[rt] + 4 * lq) * 4u, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) rsc[rt][i] = __uint_as_float(v[i]);
    }

    // epilogue: (acc - 8 sum q) * s_w * s_a
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int m = 16 * c + lrow;
      if (m >= u.M) continue;
      const int orow = u.p0 + m;
      if constexpr (PROJ == 0) {
        const int t = u.routed ? g.sorted_token[u.tok0 + m] : u.tok0 + m;
        const float sa = g.xs[t];
        const int off = 8 * g.xsum[t];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          uint32_t packed[2];
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            float h2[2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const float gv = (float)(acc[rt][c][i + d] - off) * rsc[rt][i + d] * sa;
              const float uv = (float)(acc[rt + 2][c][i + d] - off) * rsc[rt + 2][i + d] * sa;
              h2[d] = silu_mul(gv, uv);
            }
            const _Float16 a0 = (_Float16)h2[0], a1 = (_Float16)h2[1];
            packed[i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          }
          const int col = rbase[rt] + 4 * lq;
          if (col < inter)
            *reinterpret_cast<uint2*>(g.h_out + (size_t)orow * g.ldh + col) = make_uint2(packed[0], packed[1]);
          else if (col < pad_k(inter))
            *reinterpret_cast<uint2*>(g.h_out + (size_t)orow * g.ldh + col) = make_uint2(0u, 0u);
        }
      } else {
        const float sa = g.hs[orow];
        const int off = 8 * g.hsum[orow];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int col = rbase[rt] + 4 * lq;
          if (col < g.H) {
            float4 o;
            o.x = (float)(acc[rt][c][0] - off) * rsc[rt][0] * sa;
            o.y = (float)(acc[rt][c][1] - off) * rsc[rt][1] * sa;
            o.z = (float)(acc[rt][c][2] - off) * rsc[rt][2] * sa;
            o.w = (float)(acc[rt][c][3] - off) * rsc[rt][3] * sa;
            *reinterpret_cast<float4*>(g.o_out + (size_t)orow * g.H + col) = o;
          }
        }
      }
    }
  };

  if constexpr (thin) {
    if (nct > 1)
      run(ic<kBMThin / 16>{});
    else
      run(ic<1>{});
  } else {
    if constexpr (BM >= 256) {
      if (nct > 12) {
        run(ic<16>{});
        return;
      }
      if (nct > 8) {
        run(ic<12>{});
        return;
      }
    } else if constexpr (BM > 128) {
      if (nct > 8) {
        run(ic<BM / 16>{});
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

}  // namespace

template <int PROJ, int BM>
hipError_t launch_q(const GemmQArgs& g, long units, int nt, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL((moe_gemm_q_kernel<PROJ, BM, kNSq>), dim3((unsigned)(units * nt)), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* src, int ld_src, bool bf16, int rows, int split, int n,
                             int n2, int8_t* dst, int ld_dst, float* scale, int32_t* sum, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(quant_rows_kernel<true>, dim3(rows), dim3(256), 0, s, src, ld_src, split, n, n2, dst,
                       ld_dst, scale, sum);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, dim3(rows), dim3(256), 0, s, src, ld_src, split, n, n2, dst,
                       ld_dst, scale, sum);
  return hipGetLastError();
}

hipError_t launch_gemm_q(const GemmQArgs& g, int proj, int K, int E, hipStream_t s) {
  const long fat = fat_units_max(g.T, K, E, g.has_shared, kBMQ);
  const long thin = thin_units_max(g.T, K, E, g.has_shared, kBMQ);
  hipError_t e;
  if (proj == 0) {
    const int max_inter = std::max(g.routed.inter, g.has_shared ? g.shared.inter : 0);
    const int ntg = (max_inter + kGateUpPairs - 1) / kGateUpPairs;
    if ((e = launch_q<0, kBMQ>(g, fat, ntg, s)) != hipSuccess) return e;
    return launch_q<0, kBMThin>(g, thin, ntg, s);
  }
  const int ntd = (g.H + kDownRows - 1) / kDownRows;
  if ((e = launch_q<1, kBMQ>(g, fat, ntd, s)) != hipSuccess) return e;
  return launch_q<1, kBMThin>(g, thin, ntd, s);
}

}  // namespace qmoe
