// Work units of the grouped GEMMs (csrc/gemm.hip: fp16 activations;
// csrc/gemm_i8.hip: int8 activations): units of up to kBMF or kBMQ tokens of one expert
// ("fat") or kBMThin ("thin"), built on the device by build_units, and the
// mapping of work items to XCDs.
#pragma once

#include <type_traits>

#include "qmoe_device.h"

namespace qmoe {

constexpr int kBMThin = 32;
constexpr int kBMF = kGemmUnitTokensF;   // fat units of the fp16 GEMM
constexpr int kBMQ = kGemmUnitTokensQ;   // fat units of the W4A8 GEMM
// With fewer fat units than this (gate/up: 16 work items each) the fat
// launches would leave most of the chip idle, so the experts they would hold
// are cut into thin units, which run in the thin launch with the bulk of the
// work (their weights are then read once per 32 tokens).
constexpr int kFewFat = 16;
// Fat units of kBMF (kBMQ) tokens are used when there are at least kFewWide of
// them; with fewer (a skewed load: a few experts with many tokens) they are
// cut at kBMNarrow tokens, which gives more work items for the chip.
constexpr int kBMNarrow = 128;
constexpr int kFewWide = 64;
constexpr int kGateUpPairs = 128; // row pairs per gate/up unit
constexpr int kDownRows = 256;    // output rows per down unit

struct Unit {
  int e;        // expert index in its weight set (0 for the shared expert)
  int p0;       // first row of the unit in the h / O buffers
  int M;        // tokens in the unit (<= the kernel's unit rows)
  int tok0;     // routed: first sorted slot (index into sorted_token); shared: first token
  bool routed;
};

// The unit is the same for the whole workgroup; readfirstlane puts it in
// SGPRs, so that the buffer descriptors built from it are uniform (a
// descriptor in VGPRs turns every buffer load into a waterfall loop).
__device__ __forceinline__ Unit load_unit(const int4* tiles, int idx) {
  const int4 t = tiles[idx];
  Unit u;
  const int x = __builtin_amdgcn_readfirstlane(t.x);
  u.routed = x >= 0;
  u.e = u.routed ? x : 0;
  u.p0 = __builtin_amdgcn_readfirstlane(t.y);
  u.M = __builtin_amdgcn_readfirstlane(t.z);
  u.tok0 = __builtin_amdgcn_readfirstlane(t.w);
  return u;
}

// Activation rows past M start at this offset, past the range of every
// activation descriptor (the host keeps those buffers below 2 GiB), so their
// loads return zeros at every K block.
constexpr uint32_t kOOBRow = 0x80000000u;

template <int N>
using ic = std::integral_constant<int, N>;

// Work item -> (unit, n tile).  Workgroups are dispatched round-robin over
// the 8 XCDs; this maps the items that one XCD receives onto a contiguous
// range, n tile fastest, so that the n tiles of one token tile run on the same
// XCD at about the same time and share its L2 copy of the activations.
__device__ __forceinline__ int xcd_item(int L, int total) {
  const int x = L & 7, q = total >> 3, r = total & 7;
  return x * q + min(x, r) + (L >> 3);
}

// Most work units of each kind for T tokens, top-k K and E experts (the
// launches are sized to these; units past the built ones exit at once).
long fat_units_max(int T, int K, int E, bool has_shared, int bmf);
long thin_units_max(int T, int K, int E, bool has_shared, int bmf);

}  // namespace qmoe
