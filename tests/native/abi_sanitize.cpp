// Host-side checks of the C ABI (include/qmoe.h) built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the boundary code: every entry point's
// argument validation and the workspace sizing, over many configurations.
// None of these calls reaches the device (invalid calls return before any
// HIP call; sizes are host arithmetic), so no GPU is needed.  Exits non-zero
// on the first unexpected status; the sanitizers abort on any memory or
// undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "qmoe.h"

static int failures = 0;
#define EXPECT(call, want)                                                               \
  do {                                                                                   \
    const moe_status got_ = (call);                                                      \
    if (got_ != (want)) {                                                                \
      std::fprintf(stderr, "%s:%d: %s -> %s, expected %s\n", __FILE__, __LINE__, #call,   \
                   moe_status_string(got_), moe_status_string(want));                    \
      ++failures;                                                                        \
    }                                                                                    \
  } while (0)

static moe_config tiny() {
  moe_config c{};
  c.hidden = 256;
  c.moe_inter = 128;
  c.n_routed_experts = 16;
  c.n_group = 4;
  c.topk_group = 2;
  c.top_k = 4;
  c.n_shared_experts = 1;
  c.shared_inter = 128;
  c.routed_scaling_factor = 2.5f;
  c.wfmt = MOE_WFMT_INT4_G32_F16;
  return c;
}

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t(0x100000));   // aligned, never dereferenced
  const uint16_t* x = static_cast<const uint16_t*>(fake);
  const float* f = static_cast<const float*>(fake);
  int32_t* i32 = static_cast<int32_t*>(fake);
  float* fo = static_cast<float*>(fake);
  moe_qproj p{static_cast<const uint8_t*>(fake), fake, nullptr};
  moe_qexperts e{p, p, p};

  // workspace sizes over a sweep of shapes: positive, 256-aligned, monotone in T
  size_t prev = 0, bytes = 0;
  for (int H : {32, 256, 2080, 6144, 65536})
    for (int I : {32, 128, 2048})
      for (int E : {1, 16, 256})
        for (int k : {1, 4, 8}) {
          moe_config c = tiny();
          c.hidden = H;
          c.moe_inter = I;
          c.shared_inter = I;
          c.n_routed_experts = E;
          c.n_group = 1;
          c.topk_group = 1;
          c.top_k = k <= E ? k : E;
          prev = 0;
          for (int T : {0, 1, 3, 64, 4096, 262144}) {
            EXPECT(moe_workspace_size(&c, T, &bytes), MOE_OK);
            if (bytes % 256 != 0 || bytes < prev) {
              std::fprintf(stderr, "workspace size %zu at T=%d H=%d\n", bytes, T, H);
              ++failures;
            }
            prev = bytes;
          }
        }

  moe_config c = tiny();
  size_t n = 0;
  EXPECT(moe_workspace_size(&c, 8, &n), MOE_OK);
  EXPECT(moe_workspace_size(nullptr, 8, &n), MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, 8, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, -1, &n), MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, MOE_MAX_TOKENS + 1, &n), MOE_ERR_UNSUPPORTED);

  // configuration limits
  struct Bad {
    void (*mod)(moe_config&);
    moe_status want;
  } bad[] = {
      {[](moe_config& c) { c.hidden = 100; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.hidden = -32; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.moe_inter = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.n_group = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.n_group = 3; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.topk_group = 5; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.top_k = 9; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.top_k = 0x7fffffff; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.n_shared_experts = 2; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.routed_scaling_factor = NAN; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.routed_scaling_factor = INFINITY; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.wfmt = 9; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.options = 8u; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.expert_top_p = -1.0f; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.expert_top_p = NAN; }, MOE_ERR_INVALID_ARG},
      {[](moe_config& c) { c.n_routed_experts = 0x40000000; c.n_group = 1; c.topk_group = 1; },
       MOE_ERR_UNSUPPORTED},
      {[](moe_config& c) { c.hidden = 0x7fffffe0; }, MOE_ERR_UNSUPPORTED},
  };
  for (const Bad& b : bad) {
    moe_config cc = tiny();
    b.mod(cc);
    EXPECT(moe_workspace_size(&cc, 8, &n), b.want);
    EXPECT(moe_layer(&cc, 8, x, f, f, &e, &e, fake, 0, nullptr, nullptr, fake, 1 << 30, nullptr),
           b.want);
  }

  // entry points: null, misaligned and inconsistent arguments
  EXPECT(moe_workspace_size(&c, 8, &n), MOE_OK);
  EXPECT(moe_route(&c, 8, nullptr, f, nullptr, i32, fo, fake, n, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(&c, 8, x, f, nullptr, i32, fo, fake, 0, nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_route(&c, 0, x, f, nullptr, i32, fo, nullptr, 0, nullptr), MOE_OK);
  EXPECT(moe_permute(&c, 8, i32, nullptr, i32, i32, i32, i32, fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn_q4(&c, 8, x, &e, i32, nullptr, i32, i32, fo, fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn_q4(&c, 8, x, nullptr, nullptr, nullptr, nullptr, nullptr, fo, fake, n,
                           nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(&c, 8, fo, i32, fo, nullptr, fake, 3, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(&c, 0, fo, i32, fo, nullptr, fake, 0, nullptr), MOE_OK);
  moe_qexperts mis = e;
  mis.up.scale = static_cast<char*>(fake) + 2;
  EXPECT(moe_layer(&c, 8, x, f, f, &mis, &e, fake, 0, nullptr, nullptr, fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer(&c, 8, x, f, f, &e, nullptr, fake, 0, nullptr, nullptr, fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer(&c, 8, x, f, f, &e, &e, fake, 0, nullptr, nullptr, fake, n - 1, nullptr),
         MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_layer(&c, 8, x, f, f, &e, &e, static_cast<char*>(fake) + 4, 0, nullptr, nullptr,
                   fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer(&c, 0, x, f, f, &e, &e, fake, 0, nullptr, nullptr, nullptr, 0, nullptr),
         MOE_OK);
  moe_trace tr{};
  EXPECT(moe_layer_trace(&c, 8, x, f, f, &e, &e, fake, 0, nullptr, nullptr, fake, n, nullptr, &tr),
         MOE_ERR_INVALID_ARG);   // events are NULL
  EXPECT(moe_layer_trace(&c, 8, x, f, f, &e, &e, fake, 0, nullptr, nullptr, fake, n, nullptr,
                         nullptr),
         MOE_ERR_INVALID_ARG);
  uint32_t flags = 0;
  EXPECT(moe_layer_flags(static_cast<char*>(fake) + 4, &flags, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_flags(fake, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  moe_config big = tiny();
  big.hidden = 6144;
  big.moe_inter = big.shared_inter = 2048;
  big.n_routed_experts = 256;
  big.n_group = 8;
  big.topk_group = 4;
  big.top_k = 8;
  EXPECT(moe_layer_noalloc(&big, 128, x, f, f, &e, &e, fake, 0, nullptr, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_layer_noalloc(&big, 8, nullptr, f, f, &e, &e, fake, 0, nullptr, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);
  // expert cache: creation and the host-only calls need no device; invalid
  // calls return before any HIP call
  moe_expert_cache* cache = reinterpret_cast<moe_expert_cache*>(fake);
  EXPECT(moe_cache_create(&c, 0, &e, &e, &cache), MOE_ERR_INVALID_ARG);
  if (cache) ++failures;   // NULL on error
  EXPECT(moe_cache_create(&c, 17, &e, &e, &cache), MOE_ERR_INVALID_ARG);   // > E
  EXPECT(moe_cache_create(&c, 4, &mis, &e, &cache), MOE_ERR_INVALID_ARG);
  EXPECT(moe_cache_create(&c, 4, &e, nullptr, &cache), MOE_ERR_INVALID_ARG);
  EXPECT(moe_cache_create(&c, 4, &e, &e, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_cache_create(&c, 4, &e, &e, &cache), MOE_OK);
  if (cache) {
    int32_t slot = 7;
    EXPECT(moe_cache_slot_of(cache, 3, &slot), MOE_OK);
    if (slot != -1) ++failures;
    EXPECT(moe_cache_slot_of(cache, 16, &slot), MOE_ERR_INVALID_ARG);
    moe_cache_stats st{};
    EXPECT(moe_cache_get_stats(cache, &st), MOE_OK);
    if (st.calls || st.hits || st.misses || st.prefetched || st.evictions || st.bytes_loaded)
      ++failures;
    const int32_t ids[6] = {0, 1, 2, 3, 4, 16};
    int32_t loaded = 9;
    EXPECT(moe_cache_prefetch(cache, ids, 0, &loaded, nullptr), MOE_OK);
    if (loaded != 0) ++failures;
    EXPECT(moe_cache_prefetch(cache, ids, 6, &loaded, nullptr), MOE_ERR_INVALID_ARG);   // id 16
    EXPECT(moe_cache_prefetch(cache, nullptr, 2, &loaded, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_cache_pin(cache, ids, 5, nullptr), MOE_ERR_UNSUPPORTED);   // 5 experts, 4 slots
    EXPECT(moe_cache_pin(cache, ids, -1, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_cache_unpin_all(cache), MOE_OK);
    EXPECT(moe_layer_cached(cache, 8, x, f, f, &e, fake, 2, nullptr, nullptr, fake, n, nullptr),
           MOE_ERR_INVALID_ARG);   // out dtype
    EXPECT(moe_layer_cached(cache, 8, x, f, f, nullptr, fake, 0, nullptr, nullptr, fake, n, nullptr),
           MOE_ERR_INVALID_ARG);   // shared expert missing
    EXPECT(moe_layer_cached(cache, 8, x, f, f, &e, fake, 0, nullptr, nullptr, fake, n - 1, nullptr),
           MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_layer_cached(cache, 0, x, f, f, &e, fake, 0, nullptr, nullptr, nullptr, 0, nullptr),
           MOE_OK);
    EXPECT(moe_cache_destroy(cache), MOE_OK);
  }
  EXPECT(moe_layer_cached(nullptr, 1, x, f, f, &e, fake, 0, nullptr, nullptr, fake, n, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_cache_destroy(nullptr), MOE_OK);

  for (int s = 0; s <= 7; ++s)   // the values a moe_status can hold in C++
    if (!moe_status_string(static_cast<moe_status>(s))) ++failures;

  std::printf("abi_sanitize: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
