// moe_layer_noalloc: moe_layer whose workspace is a device buffer of the
// library itself, for callers that cannot allocate device memory.
//
// The buffer is a file-scope device array; every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands in for the symbol):
// the first call on a device, with that device current, asks the runtime
// for the array's device address (hipGetSymbolAddress), checks the result
// and keeps it per device, and every later use goes through that address.
// Calls on one device share the buffer and keep its last contents; moe_layer
// writes every workspace word it reads, and its first kernels clear the
// barrier words and the flags word, so nothing needs clearing here.  Calls
// that overlap on one device (two streams, two threads) race on the buffer.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

static_assert(MOE_NOALLOC_WS_BYTES % 256 == 0, "workspace alignment");
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

void* noalloc_workspace() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev].store(addr, std::memory_order_release);
    p = addr;
  }
  return p;
}

}  // namespace qmoe

extern "C" moe_status moe_layer_noalloc(const moe_config* cfg, int32_t T, const uint16_t* x,
                                        const float* router_w, const float* bias,
                                        const moe_qexperts* routed, const moe_qexperts* shared,
                                        void* y, int32_t out_dtype, int32_t* topk_ids_out,
                                        float* topk_w_out, hipStream_t stream) {
  moe_status s = qmoe::check_layer_args(cfg, T, x, router_w, routed, shared, y, out_dtype);
  if (s != MOE_OK) return s;
  size_t need = 0;
  if ((s = moe_workspace_size(cfg, T, &need)) != MOE_OK) return s;
  if (need > MOE_NOALLOC_WS_BYTES) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  void* ws = qmoe::noalloc_workspace();
  if (!ws) return MOE_ERR_HIP;
  return moe_layer(cfg, T, x, router_w, bias, routed, shared, y, out_dtype, topk_ids_out,
                   topk_w_out, ws, MOE_NOALLOC_WS_BYTES, stream);
}
