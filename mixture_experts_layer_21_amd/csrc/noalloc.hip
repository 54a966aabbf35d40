// The layer forward for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the
// workspace moe_forward takes from its caller lives here instead, in
// `scratch`, a fixed device array of the library (one copy on each GPU the
// library runs on, held until the process ends).
//
// The address of this device's copy is looked up once per device, with that
// device current, and kept; host code uses only that address (the array's
// name is a host-side stand-in, not a device address).  Nothing in the
// forward needs the scratch cleared: every byte a kernel reads was written
// earlier in the same call.  Calls that overlap on one GPU share the array
// and race.
#include <mutex>

#include "forward.h"
#include "moe.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device

void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const void* x, const void* w_r,
                                          const float* router_bias, const void* w1,
                                          const void* w2, int64_t T, int64_t H, int64_t E,
                                          int32_t top_k, int64_t F, moe_dtype dtype, void* y,
                                          int32_t* topk_ids_out, float* topk_w_out,
                                          void* stream) {
  const moe_status st =
      moe::check_forward(x, w_r, router_bias, w1, w2, T, H, E, top_k, F, dtype, dtype,
                         MOE_GATE_TOPK_SOFTMAX, y, topk_ids_out, topk_w_out);
  if (st != MOE_OK) return st;
  // no split-tile partials: the GEMMs run their leftover tiles whole
  const moe::FwdLayout L = moe::fwd_layout(T, H, E, top_k, F, dtype, false);
  if (L.total > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return MOE_ERR_LAUNCH;
  return moe::forward_body(x, w_r, router_bias, w1, w2, T, H, E, top_k, F, dtype, dtype,
                           MOE_GATE_TOPK_SOFTMAX, 0, y, topk_ids_out, topk_w_out, ws, L, false,
                           (hipStream_t)stream);
}
