// moe_layer_forward_noalloc: the whole layer forward with its workspace in a
// fixed device array of this library instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).  It runs exactly the kernels of
// moe_layer_forward (same workspace layout), so its results are the same bits.
//
// The array lives in every GPU the library runs on until the process ends.  Its
// device address is looked up once per device (with that device current) and
// kept; the array's name is never used as an address in host code.  No piece of
// the layer's workspace has to start at zero: every kernel writes what it later
// reads (logits, routing, block counts, indices, h, y_perm) within the same call,
// so nothing is cleared between calls.  Calls that overlap on one GPU share the
// array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of the array (looked up on the first call there).
moe_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F,
                                                moe_dtype dtype, const void* x, const void* w_router,
                                                const float* bias, const void* w_gate, const void* w_up,
                                                const void* w_down, void* y, float* logits_out, int32_t* topk_ids,
                                                float* topk_w, int32_t* offsets_out, void* y_perm_out, void* gu_out,
                                                void* stream) {
  // the workspace this call needs (sizes are checked; nothing is launched)
  size_t need = 0;
  moe_status st = moe_layer_forward(T, d, E, k, F, dtype, x, w_router, bias, w_gate, w_up, w_down, y, logits_out,
                                    topk_ids, topk_w, offsets_out, y_perm_out, gu_out, nullptr, &need, stream);
  if (st != MOE_OK) return st;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != MOE_OK) return st;
  size_t have = kScratchBytes;
  return moe_layer_forward(T, d, E, k, F, dtype, x, w_router, bias, w_gate, w_up, w_down, y, logits_out, topk_ids,
                           topk_w, offsets_out, y_perm_out, gu_out, ws, &have, stream);
}
