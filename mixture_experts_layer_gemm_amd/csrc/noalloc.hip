// moe_layer_forward_noalloc: the whole layer with its scratch memory in a static device array, for
// callers that cannot allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid hipMalloc). The kernels are those of moe_layer_forward; they receive the
// array's device address where moe_layer_forward passes the caller's workspace.
//
// The array is a file-scope __device__ object, so every GPU the library runs on holds its own copy
// of MOE_NOALLOC_SCRATCH_BYTES bytes until the process ends. In host code its name is only a
// host-side stand-in: the device address comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the entry point's first call there, and used everywhere after.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (null on a HIP error).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_desc* desc, const void* x, const moe_weights* weights,
                                                const float* prev_logits, float* logits_out, moe_routing* routing,
                                                void* cache, const void* residual, void* y, void* stream) {
  const size_t need = moe_workspace_bytes(desc);
  if (need == 0)   // an invalid or unsupported description: the full check returns which, launching nothing
    return moe_layer_forward(desc, x, weights, prev_logits, logits_out, routing, cache, residual, y, nullptr, 0,
                             stream);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return MOE_EHIP;
  return moe_layer_forward(desc, x, weights, prev_logits, logits_out, routing, cache, residual, y, ws,
                           (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
