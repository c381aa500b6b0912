// The layer forward with its workspace in a file-scope device array, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation). The array is this
// library's own: every GPU the library runs on holds one copy of it until the
// process ends, and every call on that GPU shares it.
//
// Host code never passes the array's name to a kernel or a copy: on the host
// that name is a stand-in, not a device address. The device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept; the kernels get that address as their workspace.

#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on its first use.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::report_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return moe::report_hip_error(e);
    if (!p) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_config* c, int64_t T, const void* x,
                                         const moe_weights* w, moe_outputs* o, void* stream) {
  size_t need = 0;
  int st = moe::layer_forward_check(c, T, x, w, o, &need);
  if (st) return st;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return moe::layer_forward_on(c, T, x, w, o, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
