// Layer group without a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace csa2_layer_group needs lives in `scratch`, a file-scope device array of
// CSA2_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device memory, so the
// array's device address is looked up once per device (with that device current) and only
// that address is handed to the kernels.  Nothing here allocates or frees memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/csa2.h"

static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)
std::mutex g_scratch_mu;

// The device address of this device's `scratch`, looked up on the first call per device.
int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" int csa2_layer_group_noalloc(const csa2_layer* layers, int n_layers, const csa2_group_cache* cache,
                                        void* stream) {
  // every argument is validated exactly as csa2_layer_group does; without a workspace it
  // stops at the workspace check when the arguments are valid, having launched nothing
  const int vr = csa2_layer_group(layers, n_layers, cache, nullptr, 0, stream);
  if (vr != CSA2_ERR_WORKSPACE) return vr;
  if (csa2_layer_group_workspace_size(cache, n_layers) > (size_t)CSA2_NOALLOC_SCRATCH_BYTES)
    return CSA2_ERR_WORKSPACE;  // this shape needs more scratch than the library holds
  const int rc = csa2_device_check();
  if (rc) return rc;
  void* ws = nullptr;
  const int sr = scratch_for_current_device(&ws);
  if (sr) return sr;
  return csa2_layer_group(layers, n_layers, cache, ws, (size_t)CSA2_NOALLOC_SCRATCH_BYTES, stream);
}
