// delta_fwd_noalloc: delta_fwd with its workspace taken from a fixed device array of this library,
// for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code its name is only a host-side stand-in, never
// a device address, so the address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to the kernels.  Calls on one device share the
// array: calls that overlap on one device race.  The forward pass ignores the workspace contents on
// entry (each kernel writes every workspace byte it later reads), so nothing needs clearing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/delta.h"

static __device__ __align__(256) unsigned char scratch[DELTA_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// The device address of `scratch` on device `dev`, looked up on the first call for that device
// with the device made current for the lookup (and the caller's current device restored).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return DELTA_ERR_HIP;
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    g_status[dev] = e;
  });
  if (g_status[dev] != hipSuccess || !g_scratch[dev]) return DELTA_ERR_HIP;
  *out = g_scratch[dev];
  return DELTA_OK;
}

}  // namespace

extern "C" int delta_fwd_noalloc(const delta_shape* s, const void* q, const void* k, const void* v,
                                 const float* beta, const float* g_log, const float* S0, void* O, float* S_final,
                                 void* stream) {
  size_t need = 0;
  int rc = delta_fwd_workspace_bytes(s, &need);
  if (rc) return rc;
  if (need > (size_t)DELTA_NOALLOC_MAX_BYTES) return DELTA_ERR_NOALLOC_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    // the device the work runs on: the stream's, or the current one for the default stream
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return DELTA_ERR_HIP;
    if ((rc = scratch_on(dev, &ws))) return rc;
  }
  return delta_fwd(s, q, k, v, beta, g_log, S0, O, S_final, ws, need, stream);
}
