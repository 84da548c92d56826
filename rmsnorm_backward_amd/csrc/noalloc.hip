// noalloc.hip -- norm_bwd_ex_static: the extended backward for callers that
// cannot allocate device memory. Its workspace (the per-group partial
// dgamma/dbeta of the two-pass reduction, or the wide-row path's recomputed
// statistics) lives in `scratch`, a static array of this library's device
// code, instead of a buffer the caller passes.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "nb_api.hpp"
#include "norm_bwd.h"

namespace {

// One copy per device the library runs on, allocated with the library's code
// object on that device and held until the process ends. Every call on a
// device shares that device's copy and leaves its last contents there; no
// call reads scratch before writing it, so nothing needs clearing.
static __device__ __align__(256) unsigned char scratch[NORM_BWD_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device, once looked up

// Host code uses the array only through the address hipGetSymbolAddress
// gives for the current device (the array's own name is a host-side stand-in).
int scratch_provider(size_t need, void** ws, size_t* ws_bytes, void* stream) {
  if (need > (size_t)NORM_BWD_STATIC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "this problem needs %zu bytes of workspace; the static scratch holds %zu "
             "(use norm_bwd_ex with a workspace of that size)",
             need, (size_t)NORM_BWD_STATIC_SCRATCH_BYTES);
    return nb::report_error(NORM_BWD_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nb::report_hip_error(e, "hipGetDevice");
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
    if (e != hipSuccess) return nb::report_hip_error(e, "hipStreamGetDevice");
    if (sd != dev)
      return nb::report_error(NORM_BWD_ERR_INVALID_ARG,
                              "the stream belongs to another device than the current one");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return nb::report_error(NORM_BWD_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return nb::report_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!p) return nb::report_error(NORM_BWD_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  *ws_bytes = (size_t)NORM_BWD_STATIC_SCRATCH_BYTES;
  return NORM_BWD_OK;
}

}  // namespace

extern "C" int norm_bwd_ex_static(const norm_bwd_args_t* a) {
  if (!a) return nb::report_error(NORM_BWD_ERR_INVALID_ARG, "args is NULL");
  if (a->workspace != nullptr || a->workspace_bytes != 0)
    return nb::report_error(NORM_BWD_ERR_INVALID_ARG,
                            "workspace must be NULL and workspace_bytes 0: norm_bwd_ex_static "
                            "uses the library's static scratch");
  return nb::run_ex(a, &scratch_provider);
}
