// msda_backward_noalloc: msda_backward with its workspace taken from a static
// device array of this file instead of the caller, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops, harnesses
// that forbid allocation).  The kernels are msda_backward's; only the workspace
// differs.
#include "msda.h"
#include "msda_launch.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB per GPU
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: host code uses only the device
// address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current.
hipError_t scratch_on(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t msda_noalloc_scratch_bytes(void) { return kScratchBytes; }

msda_status msda_backward_noalloc(const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start_index,
                                  const void *sampling_locations, const void *attention_weights,
                                  const void *grad_out, void *grad_value, void *grad_loc,
                                  void *grad_attn, const msda_dims *dims, msda_dtype dtype,
                                  msda_dtype accum_dtype, msda_scatter scatter,
                                  const int64_t *spatial_shapes_host, void *stream) {
  const size_t need =
      msda_backward_workspace_bytes(dims, dtype, accum_dtype, scatter, spatial_shapes_host);
  if (need == SIZE_MAX)  // rejected arguments: msda_backward reports why
    return msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_out, grad_value, grad_loc, grad_attn, dims, dtype,
                         accum_dtype, scatter, spatial_shapes_host, nullptr, 0, stream);
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "msda_backward_noalloc: these sizes need %zu bytes of workspace; the static scratch "
             "holds %zu", need, kScratchBytes);
    msda::set_last_error(msg);
    return MSDA_ERR_WORKSPACE;
  }
  void *ws = nullptr;
  if (need > 0) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e == hipSuccess) e = scratch_on(dev, &ws);
    if (e != hipSuccess) {
      char msg[200];
      snprintf(msg, sizeof(msg), "msda_backward_noalloc: static scratch of device %d: %s", dev,
               hipGetErrorString(e));
      msda::set_last_error(msg);
      return MSDA_ERR_HIP;
    }
  }
  return msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_weights, grad_out, grad_value, grad_loc, grad_attn, dims, dtype,
                       accum_dtype, scatter, spatial_shapes_host, ws, kScratchBytes, stream);
}

}  // extern "C"
