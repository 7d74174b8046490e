// gdn_frame_fwd_noalloc: gdn_frame_fwd for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc).  Its workspace is `scratch`, a file-scope device array
// of GDN_NOALLOC_SCRATCH_BYTES: every GPU the entry point runs on holds its
// own copy until the process ends, and every call on that GPU shares it.
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address: its address on a device comes from hipGetSymbolAddress,
// taken once per device with that device current (the first call on it) and
// kept; the kernels receive that address as their workspace argument.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, null until taken
std::mutex g_scratch_mu;

// The current device's address of `scratch` (taken on first use).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int gdn_frame_fwd_noalloc(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q,
                                     const void* k, const void* v, const float* gamma, const float* beta,
                                     const float* state_in, void* out, float* state_out, void* stream) {
  // The workspace this call needs (0 for an invalid shape: the call below
  // then reports the argument error), checked against the array's size
  // before anything touches the device's copy of it.
  const size_t need = gdn_workspace_bytes(shape, in_dtype);
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_E_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0 && scratch_ptr(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return GDN_E_HIP;
  }
  return gdn::frame_fwd_in(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, out, state_out, ws,
                           ws ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0, stream);
}
