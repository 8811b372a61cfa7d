// Allocation-free sparse decode: sda_decode_static runs sda_decode with the
// library's own device scratch array in place of a caller workspace, for
// callers that cannot allocate (code under HIP graph capture, serving loops
// that forbid hipMalloc).
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from the time the code object is loaded until
// the process ends.  In host code the name `scratch` is only a host-side
// stand-in: its device address is read once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to kernels.
//
// What the kernels keep there (the row order and row bins, the split
// partials and log-sum-exps) is written before it is read within each call,
// so nothing needs clearing between calls.  Calls that overlap on one GPU
// share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sda.h"

namespace {

static __device__ __align__(256) uint8_t scratch[SDA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, or null

// Device address of the scratch array on `device`: read once, with `device`
// current (the caller's current device is restored afterwards).
void* scratch_on(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return g_scratch[device];
  int current = -1;
  if (hipGetDevice(&current) != hipSuccess) return nullptr;
  if (current != device && hipSetDevice(device) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (current != device) (void)hipSetDevice(current);
  if (e != hipSuccess) return nullptr;
  g_scratch[device] = ptr;
  return ptr;
}

}  // namespace

extern "C" int sda_decode_static(const sda_decode_args* a, hipStream_t stream) {
  if (!a) return SDA_ERR_INVALID;
  if (a->workspace || a->workspace_bytes) return SDA_ERR_INVALID;
  // Sizes beyond the array are refused before anything touches the device.
  // (Invalid sizes give 0 here and are refused by sda_decode below.)
  if (sda_workspace_bytes(a->rows, a->heads, a->splits) > (size_t)SDA_STATIC_SCRATCH_BYTES)
    return SDA_ERR_SCRATCH;
  int device = -1;
  if (stream ? hipStreamGetDevice(stream, &device) != hipSuccess
             : hipGetDevice(&device) != hipSuccess)
    return SDA_ERR_LAUNCH;
  if (device < 0 || device >= kMaxDevices) return SDA_ERR_UNSUPPORTED;
  void* ptr = scratch_on(device);
  if (!ptr) return SDA_ERR_LAUNCH;
  sda_decode_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = SDA_STATIC_SCRATCH_BYTES;
  return sda_decode(&b, stream);
}
