// Allocation-free forward entry point of liblightning.so.
//
// la_forward_noalloc computes exactly la_forward_ex (same kernels, same
// launch plan, bit-for-bit the same results), with the segment-state
// workspace taken from a fixed array of this library's device code instead of
// a caller buffer or a stream-ordered allocation.  The array lives in device
// memory from the first use of the library on a device until the process
// ends; every call on one device shares that device's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "la_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // la.h: LA_NOALLOC_SCRATCH_BYTES

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  In host code `scratch` names a host-side stand-in, so
// kernels and copies only ever receive these addresses.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

static_assert(kScratchBytes == LA_NOALLOC_SCRATCH_BYTES, "scratch size and its public value agree");

extern "C" la_status la_forward_noalloc(const void* q, const void* k, const void* v, void* o, int64_t B,
                                        int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                                        la_dtype in_dtype, la_dtype out_dtype, const float* s_in, float* s_out,
                                        la_stream stream) {
  // la_forward_ex's own checks first (nothing touches the device on an
  // error), then the size of the plan's segment-state workspace.
  size_t need = 0;
  const la_status st = la::check_forward_args(q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in,
                                              s_out, &need);
  if (st != LA_OK) return st;
  if (need > kScratchBytes) return LA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    // The pre-pass writes every partial and the scan every segment start
    // before they are read, so the array needs no clearing between calls.
    if (device_scratch(&ws) != hipSuccess) return LA_ERR_HIP;
  }
  return la_forward_ex(q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in, s_out, ws,
                       need > 0 ? kScratchBytes : 0, stream);
}
