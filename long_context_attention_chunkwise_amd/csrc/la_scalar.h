// Device helpers of the scalar (float32 FMA) kernels: element loads and stores
// for the two storage types, float32 and bf16 held as its 16-bit pattern
// (uint16_t).  Loads widen to float32 exactly; stores round to nearest even.
// Internal to liblightning.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, int64_t i) {
  return __builtin_bit_cast(float, uint32_t(p[i]) << 16);
}
__device__ __forceinline__ void stf(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void stf(uint16_t* p, int64_t i, float x) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

}  // namespace la
