// Streaming kernels that measure the HBM bandwidth this GPU reaches in
// practice for four access mixes: read only, read + write 1:1 (a copy), read +
// write 3:2 (the byte mix of the forward output kernel: q, k, v read, o
// written) and an in-place update (read and write the same bytes, the decode
// step's pattern on its states).  They are measurement references for the benchmark, not part of
// the attention path: libla_stream.so, C ABI in include/la_stream.h.
//
// Each workgroup of 256 threads walks whole 64 KiB chunks of the source
// (grid-stride over chunks): per step every thread moves U 16-byte vectors, so
// a wave touches U fully used 1 KiB spans; loads are all issued before any
// store, and the read-only kernel folds what it reads into one word per
// thread so that no load is dead.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "la_stream.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 x) {
  if constexpr (NT) __builtin_nontemporal_store(x, p);
  else *p = x;
}

constexpr int kThreads = 256;

// Vectors per thread per step: 16 for read-only and copy (a 64 KiB chunk per
// workgroup step), 15 for the 3:2 mix (15 read, 10 written).
template <int MODE>
constexpr int units() { return MODE == 2 ? 15 : 16; }

// MODE 0: read src.  MODE 1: dst = src.  MODE 2: per step read 15 vectors of
// src and write 10 to dst (dst holds 2/3 of src's vectors).  MODE 3: update
// src in place (every vector read, changed and written back).  nchunks: whole
// steps of kThreads * units<MODE>() vectors in src.
template <int MODE, bool NT>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          size_t nchunks, unsigned* __restrict__ sink) {
  constexpr int U = units<MODE>();
  constexpr size_t kChunk = size_t(kThreads) * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * kChunk + threadIdx.x;
    u32x4 x[U];
    for (int u = 0; u < U; ++u) x[u] = ld<NT>(src + base + size_t(u) * kThreads);
    if constexpr (MODE == 0) {
      for (int u = 0; u < U; ++u) acc ^= x[u];
    } else if constexpr (MODE == 1) {
      for (int u = 0; u < U; ++u) st<NT>(dst + base + size_t(u) * kThreads, x[u]);
    } else if constexpr (MODE == 3) {
      const u32x4 one = {1u, 1u, 1u, 1u};
      for (int u = 0; u < U; ++u) st<NT>(const_cast<u32x4*>(src) + base + size_t(u) * kThreads, x[u] + one);
    } else {
      const size_t obase = c * (size_t(kThreads) * 10) + threadIdx.x;
      for (int u = 0; u < 10; ++u) st<NT>(dst + obase + size_t(u) * kThreads, x[u] ^ x[10 + u / 2]);
    }
  }
  if constexpr (MODE == 0) sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

size_t chunk_vectors(int mode) { return size_t(kThreads) * (mode == 2 ? 15 : 16); }

}  // namespace

extern "C" {

int la_stream_run(int mode, int nontemporal, const void* src, void* dst, size_t src_bytes, unsigned* sink,
                  int grid, void* stream) {
  if (mode < 0 || mode > 3 || grid <= 0 || src == nullptr || (mode == 0 && sink == nullptr)) return 1;
  if ((mode == 1 || mode == 2) && dst == nullptr) return 1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return 1;
  const size_t nchunks = src_bytes / 16 / chunk_vectors(mode);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(grid)), b(kThreads);
  const auto* a = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
#define LA_STREAM(M)                                                                                 \
  if (nontemporal) hipLaunchKernelGGL((stream_kernel<M, true>), g, b, 0, s, a, d, nchunks, sink);   \
  else hipLaunchKernelGGL((stream_kernel<M, false>), g, b, 0, s, a, d, nchunks, sink);
  if (mode == 0) {
    LA_STREAM(0)
  } else if (mode == 1) {
    LA_STREAM(1)
  } else if (mode == 2) {
    LA_STREAM(2)
  } else {
    LA_STREAM(3)
  }
#undef LA_STREAM
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

size_t la_stream_bytes_moved(int mode, size_t src_bytes) {
  if (mode < 0 || mode > 3) return 0;
  const size_t chunks = src_bytes / 16 / chunk_vectors(mode);
  const size_t read = chunks * chunk_vectors(mode) * 16;
  if (mode == 0) return read;
  if (mode == 1 || mode == 3) return 2 * read;
  return read + chunks * size_t(kThreads) * 10 * 16;
}

}  // extern "C"
