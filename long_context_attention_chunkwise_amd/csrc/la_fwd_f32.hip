// float32 causal chunkwise linear attention forward pass.
//
// Follows the block recurrence of page "如何理解MiniMax股价创历史新高？拆解国产大模型
// 技术底座" (vergex.cn), section "Lightning Attention", chunkwise teaching code:
// O_b = Q_b S + tril(Q_b K_b^T) V_b, then S += K_b^T V_b.  All arithmetic is
// float32 FMA (no reduced-precision products), so this path serves float32
// inputs at float32 accuracy.  It is the small-problem path: one workgroup per
// (batch, KV head, 32-column slice of dv) walks the whole sequence and serves
// every query head of the group, with the state slice, the block's K and V
// slice and, one head at a time, Q and the score matrix staged in LDS.  The
// state is read from s_in and written to s_out by the same workgroup, so the
// two may be the same buffer.
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;     // dv columns per workgroup
constexpr int kMaxD = 128;
constexpr int kMaxBlock = 64;

__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v, float* __restrict__ o,
                                                          const float* s_in,
                                                          float* s_out, int Hq, int Hkv,
                                                          int64_t N, int d, int dv, int C) {
  __shared__ float Qs[kMaxBlock][kMaxD + 1];
  __shared__ float Ks[kMaxBlock][kMaxD + 1];
  __shared__ float Vs[kMaxBlock][kSlice];
  __shared__ float Ps[kMaxBlock][kMaxBlock + 1];
  __shared__ float Ss[kMaxD][kSlice];

  const int nslices = dv / kSlice;
  const int slice = blockIdx.x % nslices;
  const int bg = blockIdx.x / nslices;  // b * Hkv + g
  const int g = bg % Hkv, b = bg / Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int c0 = slice * kSlice;

  const float* kh = k + int64_t(bg) * N * d;
  const float* vh = v + int64_t(bg) * N * dv;
  const int64_t sbase = int64_t(bg) * d * dv;

  for (int e = tid; e < d * kSlice; e += kThreads) {
    int i = e / kSlice, n = e % kSlice;
    Ss[i][n] = s_in ? s_in[sbase + int64_t(i) * dv + c0 + n] : 0.0f;
  }

  for (int64_t a = 0; a < N; a += C) {
    const int c = int(N - a < C ? N - a : C);
    __syncthreads();  // previous block finished with Ks/Vs/Ss
    for (int e = tid; e < c * d; e += kThreads) {
      int t = e / d, i = e % d;
      Ks[t][i] = kh[(a + t) * d + i];
    }
    for (int e = tid; e < c * kSlice; e += kThreads) {
      int t = e / kSlice, n = e % kSlice;
      Vs[t][n] = vh[(a + t) * dv + c0 + n];
    }
    for (int hh = 0; hh < G; ++hh) {
      const int64_t bh = int64_t(b) * Hq + int64_t(g) * G + hh;
      const float* qh = q + bh * N * d;
      float* oh = o + bh * N * dv;
      __syncthreads();  // previous head finished with Qs/Ps
      for (int e = tid; e < c * d; e += kThreads) {
        int t = e / d, i = e % d;
        Qs[t][i] = qh[(a + t) * d + i];
      }
      __syncthreads();
      // In-block scores with the causal mask (s <= t kept).
      for (int e = tid; e < c * c; e += kThreads) {
        int t = e / c, s = e % c;
        float acc = 0.0f;
        if (s <= t)
          for (int i = 0; i < d; ++i) acc = fmaf(Qs[t][i], Ks[s][i], acc);
        Ps[t][s] = acc;
      }
      __syncthreads();
      // O = Q S (state before this block) + P V.
      for (int e = tid; e < c * kSlice; e += kThreads) {
        int t = e / kSlice, n = e % kSlice;
        float inter = 0.0f, intra = 0.0f;
        for (int i = 0; i < d; ++i) inter = fmaf(Qs[t][i], Ss[i][n], inter);
        for (int s = 0; s <= t; ++s) intra = fmaf(Ps[t][s], Vs[s][n], intra);
        oh[(a + t) * dv + c0 + n] = inter + intra;
      }
    }
    __syncthreads();
    // S += K^T V after the block's output.
    for (int e = tid; e < d * kSlice; e += kThreads) {
      int i = e / kSlice, n = e % kSlice;
      float acc = Ss[i][n];
      for (int s = 0; s < c; ++s) acc = fmaf(Ks[s][i], Vs[s][n], acc);
      Ss[i][n] = acc;
    }
  }
  __syncthreads();
  if (s_out != nullptr) {
    for (int e = tid; e < d * kSlice; e += kThreads) {
      int i = e / kSlice, n = e % kSlice;
      s_out[sbase + int64_t(i) * dv + c0 + n] = Ss[i][n];
    }
  }
}

__global__ void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src, size_t n) {
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, dst, src, n);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, const float* s_in,
                          float* s_out, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                          int64_t block, hipStream_t stream) {
  const int64_t grid = B * Hkv * (dv / kSlice);
  hipLaunchKernelGGL(fwd_f32_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, q, k, v, o, s_in, s_out,
                     int(Hq), int(Hkv), N, int(d), int(dv), int(block));
  return hipGetLastError();
}

}  // namespace la
