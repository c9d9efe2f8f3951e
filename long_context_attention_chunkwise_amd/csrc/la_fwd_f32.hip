// float32 causal chunkwise linear attention forward pass.
//
// Follows the block recurrence of page "如何理解MiniMax股价创历史新高？拆解国产大模型
// 技术底座" (vergex.cn), section "Lightning Attention", chunkwise teaching code:
// O_b = Q_b S + tril(Q_b K_b^T) V_b, then S += K_b^T V_b.  All arithmetic is
// float32 FMA (no reduced-precision products), so this path serves float32
// inputs at float32 accuracy, and bf16 inputs (widened exactly as they are
// loaded) at the shapes the matrix-core kernels are not built for.  It is the
// small-problem path: one workgroup per
// (batch, KV head, 32-column slice of dv) walks the whole sequence and serves
// every query head of the group, with the state slice, the block's K and V
// slice and, one head at a time, Q and the score matrix staged in LDS.  The
// state is read from s_in and written to s_out by the same workgroup, so the
// two may be the same buffer.  The same kernel, with template flags, serves
// the forward variants for float32 inputs (ReLU feature map, normalisation,
// non-causal form).
#include "la_internal.h"
#include "la_scalar.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;     // dv columns per workgroup
constexpr int kMaxD = 128;
constexpr int kMaxBlock = 64;
constexpr int kFlagRelu = 1;  // same values as the bf16 kernels' flags
constexpr int kFlagNorm = 2;

// Feature-map variants (FL, the flags of the bf16 kernels) and the
// non-causal form: kRelu maps q and k through phi = ReLU as they enter LDS;
// kNorm divides output row t by phi(q_t) . z + eps, with z (d floats per KV
// head) the running sum of phi(k) kept in LDS beside the state slice (each
// slice's workgroup keeps its own copy).  Non-causal (CAUSAL false): a first
// pass sums the state (and z) over every block, a second pass forms
// o_t = phi(q_t) S_tot for every row.
//
// TI / TO: storage types of q, k, v and of o (float or bf16 bits); the
// arithmetic is float32 either way.
template <typename TI, typename TO, int FL, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                                                          const TI* __restrict__ v, TO* __restrict__ o,
                                                          const float* s_in, float* s_out, const float* z_in,
                                                          float eps, int Hq, int Hkv, int64_t N, int d, int dv,
                                                          int C) {
  constexpr bool kR = (FL & kFlagRelu) != 0;
  constexpr bool kN = (FL & kFlagNorm) != 0;
  __shared__ float Qs[kMaxBlock][kMaxD + 1];
  __shared__ float Ks[kMaxBlock][kMaxD + 1];
  __shared__ float Vs[kMaxBlock][kSlice];
  __shared__ float Ps[kMaxBlock][kMaxBlock + 1];
  __shared__ float Ss[kMaxD][kSlice];
  __shared__ float Zs[kN ? kMaxD : 1];       // z before the current block (kNorm)
  __shared__ float Den[kN ? kMaxBlock : 1];  // row denominators of the current head (kNorm)

  const int nslices = dv / kSlice;
  const int slice = blockIdx.x % nslices;
  const int bg = blockIdx.x / nslices;  // b * Hkv + g
  const int g = bg % Hkv, b = bg / Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int c0 = slice * kSlice;

  const TI* kh = k + int64_t(bg) * N * d;
  const TI* vh = v + int64_t(bg) * N * dv;
  const int64_t sbase = int64_t(bg) * d * dv;
  auto phi = [](float x) { return kR ? fmaxf(x, 0.0f) : x; };

  for (int e = tid; e < d * kSlice; e += kThreads) {
    int i = e / kSlice, n = e % kSlice;
    Ss[i][n] = s_in ? s_in[sbase + int64_t(i) * dv + c0 + n] : 0.0f;
  }
  if constexpr (kN)
    for (int i = tid; i < d; i += kThreads) Zs[i] = z_in ? z_in[int64_t(bg) * d + i] : 0.0f;

  // K and V of the block starting at a (c rows) into LDS.
  auto load_kv = [&](int64_t a, int c) {
    for (int e = tid; e < c * d; e += kThreads) {
      int t = e / d, i = e % d;
      Ks[t][i] = phi(ldf(kh, (a + t) * d + i));
    }
    for (int e = tid; e < c * kSlice; e += kThreads) {
      int t = e / kSlice, n = e % kSlice;
      Vs[t][n] = ldf(vh, (a + t) * dv + c0 + n);
    }
  };
  // S += K^T V (and z += sum of the K rows) after the block's outputs.
  auto update_state = [&](int c) {
    for (int e = tid; e < d * kSlice; e += kThreads) {
      int i = e / kSlice, n = e % kSlice;
      float acc = Ss[i][n];
      for (int s = 0; s < c; ++s) acc = fmaf(Ks[s][i], Vs[s][n], acc);
      Ss[i][n] = acc;
    }
    if constexpr (kN)
      for (int i = tid; i < d; i += kThreads) {
        float acc = Zs[i];
        for (int s = 0; s < c; ++s) acc += Ks[s][i];
        Zs[i] = acc;
      }
  };

  if constexpr (!CAUSAL) {
    for (int64_t a = 0; a < N; a += C) {
      const int c = int(N - a < C ? N - a : C);
      __syncthreads();
      load_kv(a, c);
      __syncthreads();
      update_state(c);
    }
  }

  for (int64_t a = 0; a < N; a += C) {
    const int c = int(N - a < C ? N - a : C);
    __syncthreads();  // previous block finished with Ks/Vs/Ss
    if constexpr (CAUSAL) load_kv(a, c);
    for (int hh = 0; hh < G; ++hh) {
      const int64_t bh = int64_t(b) * Hq + int64_t(g) * G + hh;
      const TI* qh = q + bh * N * d;
      TO* oh = o + bh * N * dv;
      __syncthreads();  // previous head finished with Qs/Ps/Den
      for (int e = tid; e < c * d; e += kThreads) {
        int t = e / d, i = e % d;
        Qs[t][i] = phi(ldf(qh, (a + t) * d + i));
      }
      __syncthreads();
      if constexpr (CAUSAL) {
        // In-block scores with the causal mask (s <= t kept).
        for (int e = tid; e < c * c; e += kThreads) {
          int t = e / c, s = e % c;
          float acc = 0.0f;
          if (s <= t)
            for (int i = 0; i < d; ++i) acc = fmaf(Qs[t][i], Ks[s][i], acc);
          Ps[t][s] = acc;
        }
        __syncthreads();
      }
      if constexpr (kN) {
        // denominator of row t: its weights summed without values
        for (int t = tid; t < c; t += kThreads) {
          float acc = 0.0f;
          for (int i = 0; i < d; ++i) acc = fmaf(Qs[t][i], Zs[i], acc);
          if constexpr (CAUSAL)
            for (int s = 0; s <= t; ++s) acc += Ps[t][s];
          Den[t] = acc + eps;
        }
        __syncthreads();
      }
      // O = Q S (state before this block, or the total) + P V.
      for (int e = tid; e < c * kSlice; e += kThreads) {
        int t = e / kSlice, n = e % kSlice;
        float inter = 0.0f, intra = 0.0f;
        for (int i = 0; i < d; ++i) inter = fmaf(Qs[t][i], Ss[i][n], inter);
        if constexpr (CAUSAL)
          for (int s = 0; s <= t; ++s) intra = fmaf(Ps[t][s], Vs[s][n], intra);
        float out = inter + intra;
        if constexpr (kN) out = out / Den[t];
        stf(oh, (a + t) * dv + c0 + n, out);
      }
    }
    if constexpr (CAUSAL) {
      __syncthreads();
      update_state(c);
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

// z_out[c][i] = z_in[c][i] (or 0) + sum over every token of phi(k[c][t][i]);
// one thread per (KV chain, i).  Runs after the output kernel, so z_out may be
// z_in itself.
template <typename TI, bool RELU>
__global__ void z_sum_f32(const TI* __restrict__ k, const float* z_in, float* z_out, int64_t chains, int64_t N,
                          int d) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= chains * d) return;
  const int64_t c = e / d;
  const int i = int(e % d);
  const TI* kc = k + c * N * d + i;
  float acc = z_in ? z_in[e] : 0.0f;
  for (int64_t t = 0; t < N; ++t) {
    const float x = ldf(kc, t * d);
    acc += RELU ? fmaxf(x, 0.0f) : x;
  }
  z_out[e] = acc;
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

namespace {

template <typename TI, typename TO>
hipError_t launch_scalar(const void* q, const void* k, const void* v, void* o, bool causal, bool relu, bool norm,
                         float eps, const float* s_in, float* s_out, const float* z_in, float* z_out, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                         hipStream_t stream) {
  const dim3 grid(unsigned(B * Hkv * (dv / kSlice)));
  const int iHq = int(Hq), iHkv = int(Hkv), id = int(d), idv = int(dv), ib = int(block);
  const TI* qt = static_cast<const TI*>(q);
  const TI* kt = static_cast<const TI*>(k);
  const TI* vt = static_cast<const TI*>(v);
  TO* ot = static_cast<TO*>(o);
#define LA_F32V(FL, CAUSAL)                                                                                     \
  hipLaunchKernelGGL((fwd_f32_kernel<TI, TO, FL, CAUSAL>), grid, dim3(kThreads), 0, stream, qt, kt, vt, ot, s_in, \
                     s_out, z_in, eps, iHq, iHkv, N, id, idv, ib)
  const int fl = (relu ? kFlagRelu : 0) | (norm ? kFlagNorm : 0);
  switch (fl + (causal ? 4 : 0)) {
    case 0: LA_F32V(0, false); break;
    case 1: LA_F32V(1, false); break;
    case 2: LA_F32V(2, false); break;
    case 3: LA_F32V(3, false); break;
    case 4: LA_F32V(0, true); break;
    case 5: LA_F32V(1, true); break;
    case 6: LA_F32V(2, true); break;
    default: LA_F32V(3, true); break;
  }
#undef LA_F32V
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !norm || z_out == nullptr) return e;
  const int64_t nz = B * Hkv * d;
  if (relu)
    hipLaunchKernelGGL((z_sum_f32<TI, true>), dim3(unsigned((nz + 255) / 256)), dim3(256), 0, stream, kt, z_in,
                       z_out, B * Hkv, N, id);
  else
    hipLaunchKernelGGL((z_sum_f32<TI, false>), dim3(unsigned((nz + 255) / 256)), dim3(256), 0, stream, kt, z_in,
                       z_out, B * Hkv, N, id);
  return hipGetLastError();
}

}  // namespace

namespace {

// State-only pass on float32 FMA: s_out[c] = s_in[c] + sum over the G input
// chains c G .. c G + G - 1 and all N tokens of k_t^T v_t (the forward's state:
// G = 1, k and v of KV head c; the backward's: G query heads' q and dO).
// Workgroup (c, i-tile) owns
// rows [16 it, 16 it + 16) of the d x dv state, all dv columns; thread t owns
// column t % 128 of rows 16 it + 8 (t / 128) + {0..7}.  The sequence is walked
// in 64-token chunks staged in LDS.  s_out may be s_in (each entry is read
// and written by one thread).
template <typename TI>
__global__ __launch_bounds__(kThreads) void state_total_f32(const TI* __restrict__ k, const TI* __restrict__ v,
                                                           const float* s_in, float* s_out, int64_t N, int d,
                                                           int dv, int G) {
  constexpr int CH = 64, RT = 16;
  __shared__ float Ks[CH][RT];
  __shared__ float Vs[CH][kMaxD];
  const int nit = (d + RT - 1) / RT;
  const int64_t c = blockIdx.x / nit;
  const int i0 = (blockIdx.x % nit) * RT;
  const int tid = threadIdx.x;
  const int j = tid % kMaxD, rg = tid / kMaxD;
  float acc[8];
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  for (int h = 0; h < G; ++h) {
  const TI* kc = k + (c * G + h) * N * d;
  const TI* vc = v + (c * G + h) * N * dv;
  for (int64_t t0 = 0; t0 < N; t0 += CH) {
    for (int e = tid; e < CH * RT; e += kThreads) {
      const int tt = e / RT, ii = e % RT;
      const int64_t t = t0 + tt;
      Ks[tt][ii] = (t < N && i0 + ii < d) ? ldf(kc, t * d + i0 + ii) : 0.0f;
    }
    for (int e = tid; e < CH * kMaxD; e += kThreads) {
      const int tt = e / kMaxD, jj = e % kMaxD;
      const int64_t t = t0 + tt;
      Vs[tt][jj] = (t < N && jj < dv) ? ldf(vc, t * dv + jj) : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < CH; ++tt) {
      const float vv = Vs[tt][j];
      for (int r = 0; r < 8; ++r) acc[r] = fmaf(Ks[tt][8 * rg + r], vv, acc[r]);
    }
    __syncthreads();
  }
  }
  if (j < dv)
    for (int r = 0; r < 8; ++r) {
      const int i = i0 + 8 * rg + r;
      if (i < d) {
        const int64_t idx = (c * d + i) * dv + j;
        s_out[idx] = (s_in ? s_in[idx] : 0.0f) + acc[r];
      }
    }
}

}  // namespace

hipError_t launch_state_total_f32(const void* k, const void* v, bool in_bf16, const float* s_in, float* s_out,
                                  int64_t chains, int G, int64_t N, int64_t d, int64_t dv, hipStream_t stream) {
  if (d < 1 || d > kMaxD || dv < 1 || dv > kMaxD || G < 1) return hipErrorInvalidValue;
  const dim3 grid(unsigned(chains * ((d + 15) / 16)));
  if (in_bf16)
    hipLaunchKernelGGL((state_total_f32<uint16_t>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), s_in, s_out, N, int(d),
                       int(dv), G);
  else
    hipLaunchKernelGGL((state_total_f32<float>), grid, dim3(kThreads), 0, stream, static_cast<const float*>(k),
                       static_cast<const float*>(v), s_in, s_out, N, int(d), int(dv), G);
  return hipGetLastError();
}

hipError_t launch_fwd_f32_variant(const void* q, const void* k, const void* v, void* o, bool in_bf16,
                                  bool out_bf16, bool causal, bool relu, bool norm, float eps, const float* s_in,
                                  float* s_out, const float* z_in, float* z_out, int64_t B, int64_t Hq,
                                  int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                                  hipStream_t stream) {
  if (in_bf16)
    return out_bf16 ? launch_scalar<uint16_t, uint16_t>(q, k, v, o, causal, relu, norm, eps, s_in, s_out, z_in,
                                                         z_out, B, Hq, Hkv, N, d, dv, block, stream)
                    : launch_scalar<uint16_t, float>(q, k, v, o, causal, relu, norm, eps, s_in, s_out, z_in,
                                                      z_out, B, Hq, Hkv, N, d, dv, block, stream);
  return out_bf16 ? launch_scalar<float, uint16_t>(q, k, v, o, causal, relu, norm, eps, s_in, s_out, z_in, z_out, B,
                                                    Hq, Hkv, N, d, dv, block, stream)
                  : launch_scalar<float, float>(q, k, v, o, causal, relu, norm, eps, s_in, s_out, z_in, z_out, B, Hq,
                                                 Hkv, N, d, dv, block, stream);
}

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, bool in_bf16, bool out_bf16,
                          const float* s_in, float* s_out, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                          int64_t dv, int64_t block, hipStream_t stream) {
  return launch_fwd_f32_variant(q, k, v, o, in_bf16, out_bf16, true, false, false, 0.0f, s_in, s_out, nullptr,
                                nullptr, B, Hq, Hkv, N, d, dv, block, stream);
}

}  // namespace la
