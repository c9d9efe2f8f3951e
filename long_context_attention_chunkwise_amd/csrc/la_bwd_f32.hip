// float32 backward pass of causal chunkwise linear attention.
//
// Gradients of the forward of page "如何理解MiniMax股价创历史新高？拆解国产大模型技术
// 底座" (vergex.cn), section "Lightning Attention", chunkwise teaching code, with
// query head h reading KV head h / (Hq / Hkv) (page "MiniMax-01与Lightning
// Attention", section 1.1 table).  The pages give no backward; differentiating
// o_t = q_t . s_in + sum_{s<=t} (q_t . k_s) v_s and s_out = s_in + sum_s k_s^T v_s
// gives, per KV head, with the state R = ds_out + sum over later tokens and the
// group's query heads of q^T dO:
//     dQ_b = dO_b s_in^T + (forward over (dO, V, K))   -- the forward kernel
//     dV_b = K_b R + sum_h triu(K_b Q_hb^T) dO_hb
//     dK_b = V_b R^T + sum_h triu(V_b dO_hb^T) Q_hb
//     R   <- R + sum_h Q_hb^T dO_hb                    (after the block)
// walked from the last block to the first; ds_in is the final R.
//
// All arithmetic is float32 FMA, so this path serves float32 inputs at float32
// accuracy, and bf16 inputs (widened exactly as they are loaded) at the shapes
// the matrix-core kernels are not built for.  Like the float32 forward it is
// the small-problem path: one
// workgroup per (batch, KV head, 32-column slice) walks the whole sequence
// backwards and serves every query head of the group.  The dV kernel slices
// dv (it holds R's columns of its slice); the dK kernel slices d (it holds R's
// rows of its slice); each recomputes the score block it needs.
#include "la_internal.h"
#include "la_scalar.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;
constexpr int kMaxD = 128;
constexpr int kMaxBlock = 64;

// dV[:, c0:c0+32] and ds_in[:, c0:c0+32].  TI / TG: storage types of the
// inputs and of the gradients (float or bf16 bits); float32 arithmetic.
template <typename TI, typename TG>
__global__ __launch_bounds__(kThreads) void bwd_dv_f32(const TI* __restrict__ q, const TI* __restrict__ k,
                                                      const TI* __restrict__ dout, TG* __restrict__ dvg,
                                                      const float* ds_out, float* ds_in, int Hq, int Hkv,
                                                      int64_t N, int d, int dv, int C) {
  __shared__ float Ks[kMaxBlock][kMaxD + 1];    // K_b
  __shared__ float Qs[kMaxBlock][kMaxD + 1];    // Q_hb
  __shared__ float Os[kMaxBlock][kSlice];       // dO_hb, this slice's columns
  __shared__ float Xs[kMaxBlock][kMaxBlock + 1];  // X[s][t] = k_s . q_t for t >= s, else 0
  __shared__ float Rs[kMaxD][kSlice];           // R, this slice's columns
  __shared__ float As[kMaxBlock][kSlice];       // dV rows of the block

  const int nslices = dv / kSlice;
  const int slice = blockIdx.x % nslices;
  const int bg = blockIdx.x / nslices;  // b * Hkv + g
  const int g = bg % Hkv, b = bg / Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int c0 = slice * kSlice;
  const TI* kh = k + int64_t(bg) * N * d;
  const int64_t sbase = int64_t(bg) * d * dv;

  for (int e = tid; e < d * kSlice; e += kThreads) {
    const int i = e / kSlice, n = e % kSlice;
    Rs[i][n] = ds_out ? ds_out[sbase + int64_t(i) * dv + c0 + n] : 0.0f;
  }
  const int64_t nblocks = (N + C - 1) / C;
  for (int64_t blk = nblocks - 1; blk >= 0; --blk) {
    const int64_t a = blk * C;
    const int c = int(N - a < C ? N - a : C);
    __syncthreads();  // the previous block's stores and R updates are done
    for (int e = tid; e < c * d; e += kThreads) {
      const int t = e / d, i = e % d;
      Ks[t][i] = ldf(kh, (a + t) * d + i);
    }
    __syncthreads();
    // inter: K_b R with R over later tokens only
    for (int e = tid; e < c * kSlice; e += kThreads) {
      const int s = e / kSlice, n = e % kSlice;
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) acc = fmaf(Ks[s][i], Rs[i][n], acc);
      As[s][n] = acc;
    }
    for (int hh = 0; hh < G; ++hh) {
      const int64_t bh = int64_t(b) * Hq + int64_t(g) * G + hh;
      __syncthreads();  // the inter term and the previous head are done with Qs, Os, Xs, Rs
      for (int e = tid; e < c * d; e += kThreads) {
        const int t = e / d, i = e % d;
        Qs[t][i] = ldf(q, (bh * N + a + t) * d + i);
      }
      for (int e = tid; e < c * kSlice; e += kThreads) {
        const int t = e / kSlice, n = e % kSlice;
        Os[t][n] = ldf(dout, (bh * N + a + t) * dv + c0 + n);
      }
      __syncthreads();
      for (int e = tid; e < c * c; e += kThreads) {
        const int s = e / c, t = e % c;
        float acc = 0.0f;
        if (t >= s)
          for (int i = 0; i < d; ++i) acc = fmaf(Ks[s][i], Qs[t][i], acc);
        Xs[s][t] = acc;
      }
      __syncthreads();
      // intra: dV[s] += sum_{t >= s} X[s][t] dO[t];  R += Q^T dO (each thread its own elements)
      for (int e = tid; e < c * kSlice; e += kThreads) {
        const int s = e / kSlice, n = e % kSlice;
        float acc = As[s][n];
        for (int t = s; t < c; ++t) acc = fmaf(Xs[s][t], Os[t][n], acc);
        As[s][n] = acc;
      }
      for (int e = tid; e < d * kSlice; e += kThreads) {
        const int i = e / kSlice, n = e % kSlice;
        float acc = Rs[i][n];
        for (int t = 0; t < c; ++t) acc = fmaf(Qs[t][i], Os[t][n], acc);
        Rs[i][n] = acc;
      }
    }
    __syncthreads();
    for (int e = tid; e < c * kSlice; e += kThreads) {
      const int s = e / kSlice, n = e % kSlice;
      stf(dvg, (int64_t(bg) * N + a + s) * dv + c0 + n, As[s][n]);
    }
  }
  __syncthreads();
  if (ds_in != nullptr)
    for (int e = tid; e < d * kSlice; e += kThreads) {
      const int i = e / kSlice, n = e % kSlice;
      ds_in[sbase + int64_t(i) * dv + c0 + n] = Rs[i][n];
    }
}

// dK[:, c0:c0+32].
template <typename TI, typename TG>
__global__ __launch_bounds__(kThreads) void bwd_dk_f32(const TI* __restrict__ q, const TI* __restrict__ v,
                                                      const TI* __restrict__ dout, TG* __restrict__ dkg,
                                                      const float* ds_out, int Hq, int Hkv, int64_t N, int d,
                                                      int dv, int C) {
  __shared__ float Vs[kMaxBlock][kMaxD + 1];    // V_b
  __shared__ float Os[kMaxBlock][kMaxD + 1];    // dO_hb
  __shared__ float Qs[kMaxBlock][kSlice];       // Q_hb, this slice's columns
  __shared__ float Ys[kMaxBlock][kMaxBlock + 1];  // Y[s][t] = v_s . dO_t for t >= s, else 0
  __shared__ float Rr[kSlice][kMaxD + 1];       // R, this slice's rows
  __shared__ float As[kMaxBlock][kSlice];       // dK rows of the block

  const int nslices = d / kSlice;
  const int slice = blockIdx.x % nslices;
  const int bg = blockIdx.x / nslices;
  const int g = bg % Hkv, b = bg / Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int c0 = slice * kSlice;
  const TI* vh = v + int64_t(bg) * N * dv;
  const int64_t sbase = int64_t(bg) * d * dv;

  for (int e = tid; e < kSlice * dv; e += kThreads) {
    const int i = e / dv, n = e % dv;
    Rr[i][n] = ds_out ? ds_out[sbase + int64_t(c0 + i) * dv + n] : 0.0f;
  }
  const int64_t nblocks = (N + C - 1) / C;
  for (int64_t blk = nblocks - 1; blk >= 0; --blk) {
    const int64_t a = blk * C;
    const int c = int(N - a < C ? N - a : C);
    __syncthreads();
    for (int e = tid; e < c * dv; e += kThreads) {
      const int t = e / dv, n = e % dv;
      Vs[t][n] = ldf(vh, (a + t) * dv + n);
    }
    __syncthreads();
    // inter: V_b R^T over this slice's rows of R
    for (int e = tid; e < c * kSlice; e += kThreads) {
      const int s = e / kSlice, i = e % kSlice;
      float acc = 0.0f;
      for (int n = 0; n < dv; ++n) acc = fmaf(Vs[s][n], Rr[i][n], acc);
      As[s][i] = acc;
    }
    for (int hh = 0; hh < G; ++hh) {
      const int64_t bh = int64_t(b) * Hq + int64_t(g) * G + hh;
      __syncthreads();
      for (int e = tid; e < c * dv; e += kThreads) {
        const int t = e / dv, n = e % dv;
        Os[t][n] = ldf(dout, (bh * N + a + t) * dv + n);
      }
      for (int e = tid; e < c * kSlice; e += kThreads) {
        const int t = e / kSlice, i = e % kSlice;
        Qs[t][i] = ldf(q, (bh * N + a + t) * d + c0 + i);
      }
      __syncthreads();
      for (int e = tid; e < c * c; e += kThreads) {
        const int s = e / c, t = e % c;
        float acc = 0.0f;
        if (t >= s)
          for (int n = 0; n < dv; ++n) acc = fmaf(Vs[s][n], Os[t][n], acc);
        Ys[s][t] = acc;
      }
      __syncthreads();
      for (int e = tid; e < c * kSlice; e += kThreads) {
        const int s = e / kSlice, i = e % kSlice;
        float acc = As[s][i];
        for (int t = s; t < c; ++t) acc = fmaf(Ys[s][t], Qs[t][i], acc);
        As[s][i] = acc;
      }
      for (int e = tid; e < kSlice * dv; e += kThreads) {
        const int i = e / dv, n = e % dv;
        float acc = Rr[i][n];
        for (int t = 0; t < c; ++t) acc = fmaf(Qs[t][i], Os[t][n], acc);
        Rr[i][n] = acc;
      }
    }
    __syncthreads();
    for (int e = tid; e < c * kSlice; e += kThreads) {
      const int s = e / kSlice, i = e % kSlice;
      stf(dkg, (int64_t(bg) * N + a + s) * d + c0 + i, As[s][i]);
    }
  }
}

// out[c][n][i] = in[c][i][n] for count states of d x dv.
__global__ void transpose_f32(const float* __restrict__ in, float* __restrict__ out, int64_t count, int d, int dv) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per = int64_t(d) * dv;
  if (e >= count * per) return;
  const int64_t c = e / per, r = e % per;
  const int i = int(r / dv), n = int(r % dv);
  out[c * per + int64_t(n) * d + i] = in[e];
}

}  // namespace

size_t bwd_f32_workspace_floats(int64_t B, int64_t Hkv, int64_t d, int64_t dv) {
  return size_t(B * Hkv) * size_t(d * dv);
}

namespace {

template <typename TI, typename TG>
void launch_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dvg,
                 const float* ds_out, float* ds_in, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 int64_t dv, int64_t block, hipStream_t stream) {
  const TI *qt = static_cast<const TI*>(q), *kt = static_cast<const TI*>(k), *vt = static_cast<const TI*>(v);
  const TI* ot = static_cast<const TI*>(dout);
  // dK first: it reads ds_out, which the dV kernel may overwrite (ds_in may be
  // ds_out itself; each dV workgroup reads and writes only its own columns).
  hipLaunchKernelGGL((bwd_dk_f32<TI, TG>), dim3(unsigned(B * Hkv * (d / kSlice))), dim3(kThreads), 0, stream, qt,
                     vt, ot, static_cast<TG*>(dk), ds_out, int(Hq), int(Hkv), N, int(d), int(dv), int(block));
  hipLaunchKernelGGL((bwd_dv_f32<TI, TG>), dim3(unsigned(B * Hkv * (dv / kSlice))), dim3(kThreads), 0, stream, qt,
                     kt, ot, static_cast<TG*>(dvg), ds_out, ds_in, int(Hq), int(Hkv), N, int(d), int(dv),
                     int(block));
}

}  // namespace

hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                          void* dvg, bool in_bf16, bool grad_bf16, const float* s_in, const float* ds_out,
                          float* ds_in, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                          int64_t block, float* workspace, hipStream_t stream) {
  // dQ: the scalar forward over (queries dO, keys V, values K) from s_in^T
  const float* s_t = nullptr;
  if (s_in != nullptr) {
    const int64_t n = B * Hkv * d * dv;
    hipLaunchKernelGGL(transpose_f32, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, s_in, workspace,
                       B * Hkv, int(d), int(dv));
    s_t = workspace;
  }
  hipError_t e = launch_fwd_f32(dout, v, k, dq, in_bf16, grad_bf16, s_t, nullptr, B, Hq, Hkv, N, dv, d, block,
                                stream);
  if (e != hipSuccess) return e;
  if (in_bf16) {
    if (grad_bf16) launch_dkdv<uint16_t, uint16_t>(q, k, v, dout, dk, dvg, ds_out, ds_in, B, Hq, Hkv, N, d, dv, block, stream);
    else launch_dkdv<uint16_t, float>(q, k, v, dout, dk, dvg, ds_out, ds_in, B, Hq, Hkv, N, d, dv, block, stream);
  } else {
    if (grad_bf16) launch_dkdv<float, uint16_t>(q, k, v, dout, dk, dvg, ds_out, ds_in, B, Hq, Hkv, N, d, dv, block, stream);
    else launch_dkdv<float, float>(q, k, v, dout, dk, dvg, ds_out, ds_in, B, Hq, Hkv, N, d, dv, block, stream);
  }
  return hipGetLastError();
}

}  // namespace la
