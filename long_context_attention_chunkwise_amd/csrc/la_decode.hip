// Batched single-token decode step of causal linear attention.
//
// Page "MiniMax-01与Lightning Attention", section 4.1 table: the key-value
// state is updated incrementally and the history is not kept.  Per (batch,
// KV head) state S (d x dv, float32):
//     S <- S + k^T v                 (rank-one update, in place)
//     o_h = q_h S   for the query heads h of the group (reads the updated S)
// The step is bound by HBM bandwidth: each state is streamed from HBM once and
// written back once, and the G query-head products are formed from the same
// registers on the way (one pass, no second read of S).
//
// One workgroup of 512 threads per state (measured against 128, 256 and 1024
// at d = dv = 128: 512 streams fastest).  Groups of more than eight query
// heads are served in chunks of eight: the first launch updates the state and
// serves the first chunk, each further launch re-reads the updated state
// without writing it and serves the next chunk (stream order keeps them in
// sequence).  Thread (row group rg, column group
// cg) owns columns [4cg, 4cg+4) of rows rg, rg + nrg, ...: a wave reads whole
// 512-byte rows with 16-byte accesses.  Per-thread partial products over its
// rows are reduced in a fixed order, so results are deterministic: at dv = 128
// first inside each wave (its two row groups, by a lane exchange), then over
// the eight waves through LDS; at other dv over all row groups through LDS.
// (Both reductions measured the same, 195.3 and 195.6 us per step on the
// 256-sequence workload: the step is bound by streaming the states.)
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 512;
constexpr int kMaxD = 128;
constexpr int kMaxDV = 128;
constexpr int kMaxChunk = 8;  // query heads per launch

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The state is touched once per step: streaming (non-temporal) accesses keep
// it from displacing other data in the caches and measured faster on gfx950.
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ void store_stream(float4* p, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

template <bool IN_BF16>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if (IN_BF16) {
    const uint32_t bits = uint32_t(static_cast<const uint16_t*>(p)[i]) << 16;
    return __builtin_bit_cast(float, bits);
  }
  return static_cast<const float*>(p)[i];
}

// One state's step (state bg = b * Hkv + g).  G: query heads served by this
// launch.  CHUNKED: one chunk [h0, h0 + G) of a larger group of Gfull heads
// (otherwise the whole group, Gfull = G, h0 = 0);
// UPDATE: add k^T v to the state and write it back (otherwise read only).
// WRED (wave-level reduction, dv = 128 only: a wave is two row groups of 32
// column groups): the two row groups of each wave are first added with a
// cross-half lane exchange, so only the eight waves' partials pass through
// LDS; otherwise every row group's partial does.
template <int G, bool IN_BF16, bool OUT_F32, bool CHUNKED, bool UPDATE, bool WRED = false>
__device__ __forceinline__ void decode_body(float* __restrict__ S, const void* __restrict__ q,
                                                         const void* __restrict__ k, const void* __restrict__ v,
                                                         void* __restrict__ o, int Hkv, int d, int dv, int Gfull,
                                                         int h0, int bg_in) {
  __shared__ float qs[G][kMaxD];
  __shared__ float ks[kMaxD];
  __shared__ float vs[kMaxDV];
  __shared__ float4 red[(WRED ? kThreads / 2 : kThreads) * G];  // [row group or wave][head][column group]

  const int bg = bg_in;  // b * Hkv + g
  const int tid = threadIdx.x;
  // first query head served, flattened over batch
  const int64_t hq0 = CHUNKED ? int64_t(bg) * Gfull + h0 : int64_t(bg) * G;
  if (UPDATE) {
    for (int i = tid; i < d; i += kThreads) ks[i] = load_in<IN_BF16>(k, int64_t(bg) * d + i);
    for (int i = tid; i < dv; i += kThreads) vs[i] = load_in<IN_BF16>(v, int64_t(bg) * dv + i);
  }
  for (int i = tid; i < G * d; i += kThreads) qs[i / d][i % d] = load_in<IN_BF16>(q, hq0 * d + i);
  __syncthreads();

  const int ncg = dv / 4;        // column groups
  const int nrg = kThreads / ncg;  // row groups
  const int cg = tid % ncg, rg = tid / ncg;
  float4 acc[G];
  for (int h = 0; h < G; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);

  if (rg < nrg) {
    float4* Sg = reinterpret_cast<float4*>(S + int64_t(bg) * d * dv);
    const float4 v4 = UPDATE ? make_float4(vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3])
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int r = rg; r < d; r += nrg) {
      float4 s = load_stream(&Sg[r * ncg + cg]);
      if (UPDATE) {
        const float kr = ks[r];
        s.x = fmaf(kr, v4.x, s.x);
        s.y = fmaf(kr, v4.y, s.y);
        s.z = fmaf(kr, v4.z, s.z);
        s.w = fmaf(kr, v4.w, s.w);
        store_stream(&Sg[r * ncg + cg], s);
      }
      for (int h = 0; h < G; ++h) {
        const float qr = qs[h][r];
        acc[h].x = fmaf(qr, s.x, acc[h].x);
        acc[h].y = fmaf(qr, s.y, acc[h].y);
        acc[h].z = fmaf(qr, s.z, acc[h].z);
        acc[h].w = fmaf(qr, s.w, acc[h].w);
      }
    }
    if constexpr (!WRED)
      for (int h = 0; h < G; ++h) red[(rg * G + h) * ncg + cg] = acc[h];
  }
  if constexpr (WRED) {
    // lanes i and i + 32 of a wave hold row groups 2w and 2w + 1 of the same
    // column group: add the upper half into the lower, which publishes the
    // wave's partial (row groups 2w, 2w + 1 in that order)
    const int wv = tid >> 6;
    for (int h = 0; h < G; ++h) {
      float4 x = acc[h];
      x.x += __shfl_down(x.x, 32);
      x.y += __shfl_down(x.y, 32);
      x.z += __shfl_down(x.z, 32);
      x.w += __shfl_down(x.w, 32);
      if ((tid & 63) < 32) red[(wv * G + h) * ncg + cg] = x;
    }
  }
  __syncthreads();

  // o[h][4c..4c+3] = sum over row groups (or waves), in order.
  constexpr int kParts = WRED ? kThreads / 64 : 0;
  const int nparts = WRED ? kParts : nrg;
  for (int e = tid; e < G * ncg; e += kThreads) {
    const int h = e / ncg, c = e % ncg;
    float4 sum = red[h * ncg + c];
    for (int r = 1; r < nparts; ++r) {
      const float4 x = red[(r * G + h) * ncg + c];
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const int64_t off = (hq0 + h) * dv + 4 * c;
    if (OUT_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(o) + off) = sum;
    } else {
      uint16_t* ob = static_cast<uint16_t*>(o) + off;
      const float vals[4] = {sum.x, sum.y, sum.z, sum.w};
      for (int i = 0; i < 4; ++i) {
        __bf16 hb = (__bf16)vals[i];
        ob[i] = __builtin_bit_cast(uint16_t, hb);
      }
    }
  }
}

// One workgroup per state, written as a loop over states with the grid's
// stride (one pass per workgroup as launched): the compiler schedules this
// form's loads and stores differently, measured 190.3 against 192.2 us per
// step on the 256-sequence workload (same results bit for bit); grids of two
// to four workgroups per compute unit that loop over several states each
// measured slower (193.5-215 us).
template <int G, bool IN_BF16, bool OUT_F32, bool CHUNKED, bool UPDATE, bool WRED = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(float* __restrict__ S, const void* __restrict__ q,
                                                         const void* __restrict__ k, const void* __restrict__ v,
                                                         void* __restrict__ o, int Hkv, int d, int dv, int Gfull,
                                                         int h0, int nstates) {
  for (int bg = blockIdx.x; bg < nstates; bg += gridDim.x) {
    decode_body<G, IN_BF16, OUT_F32, CHUNKED, UPDATE, WRED>(S, q, k, v, o, Hkv, d, dv, Gfull, h0, bg);
    __syncthreads();
  }
}

template <int G, bool CHUNKED, bool UPDATE>
hipError_t launch_g(float* S, const void* q, const void* k, const void* v, void* o, bool in_bf16, bool out_f32,
                    int64_t B, int64_t Hkv, int64_t d, int64_t dv, int Gfull, int h0, hipStream_t stream) {
  const int64_t ns = B * Hkv;
  const dim3 grid(static_cast<unsigned>(ns)), block(kThreads);
  const int iHkv = int(Hkv), id = int(d), idv = int(dv);
  // dv = 128: the wave-level reduction (each wave is exactly two row groups)
#define LA_DEC(BF, F32, WR)                                                                                       \
  hipLaunchKernelGGL((decode_kernel<G, BF, F32, CHUNKED, UPDATE, WR>), grid, block, 0, stream, S, q, k, v, o, iHkv, \
                     id, idv, Gfull, h0, int(ns))
  if (dv == kMaxDV) {
    if (in_bf16) {
      if (out_f32) LA_DEC(true, true, true);
      else LA_DEC(true, false, true);
    } else {
      if (out_f32) LA_DEC(false, true, true);
      else LA_DEC(false, false, true);
    }
  } else if (in_bf16) {
    if (out_f32) LA_DEC(true, true, false);
    else LA_DEC(true, false, false);
  } else {
    if (out_f32) LA_DEC(false, true, false);
    else LA_DEC(false, false, false);
  }
#undef LA_DEC
  return hipGetLastError();
}

// The first chunk of a group of more than eight heads (state update) or a
// later one (read only), of g heads starting at h0.
template <bool UPDATE>
hipError_t launch_chunk(int g, float* S, const void* q, const void* k, const void* v, void* o, bool in_bf16,
                        bool out_f32, int64_t B, int64_t Hkv, int64_t d, int64_t dv, int Gfull, int h0,
                        hipStream_t stream) {
  switch (g) {
#define LA_C(N)                                                                                                 \
  case N: return launch_g<N, true, UPDATE>(S, q, k, v, o, in_bf16, out_f32, B, Hkv, d, dv, Gfull, h0, stream);
    LA_C(1) LA_C(2) LA_C(3) LA_C(4) LA_C(5) LA_C(6) LA_C(7) LA_C(8)
#undef LA_C
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(float* S, const void* q, const void* k, const void* v, void* o, bool in_bf16,
                         bool out_f32, int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t dv,
                         hipStream_t stream) {
  const int64_t G = Hq / Hkv;
  if (G > kMaxChunk) {
    const int Gf = int(G);
    hipError_t e = launch_chunk<true>(kMaxChunk, S, q, k, v, o, in_bf16, out_f32, B, Hkv, d, dv, Gf, 0, stream);
    for (int h0 = kMaxChunk; e == hipSuccess && h0 < Gf; h0 += kMaxChunk) {
      const int g = Gf - h0 < kMaxChunk ? Gf - h0 : kMaxChunk;
      e = launch_chunk<false>(g, S, q, k, v, o, in_bf16, out_f32, B, Hkv, d, dv, Gf, h0, stream);
    }
    return e;
  }
  switch (G) {
#define LA_G(N) \
  case N: return launch_g<N, false, true>(S, q, k, v, o, in_bf16, out_f32, B, Hkv, d, dv, N, 0, stream);
    LA_G(1) LA_G(2) LA_G(3) LA_G(4) LA_G(5) LA_G(6) LA_G(7) LA_G(8)
#undef LA_G
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
