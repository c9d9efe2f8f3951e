// Backward pass of causal chunkwise linear attention: dK and dV (gfx950).
//
// The forward (page "如何理解MiniMax股价创历史新高？拆解国产大模型技术底座",
// vergex.cn, section "Lightning Attention", chunkwise teaching code) is
// o_t = sum_{s<=t} (q_t . k_s) v_s with query head h reading KV head
// h / (Hq / Hkv) (page "MiniMax-01与Lightning Attention", section 1.1 table).
// The pages give no backward; differentiating that sum gives, per KV head,
//     dk_s = sum_h sum_{t>=s} (v_s . dO_ht) q_ht
//     dv_s = sum_h sum_{t>=s} (k_s . q_ht) dO_ht
// an anti-causal recurrence whose state R = sum over later tokens and the
// group's query heads of q^T dO (d x dv) serves both:
//     dV_b = K_b R + sum_h triu(K_b Q_hb^T) dO_hb
//     dK_b = V_b R^T + sum_h triu(V_b dO_hb^T) Q_hb
//     R   <- R + sum_h Q_hb^T dO_hb            (after the block)
// walked from the last block to the first.  (dQ is the causal forward on
// (dO, V, K) and runs on the forward kernels.)
//
// Design for MI355X: one workgroup of four waves (one per SIMD) per (batch,
// KV head, sequence segment); segment j starts from the sum over later
// segments, produced by the forward's pre-pass kernel run on (Q, dO) pairs and
// a reverse scan here.  Wave w owns dV columns, dK columns and state columns
// [32w, 32w+32); the fp32 state stays in VGPRs and is rounded to bf16 once
// per block into an n-major LDS copy for the inter terms.  Query heads are
// processed one at a time through LDS; the next head's (or next block's)
// tiles are loaded into registers while the current one computes.  Products
// are v_mfma_f32_16x16x32_bf16 with the transposed-product layout of the
// forward kernel: the accumulators of the masked score tiles X^T = Q K^T and
// Y^T = dO V^T are the B operands of the token-contracting products, shared
// between waves through LDS in operand order.
#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

using namespace mfma16;

constexpr int kThreads = 256;
constexpr int DD = D * DV;

// Two row-major [64][128] bf16 tiles of one block: thread tid moves rows
// tid/16 + 16i (i < 4), 16-byte chunk tid%16; rows at or past N are zero.
struct PairRegs {
  uint4 a[4], b[4];
};

__device__ __forceinline__ void load_pair(PairRegs& r, const uint16_t* ah, const uint16_t* bh, int64_t blk,
                                          int64_t N, int tid) {
  const int c = tid & 15;
  for (int i = 0; i < 4; ++i) {
    const int64_t t = blk * C + (tid >> 4) + 16 * i;
    if (t < N) {
      r.a[i] = ld_stream16(ah + t * D + 8 * c);
      r.b[i] = ld_stream16(bh + t * DV + 8 * c);
    } else {
      r.a[i] = make_uint4(0, 0, 0, 0);
      r.b[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void store_pair(const PairRegs& r, uint16_t* as, uint16_t* bs, int tid) {
  const int c = tid & 15;
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 16 * i;
    *reinterpret_cast<uint4*>(as + row * ROWKV + 8 * c) = r.a[i];
    *reinterpret_cast<uint4*>(bs + row * ROWKV + 8 * c) = r.b[i];
  }
}

// Keep the entries of a diagonal score tile with query position t >= key
// position s: entry (t = 4grp + i, s = l16) of the tile.
__device__ __forceinline__ floatx4 keep_query_after_key(floatx4 x, int l16, int grp) {
  for (int i = 0; i < 4; ++i)
    if (4 * grp + i < l16) x[i] = 0.0f;
  return x;
}

struct __align__(16) BwdSmem {
  uint16_t k[C * ROWKV];    // K_b   [s][d]
  uint16_t v[C * ROWKV];    // V_b   [s][n]
  uint16_t q[C * ROWKV];    // Q_hb  [t][d]  (one query head at a time)
  uint16_t o[C * ROWKV];    // dO_hb [t][n]
  uint16_t rt[DV * ROWST];  // bf16 copy of R, n-major: rt[n][i]
  bf16x8 xb[2][8][64];      // X^T / Y^T operand packs: [X or Y][4p + s-tile][lane]
};

template <bool OUT_F32>
__device__ __forceinline__ void store_row4(void* base, int64_t off, floatx4 x) {
  if (OUT_F32)
    *reinterpret_cast<floatx4*>(static_cast<float*>(base) + off) = x;
  else
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(base) + off) = to_bf16x4(x);
}

template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, void* __restrict__ dk, void* __restrict__ dvg,
    const float* __restrict__ rstarts, float* __restrict__ ds_in, int Hq, int Hkv, int64_t N,
    int64_t nblocks, int64_t blocks_per_seg, int P) {
  __shared__ BwdSmem sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int bg = blockIdx.x / P;  // b * Hkv + g
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;

  const uint16_t* kh = k + int64_t(bg) * N * D;
  const uint16_t* vh = v + int64_t(bg) * N * DV;
  const uint16_t* qg = q + (int64_t(b) * Hq + int64_t(g) * G) * N * D;        // head 0 of the group
  const uint16_t* og = dout + (int64_t(b) * Hq + int64_t(g) * G) * N * DV;

  // State of the later tokens, wave w's columns [32w, 32w+32).
  const float* r0 = rstarts ? rstarts + (int64_t(bg) * P + seg) * DD : nullptr;
  floatx4 racc[2][8];
  for (int jn = 0; jn < 2; ++jn)
    for (int it = 0; it < 8; ++it)
      for (int i = 0; i < 4; ++i)
        racc[jn][it][i] = r0 ? r0[(16 * it + 4 * grp + i) * DV + 32 * w + 16 * jn + l16] : 0.0f;
  for (int jn = 0; jn < 2; ++jn)
    for (int it = 0; it < 8; ++it)
      *reinterpret_cast<bf16x4*>(&sm.rt[(32 * w + 16 * jn + l16) * ROWST + 16 * it + 4 * grp]) =
          to_bf16x4(racc[jn][it]);

  PairRegs kv, qd;
  if (blk1 > blk0) {
    load_pair(kv, kh, vh, blk1 - 1, N, tid);
    load_pair(qd, qg, og, blk1 - 1, N, tid);
  }
  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t blk = blk1 - 1; blk >= blk0; --blk) {
    store_pair(kv, sm.k, sm.v, tid);
    if (blk - 1 >= blk0) load_pair(kv, kh, vh, blk - 1, N, tid);

    floatx4 adv[2][4], adk[2][4];  // dV^T / dK^T tiles: [column tile of 32w + 16j][s-tile]
    for (int j = 0; j < 2; ++j)
      for (int si = 0; si < 4; ++si) {
        adv[j][si] = z4;
        adk[j][si] = z4;
      }

    for (int h = 0; h < G; ++h) {
      store_pair(qd, sm.q, sm.o, tid);
      __syncthreads();  // K/V, this head's Q/dO and the state copy are in LDS
      {
        const bool last = h + 1 == G;
        const int64_t nb = last ? blk - 1 : blk;
        const int nh = last ? 0 : h + 1;
        if (nb >= blk0) load_pair(qd, qg + int64_t(nh) * N * D, og + int64_t(nh) * N * DV, nb, N, tid);
      }

      if (h == 0) {
        // inter: dV^T[n][s] += sum_i R[i][n] K[s][i];  dK^T[i][s] += sum_n R[i][n] V[s][n]
        for (int p = 0; p < 4; ++p) {
          bf16x8 ra[2], rb[2];
          for (int j = 0; j < 2; ++j) {
            ra[j] = ld_lds16(sm.rt + (32 * w + 16 * j + l16) * ROWST + 32 * p + 8 * grp);
            rb[j] = tr_operand(sm.rt, p, 32 * w + 16 * j, l16, grp, 4, ROWST);
          }
          for (int si = 0; si < 4; ++si) {
            const uint16_t* krow = sm.k + (16 * si + l16) * ROWKV;
            const uint16_t* vrow = sm.v + (16 * si + l16) * ROWKV;
            const bf16x8 bk = ld_lds16(krow + 32 * p + 8 * grp);
            // V[s] at the transpose load's slots 32p + 4grp + {0..3}, 32p + 16 + 4grp + {0..3}
            const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 4 * grp);
            const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 16 + 4 * grp);
            bf16x8 bv;
            for (int i = 0; i < 4; ++i) {
              bv[i] = v0[i];
              bv[i + 4] = v1[i];
            }
            for (int j = 0; j < 2; ++j) {
              adv[j][si] = mfma(ra[j], bk, adv[j][si]);
              adk[j][si] = mfma(rb[j], bv, adk[j][si]);
            }
          }
        }
      }

      // scores of key tile s-tile = w: X^T[t][s] = Q[t].K[s], Y^T[t][s] = dO[t].V[s]
      // for query tiles t-tile >= w, masked to t >= s on the diagonal tile.
      {
        floatx4 xt[4], yt[4];
        for (int ti = 0; ti < 4; ++ti) {
          xt[ti] = z4;
          yt[ti] = z4;
        }
        for (int ds = 0; ds < 4; ++ds) {
          const bf16x8 bk = ld_lds16(sm.k + (16 * w + l16) * ROWKV + 32 * ds + 8 * grp);
          const bf16x8 bv = ld_lds16(sm.v + (16 * w + l16) * ROWKV + 32 * ds + 8 * grp);
          for (int ti = 0; ti < 4; ++ti) {
            if (ti < w) continue;
            const bf16x8 aq = ld_lds16(sm.q + (16 * ti + l16) * ROWKV + 32 * ds + 8 * grp);
            const bf16x8 ao = ld_lds16(sm.o + (16 * ti + l16) * ROWKV + 32 * ds + 8 * grp);
            xt[ti] = mfma(aq, bk, xt[ti]);
            yt[ti] = mfma(ao, bv, yt[ti]);
          }
        }
        for (int ti = 0; ti < 4; ++ti)
          if (ti == w) {
            xt[ti] = keep_query_after_key(xt[ti], l16, grp);
            yt[ti] = keep_query_after_key(yt[ti], l16, grp);
          }
        // operand packs for token steps p = 0 (t-tiles 0, 1) and p = 1 (t-tiles 2, 3)
        for (int p = 0; p < 2; ++p) {
          if (2 * p + 1 < w) continue;  // both t-tiles before the key tile: all zero, never read
          const floatx4 xlo = (2 * p >= w) ? xt[2 * p] : z4, ylo = (2 * p >= w) ? yt[2 * p] : z4;
          sm.xb[0][4 * p + w][lane] = pack_tiles(xlo, xt[2 * p + 1]);
          sm.xb[1][4 * p + w][lane] = pack_tiles(ylo, yt[2 * p + 1]);
        }
      }
      __syncthreads();  // every wave's score packs are in LDS

      // intra: dV^T[n][s] += sum_t dO[t][n] X^T[t][s];  dK^T[i][s] += sum_t Q[t][i] Y^T[t][s]
      // and the state update R[i][n] += sum_t Q[t][i] dO[t][n]
      for (int p = 0; p < 2; ++p) {
        bf16x8 ao[2], aq[2];
        for (int j = 0; j < 2; ++j) {
          ao[j] = tr_operand(sm.o, p, 32 * w + 16 * j, l16, grp);
          aq[j] = tr_operand(sm.q, p, 32 * w + 16 * j, l16, grp);
        }
        for (int si = 0; si < 4; ++si) {
          if (p == 0 && si >= 2) continue;  // tokens 0..31 are all before key tiles 2, 3
          const bf16x8 bx = sm.xb[0][4 * p + si][lane];
          const bf16x8 by = sm.xb[1][4 * p + si][lane];
          for (int j = 0; j < 2; ++j) {
            adv[j][si] = mfma(ao[j], bx, adv[j][si]);
            adk[j][si] = mfma(aq[j], by, adk[j][si]);
          }
        }
        for (int it = 0; it < 8; ++it) {
          const bf16x8 qa = tr_operand(sm.q, p, 16 * it, l16, grp);
          racc[0][it] = mfma(qa, ao[0], racc[0][it]);
          racc[1][it] = mfma(qa, ao[1], racc[1][it]);
        }
      }
      __syncthreads();  // Q/dO and the packs may be overwritten
    }

    // dV, dK rows of the block: tile (j, si) holds columns 32w + 16j + 4grp + {0..3} of row 16si + l16
    for (int si = 0; si < 4; ++si) {
      const int64_t s = blk * C + 16 * si + l16;
      if (s < N)
        for (int j = 0; j < 2; ++j) {
          const int64_t off = (int64_t(bg) * N + s) * DV + 32 * w + 16 * j + 4 * grp;
          store_row4<OUT_F32>(dvg, off, adv[j][si]);
          store_row4<OUT_F32>(dk, off, adk[j][si]);
        }
    }
    // bf16 copy of the updated state for the next (earlier) block's inter terms
    for (int jn = 0; jn < 2; ++jn)
      for (int it = 0; it < 8; ++it)
        *reinterpret_cast<bf16x4*>(&sm.rt[(32 * w + 16 * jn + l16) * ROWST + 16 * it + 4 * grp]) =
            to_bf16x4(racc[jn][it]);
  }

  if (ds_in != nullptr && seg == 0) {
    float* so = ds_in + int64_t(bg) * DD;
    for (int jn = 0; jn < 2; ++jn)
      for (int it = 0; it < 8; ++it)
        for (int i = 0; i < 4; ++i) so[(16 * it + 4 * grp + i) * DV + 32 * w + 16 * jn + l16] = racc[jn][it][i];
  }
}

// rstarts[c][j] = ds_out[c] + sum over segments i > j and the G query heads of
// chain c of the pre-pass partials (partial index ((c G + h)(P - 1) + i - 1) R
// + r), in a fixed order.
__global__ __launch_bounds__(256) void scan_rstarts(const float* __restrict__ partial, float* __restrict__ rstarts,
                                                    const float* ds_out, int G, int P, int R) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t c = gid / DD;
  const int e = int(gid % DD);
  float run = ds_out ? ds_out[c * DD + e] : 0.0f;
  for (int j = P - 1; j >= 0; --j) {
    rstarts[(c * P + j) * DD + e] = run;
    if (j >= 1)
      for (int h = 0; h < G; ++h)
        for (int r = 0; r < R; ++r) run += partial[(((c * G + h) * (P - 1) + (j - 1)) * R + r) * DD + e];
  }
}

// out[c][n][i] = in[c][i][n] for 128 x 128 states, through 32 x 32 LDS tiles.
// Workgroup 16c + t moves tile t of state c.
__global__ __launch_bounds__(256) void transpose_states(const float* __restrict__ in, float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int64_t c = blockIdx.x >> 4;
  const int bx = blockIdx.x & 3, by = (blockIdx.x >> 2) & 3;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int j = ty; j < 32; j += 8) tile[j][tx] = in[c * DD + (by * 32 + j) * DV + bx * 32 + tx];
  __syncthreads();
  for (int j = ty; j < 32; j += 8) out[c * DD + (bx * 32 + j) * D + by * 32 + tx] = tile[tx][j];
}

}  // namespace

hipError_t launch_transpose_states(const float* in, float* out, int64_t count, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_states, dim3(unsigned(16 * count)), dim3(256), 0, stream, in, out);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dvg,
                         bool out_f32, const float* ds_out, float* ds_in, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, const BwdPlan& plan, float* workspace_f, hipStream_t stream) {
  float* partial = workspace_f;
  float* rstarts = partial + plan.partial_floats;
  const float* rs = ds_out;  // one segment: it starts from ds_out
  if (plan.P > 1) {
    hipError_t e = launch_state_parts(q, dout, partial, B * Hq, N, plan.nblocks, plan.blocks_per_seg,
                                      plan.blocks_per_part, plan.P, plan.R, 1, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_rstarts, dim3(unsigned(B * Hkv * DD / 256)), dim3(256), 0, stream, partial, rstarts,
                       ds_out, int(Hq / Hkv), plan.P, plan.R);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    rs = rstarts;
  }
  const dim3 grid(unsigned(B * Hkv * plan.P));
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* o16 = static_cast<const uint16_t*>(dout);
  if (out_f32)
    hipLaunchKernelGGL((bwd_kv_kernel<true>), grid, dim3(kThreads), 0, stream, q16, k16, v16, o16, dk, dvg, rs,
                       ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<false>), grid, dim3(kThreads), 0, stream, q16, k16, v16, o16, dk, dvg, rs,
                       ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
  return hipGetLastError();
}

}  // namespace la
