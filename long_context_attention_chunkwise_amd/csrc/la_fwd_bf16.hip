// bf16 matrix-core forward pass of causal chunkwise linear attention (gfx950).
//
// Method: page "如何理解MiniMax股价创历史新高？拆解国产大模型技术底座" (vergex.cn),
// section "Lightning Attention", chunkwise teaching code.  For each 64-token
// block b of a head:
//     inter = Q_b S                 (S = state before the block)
//     intra = tril(Q_b K_b^T) V_b   (diagonal kept)
//     O_b   = inter + intra
//     S    <- S + K_b^T V_b
// Query head h reads KV head h / (Hq / Hkv) (page "MiniMax-01与Lightning
// Attention", section 1.1 table: 128 heads over 32 KV heads), so the state is
// kept once per KV head and shared by the group's query heads.
//
// Design for MI355X:
//  * One workgroup owns one (batch, KV head, query-head subgroup, sequence
//    segment) and walks its segment block by block.  The float32 state lives
//    in VGPRs for the whole walk as 16x16 MFMA accumulator tiles, each wave
//    owning a slice of its columns.
//  * All products run on v_mfma_f32_16x16x32_bf16 with float32 accumulation.
//    Every product is computed transposed (O^T, P^T = K Q^T) so that the
//    accumulator layout of one product is directly the operand layout of the
//    next: the P^T tiles feed V^T P^T without a shuffle, and the state tiles
//    are written once per block, rounded to bf16, into an n-major LDS copy
//    that the Q S product reads with 16-byte loads.
//  * K and V stay row-major in LDS; the token-contracting products (K^T V and
//    V^T P^T) read their operands with the gfx950 LDS transpose load
//    (ds_read_b64_tr_b16), so nothing is transposed in memory.
//  * Q goes straight from HBM into operand registers (each Q row is read by
//    exactly one wave).
//  * Two layouts.  fwd_bf16_main (eight waves, groups of one or two query
//    heads): K, V and the bf16 state are double-buffered in LDS, one barrier
//    per block, wave w owns state columns [16w, 16w+16).  fwd_bf16_g4 (four
//    waves, groups of four query heads, the 128/32-head shape, head size 128
//    or 64; at 64 also one or two query heads per workgroup): one wave per
//    query head, single-buffered LDS, described above the kernel.
//  * The sequence split into segments needs each segment's starting state:
//    a pre-pass (state_parts) sums K_b^T V_b over parts of every segment but
//    the last, and a scan (scan_starts) adds the parts up (s_in first, then
//    parts in order), exact by associativity of the sums.
//  * fwd_noncausal serves the non-causal variant (head size 128 or 64): every
//    output row reads the total state, which the same pre-pass computes.
#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

using namespace mfma16;


constexpr int kMainThreads = 512;
constexpr int kPartThreads = 256;
// Pre-pass workgroups resident per compute unit (registers: two load slots).
constexpr int part_wgs_per_cu(int hd) { return hd == 128 ? 2 : 3; }

// Shifted segment boundaries (plan flag `shifted`): the inner boundaries of
// KV chain c sit seg_shift(c) blocks before the multiples of the segment
// length, an odd number from -15 to 15 over sixteen chains.  All workgroups
// walk their segments in step, so with plain boundaries every chain's q, o,
// k and v streams stand at the same offsets at the same moment, and a
// placement of the caller's buffers in which those offsets collide in the
// memory system slows every workgroup at once (measured at 1M tokens: one
// (q, o) buffer pair 17.9 ms against 16.1-16.8 for others); sixteen phases
// of two blocks each spread the collisions (17.0-17.4 ms for that pair).
__device__ __forceinline__ int64_t seg_shift(int64_t c) { return (c % 16 - 8) * 2 + 1; }

// First block of segment j of chain c (j < P; segment P - 1 ends at nblocks).
__device__ __forceinline__ int64_t seg_first(int64_t j, int64_t blocks_per_seg, int64_t shift) {
  return j == 0 ? 0 : j * blocks_per_seg - shift;
}

struct __align__(16) MainSmem {
  uint16_t k[2][C * ROWKV];
  uint16_t v[2][C * ROWKV];
  uint16_t st[2][DV * ROWST];  // bf16 copy of the state, n-major: st[n][d]
};

// One block's K and V: 64 rows x 256 bytes each; thread tid moves rows
// tid/16 and tid/16 + 32, 16-byte chunk tid%16.
struct KVRegs {
  uint4 k[2], v[2];
};

__device__ __forceinline__ void load_kv(KVRegs& r, const uint16_t* kh, const uint16_t* vh, int64_t blk,
                                        int64_t N, int tid) {
  const int c = tid & 15;
  for (int i = 0; i < 2; ++i) {
    const int64_t t = blk * C + (tid >> 4) + 32 * i;
    if (t < N) {
      r.k[i] = *reinterpret_cast<const uint4*>(kh + t * D + 8 * c);
      r.v[i] = *reinterpret_cast<const uint4*>(vh + t * DV + 8 * c);
    } else {
      r.k[i] = make_uint4(0, 0, 0, 0);
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void store_kv(const KVRegs& r, uint16_t* ks, uint16_t* vs, int tid) {
  const int c = tid & 15;
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 4) + 32 * i;
    *reinterpret_cast<uint4*>(ks + row * ROWKV + 8 * c) = r.k[i];
    *reinterpret_cast<uint4*>(vs + row * ROWKV + 8 * c) = r.v[i];
  }
}

//
// Feature-map variants (FL) as in fwd_bf16_g4: kRelu applies phi = ReLU to
// the Q operands and to K as it enters LDS; kNorm divides output row t by
// phi(q_t) . z_t + eps, with the in-block part of z_t from the float32 score
// tiles the wave already holds for its rows and the earlier part from z (d
// floats, double-buffered in LDS like the state copy; wave w accumulates
// entries [16w, 16w+16) as K^T times a ones operand).
template <int GW, bool OUT_F32, int FL>
__global__ __launch_bounds__(kMainThreads, 1) void fwd_bf16_main(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ o, const float* starts, const float* s_in, float* s_out, int Hq, int Hkv, int subgroups,
    int64_t N, int64_t nblocks, int64_t blocks_per_seg, int P, const float* zstarts, const float* z_in,
    float* z_out, float eps) {
  constexpr bool kN = (FL & kNorm) != 0;
  constexpr bool kR = (FL & kRelu) != 0;
  __shared__ MainSmem sm;
  __shared__ __align__(16) float zs[2][kN ? D : 4];

  constexpr int WPH = 8 / GW;  // waves per query head
  constexpr int NT = 2 * GW;   // 16-column output tiles per wave

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int chain = blockIdx.x / P;
  const int sub = chain % subgroups;
  const int bg = chain / subgroups;  // b * Hkv + g
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;

  // Wave role: query head hw of the subgroup, row tiles {ta, tb} of every
  // block (the pairing {0,3} / {1,2} balances the causal work), output
  // columns [16*nt0, 16*(nt0+NT)).
  const int hw = w / WPH, sw = w % WPH;
  const int ta = sw & 1, tb = 3 - (sw & 1);
  const int nt0 = (sw >> 1) * NT;

  const int64_t head = int64_t(b) * Hq + int64_t(g) * G + int64_t(sub) * GW + hw;
  const uint16_t* qh = q + head * N * D;
  const uint16_t* kh = k + int64_t(bg) * N * D;
  const uint16_t* vh = v + int64_t(bg) * N * DV;

  // Starting state of the segment (float32), wave w's column tile.
  const float* s0 = starts ? starts + (int64_t(bg) * P + seg) * (D * DV)
                           : (s_in ? s_in + int64_t(bg) * (D * DV) : nullptr);
  floatx4 sacc[8];
  for (int dt = 0; dt < 8; ++dt)
    for (int i = 0; i < 4; ++i)
      sacc[dt][i] = s0 ? s0[(16 * dt + 4 * grp + i) * DV + 16 * w + l16] : 0.0f;

  // normaliser sums, entries 16w + 4grp + i (every column equal)
  floatx4 zacc = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kN) {
    const float* z0 = zstarts ? zstarts + (int64_t(bg) * P + seg) * D : (z_in ? z_in + int64_t(bg) * D : nullptr);
    if (z0 != nullptr)
      for (int i = 0; i < 4; ++i) zacc[i] = z0[16 * w + 4 * grp + i];
    if (l16 == 0) *reinterpret_cast<floatx4*>(&zs[0][16 * w + 4 * grp]) = zacc;
  }

  if (blk0 < blk1) {
    KVRegs kv;
    load_kv(kv, kh, vh, blk0, N, tid);
    if constexpr (kR)
      for (int i = 0; i < 2; ++i) kv.k[i] = relu_bf16x8(kv.k[i]);
    store_kv(kv, sm.k[0], sm.v[0], tid);
  }
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<bf16x4*>(&sm.st[0][(16 * w + l16) * ROWST + 16 * dt + 4 * grp]) = to_bf16x4(sacc[dt]);

  bf16x8 qa[2][4], qn[2][4];
  auto load_q = [&](bf16x8 (&dst)[2][4], int64_t blk) {
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t t = blk * C + 16 * (tt ? tb : ta) + l16;
      for (int ds = 0; ds < 4; ++ds)
        dst[tt][ds] = (t < N) ? ld_global16(qh + t * D + 32 * ds + 8 * grp) : zero_bf16x8();
    }
  };
  if (blk0 < blk1) load_q(qa, blk0);
  __syncthreads();

  // qa holds this block's Q operands; the next block's Q is loaded into qn at
  // the start, so it has a whole block to arrive.
  for (int64_t blk = blk0; blk < blk1; ++blk) {
    const int cur = int(blk - blk0) & 1;
    const bool has_next = blk + 1 < blk1;
    const uint16_t* ks = sm.k[cur];
    const uint16_t* vs = sm.v[cur];
    const uint16_t* st = sm.st[cur];
    if constexpr (kR)
      for (int tt = 0; tt < 2; ++tt)
        for (int ds = 0; ds < 4; ++ds) qa[tt][ds] = relu_bf16x8(qa[tt][ds]);

    KVRegs kvn;
    if (has_next) {
      load_q(qn, blk + 1);
      load_kv(kvn, kh, vh, blk + 1, N, tid);
    }

    // inter: O^T[n][t] = sum_d S[d][n] Q[t][d]  (state before this block)
    floatx4 acc[2][NT];
    for (int tt = 0; tt < 2; ++tt)
      for (int j = 0; j < NT; ++j) acc[tt][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int ds = 0; ds < 4; ++ds) {
      for (int j = 0; j < NT; ++j) {
        const bf16x8 sa = ld_lds16(st + (16 * (nt0 + j) + l16) * ROWST + 32 * ds + 8 * grp);
        acc[0][j] = mfma(sa, qa[0][ds], acc[0][j]);
        acc[1][j] = mfma(sa, qa[1][ds], acc[1][j]);
      }
    }

    // scores: P^T[s][t] = sum_d K[s][d] Q[t][d] for s-tiles up to each t-tile
    floatx4 pa[2], pb[4];
    for (int i = 0; i < 2; ++i) pa[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < 4; ++i) pb[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int ds = 0; ds < 4; ++ds) {
      for (int si = 0; si < 4; ++si) {
        if (si > tb) continue;
        const bf16x8 ka = ld_lds16(ks + (16 * si + l16) * ROWKV + 32 * ds + 8 * grp);
        if (si <= ta) pa[si] = mfma(ka, qa[0][ds], pa[si]);
        pb[si] = mfma(ka, qa[1][ds], pb[si]);
      }
    }

    // causal mask on the diagonal tiles, then bf16 operands for V^T P^T
    if (ta == 0) pa[0] = causal_mask(pa[0], l16, grp);
    else pa[1] = causal_mask(pa[1], l16, grp);
    if (tb == 2) pb[2] = causal_mask(pb[2], l16, grp);
    else pb[3] = causal_mask(pb[3], l16, grp);
    float inv[2];  // normaliser of rows 16ta + l16 and 16tb + l16 (kNorm only)
    (void)inv;
    if constexpr (kN) {
      // this lane's share of sum_s P^T[s][t] over s <= t, plus phi(q_t) . z
      // over this lane's 32 entries of q_t; the four lane groups then add up
      float den[2];
      den[0] = (pa[0][0] + pa[0][1]) + (pa[0][2] + pa[0][3]);
      if (ta == 1) den[0] += (pa[1][0] + pa[1][1]) + (pa[1][2] + pa[1][3]);
      den[1] = 0.0f;
      for (int si = 0; si < 4; ++si)
        if (si <= tb) den[1] += (pb[si][0] + pb[si][1]) + (pb[si][2] + pb[si][3]);
      const float* zc = zs[cur];
      for (int ds = 0; ds < 4; ++ds) {
        const floatx4 za = *reinterpret_cast<const floatx4*>(&zc[32 * ds + 8 * grp]);
        const floatx4 zb = *reinterpret_cast<const floatx4*>(&zc[32 * ds + 8 * grp + 4]);
        for (int tt = 0; tt < 2; ++tt) {
          float dsum = 0.0f;
          for (int j = 0; j < 4; ++j)
            dsum += float(qa[tt][ds][j]) * za[j] + float(qa[tt][ds][j + 4]) * zb[j];
          den[tt] += dsum;
        }
      }
      for (int tt = 0; tt < 2; ++tt) {
        float x = den[tt];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        inv[tt] = 1.0f / (x + eps);
      }
    }
    const floatx4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const bf16x8 pA0 = pack_tiles(pa[0], ta == 1 ? pa[1] : zero4);
    const bf16x8 pB0 = pack_tiles(pb[0], pb[1]);
    const bf16x8 pB1 = pack_tiles(pb[2], tb == 3 ? pb[3] : zero4);

    // intra: O^T[n][t] += sum_s V[s][n] P^T[s][t]
    for (int j = 0; j < NT; ++j) {
      const bf16x8 va0 = tr_operand(vs, 0, 16 * (nt0 + j), l16, grp);
      const bf16x8 va1 = tr_operand(vs, 1, 16 * (nt0 + j), l16, grp);
      acc[0][j] = mfma(va0, pA0, acc[0][j]);
      acc[1][j] = mfma(va0, pB0, acc[1][j]);
      acc[1][j] = mfma(va1, pB1, acc[1][j]);
    }

    if constexpr (kN)
      for (int tt = 0; tt < 2; ++tt)
        for (int j = 0; j < NT; ++j)
          for (int i = 0; i < 4; ++i) acc[tt][j][i] *= inv[tt];

    // store O rows (each lane: 4 consecutive columns of one row per tile)
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t t = blk * C + 16 * (tt ? tb : ta) + l16;
      if (t < N) {
        for (int j = 0; j < NT; ++j) {
          const int64_t off = (head * N + t) * DV + 16 * (nt0 + j) + 4 * grp;
          if (OUT_F32)
            *reinterpret_cast<floatx4*>(static_cast<float*>(o) + off) = acc[tt][j];
          else
            *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(o) + off) = to_bf16x4(acc[tt][j]);
        }
      }
    }

    // state update: S[:, 16w:16w+16] += K_b^T V_b, then its bf16 copy
    {
      const bf16x8 vb0 = tr_operand(vs, 0, 16 * w, l16, grp);
      const bf16x8 vb1 = tr_operand(vs, 1, 16 * w, l16, grp);
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 k0 = tr_operand(ks, 0, 16 * dt, l16, grp);
        const bf16x8 k1 = tr_operand(ks, 1, 16 * dt, l16, grp);
        sacc[dt] = mfma(k0, vb0, sacc[dt]);
        sacc[dt] = mfma(k1, vb1, sacc[dt]);
      }
      uint16_t* stn = sm.st[cur ^ 1];
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<bf16x4*>(&stn[(16 * w + l16) * ROWST + 16 * dt + 4 * grp]) = to_bf16x4(sacc[dt]);
      if constexpr (kN) {
        for (int p = 0; p < 2; ++p) zacc = mfma(tr_operand(ks, p, 16 * w, l16, grp), ones_bf16x8(), zacc);
        if (l16 == 0) *reinterpret_cast<floatx4*>(&zs[cur ^ 1][16 * w + 4 * grp]) = zacc;
      }
    }
    if (has_next) {
      if constexpr (kR)
        for (int i = 0; i < 2; ++i) kvn.k[i] = relu_bf16x8(kvn.k[i]);
      store_kv(kvn, sm.k[cur ^ 1], sm.v[cur ^ 1], tid);
      for (int tt = 0; tt < 2; ++tt)
        for (int ds = 0; ds < 4; ++ds) qa[tt][ds] = qn[tt][ds];
    }
    __syncthreads();
  }

  if (s_out != nullptr && seg == P - 1 && sub == 0) {
    float* so = s_out + int64_t(bg) * (D * DV);
    for (int dt = 0; dt < 8; ++dt)
      for (int i = 0; i < 4; ++i) so[(16 * dt + 4 * grp + i) * DV + 16 * w + l16] = sacc[dt][i];
  }
  if constexpr (kN)
    if (z_out != nullptr && seg == P - 1 && sub == 0 && l16 == 0)
      for (int i = 0; i < 4; ++i) z_out[int64_t(bg) * D + 16 * w + 4 * grp + i] = zacc[i];
}

// K and V tiles of a head size HD (d = dv = HD): 256 threads move the 64
// rows of HD bf16 values in 16-byte chunks, HD / 8 chunks per row; thread tid
// takes chunk tid % (HD / 8) of rows tid / (HD / 8) + (2048 / HD) i.
template <int HD>
struct KVTile {
  uint4 k[HD / 32], v[HD / 32];
};

template <int HD>
__device__ __forceinline__ void load_kv_tile(KVTile<HD>& r, const uint16_t* kh, const uint16_t* vh, int64_t blk,
                                             int64_t N, int tid) {
  constexpr int CPR = HD / 8, RPP = 256 / CPR;
  const int c = tid % CPR;
  for (int i = 0; i < HD / 32; ++i) {
    const int64_t t = blk * C + tid / CPR + RPP * i;
    if (t < N) {
      r.k[i] = ld_stream16(kh + t * HD + 8 * c);
      r.v[i] = ld_stream16(vh + t * HD + 8 * c);
    } else {
      r.k[i] = make_uint4(0, 0, 0, 0);
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int HD>
__device__ __forceinline__ void store_kv_tile(const KVTile<HD>& r, uint16_t* ks, uint16_t* vs, int tid) {
  constexpr int CPR = HD / 8, RPP = 256 / CPR, PITCH = HD + 16;
  const int c = tid % CPR;
  for (int i = 0; i < HD / 32; ++i) {
    const int row = tid / CPR + RPP * i;
    *reinterpret_cast<uint4*>(ks + row * PITCH + 8 * c) = r.k[i];
    *reinterpret_cast<uint4*>(vs + row * PITCH + 8 * c) = r.v[i];
  }
}

// ---------------------------------------------------------------------------
// Four-wave kernel for groups of four query heads (the 128/32-head shape;
// head size d = dv = HD, 128 or 64).  One wave per SIMD: wave h computes every
// row of the block for query head h of the group (each wave reads the bf16
// state once per block: half the LDS traffic of the eight-wave layout) and
// owns state columns [h HD/4, (h+1) HD/4).
//
// Output columns are processed in quarters of 32 as two interleaved 16-column
// tiles (columns 32m + 8j + {0..3} and 32m + 8j + {4..7}, j = 0..3), so each
// lane holds 8 consecutive columns of one row and stores 16 bytes, and only
// 32 accumulator registers are live at a time.
//
// LDS tiles are single-buffered (70 KiB).  The next block's Q and K/V loads
// are issued once the current block's Q operands are dead (after the output
// products), so they overlap the state update and the barriers without
// competing with the matrix-heavy phase.  Three barriers per block: K/V and
// the state are published, the inter term has finished reading the state,
// and the state update has finished reading K/V.
// ---------------------------------------------------------------------------
//
// Feature-map variants (FL): kRelu applies phi = ReLU to the Q operands and
// to K as it enters LDS.  kNorm divides each output row t by
// phi(q_t) . z_t + eps, where z_t = z at the segment start + sum of phi(k_s)
// over s <= t: the in-block part is the column sum of the float32 P^T tiles,
// the earlier part phi(q_t) . z with z (float32, d entries) kept like the
// state: wave w accumulates entries [32w, 32w+32) on the matrix cores (K^T
// times a ones operand) and publishes them in LDS once per block.
//
// PARTIAL (head size 64, groups of one or two query heads, or any group size
// not a multiple of four): a workgroup serves gw < 4 query heads.  Waves w >=
// gw have no head: they skip the Q loads, scores and outputs (a wave-uniform
// branch) but keep their share of the state update and its barriers.
//
// o may be q itself (in-place output): q and o are therefore not restrict.
// Each query row is loaded into the wave's operand registers before that
// wave writes the same output row, and never read again.
//
// RS (the backward's dQ pass, which runs this kernel over queries dO, keys V
// and values K): the workgroup also sums R = sum_t x_t^T q_t over its segment
// and the group's query heads, x being a second [head][N][HD] input (the
// forward's queries), and writes R to rpart (float32, HD x HD, entry [i][j] =
// sum x[t][i] q[t][j]) at index chain (P - 1) + seg - 1; segment 0 skips it.
// The reverse recurrence starts each segment from the sum of these over the
// later segments, so the backward reads dO once for dQ and R together.  Wave h
// writes head h's x and q rows to LDS, half a block at a time, and wave w sums
// columns [w HD/4, (w+1) HD/4) of R over all four heads with the same
// transpose-load products as the state update.  One more barrier per block:
// the two halves take two write/read rounds of the staging tiles.
template <bool OUT_F32, int FL, int HD = 128, bool PARTIAL = false, bool RS = false>
__global__ __launch_bounds__(256, 1) void fwd_bf16_g4(
    const uint16_t* q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* o, const float* starts, const float* s_in, float* s_out, int Hq, int Hkv, int subgroups,
    int64_t N, int64_t nblocks, int64_t blocks_per_seg, int P, const float* zstarts, const float* z_in,
    float* z_out, float eps, int gw, const uint16_t* __restrict__ qx, float* __restrict__ rpart, int shifted) {
  constexpr bool kN = (FL & kNorm) != 0;
  constexpr bool kR = (FL & kRelu) != 0;
  static_assert(!RS || (FL == 0 && !PARTIAL), "R sums: plain forward over four query heads");
  // Head size HD = d = dv (64 or 128): 32-wide chunks of d, 16-row tiles of
  // the state, 32-column output quarters, state columns per wave and their
  // 16-column tiles; LDS pitches as for 128 (16 and 8 elements of padding).
  static_assert(HD == 64 || HD == 128, "head sizes 64 and 128");
  constexpr int NDS = HD / 32, NDT = HD / 16, NM = HD / 32, WC = HD / 4, NJ = WC / 16;
  constexpr int RKV = HD + 16, RST = HD + 8;
  __shared__ __align__(16) uint16_t ks[C * RKV];
  __shared__ __align__(16) uint16_t vs[C * RKV];
  __shared__ __align__(16) uint16_t st[HD * RST];
  __shared__ __align__(16) float zs[kN ? HD : 4];
  // RS staging: tile 2h holds x rows, tile 2h + 1 q rows of head h (32 rows)
  __shared__ __align__(16) uint16_t xs[RS ? 8 * 32 * RKV : 8];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int chain = blockIdx.x / P;
  const int sub = chain % subgroups;
  const int bg = chain / subgroups;  // b * Hkv + g
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t shift = shifted ? seg_shift(bg) : 0;
  const int64_t blk0 = seg_first(seg, blocks_per_seg, shift);
  const int64_t blk_end = seg == P - 1 ? nblocks : seg_first(seg + 1, blocks_per_seg, shift);
  const int64_t blk1 = blk_end < nblocks ? blk_end : nblocks;
  const bool rs_on = RS && seg > 0;

  // query heads of this workgroup: 4, or gw when PARTIAL (waves w >= gw idle)
  const int gsz = PARTIAL ? gw : 4;
  const bool act = !PARTIAL || __builtin_amdgcn_readfirstlane(w) < gsz;
  const int64_t head = int64_t(b) * Hq + int64_t(g) * G + int64_t(sub) * gsz + (act ? w : 0);
  const uint16_t* qh = q + head * N * HD;
  const uint16_t* xh = RS ? qx + head * N * HD : nullptr;
  const uint16_t* kh = k + int64_t(bg) * N * HD;
  const uint16_t* vh = v + int64_t(bg) * N * HD;
  const int nlane = 8 * (l16 >> 2) + (l16 & 3);

  const float* s0 = starts ? starts + (int64_t(bg) * P + seg) * (HD * HD)
                           : (s_in ? s_in + int64_t(bg) * (HD * HD) : nullptr);
  floatx4 sacc[NJ][NDT];
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt)
      for (int i = 0; i < 4; ++i)
        sacc[jn][dt][i] = s0 ? s0[(16 * dt + 4 * grp + i) * HD + WC * w + 16 * jn + l16] : 0.0f;
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<bf16x4*>(&st[(WC * w + 16 * jn + l16) * RST + 16 * dt + 4 * grp]) =
          to_bf16x4(sacc[jn][dt]);

  // normaliser sums, entries WC w + 16jj + 4grp + i (every column equal)
  floatx4 zacc[NJ];
  for (int jj = 0; jj < NJ; ++jj) zacc[jj] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kN) {
    const float* z0 = zstarts ? zstarts + (int64_t(bg) * P + seg) * HD : (z_in ? z_in + int64_t(bg) * HD : nullptr);
    if (z0 != nullptr)
      for (int jj = 0; jj < NJ; ++jj)
        for (int i = 0; i < 4; ++i) zacc[jj][i] = z0[WC * w + 16 * jj + 4 * grp + i];
    if (l16 == 0)
      for (int jj = 0; jj < NJ; ++jj)
        *reinterpret_cast<floatx4*>(&zs[WC * w + 16 * jj + 4 * grp]) = zacc[jj];
  }

  bf16x8 qa[4][NDS];
  bf16x8 xa[4][NDS];        // RS: x rows, in qa's layout
  floatx4 racc[NJ][NDT];    // RS: R[16dt + 4grp + i][WC w + 16jn + l16]
  if constexpr (RS)
    for (int jn = 0; jn < NJ; ++jn)
      for (int dt = 0; dt < NDT; ++dt) racc[jn][dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  KVTile<HD> kv;
  auto load_q = [&](int64_t blk) {
    if (act) {
      for (int ti = 0; ti < 4; ++ti) {
        const int64_t t = blk * C + 16 * ti + l16;
        for (int ds = 0; ds < NDS; ++ds)
          qa[ti][ds] = (t < N) ? ld_global16(qh + t * HD + 32 * ds + 8 * grp) : zero_bf16x8();
      }
    } else {
      for (int ti = 0; ti < 4; ++ti)
        for (int ds = 0; ds < NDS; ++ds) qa[ti][ds] = zero_bf16x8();
    }
  };
  // RS: x rows 32 half .. 32 half + 31 of block blk
  auto load_x_half = [&](int64_t blk, int half) {
    for (int tj = 0; tj < 2; ++tj) {
      const int ti = 2 * half + tj;
      const int64_t t = blk * C + 16 * ti + l16;
      for (int ds = 0; ds < NDS; ++ds)
        xa[ti][ds] = (t < N) ? ld_global16(xh + t * HD + 32 * ds + 8 * grp) : zero_bf16x8();
    }
  };
  // RS: wave w stages rows 32 half .. 32 half + 31 of its head's x and q.
  auto stage_half = [&](int half) {
    uint16_t* xt = xs + (2 * w) * (32 * RKV);
    uint16_t* qt = xt + 32 * RKV;
    for (int tj = 0; tj < 2; ++tj)
      for (int ds = 0; ds < NDS; ++ds) {
        const int off = (16 * tj + l16) * RKV + 32 * ds + 8 * grp;
        *reinterpret_cast<bf16x8*>(xt + off) = xa[2 * half + tj][ds];
        *reinterpret_cast<bf16x8*>(qt + off) = qa[2 * half + tj][ds];
      }
  };
  // RS: R[:, WC w : WC w + WC] += sum over the four heads of the staged
  // x^T q (32 tokens: one token-contracting step).
  auto r_sum_half = [&]() {
    for (int h = 0; h < 4; ++h) {
      const uint16_t* xt = xs + (2 * h) * (32 * RKV);
      const uint16_t* qt = xt + 32 * RKV;
      bf16x8 qb[NJ];
      for (int jn = 0; jn < NJ; ++jn) qb[jn] = tr_operand(qt, 0, WC * w + 16 * jn, l16, grp, 4, RKV);
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 xt_op = tr_operand(xt, 0, 16 * dt, l16, grp, 4, RKV);
        for (int jn = 0; jn < NJ; ++jn) racc[jn][dt] = mfma(xt_op, qb[jn], racc[jn][dt]);
      }
    }
  };
  // The block walk, compiled separately with and without the R sums so that
  // segment 0 (no sums) keeps the plain kernel's registers.
  auto walk = [&](auto ron) {
    constexpr bool RON = decltype(ron)::value;
    if (blk0 < blk1) {
      load_kv_tile<HD>(kv, kh, vh, blk0, N, tid);
      load_q(blk0);
      if constexpr (RON) {
        load_x_half(blk0, 0);
        load_x_half(blk0, 1);
      }
    }
    for (int64_t blk = blk0; blk < blk1; ++blk) {
      if constexpr (kR) {
        for (int i = 0; i < HD / 32; ++i) kv.k[i] = relu_bf16x8(kv.k[i]);
        for (int ti = 0; ti < 4; ++ti)
          for (int ds = 0; ds < NDS; ++ds) qa[ti][ds] = relu_bf16x8(qa[ti][ds]);
      }
      store_kv_tile<HD>(kv, ks, vs, tid);
      if constexpr (RON) {
        // With the R sums, the next block's K/V and first x half go out as
        // soon as their registers are free (measured 0.4 ms faster per 1M-token
        // backward than loading everything after the outputs).
        stage_half(0);
        if (blk + 1 < blk1) {
          load_kv_tile<HD>(kv, kh, vh, blk + 1, N, tid);
          load_x_half(blk + 1, 0);
        }
      }
      __syncthreads();  // K, V and the state of the previous block are in LDS

      // scores, one P^T tile at a time, packed to bf16 operands right away
      const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (act) {
      bf16x8 pop[4][2];
      float inv[4];  // 1 / normaliser of row 16ti + l16 (kNorm only)
      (void)inv;
      for (int ti = 0; ti < 4; ++ti) {
        floatx4 pt[4];
        for (int si = 0; si <= ti; ++si) {
          pt[si] = z4;
          for (int ds = 0; ds < NDS; ++ds)
            pt[si] = mfma(ld_lds16(ks + (16 * si + l16) * RKV + 32 * ds + 8 * grp), qa[ti][ds], pt[si]);
        }
        pt[ti] = causal_mask(pt[ti], l16, grp);
        pop[ti][0] = pack_tiles(pt[0], ti >= 1 ? pt[1] : z4);
        if (ti >= 2) pop[ti][1] = pack_tiles(pt[2], ti == 3 ? pt[3] : z4);
      }
      if constexpr (kN) {
        // Denominators on the matrix cores, as one more 16-column output
        // tile: rows 0-7 of its A operand hold the high bf16 part of z and
        // ones against the bf16 score operands the numerator uses, rows 8-15
        // the low part of z (z = hi + lo to about 16 significant bits), so
        // output row 0 of column t is phi(q_t) . z_hi + sum_s P^T[s][t] and
        // row 8 is phi(q_t) . z_lo; lane (l16, grp) holds rows 4grp.., and
        // lanes l and l ^ 32 hold rows 0 and 8 of column 16ti + l16.
        const bool hi_row = l16 < 8;
        bf16x8 za_op[NDS];
        for (int ds = 0; ds < NDS; ++ds) {
          const floatx4 za = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp]);
          const floatx4 zb = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp + 4]);
          for (int j = 0; j < 4; ++j) {
            const __bf16 ha = (__bf16)za[j], hb = (__bf16)zb[j];
            za_op[ds][j] = hi_row ? ha : (__bf16)(za[j] - float(ha));
            za_op[ds][j + 4] = hi_row ? hb : (__bf16)(zb[j] - float(hb));
          }
        }
        const bf16x8 ones = hi_row ? ones_bf16x8() : zero_bf16x8();
        for (int ti = 0; ti < 4; ++ti) {
          floatx4 dt = mfma(ones, pop[ti][0], z4);
          if (ti >= 2) dt = mfma(ones, pop[ti][1], dt);
          for (int ds = 0; ds < NDS; ++ds) dt = mfma(za_op[ds], qa[ti][ds], dt);
          inv[ti] = 1.0f / ((dt[0] + __shfl_xor(dt[0], 32)) + eps);
        }
      }

      // Output columns in quarters of 32 (one interleaved column pair m), so
      // only 32 accumulator registers are live at a time; bf16 outputs of an
      // even quarter wait packed for the odd one.
      bf16x8 held[4];
      for (int m = 0; m < NM; ++m) {
        floatx4 acc[2][4];
        for (int h2 = 0; h2 < 2; ++h2)
          for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = z4;
        // inter: O^T[n][t] = sum_d S[d][n] Q[t][d] (state before the block)
        for (int ds = 0; ds < NDS; ++ds)
          for (int h2 = 0; h2 < 2; ++h2) {
            const bf16x8 sa = ld_lds16(st + (32 * m + 4 * h2 + nlane) * RST + 32 * ds + 8 * grp);
            for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = mfma(sa, qa[ti][ds], acc[h2][ti]);
          }
        // intra: O^T[n][t] += sum_s V[s][n] P^T[s][t]
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 va0 = tr_operand(vs, 0, 32 * m + 4 * h2, l16, grp, 8, RKV);
          const bf16x8 va1 = tr_operand(vs, 1, 32 * m + 4 * h2, l16, grp, 8, RKV);
          for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = mfma(va0, pop[ti][0], acc[h2][ti]);
          acc[h2][2] = mfma(va1, pop[2][1], acc[h2][2]);
          acc[h2][3] = mfma(va1, pop[3][1], acc[h2][3]);
        }
        if constexpr (kN)
          for (int h2 = 0; h2 < 2; ++h2)
            for (int ti = 0; ti < 4; ++ti)
              for (int i = 0; i < 4; ++i) acc[h2][ti][i] *= inv[ti];
        if constexpr (OUT_F32 || RS) {
          // (the dQ pass with the R sums: whole-line stores measured 0.9 ms
          // slower per 1M-token backward there, so it stores each quarter)
          for (int ti = 0; ti < 4; ++ti) {
            const int64_t t = blk * C + 16 * ti + l16;
            if (t < N) {
              const int64_t off = (head * N + t) * HD + 32 * m + 8 * grp;
              if constexpr (OUT_F32) {
                float* op = static_cast<float*>(o) + off;
                *reinterpret_cast<floatx4*>(op) = acc[0][ti];
                *reinterpret_cast<floatx4*>(op + 4) = acc[1][ti];
              } else {
                *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(o) + off) = pack_tiles(acc[0][ti], acc[1][ti]);
              }
            }
          }
        } else if ((m & 1) == 0) {
          for (int ti = 0; ti < 4; ++ti) held[ti] = pack_tiles(acc[0][ti], acc[1][ti]);
        } else {
          // quarters m - 1 and m make one 128-byte line of every row: whole
          // lines per store (measured 2-3.5% faster at 1M tokens than storing
          // each quarter's half lines, and no partial-line write-backs)
          uint16_t* line = static_cast<uint16_t*>(o) + head * N * HD + 64 * (m >> 1);
          for (int ti = 0; ti < 4; ++ti)
            store_lines(line, HD, blk * C + 16 * ti, N, held[ti], pack_tiles(acc[0][ti], acc[1][ti]), l16, grp);
        }
      }
      }  // act
      if constexpr (!RON) {
        // The next block's loads go out now (Q operands are no longer needed),
        // so they overlap the state update and the barriers.
        if (blk + 1 < blk1) {
          load_kv_tile<HD>(kv, kh, vh, blk + 1, N, tid);
          load_q(blk + 1);
        }
        __syncthreads();  // every wave has finished reading the state
      } else {
        r_sum_half();
        __syncthreads();  // the state and the first staged half are read
        stage_half(1);
        if (blk + 1 < blk1) {
          load_q(blk + 1);
          load_x_half(blk + 1, 1);
        }
      }

      // state update: S[:, WC w:WC w+WC] += K_b^T V_b, then its bf16 copy
      {
        bf16x8 vb[NJ][2];
        for (int jn = 0; jn < NJ; ++jn)
          for (int p = 0; p < 2; ++p) vb[jn][p] = tr_operand(vs, p, WC * w + 16 * jn, l16, grp, 4, RKV);
        for (int dt = 0; dt < NDT; ++dt)
          for (int p = 0; p < 2; ++p) {
            const bf16x8 kt = tr_operand(ks, p, 16 * dt, l16, grp, 4, RKV);
            for (int jn = 0; jn < NJ; ++jn) sacc[jn][dt] = mfma(kt, vb[jn][p], sacc[jn][dt]);
          }
        for (int jn = 0; jn < NJ; ++jn)
          for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<bf16x4*>(&st[(WC * w + 16 * jn + l16) * RST + 16 * dt + 4 * grp]) =
                to_bf16x4(sacc[jn][dt]);
        if constexpr (kN) {
          for (int p = 0; p < 2; ++p)
            for (int jj = 0; jj < NJ; ++jj)
              zacc[jj] = mfma(tr_operand(ks, p, WC * w + 16 * jj, l16, grp, 4, RKV), ones_bf16x8(), zacc[jj]);
          if (l16 == 0)
            for (int jj = 0; jj < NJ; ++jj)
              *reinterpret_cast<floatx4*>(&zs[WC * w + 16 * jj + 4 * grp]) = zacc[jj];
        }
      }
      __syncthreads();  // K and V are free for the next block
      if constexpr (RON) {
        r_sum_half();
        __syncthreads();  // the staging tiles are free for the next block
      }
    }
  };
  if constexpr (RS) {
    if (rs_on) walk(std::integral_constant<bool, true>{});
    else walk(std::integral_constant<bool, false>{});
  } else {
    walk(std::integral_constant<bool, false>{});
  }

  if constexpr (RS)
    if (rs_on) {
      float* rp = rpart + (int64_t(chain) * (P - 1) + seg - 1) * (HD * HD);
      for (int jn = 0; jn < NJ; ++jn)
        for (int dt = 0; dt < NDT; ++dt)
          for (int i = 0; i < 4; ++i) rp[(16 * dt + 4 * grp + i) * HD + WC * w + 16 * jn + l16] = racc[jn][dt][i];
    }

  if (s_out != nullptr && seg == P - 1 && sub == 0) {
    float* so = s_out + int64_t(bg) * (HD * HD);
    for (int jn = 0; jn < NJ; ++jn)
      for (int dt = 0; dt < NDT; ++dt)
        for (int i = 0; i < 4; ++i) so[(16 * dt + 4 * grp + i) * HD + WC * w + 16 * jn + l16] = sacc[jn][dt][i];
  }
  if constexpr (kN)
    if (z_out != nullptr && seg == P - 1 && sub == 0 && l16 == 0)
      for (int jj = 0; jj < NJ; ++jj)
        for (int i = 0; i < 4; ++i) z_out[int64_t(bg) * HD + WC * w + 16 * jj + 4 * grp + i] = zacc[jj][i];
}

// ---------------------------------------------------------------------------
// One-wave workgroups for one query head per KV head at head size 64 (d = dv
// = 64, Hq = Hkv).  With a single query head, the four-wave kernel keeps three
// waves idle; here each wave is a workgroup of its own that owns one (batch,
// head, segment): the head's whole 64 x 64 float32 state in VGPRs (16
// accumulator tiles), its own K/V tiles and bf16 state copy in LDS (30 KiB),
// so no wave ever waits for another, and four of them share a compute unit
// (the host plans four segments per unit: 32 per chain for 32 heads).  The
// block step is the four-wave kernel's with the wave owning every state
// column: scores P^T = K Q^T, outputs O^T = S^T Q^T + V^T P^T in two 32-column
// quarters, then S += K^T V and its bf16 copy.
//
// Flags (causal feature-map variants), as in the four-wave kernel: kRelu
// applies phi = ReLU to q and to k before it enters LDS; kNorm divides each
// output row by phi(q_t) . z + eps, z (64 floats) running beside the state:
// kept in float32 accumulator tiles (K^T times a ones operand), published in
// LDS once per block, and read back in operand layout for the denominators.
// ---------------------------------------------------------------------------
template <bool OUT_F32, int FL = 0>
__global__ __launch_bounds__(64, 1) void fwd_bf16_solo(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, void* __restrict__ o,
                                                       const float* starts, const float* s_in, float* s_out,
                                                       int64_t N, int64_t nblocks, int64_t blocks_per_seg, int P,
                                                       const float* zstarts, const float* z_in, float* z_out,
                                                       float eps) {
  constexpr bool kN = (FL & kNorm) != 0;
  constexpr bool kR = (FL & kRelu) != 0;
  constexpr int HD = 64, NDS = HD / 32, NDT = HD / 16, NM = HD / 32, NJ = HD / 16;
  constexpr int RKV = HD + 16, RST = HD + 8, CPR = HD / 8, RPI = 64 / CPR, NLD = C / RPI;
  __shared__ __align__(16) uint16_t ks[C * RKV];
  __shared__ __align__(16) uint16_t vs[C * RKV];
  __shared__ __align__(16) uint16_t st[HD * RST];
  __shared__ __align__(16) float zs[kN ? HD : 4];

  const int lane = threadIdx.x, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int64_t bh = blockIdx.x / P;  // b * H + h: query head h reads KV head h
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;
  const uint16_t* qh = q + bh * N * HD;
  const uint16_t* kh = k + bh * N * HD;
  const uint16_t* vh = v + bh * N * HD;
  const int nlane = 8 * (l16 >> 2) + (l16 & 3);

  // state tile (jn, dt): rows 16 dt + 4 grp + i, column 16 jn + l16
  const float* s0 = starts ? starts + (bh * P + seg) * (HD * HD) : (s_in ? s_in + bh * (HD * HD) : nullptr);
  floatx4 sacc[NJ][NDT];
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt)
      for (int i = 0; i < 4; ++i) sacc[jn][dt][i] = s0 ? s0[(16 * dt + 4 * grp + i) * HD + 16 * jn + l16] : 0.0f;
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<bf16x4*>(&st[(16 * jn + l16) * RST + 16 * dt + 4 * grp]) = to_bf16x4(sacc[jn][dt]);

  // normaliser sums, entries 16jj + 4grp + i (every column equal)
  floatx4 zacc[NJ];
  for (int jj = 0; jj < NJ; ++jj) zacc[jj] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kN) {
    const float* z0 = zstarts ? zstarts + (bh * P + seg) * HD : (z_in ? z_in + bh * HD : nullptr);
    if (z0 != nullptr)
      for (int jj = 0; jj < NJ; ++jj)
        for (int i = 0; i < 4; ++i) zacc[jj][i] = z0[16 * jj + 4 * grp + i];
    if (l16 == 0)
      for (int jj = 0; jj < NJ; ++jj) *reinterpret_cast<floatx4*>(&zs[16 * jj + 4 * grp]) = zacc[jj];
  }

  // one block's K and V: lane moves chunk lane % CPR of rows lane / CPR + RPI i
  uint4 kr[NLD], vr[NLD];
  bf16x8 qa[4][NDS];
  auto load_block = [&](int64_t blk) {
    const int c = lane % CPR;
    for (int i = 0; i < NLD; ++i) {
      const int64_t t = blk * C + lane / CPR + RPI * i;
      if (t < N) {
        kr[i] = ld_stream16(kh + t * HD + 8 * c);
        vr[i] = ld_stream16(vh + t * HD + 8 * c);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
    for (int ti = 0; ti < 4; ++ti) {
      const int64_t t = blk * C + 16 * ti + l16;
      for (int ds = 0; ds < NDS; ++ds)
        qa[ti][ds] = (t < N) ? ld_global16(qh + t * HD + 32 * ds + 8 * grp) : zero_bf16x8();
    }
  };
  if (blk0 < blk1) load_block(blk0);
  for (int64_t blk = blk0; blk < blk1; ++blk) {
    if constexpr (kR) {
      for (int i = 0; i < NLD; ++i) kr[i] = relu_bf16x8(kr[i]);
      for (int ti = 0; ti < 4; ++ti)
        for (int ds = 0; ds < NDS; ++ds) qa[ti][ds] = relu_bf16x8(qa[ti][ds]);
    }
    {
      const int c = lane % CPR;
      for (int i = 0; i < NLD; ++i) {
        const int row = lane / CPR + RPI * i;
        *reinterpret_cast<uint4*>(ks + row * RKV + 8 * c) = kr[i];
        *reinterpret_cast<uint4*>(vs + row * RKV + 8 * c) = vr[i];
      }
    }
    __syncthreads();  // (one wave: orders the tile stores before the reads below)

    const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 pop[4][2];
    for (int ti = 0; ti < 4; ++ti) {
      floatx4 pt[4];
      for (int si = 0; si <= ti; ++si) {
        pt[si] = z4;
        for (int ds = 0; ds < NDS; ++ds)
          pt[si] = mfma(ld_lds16(ks + (16 * si + l16) * RKV + 32 * ds + 8 * grp), qa[ti][ds], pt[si]);
      }
      pt[ti] = causal_mask(pt[ti], l16, grp);
      pop[ti][0] = pack_tiles(pt[0], ti >= 1 ? pt[1] : z4);
      if (ti >= 2) pop[ti][1] = pack_tiles(pt[2], ti == 3 ? pt[3] : z4);
    }
    float inv[4];  // 1 / normaliser of row 16ti + l16 (kNorm only)
    (void)inv;
    if constexpr (kN) {
      // denominators as one more MFMA output tile, formed as in the
      // four-wave kernel: rows 0-7 of the A operand hold z's high bf16 part
      // and ones, rows 8-15 its low part; lanes l and l ^ 32 add up
      const bool hi_row = l16 < 8;
      const bf16x8 ones = hi_row ? ones_bf16x8() : zero_bf16x8();
      floatx4 dt[4];
      for (int ti = 0; ti < 4; ++ti) {
        dt[ti] = mfma(ones, pop[ti][0], z4);
        if (ti >= 2) dt[ti] = mfma(ones, pop[ti][1], dt[ti]);
      }
      for (int ds = 0; ds < NDS; ++ds) {
        const floatx4 za = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp]);
        const floatx4 zb = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp + 4]);
        bf16x8 zop;
        for (int j = 0; j < 4; ++j) {
          const __bf16 ha = (__bf16)za[j], hb = (__bf16)zb[j];
          zop[j] = hi_row ? ha : (__bf16)(za[j] - float(ha));
          zop[j + 4] = hi_row ? hb : (__bf16)(zb[j] - float(hb));
        }
        for (int ti = 0; ti < 4; ++ti) dt[ti] = mfma(zop, qa[ti][ds], dt[ti]);
      }
      for (int ti = 0; ti < 4; ++ti) inv[ti] = 1.0f / ((dt[ti][0] + __shfl_xor(dt[ti][0], 32)) + eps);
    }
    bf16x8 held[4];  // bf16 outputs of quarter 0, stored with quarter 1
    for (int m = 0; m < NM; ++m) {
      floatx4 acc[2][4];
      for (int h2 = 0; h2 < 2; ++h2)
        for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = z4;
      // inter: O^T[n][t] = sum_d S[d][n] Q[t][d] (state before the block)
      for (int ds = 0; ds < NDS; ++ds)
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 sa = ld_lds16(st + (32 * m + 4 * h2 + nlane) * RST + 32 * ds + 8 * grp);
          for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = mfma(sa, qa[ti][ds], acc[h2][ti]);
        }
      // intra: O^T[n][t] += sum_s V[s][n] P^T[s][t]
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 va0 = tr_operand(vs, 0, 32 * m + 4 * h2, l16, grp, 8, RKV);
        const bf16x8 va1 = tr_operand(vs, 1, 32 * m + 4 * h2, l16, grp, 8, RKV);
        for (int ti = 0; ti < 4; ++ti) acc[h2][ti] = mfma(va0, pop[ti][0], acc[h2][ti]);
        acc[h2][2] = mfma(va1, pop[2][1], acc[h2][2]);
        acc[h2][3] = mfma(va1, pop[3][1], acc[h2][3]);
      }
      if constexpr (kN)
        for (int h2 = 0; h2 < 2; ++h2)
          for (int ti = 0; ti < 4; ++ti)
            for (int i = 0; i < 4; ++i) acc[h2][ti][i] *= inv[ti];
      if constexpr (OUT_F32) {
        for (int ti = 0; ti < 4; ++ti) {
          const int64_t t = blk * C + 16 * ti + l16;
          if (t < N) {
            float* op = static_cast<float*>(o) + (bh * N + t) * HD + 32 * m + 8 * grp;
            *reinterpret_cast<floatx4*>(op) = acc[0][ti];
            *reinterpret_cast<floatx4*>(op + 4) = acc[1][ti];
          }
        }
      } else if ((m & 1) == 0) {
        for (int ti = 0; ti < 4; ++ti) held[ti] = pack_tiles(acc[0][ti], acc[1][ti]);
      } else {
        // the two quarters make one 128-byte line of every row: whole lines
        uint16_t* line = static_cast<uint16_t*>(o) + bh * N * HD + 64 * (m >> 1);
        for (int ti = 0; ti < 4; ++ti)
          store_lines(line, HD, blk * C + 16 * ti, N, held[ti], pack_tiles(acc[0][ti], acc[1][ti]), l16, grp);
      }
    }
    // the next block's loads go out once this block's Q operands are dead
    if (blk + 1 < blk1) load_block(blk + 1);

    // state update: S += K_b^T V_b (every column), then its bf16 copy
    {
      bf16x8 vb[NJ][2];
      for (int jn = 0; jn < NJ; ++jn)
        for (int p = 0; p < 2; ++p) vb[jn][p] = tr_operand(vs, p, 16 * jn, l16, grp, 4, RKV);
      for (int dt = 0; dt < NDT; ++dt)
        for (int p = 0; p < 2; ++p) {
          const bf16x8 kt = tr_operand(ks, p, 16 * dt, l16, grp, 4, RKV);
          for (int jn = 0; jn < NJ; ++jn) sacc[jn][dt] = mfma(kt, vb[jn][p], sacc[jn][dt]);
        }
      for (int jn = 0; jn < NJ; ++jn)
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<bf16x4*>(&st[(16 * jn + l16) * RST + 16 * dt + 4 * grp]) = to_bf16x4(sacc[jn][dt]);
      if constexpr (kN) {
        // z += K_b^T 1 (after this block's denominators have read z)
        for (int p = 0; p < 2; ++p)
          for (int jj = 0; jj < NJ; ++jj)
            zacc[jj] = mfma(tr_operand(ks, p, 16 * jj, l16, grp, 4, RKV), ones_bf16x8(), zacc[jj]);
        if (l16 == 0)
          for (int jj = 0; jj < NJ; ++jj) *reinterpret_cast<floatx4*>(&zs[16 * jj + 4 * grp]) = zacc[jj];
      }
    }
    __syncthreads();  // (one wave: the tile reads above precede the next block's stores)
  }

  if (s_out != nullptr && seg == P - 1) {
    float* so = s_out + bh * (HD * HD);
    for (int jn = 0; jn < NJ; ++jn)
      for (int dt = 0; dt < NDT; ++dt)
        for (int i = 0; i < 4; ++i) so[(16 * dt + 4 * grp + i) * HD + 16 * jn + l16] = sacc[jn][dt][i];
  }
  if constexpr (kN)
    if (z_out != nullptr && seg == P - 1 && l16 == 0)
      for (int jj = 0; jj < NJ; ++jj)
        for (int i = 0; i < 4; ++i) z_out[bh * HD + 16 * jj + 4 * grp + i] = zacc[jj][i];
}

// Pre-pass: partial[c][j][r] = sum of K_b^T V_b over part r of segment
// j + seg_offset of chain c, for j < P - 1 (the forward sums every segment but
// the last with seg_offset 0; the backward every segment but the first with
// seg_offset 1).  Four waves; wave w owns state columns [w HD/4, (w+1) HD/4)
// (head size HD = d = dv, 128 or 64).  A pure HBM stream: the K/V tile is
// single-buffered in LDS (36 KiB at HD = 128) and the next two blocks' loads
// are in flight in two register slots while a block is multiplied; two
// workgroups share a CU at HD = 128 (148 + 32 registers per wave), three at
// 64.  (At 128, two slots and two workgroups per CU measured 0.6 ms faster
// per 1M-token backward than one slot and three.)
//
// Flags (feature-map variants): kRelu applies phi = ReLU to k as it enters
// LDS; kNorm also writes zpart[c][j][r] = sum of phi(k_b) over the part
// (wave w: entries [32w, 32w+32), as K^T times a ones operand on the matrix
// cores).
template <int FL, int HD = 128>
__global__ __launch_bounds__(kPartThreads, part_wgs_per_cu(HD)) void state_parts(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           float* __restrict__ partial,
                                                           float* __restrict__ zpart, int64_t N,
                                                           int64_t nblocks, int64_t blocks_per_seg,
                                                           int64_t blocks_per_part, int P, int R,
                                                           int seg_offset, int shifted) {
  // head size HD = d = dv (64 or 128), as in fwd_bf16_g4
  constexpr int NDT = HD / 16, WC = HD / 4, NJ = WC / 16, RKV = HD + 16, CPR = HD / 8, RPP = 256 / CPR;
  __shared__ __align__(16) uint16_t ksm[C * RKV];
  __shared__ __align__(16) uint16_t vsm[C * RKV];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int per_chain = (P - 1) * R;
  const int c = blockIdx.x / per_chain;
  const int rem = blockIdx.x % per_chain;
  const int j = rem / R, r = rem % R;
  const int64_t js = int64_t(j) + seg_offset;  // segment summed by this part
  // shifted boundaries (pre-passes of the forward and the causal variants,
  // js + 1 < P): the last part runs to the segment's end, which may lie up to
  // 15 blocks past R parts
  const int64_t shift = shifted ? seg_shift(c) : 0;
  const int64_t seg_end = seg_first(js + 1, blocks_per_seg, shift);
  int64_t b0 = seg_first(js, blocks_per_seg, shift) + int64_t(r) * blocks_per_part;
  int64_t b1 = r == R - 1 ? seg_end : b0 + blocks_per_part;
  if (b1 > seg_end) b1 = seg_end;
  if (b1 > nblocks) b1 = nblocks;

  const uint16_t* kh = k + int64_t(c) * N * HD;
  const uint16_t* vh = v + int64_t(c) * N * HD;

  floatx4 acc[NJ][NDT];
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt) acc[jn][dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 zacc[NJ];
  for (int jj = 0; jj < NJ; ++jj) zacc[jj] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int ch = tid % CPR;
  auto load = [&](int64_t blk, uint4 (&kr)[HD / 32], uint4 (&vr)[HD / 32]) {
    for (int i = 0; i < HD / 32; ++i) {
      const int64_t t = blk * C + tid / CPR + RPP * i;
      if (t < N) {
        kr[i] = ld_stream16(kh + t * HD + 8 * ch);
        vr[i] = ld_stream16(vh + t * HD + 8 * ch);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store = [&](const uint4 (&kr)[HD / 32], const uint4 (&vr)[HD / 32]) {
    for (int i = 0; i < HD / 32; ++i) {
      const int row = tid / CPR + RPP * i;
      *reinterpret_cast<uint4*>(&ksm[row * RKV + 8 * ch]) = (FL & kRelu) ? relu_bf16x8(kr[i]) : kr[i];
      *reinterpret_cast<uint4*>(&vsm[row * RKV + 8 * ch]) = vr[i];
    }
  };

  // Two register slots; blocks past the part are loaded too (zeros past N,
  // unused otherwise) so that every path issues the same loads.
  constexpr int NSL = 2;
  int64_t blk = b0;
  uint4 kr[NSL][HD / 32], vr[NSL][HD / 32];
  for (int sl = 0; sl < NSL; ++sl) load(b0 + sl, kr[sl], vr[sl]);
  auto body = [&](int sl) __attribute__((always_inline)) {
    store(kr[sl], vr[sl]);
    __syncthreads();  // the block's K and V are in LDS
    load(blk + NSL, kr[sl], vr[sl]);
    for (int p = 0; p < 2; ++p) {
      bf16x8 vb[NJ];
      for (int jn = 0; jn < NJ; ++jn) vb[jn] = tr_operand(vsm, p, WC * w + 16 * jn, l16, grp, 4, RKV);
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 ka = tr_operand(ksm, p, 16 * dt, l16, grp, 4, RKV);
        for (int jn = 0; jn < NJ; ++jn) acc[jn][dt] = mfma(ka, vb[jn], acc[jn][dt]);
      }
      if constexpr ((FL & kNorm) != 0)
        for (int jj = 0; jj < NJ; ++jj)
          zacc[jj] = mfma(tr_operand(ksm, p, WC * w + 16 * jj, l16, grp, 4, RKV), ones_bf16x8(), zacc[jj]);
    }
    __syncthreads();  // every wave is done with this block's K and V
    ++blk;
  };
  // whole rounds of NSL blocks in the loop, the remainder after it (a
  // conditional step inside the loop would make the compiler wait for every
  // load in flight before each store)
  while (blk + NSL <= b1)
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) body(sl);
  if (blk < b1) body(0);
  if constexpr ((FL & kNorm) != 0) {
    // every column of the ones product holds the sum; lanes of column 0 write it
    float* zo = zpart + ((int64_t(c) * (P - 1) + j) * R + r) * HD;
    if (l16 == 0)
      for (int jj = 0; jj < NJ; ++jj)
        for (int i = 0; i < 4; ++i) zo[WC * w + 16 * jj + 4 * grp + i] = zacc[jj][i];
  }

  float* out = partial + ((int64_t(c) * (P - 1) + j) * R + r) * (HD * HD);
  for (int jn = 0; jn < NJ; ++jn)
    for (int dt = 0; dt < NDT; ++dt)
      for (int i = 0; i < 4; ++i) out[(16 * dt + 4 * grp + i) * HD + WC * w + 16 * jn + l16] = acc[jn][dt][i];
}

// starts[c][j] = s_in[c] + sum over segments i < j and parts r of partial[c][i][r],
// accumulated in that fixed order; E elements per chain (d*dv for the state,
// d for the normaliser sums), `total` threads.  A thread's partials are
// independent loads, issued kScanBatch at a time ahead of the additions (the
// batch's tail re-reads the last partial instead of branching, which would
// make the compiler wait for each load before the next), so a scan waits a
// few memory latencies instead of one per partial.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(256) void scan_starts(const float* __restrict__ partial, float* __restrict__ starts,
                                                   const float* s_in, int P, int R, int E, int64_t total) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= total) return;
  const int64_t c = gid / E;
  const int e = int(gid % E);
  const int n = (P - 1) * R;  // the chain's partials, in summation order
  const float* pc = partial + c * n * E + e;
  float* sc = starts + c * P * E + e;
  float run = s_in ? s_in[c * E + e] : 0.0f;
  sc[0] = run;
  int r = 0, j = 0;
  for (int b = 0; b < n; b += kScanBatch) {
    float x[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) x[i] = pc[int64_t(b + i < n ? b + i : n - 1) * E];  // no branch
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (b + i < n) {
        run += x[i];
        if (++r == R) {
          r = 0;
          sc[int64_t(++j) * E] = run;
        }
      }
  }
}

// s_out[c][e] = s_in[c][e] (0 without s_in) + sum over r < R of
// partial[c][r][e], added in order of r; E elements per state.  s_out may be
// s_in (each thread reads its element before writing it).  Loads are batched
// as in scan_starts.
__global__ __launch_bounds__(256) void sum_parts(const float* __restrict__ partial, const float* s_in, float* s_out,
                                                 int R, int E, int64_t total) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= total) return;
  const int64_t c = gid / E;
  const int e = int(gid % E);
  const float* pc = partial + c * R * E + e;
  float run = s_in ? s_in[gid] : 0.0f;
  for (int b = 0; b < R; b += kScanBatch) {
    float x[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) x[i] = pc[int64_t(b + i < R ? b + i : R - 1) * E];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (b + i < R) run += x[i];
  }
  s_out[gid] = run;
}

// ---------------------------------------------------------------------------
// Non-causal variant (LinearAttentionCore of page "MiniMax-01与Lightning
// Attention", section 2.2): o_t = phi(q_t) . S_tot for every t, with S_tot =
// s_in + sum over all tokens of phi(k_s)^T v_s, optionally divided by
// phi(q_t) . z_tot + eps.  With the state fixed every block is independent:
// a streaming product Q S_tot per query head (read q, write o) with no
// barrier in the loop; the next step's Q operands load while the current
// step multiplies.  Grid: B * Hkv * (G/GW) * P workgroups of eight waves (two
// per SIMD) serving GW = 4, 2 or 1 query heads of a KV head's group: wave w
// takes query head w % GW and 16-token query tiles {2(w/GW), 2(w/GW) + 1} of
// each step of 4/GW blocks (one block for GW = 4).  S_tot comes in float32
// from the pre-pass and is rounded once to the bf16 n-major LDS layout of the
// causal kernel's state copy.  Built for head sizes 128 and 64, GW = 4, 2, 1.
// ---------------------------------------------------------------------------
template <int GW, bool OUT_F32, int FL, int HD = 128>
__global__ __launch_bounds__(512, 1) void fwd_noncausal(
    const uint16_t* __restrict__ q, void* __restrict__ o, const float* __restrict__ stot,
    const float* __restrict__ ztot, int64_t tot_stride, float* s_out, float* z_out, int Hq, int Hkv,
    int subgroups, int64_t N, int64_t nblocks, int64_t blocks_per_seg, int P, float eps) {
  constexpr bool kN = (FL & kNorm) != 0;
  constexpr bool kR = (FL & kRelu) != 0;
  // head size HD = d = dv (64 or 128): NDS 32-wide chunks of d, state rows at RST
  static_assert(HD == 64 || HD == 128, "head size 64 or 128");
  constexpr int NDS = HD / 32, RST = HD + 8, HH = HD * HD;
  __shared__ __align__(16) uint16_t st[HD * RST];
  __shared__ __align__(16) float zs[kN ? HD : 4];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int hw = w % GW, t0 = 2 * (w / GW);               // head in the subgroup, first query tile
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int chain = blockIdx.x / P;
  const int sub = chain % subgroups;
  const int bg = chain / subgroups;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;
  const int64_t head = int64_t(b) * Hq + int64_t(g) * G + int64_t(sub) * GW + hw;
  const uint16_t* qh = q + head * N * HD;
  const int nlane = 8 * (l16 >> 2) + (l16 & 3);
  constexpr int SB = 4 / GW;  // blocks per step
  // tokens of this segment (a step of several blocks may run past its end)
  const int64_t tend = GW == 4 ? N : (blk1 * C < N ? blk1 * C : N);

  // wave w < HD/16 rounds state columns [16w, 16w+16) (all eight at 128)
  const float* S = stot + int64_t(bg) * tot_stride * HH;
  if (HD == 128 || w < HD / 16)
    for (int dt = 0; dt < HD / 16; ++dt) {
      floatx4 x;
      for (int i = 0; i < 4; ++i) x[i] = S[(16 * dt + 4 * grp + i) * HD + 16 * w + l16];
      *reinterpret_cast<bf16x4*>(&st[(16 * w + l16) * RST + 16 * dt + 4 * grp]) = to_bf16x4(x);
      if (s_out != nullptr && seg == 0 && sub == 0)
        for (int i = 0; i < 4; ++i) s_out[int64_t(bg) * HH + (16 * dt + 4 * grp + i) * HD + 16 * w + l16] = x[i];
    }
  if constexpr (kN) {
    const float* Z = ztot + int64_t(bg) * tot_stride * HD;
    if (tid < HD) {
      zs[tid] = Z[tid];
      if (z_out != nullptr && seg == 0 && sub == 0) z_out[int64_t(bg) * HD + tid] = Z[tid];
    }
  }
  __syncthreads();  // S_tot (and z_tot) are in LDS

  auto load_q = [&](bf16x8 (&qa)[2][NDS], int64_t blk) {
    for (int tj = 0; tj < 2; ++tj) {
      const int64_t t = blk * C + 16 * (t0 + tj) + l16;
      for (int ds = 0; ds < NDS; ++ds)
        qa[tj][ds] = (t < tend) ? ld_global16(qh + t * HD + 32 * ds + 8 * grp) : zero_bf16x8();
    }
  };
  bf16x8 qa[2][NDS], qn[2][NDS];
  if (blk0 < blk1) load_q(qa, blk0);
  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t blk = blk0; blk < blk1; blk += SB) {
    // The state operands are re-read from LDS every step rather than held in
    // registers across the loop: holding them leaves the normalised forms too
    // few registers (they spill) and measured no faster for the others.
    asm volatile("" ::: "memory");
    if (blk + SB < blk1) load_q(qn, blk + SB);
    if constexpr (kR)
      for (int tj = 0; tj < 2; ++tj)
        for (int ds = 0; ds < NDS; ++ds) qa[tj][ds] = relu_bf16x8(qa[tj][ds]);
    float inv[2];
    (void)inv;
    if constexpr (kN) {
      float den[2] = {0.0f, 0.0f};
      for (int ds = 0; ds < NDS; ++ds) {
        const floatx4 za = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp]);
        const floatx4 zb = *reinterpret_cast<const floatx4*>(&zs[32 * ds + 8 * grp + 4]);
        for (int tj = 0; tj < 2; ++tj)
          for (int j = 0; j < 4; ++j)
            den[tj] += float(qa[tj][ds][j]) * za[j] + float(qa[tj][ds][j + 4]) * zb[j];
      }
      for (int tj = 0; tj < 2; ++tj) {
        float x = den[tj];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        inv[tj] = 1.0f / (x + eps);
      }
    }
    bf16x8 held[2];  // bf16 outputs of an even quarter, stored with the odd one
    for (int m = 0; m < HD / 32; ++m) {
      floatx4 acc[2][2];
      for (int h2 = 0; h2 < 2; ++h2)
        for (int tj = 0; tj < 2; ++tj) acc[h2][tj] = z4;
      for (int ds = 0; ds < NDS; ++ds)
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 sa = ld_lds16(st + (32 * m + 4 * h2 + nlane) * RST + 32 * ds + 8 * grp);
          for (int tj = 0; tj < 2; ++tj) acc[h2][tj] = mfma(sa, qa[tj][ds], acc[h2][tj]);
        }
      if constexpr (kN)
        for (int h2 = 0; h2 < 2; ++h2)
          for (int tj = 0; tj < 2; ++tj)
            for (int i = 0; i < 4; ++i) acc[h2][tj][i] *= inv[tj];
      if constexpr (OUT_F32) {
        for (int tj = 0; tj < 2; ++tj) {
          const int64_t t = blk * C + 16 * (t0 + tj) + l16;
          if (t < tend) {
            float* op = static_cast<float*>(o) + (head * N + t) * HD + 32 * m + 8 * grp;
            *reinterpret_cast<floatx4*>(op) = acc[0][tj];
            *reinterpret_cast<floatx4*>(op + 4) = acc[1][tj];
          }
        }
      } else if ((m & 1) == 0) {
        for (int tj = 0; tj < 2; ++tj) held[tj] = pack_tiles(acc[0][tj], acc[1][tj]);
      } else {
        // two quarters make one 128-byte line of every row: whole lines
        uint16_t* line = static_cast<uint16_t*>(o) + head * N * HD + 64 * (m >> 1);
        for (int tj = 0; tj < 2; ++tj)
          store_lines(line, HD, blk * C + 16 * (t0 + tj), tend, held[tj], pack_tiles(acc[0][tj], acc[1][tj]), l16,
                      grp);
      }
    }
    for (int tj = 0; tj < 2; ++tj)
      for (int ds = 0; ds < NDS; ++ds) qa[tj][ds] = qn[tj][ds];
  }
}

// gw: query heads per workgroup (4; 1 or 2 with PARTIAL)
template <bool OUT_F32, int FL = 0, int HD = 128, bool PARTIAL = false, bool RS = false>
void launch_g4(dim3 grid, hipStream_t stream, const void* q, const void* k, const void* v, void* o,
               const float* starts, const float* s_in, float* s_out, int Hq, int Hkv, int subgroups, int64_t N,
               int64_t nblocks, int64_t bps, int P, const float* zstarts = nullptr, const float* z_in = nullptr,
               float* z_out = nullptr, float eps = 0.0f, int gw = 4, const void* qx = nullptr,
               float* rpart = nullptr, bool shifted = false) {
  hipLaunchKernelGGL((fwd_bf16_g4<OUT_F32, FL, HD, PARTIAL, RS>), grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, starts, s_in, s_out, Hq, Hkv, subgroups, N, nblocks, bps,
                     P, zstarts, z_in, z_out, eps, gw, static_cast<const uint16_t*>(qx), rpart, int(shifted));
}

template <int GW, bool OUT_F32, int FL = 0>
void launch_main(dim3 grid, hipStream_t stream, const void* q, const void* k, const void* v, void* o,
                 const float* starts, const float* s_in, float* s_out, int Hq, int Hkv, int subgroups, int64_t N,
                 int64_t nblocks, int64_t bps, int P, const float* zstarts = nullptr, const float* z_in = nullptr,
                 float* z_out = nullptr, float eps = 0.0f) {
  hipLaunchKernelGGL((fwd_bf16_main<GW, OUT_F32, FL>), grid, dim3(kMainThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), o, starts, s_in, s_out, Hq, Hkv, subgroups, N, nblocks, bps,
                     P, zstarts, z_in, z_out, eps);
}

}  // namespace

hipError_t launch_segment_states(const void* k, const void* v, const float* s_in, int64_t B, int64_t Hkv,
                                 int64_t N, const Bf16Plan& plan, void* workspace, hipStream_t stream) {
  const int64_t kv_chains = B * Hkv;
  float* partial = static_cast<float*>(workspace);
  float* starts = partial + plan.partial_floats;
  if (plan.hd != 128 && plan.hd != 64) return hipErrorInvalidValue;
  if (plan.P > 1) {
    const dim3 grid(unsigned(kv_chains * (plan.P - 1) * plan.R));
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    if (plan.hd == 64)
      hipLaunchKernelGGL((state_parts<0, 64>), grid, dim3(kPartThreads), 0, stream, k16, v16, partial, nullptr, N,
                         plan.nblocks, plan.blocks_per_seg, plan.blocks_per_part, plan.P, plan.R, 0,
                         int(plan.shifted));
    else
      hipLaunchKernelGGL((state_parts<0, 128>), grid, dim3(kPartThreads), 0, stream, k16, v16, partial, nullptr, N,
                         plan.nblocks, plan.blocks_per_seg, plan.blocks_per_part, plan.P, plan.R, 0,
                         int(plan.shifted));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int E = plan.hd * plan.hd;
  const int64_t total = kv_chains * E;
  hipLaunchKernelGGL(scan_starts, dim3(unsigned((total + 255) / 256)), dim3(256), 0, stream, partial, starts, s_in,
                     plan.P, plan.R, E, total);
  return hipGetLastError();
}

hipError_t launch_state_total_bf16(const void* a, const void* b, const float* s_in, float* s_out, int64_t chains,
                                   int G, int64_t N, const StatePlan& plan, float* workspace, hipStream_t stream) {
  // one summed segment (the whole sequence) of each of the chains * G input
  // chains in plan.R parts; output chain c sums input chains c G .. c G + G - 1
  hipError_t e = launch_state_parts(a, b, workspace, chains * G, N, plan.nblocks, plan.nblocks, plan.blocks_per_part,
                                    2, plan.R, 0, plan.hd, stream);
  if (e != hipSuccess) return e;
  const int E = plan.hd * plan.hd;
  const int64_t total = chains * E;
  hipLaunchKernelGGL(sum_parts, dim3(unsigned((total + 255) / 256)), dim3(256), 0, stream, workspace, s_in, s_out,
                     G * plan.R, E, total);
  return hipGetLastError();
}

hipError_t launch_state_parts(const void* a, const void* b, float* partial, int64_t chains, int64_t N,
                              int64_t nblocks, int64_t blocks_per_seg, int64_t blocks_per_part, int P, int R,
                              int seg_offset, int hd, hipStream_t stream) {
  const dim3 grid(unsigned(chains * (P - 1) * R));
  const auto* a16 = static_cast<const uint16_t*>(a);
  const auto* b16 = static_cast<const uint16_t*>(b);
  if (hd == 64)
    hipLaunchKernelGGL((state_parts<0, 64>), grid, dim3(kPartThreads), 0, stream, a16, b16, partial, nullptr, N,
                       nblocks, blocks_per_seg, blocks_per_part, P, R, seg_offset, 0);
  else if (hd == 128)
    hipLaunchKernelGGL((state_parts<0, 128>), grid, dim3(kPartThreads), 0, stream, a16, b16, partial, nullptr, N,
                       nblocks, blocks_per_seg, blocks_per_part, P, R, seg_offset, 0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {

template <int FL, int HD>
hipError_t variant_states(const void* k, const void* v, const float* s_in, const float* z_in, int64_t kv_chains,
                          int64_t N, const VarPlan& vp, float* ws, hipStream_t stream) {
  // Segment starts (causal) or the totals (non-causal: the scan over Ppre + 1
  // entries ends with the sum over every segment).
  const Bf16Plan& p = vp.base;
  const int Ppre = vp.causal ? p.P : p.P + 1;
  float* partial = ws;
  float* starts = partial + vp.partial_floats;
  float* zpart = starts + vp.start_floats;
  float* zstarts = zpart + vp.zpart_floats;
  if (Ppre > 1) {
    hipLaunchKernelGGL((state_parts<FL, HD>), dim3(unsigned(kv_chains * (Ppre - 1) * p.R)), dim3(kPartThreads), 0,
                       stream, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), partial, zpart, N,
                       p.nblocks, p.blocks_per_seg, p.blocks_per_part, Ppre, p.R, 0, int(p.shifted));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = kv_chains * HD * HD;
  hipLaunchKernelGGL(scan_starts, dim3(unsigned((total + 255) / 256)), dim3(256), 0, stream, partial, starts, s_in,
                     Ppre, p.R, HD * HD, total);
  if ((FL & kNorm) != 0) {
    const int64_t zt = kv_chains * HD;
    hipLaunchKernelGGL(scan_starts, dim3(unsigned((zt + 255) / 256)), dim3(256), 0, stream, zpart, zstarts, z_in,
                       Ppre, p.R, HD, zt);
  }
  return hipGetLastError();
}

template <bool OUT_F32, int FL>
hipError_t variant_outputs(const void* q, const void* k, const void* v, void* o, const float* s_in, float* s_out,
                           const float* z_in, float* z_out, float eps, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                           const VarPlan& vp, float* ws, hipStream_t stream) {
  const Bf16Plan& p = vp.base;
  const float* starts = ws + vp.partial_floats;
  const float* zstarts = starts + vp.start_floats + vp.zpart_floats;
  const int iHq = int(Hq), iHkv = int(Hkv);
  if (vp.causal) {
    const dim3 grid(unsigned(B * Hkv * p.subgroups * p.P));
    const bool st = p.use_starts;
    const float* zs = (FL & kNorm) && st ? zstarts : nullptr;
    const float* zi = (FL & kNorm) && !st ? z_in : nullptr;
#define LA_VAR(LAUNCH)                                                                                              \
  LAUNCH(grid, stream, q, k, v, o, st ? starts : nullptr, st ? nullptr : s_in, s_out, iHq, iHkv, p.subgroups, N, \
         p.nblocks, p.blocks_per_seg, p.P, zs, zi, z_out, eps)
    if (p.solo) {
      hipLaunchKernelGGL((fwd_bf16_solo<OUT_F32, FL>), grid, dim3(64), 0, stream, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), o,
                         st ? starts : nullptr, st ? nullptr : s_in, s_out, N, p.nblocks, p.blocks_per_seg, p.P, zs,
                         zi, z_out, eps);
    } else if (p.hd == 64) {
      if (p.gw == 4)
        launch_g4<OUT_F32, FL, 64>(grid, stream, q, k, v, o, st ? starts : nullptr, st ? nullptr : s_in, s_out, iHq,
                                   iHkv, p.subgroups, N, p.nblocks, p.blocks_per_seg, p.P, zs, zi, z_out, eps, 4,
                                   nullptr, nullptr, p.shifted);
      else
        launch_g4<OUT_F32, FL, 64, true>(grid, stream, q, k, v, o, st ? starts : nullptr, st ? nullptr : s_in,
                                         s_out, iHq, iHkv, p.subgroups, N, p.nblocks, p.blocks_per_seg, p.P, zs, zi,
                                         z_out, eps, p.gw);
    } else if (p.gw == 4) {
      launch_g4<OUT_F32, FL>(grid, stream, q, k, v, o, st ? starts : nullptr, st ? nullptr : s_in, s_out, iHq, iHkv,
                             p.subgroups, N, p.nblocks, p.blocks_per_seg, p.P, zs, zi, z_out, eps, 4, nullptr,
                             nullptr, p.shifted);
    } else if (p.gw == 2) LA_VAR((launch_main<2, OUT_F32, FL>));
    else LA_VAR((launch_main<1, OUT_F32, FL>));
#undef LA_VAR
  } else {
    // totals sit at entry P of each chain's P + 1 scanned entries
    const int64_t stride = p.P + 1;
    const dim3 grid(unsigned(B * Hkv * p.subgroups * vp.P_out));
#define LA_NC(GW, HD)                                                                                               \
  hipLaunchKernelGGL((fwd_noncausal<GW, OUT_F32, FL, HD>), grid, dim3(512), 0, stream,                              \
                     static_cast<const uint16_t*>(q), o, starts + p.P * (HD * HD), zstarts + p.P * HD, stride, s_out, \
                     z_out, iHq, iHkv, p.subgroups, N, p.nblocks, vp.bps_out, vp.P_out, eps)
    if (p.hd == 64) {
      if (p.gw == 4) LA_NC(4, 64);
      else if (p.gw == 2) LA_NC(2, 64);
      else LA_NC(1, 64);
    } else if (p.gw == 4) LA_NC(4, 128);
    else if (p.gw == 2) LA_NC(2, 128);
    else LA_NC(1, 128);
#undef LA_NC
  }
  return hipGetLastError();
}

template <int FL>
hipError_t variant_run(const void* q, const void* k, const void* v, void* o, bool out_f32, const float* s_in,
                       float* s_out, const float* z_in, float* z_out, float eps, int64_t B, int64_t Hq, int64_t Hkv,
                       int64_t N, const VarPlan& vp, float* ws, hipStream_t stream) {
  if (vp.base.hd != 128 && vp.base.hd != 64) return hipErrorInvalidValue;
  if (!vp.causal || vp.base.use_starts) {
    hipError_t e = vp.base.hd == 64 ? variant_states<FL, 64>(k, v, s_in, z_in, B * Hkv, N, vp, ws, stream)
                                    : variant_states<FL, 128>(k, v, s_in, z_in, B * Hkv, N, vp, ws, stream);
    if (e != hipSuccess) return e;
  }
  return out_f32 ? variant_outputs<true, FL>(q, k, v, o, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp, ws, stream)
                 : variant_outputs<false, FL>(q, k, v, o, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp, ws,
                                              stream);
}

}  // namespace

hipError_t launch_variant(const void* q, const void* k, const void* v, void* o, bool out_f32, bool relu,
                          const float* s_in, float* s_out, const float* z_in, float* z_out, float eps, int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t N, const VarPlan& vp, void* workspace,
                          hipStream_t stream) {
  float* ws = static_cast<float*>(workspace);
  if (vp.norm)
    return relu ? variant_run<kRelu | kNorm>(q, k, v, o, out_f32, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp,
                                             ws, stream)
                : variant_run<kNorm>(q, k, v, o, out_f32, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp, ws,
                                     stream);
  return relu ? variant_run<kRelu>(q, k, v, o, out_f32, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp, ws,
                                   stream)
              : variant_run<0>(q, k, v, o, out_f32, s_in, s_out, z_in, z_out, eps, B, Hq, Hkv, N, vp, ws, stream);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, bool out_f32, const float* s_in,
                           float* s_out, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, const Bf16Plan& plan,
                           const void* workspace, hipStream_t stream) {
  const int64_t kv_chains = B * Hkv;
  const float* starts = plan.use_starts ? static_cast<const float*>(workspace) + plan.partial_floats : nullptr;
  const dim3 grid(unsigned(kv_chains * plan.subgroups * plan.P));
  const int iHq = int(Hq), iHkv = int(Hkv);
#define LA_MAIN(GW, F32)                                                                                      \
  launch_main<GW, F32>(grid, stream, q, k, v, o, starts, plan.use_starts ? nullptr : s_in, s_out, iHq, iHkv, \
                       plan.subgroups, N, plan.nblocks, plan.blocks_per_seg, plan.P)
  if (plan.solo) {
    // head size 64, one query head per KV head: one-wave workgroups
    if (plan.hd != 64) return hipErrorInvalidValue;
    const auto* q16 = static_cast<const uint16_t*>(q);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const float* si = plan.use_starts ? nullptr : s_in;
    if (out_f32)
      hipLaunchKernelGGL((fwd_bf16_solo<true>), grid, dim3(64), 0, stream, q16, k16, v16, o, starts, si, s_out, N,
                         plan.nblocks, plan.blocks_per_seg, plan.P, nullptr, nullptr, nullptr, 0.0f);
    else
      hipLaunchKernelGGL((fwd_bf16_solo<false>), grid, dim3(64), 0, stream, q16, k16, v16, o, starts, si, s_out, N,
                         plan.nblocks, plan.blocks_per_seg, plan.P, nullptr, nullptr, nullptr, 0.0f);
  } else if (plan.hd == 64) {
    // head size 64: the four-wave kernel, with gw = 1 or 2 query heads per
    // workgroup (idle waves) for groups that are not a multiple of four
    const float* si = plan.use_starts ? nullptr : s_in;
#define LA_G64(F32, PART)                                                                                     \
  launch_g4<F32, 0, 64, PART>(grid, stream, q, k, v, o, starts, si, s_out, iHq, iHkv, plan.subgroups, N,     \
                              plan.nblocks, plan.blocks_per_seg, plan.P, nullptr, nullptr, nullptr, 0.0f, plan.gw, \
                              nullptr, nullptr, plan.shifted)
    if (plan.gw == 4) {
      if (out_f32) LA_G64(true, false); else LA_G64(false, false);
    } else {
      if (out_f32) LA_G64(true, true); else LA_G64(false, true);
    }
#undef LA_G64
  } else if (plan.hd != 128) {
    return hipErrorInvalidValue;
  } else if (plan.gw == 4) {
    const float* si = plan.use_starts ? nullptr : s_in;
    if (out_f32)
      launch_g4<true>(grid, stream, q, k, v, o, starts, si, s_out, iHq, iHkv, plan.subgroups, N, plan.nblocks,
                      plan.blocks_per_seg, plan.P, nullptr, nullptr, nullptr, 0.0f, 4, nullptr, nullptr,
                      plan.shifted);
    else
      launch_g4<false>(grid, stream, q, k, v, o, starts, si, s_out, iHq, iHkv, plan.subgroups, N, plan.nblocks,
                       plan.blocks_per_seg, plan.P, nullptr, nullptr, nullptr, 0.0f, 4, nullptr, nullptr,
                       plan.shifted);
  } else if (plan.gw == 2) {
    if (out_f32) LA_MAIN(2, true); else LA_MAIN(2, false);
  } else {
    if (out_f32) LA_MAIN(1, true); else LA_MAIN(1, false);
  }
#undef LA_MAIN
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_rsum(const void* q, const void* k, const void* v, void* o, bool out_f32,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, const Bf16Plan& plan,
                                const void* workspace, const void* x, float* rpart, hipStream_t stream) {
  if (plan.hd != 128 || plan.gw != 4 || plan.solo || plan.P < 2 || !plan.use_starts) return hipErrorInvalidValue;
  const float* starts = static_cast<const float*>(workspace) + plan.partial_floats;
  const dim3 grid(unsigned(B * Hkv * plan.subgroups * plan.P));
  if (out_f32)
    launch_g4<true, 0, 128, false, true>(grid, stream, q, k, v, o, starts, nullptr, nullptr, int(Hq), int(Hkv),
                                         plan.subgroups, N, plan.nblocks, plan.blocks_per_seg, plan.P, nullptr,
                                         nullptr, nullptr, 0.0f, 4, x, rpart);
  else
    launch_g4<false, 0, 128, false, true>(grid, stream, q, k, v, o, starts, nullptr, nullptr, int(Hq), int(Hkv),
                                          plan.subgroups, N, plan.nblocks, plan.blocks_per_seg, plan.P, nullptr,
                                          nullptr, nullptr, 0.0f, 4, x, rpart);
  return hipGetLastError();
}

}  // namespace la
