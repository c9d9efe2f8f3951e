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
// Design for MI355X (head size 128): one workgroup of eight waves per (batch,
// KV head, sequence segment); segment j starts from the sum over later
// segments, produced by the forward's pre-pass kernel run on (Q, dO) pairs
// and a reverse scan here.  On SIMD s, wave s is a gradient wave and wave
// s + 4 a state wave:
//  * gradient waves 0 and 1 hold dV^T of key tiles {0, 3} and {1, 2} of the
//    block, waves 2 and 3 dK^T of the same pairs (pairing key tile j with
//    3 - j evens out the causal work).  A gradient wave computes the score
//    tiles of its own keys (X^T = Q K^T for dV, Y^T = dO V^T for dK), which
//    stay in registers as the operands of its intra products, and the inter
//    products from the bf16 copy of R;
//  * the state waves hold R (128 x 128, float32) in four sets of 16 tiles,
//    update them per query head and round them once per block into an
//    n-major bf16 LDS copy.
// Each SIMD thus does 92 matrix products per query head, split 60 / 32
// between its two waves, and one wave's LDS waits overlap the other's
// products.  The block's K/V pair and each query head's Q/dO pair form one
// stream of 32 KiB items through two register slots and three LDS buffers
// (the block's K/V keeps one, its heads alternate between the other two), so
// one barrier per item suffices.  Products are v_mfma_f32_16x16x32_bf16 in
// the transposed-product layout of the forward kernel.
#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

using namespace mfma16;

constexpr int kThreads = 512;  // eight waves, two per SIMD
constexpr int kSlots = 2;      // 32 KiB items in flight per workgroup (register slots)
constexpr int DD = D * DV;

__device__ __forceinline__ u32x4 ld_stream_v(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

struct __align__(16) BwdSmem {
  // Three buffers of one item each (two [64][128] bf16 tiles, row-major).
  uint16_t t[3][2][C * ROWKV];
  uint16_t rt[DV * ROWST];  // bf16 copy of R, n-major: rt[n][i]
};

template <bool OUT_F32>
__device__ __forceinline__ void store_row4(void* base, int64_t off, floatx4 x) {
  if (OUT_F32)
    *reinterpret_cast<floatx4*>(static_cast<float*>(base) + off) = x;
  else
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(base) + off) = to_bf16x4(x);
}

// Two row-major [64][128] bf16 tiles of one block (a K/V or a Q/dO pair):
// thread tid moves rows tid/16 + 32i (i < 2), 16-byte chunk tid%16.  `rows`
// (1..64) is the number of the block's tokens before N; rows past it re-read
// the last valid row (every load is issued on every path, so the compiler
// counts the loads in flight exactly) and are stored to LDS as zeros.
struct PairRegs8 {
  u32x4 a[2], b[2];
};

__device__ __forceinline__ void load_pair8(PairRegs8& r, const uint16_t* ab, const uint16_t* bb, int rows, int tid) {
  const int c = tid & 15;
  for (int i = 0; i < 2; ++i) {
    int row = (tid >> 4) + 32 * i;
    row = row < rows ? row : rows - 1;
    r.a[i] = ld_stream_v(ab + row * D + 8 * c);
    r.b[i] = ld_stream_v(bb + row * DV + 8 * c);
  }
}

__device__ __forceinline__ void store_pair8(const PairRegs8& r, uint16_t* as, uint16_t* bs, int rows, int tid) {
  const int c = tid & 15;
  if (rows == C) {
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 4) + 32 * i;
      *reinterpret_cast<u32x4*>(as + row * ROWKV + 8 * c) = r.a[i];
      *reinterpret_cast<u32x4*>(bs + row * ROWKV + 8 * c) = r.b[i];
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 4) + 32 * i;
      *reinterpret_cast<u32x4*>(as + row * ROWKV + 8 * c) = row < rows ? r.a[i] : z;
      *reinterpret_cast<u32x4*>(bs + row * ROWKV + 8 * c) = row < rows ? r.b[i] : z;
    }
  }
}

// Diagonal X^T / Y^T tile (entry i of lane (l16, grp): token 4grp + i, key
// l16 within the tile): keep token >= key.
__device__ __forceinline__ floatx4 causal_mask_t(floatx4 x, int l16, int grp) {
  for (int i = 0; i < 4; ++i)
    if (4 * grp + i < l16) x[i] = 0.0f;
  return x;
}

// Operand with a straight contraction order from a row-major [k][col] LDS
// tile: lane (l16, grp) gets column col0 + l16 at rows k0 + 8grp + {0..7}
// (the order of a plain 16-byte row load of the transposed tile).
__device__ __forceinline__ bf16x8 tr_operand_lin(const uint16_t* tile, int k0, int col0, int l16, int grp,
                                                 int pitch) {
  const int r = k0 + 8 * grp + (l16 >> 2);
  const int c = col0 + 4 * (l16 & 3);
  const bf16x4 lo = ld_lds_tr(tile + r * pitch + c);
  const bf16x4 hi = ld_lds_tr(tile + (r + 4) * pitch + c);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  void* dk;
  void* dvg;
  const float* rstarts;
  float* ds_in;
  int Hq, Hkv;
  int64_t N, nblocks, blocks_per_seg;
  int P;
};

// Tile m (0..15) of the part of R held by state wave (SIDE, PAIR): its row
// and column tile.  SIDE 0 takes row tiles 2 PAIR, 2 PAIR + 1 (all columns),
// updated with Q^T of those rows and dO^T of every column; SIDE 1 row tiles
// 4..7 of column tiles 4 PAIR .. 4 PAIR + 3.
template <int SIDE, int PAIR>
__device__ constexpr int r_row(int m) { return SIDE == 0 ? 2 * PAIR + m / 8 : 4 + m / 4; }
template <int SIDE, int PAIR>
__device__ constexpr int r_col(int m) { return SIDE == 0 ? m % 8 : 4 * PAIR + m % 4; }

// The whole reverse walk of one wave.  Gradient wave (STATE false): SIDE 0
// holds dV of key tiles PAIR and 3 - PAIR (scores X^T = Q K^T, contraction
// operands dO^T), SIDE 1 dK of the same keys (Y^T = dO V^T, operands Q^T).
// State wave (STATE true): tiles r_row/r_col<SIDE, PAIR> of R.  Every wave
// runs the same sequence of barriers.
template <bool OUT_F32, int SIDE, int PAIR, bool STATE, int NS>
__device__ __forceinline__ void bwd_kv_wave(const BwdArgs& A, BwdSmem& sm) {
  constexpr int KA = PAIR, KB = 3 - PAIR;  // key tiles (KA < 2 <= KB)
  const int tid = threadIdx.x;
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % A.P;
  const int bg = blockIdx.x / A.P;
  const int b = bg / A.Hkv, g = bg % A.Hkv;
  const int G = A.Hq / A.Hkv;
  const int64_t N = A.N;
  const int64_t blk0 = int64_t(seg) * A.blocks_per_seg;
  const int64_t blk1 = blk0 + A.blocks_per_seg < A.nblocks ? blk0 + A.blocks_per_seg : A.nblocks;

  const uint16_t* kh = A.k + int64_t(bg) * N * D;
  const uint16_t* vh = A.v + int64_t(bg) * N * DV;
  const uint16_t* qg = A.q + (int64_t(b) * A.Hq + int64_t(g) * G) * N * D;
  const uint16_t* og = A.dout + (int64_t(b) * A.Hq + int64_t(g) * G) * N * DV;

  // state wave: R tile m holds rows 16 r_row(m) + 4grp + i, column 16 r_col(m) + l16
  constexpr int NR = STATE ? 16 : 1;
  floatx4 racc[NR];
  auto write_rt = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NR; ++m)
      *reinterpret_cast<bf16x4*>(
          &sm.rt[(16 * r_col<SIDE, PAIR>(m) + l16) * ROWST + 16 * r_row<SIDE, PAIR>(m) + 4 * grp]) =
          to_bf16x4(racc[m]);
  };
  if constexpr (STATE) {
    const float* r0 = A.rstarts ? A.rstarts + (int64_t(bg) * A.P + seg) * DD : nullptr;
#pragma unroll
    for (int m = 0; m < NR; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        racc[m][i] = r0 ? r0[(16 * r_row<SIDE, PAIR>(m) + 4 * grp + i) * DV + 16 * r_col<SIDE, PAIR>(m) + l16] : 0.0f;
    write_rt();
  }

  const int per_blk = G + 1;
  int64_t ld_blk = blk1 - 1;
  int ld_r = 0;
  auto load_next = [&](PairRegs8& r) __attribute__((always_inline)) {
    const int rows = int(N - ld_blk * C < C ? N - ld_blk * C : C);
    const uint16_t* a = ld_r == 0 ? kh : qg + int64_t(ld_r - 1) * N * D;
    const uint16_t* bb = ld_r == 0 ? vh : og + int64_t(ld_r - 1) * N * DV;
    load_pair8(r, a + ld_blk * C * D, bb + ld_blk * C * DV, rows, tid);
    if (ld_blk > blk0 || ld_r < G) {
      if (++ld_r == per_blk) {
        ld_r = 0;
        --ld_blk;
      }
    }
  };

  const int64_t nitems = (blk1 - blk0) * per_blk;
  PairRegs8 slot[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (i < nitems) load_next(slot[i]);

  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  // gradient wave: acc[0][t] / acc[1][t] = dV^T (SIDE 0) or dK^T (SIDE 1) of
  // key tile KA / KB, rows 16t + 4grp + i, column 16 key + l16
  constexpr int NA = STATE ? 1 : 8;
  floatx4 acc[2][NA];
  int64_t blk = blk1 - 1;
  int r_in = 0;
  // Buffer of the current block's K/V and of the last query-head item.  Each
  // item goes to the third buffer: the other two may still be read by waves
  // that have not finished the previous item, and every earlier reader of the
  // third one has passed the previous item's barrier.
  int kvb = 0, hlast = 1;

  auto step = [&](PairRegs8& cur) __attribute__((always_inline)) {
    const int rows = int(N - blk * C < C ? N - blk * C : C);
    const int nb = 3 - kvb - hlast;
    store_pair8(cur, sm.t[nb][0], sm.t[nb][1], rows, tid);
    __syncthreads();  // the item is in LDS
    load_next(cur);
    if (r_in == 0) {
      kvb = nb;
      if constexpr (!STATE) {
        // inter terms from the bf16 copy of R (the state after the later blocks)
        const uint16_t* kv = sm.t[nb][SIDE] + l16 * ROWKV + 8 * grp;  // K rows (SIDE 0) or V rows
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 ba = ld_lds16(kv + 16 * KA * ROWKV + 32 * kk);
          const bf16x8 bb = ld_lds16(kv + 16 * KB * ROWKV + 32 * kk);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const bf16x8 r = SIDE == 0 ? ld_lds16(sm.rt + (16 * t + l16) * ROWST + 32 * kk + 8 * grp)
                                       : tr_operand_lin(sm.rt, 32 * kk, 16 * t, l16, grp, ROWST);
            acc[0][t] = mfma(r, ba, kk ? acc[0][t] : z4);
            acc[1][t] = mfma(r, bb, kk ? acc[1][t] : z4);
          }
        }
      }
      r_in = 1;
      return;
    }
    const int h = r_in - 1;
    hlast = nb;
    const uint16_t* sq = sm.t[nb][0];
    const uint16_t* so = sm.t[nb][1];

    if constexpr (STATE) {
      // R[i][n] += sum_t Q[t][i] dO[t][n] on this SIMD's 16 tiles
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if constexpr (SIDE == 0) {
          bf16x8 qa[2];  // Q^T of row tiles 2 PAIR, 2 PAIR + 1
#pragma unroll
          for (int m = 0; m < 2; ++m) qa[m] = tr_operand(sq, p, 16 * (2 * PAIR + m), l16, grp);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const bf16x8 ot = tr_operand(so, p, 16 * t, l16, grp);
#pragma unroll
            for (int m = 0; m < 2; ++m) racc[8 * m + t] = mfma(qa[m], ot, racc[8 * m + t]);
          }
        } else {
          bf16x8 ob[4];  // dO^T of column tiles 4 PAIR .. 4 PAIR + 3
#pragma unroll
          for (int c = 0; c < 4; ++c) ob[c] = tr_operand(so, p, 16 * (4 * PAIR + c), l16, grp);
#pragma unroll
          for (int t = 4; t < 8; ++t) {
            const bf16x8 qt = tr_operand(sq, p, 16 * t, l16, grp);
#pragma unroll
            for (int c = 0; c < 4; ++c) racc[4 * (t - 4) + c] = mfma(qt, ob[c], racc[4 * (t - 4) + c]);
          }
        }
      }
      if (h == G - 1) {
        write_rt();
        r_in = 0;
        --blk;
      } else {
        ++r_in;
      }
      return;
    } else {
      const uint16_t* srow = sm.t[nb][SIDE];      // score rows: Q (SIDE 0) or dO
      const uint16_t* scol = sm.t[nb][1 - SIDE];  // contraction operands: dO (SIDE 0) or Q
      const uint16_t* kv = sm.t[kvb][SIDE] + l16 * ROWKV + 8 * grp;
      // all score tiles of the head first (independent product chains):
      // sc[ti] of key tile KA for query tiles ti = KA..3, sb[u] of KB for
      // query tiles 2 + u; entry i of a tile holds t = 16ti + 4grp + i, key l16
      floatx4 sc[4] = {z4, z4, z4, z4}, sb[2] = {z4, z4};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const bf16x8 ba = ld_lds16(kv + 16 * KA * ROWKV + 32 * ds);
        const bf16x8 bb = ld_lds16(kv + 16 * KB * ROWKV + 32 * ds);
#pragma unroll
        for (int ti = KA; ti < 4; ++ti) {
          const bf16x8 a = ld_lds16(srow + (16 * ti + l16) * ROWKV + 32 * ds + 8 * grp);
          sc[ti] = mfma(a, ba, sc[ti]);
          if (ti >= KB) sb[ti - 2] = mfma(a, bb, sb[ti - 2]);
        }
      }
      sc[KA] = causal_mask_t(sc[KA], l16, grp);
      sb[KB - 2] = causal_mask_t(sb[KB - 2], l16, grp);
      const bf16x8 pa[2] = {pack_tiles(sc[0], sc[1]), pack_tiles(sc[2], sc[3])};
      const bf16x8 pb = pack_tiles(sb[0], sb[1]);
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 ct = tr_operand(scol, p, 16 * t, l16, grp);
          acc[0][t] = mfma(ct, pa[p], acc[0][t]);
          if (p == 1) acc[1][t] = mfma(ct, pb, acc[1][t]);
        }
      if (h == G - 1) {
        void* out = SIDE == 0 ? A.dvg : A.dk;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int64_t s = blk * C + 16 * (e ? KB : KA) + l16;
          if (s < N) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
              store_row4<OUT_F32>(out, (int64_t(bg) * N + s) * DV + 16 * t + 4 * grp, acc[e][t]);
          }
        }
        r_in = 0;
        --blk;
      } else {
        ++r_in;
      }
    }
  };

  int64_t n = 0;
  for (; n + NS <= nitems; n += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) step(slot[i]);
  }
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (n + i < nitems) step(slot[i]);

  if constexpr (STATE) {
    if (A.ds_in != nullptr && seg == 0) {
      float* so = A.ds_in + int64_t(bg) * DD;
#pragma unroll
      for (int m = 0; m < NR; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          so[(16 * r_row<SIDE, PAIR>(m) + 4 * grp + i) * DV + 16 * r_col<SIDE, PAIR>(m) + l16] = racc[m][i];
    }
  }
}

template <bool OUT_F32, int NS>
__global__ __launch_bounds__(kThreads, 1) void bwd_kv_kernel(BwdArgs args) {
  __shared__ BwdSmem sm;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (w) {
    case 0: bwd_kv_wave<OUT_F32, 0, 0, false, NS>(args, sm); break;
    case 1: bwd_kv_wave<OUT_F32, 0, 1, false, NS>(args, sm); break;
    case 2: bwd_kv_wave<OUT_F32, 1, 0, false, NS>(args, sm); break;
    case 3: bwd_kv_wave<OUT_F32, 1, 1, false, NS>(args, sm); break;
    case 4: bwd_kv_wave<OUT_F32, 0, 0, true, NS>(args, sm); break;
    case 5: bwd_kv_wave<OUT_F32, 0, 1, true, NS>(args, sm); break;
    case 6: bwd_kv_wave<OUT_F32, 1, 0, true, NS>(args, sm); break;
    default: bwd_kv_wave<OUT_F32, 1, 1, true, NS>(args, sm); break;
  }
}

// ---------------------------------------------------------------------------
// Head size 64 (d = dv = 64), column-split form, used for one query head per
// KV head: four waves, one per SIMD.  Wave w owns columns [16w, 16w+16) of
// dV, dK and R and computes both score tiles of key tile w for all four query
// tiles, X^T = Q K^T and Y^T = dO V^T, published in LDS as bf16 operand packs
// that every wave reads for its columns (three barriers per query head).  The
// K/V pair and each head's (Q, dO) pair form one stream of 16 KiB items over
// two register slots; the K/V item is stored without a barrier of its own,
// its inter products run with the block's first head.  LDS: four 64 x 64
// tiles (160-byte rows), the bf16 copy of R and the packs = 65 KiB, so two
// workgroups share a compute unit (the host plans two segments per unit at
// this head size).
// ---------------------------------------------------------------------------
constexpr int H64 = 64;
constexpr int ROW64 = H64 + 16;  // LDS row pitch of the 64-wide tiles (elements)
constexpr int RST64 = H64 + 8;   // LDS row pitch of the bf16 copy of R
constexpr int DD64 = H64 * H64;

struct __align__(16) BwdSmem64 {
  uint16_t k[C * ROW64];    // K_b   [s][d]
  uint16_t v[C * ROW64];    // V_b   [s][n]
  uint16_t q[C * ROW64];    // Q_hb  [t][d]
  uint16_t o[C * ROW64];    // dO_hb [t][n]
  uint16_t rt[H64 * RST64]; // bf16 copy of R, n-major: rt[n][i]
  bf16x8 xb[2][8][64];      // X^T / Y^T operand packs: [X or Y][4p + s-tile][lane]
};

// Two row-major [64][64] bf16 tiles of one block moved by 256 threads: rows
// tid/8 + 32i (i < 2), 16-byte chunk tid%8; rows past `rows` re-read the last
// valid row and are stored to LDS as zeros.
struct PairRegs64 {
  u32x4 a[2], b[2];
};

__device__ __forceinline__ void load_pair64(PairRegs64& r, const uint16_t* ab, const uint16_t* bb, int rows, int tid) {
  const int c = tid & 7;
  for (int i = 0; i < 2; ++i) {
    int row = (tid >> 3) + 32 * i;
    row = row < rows ? row : rows - 1;
    r.a[i] = ld_stream_v(ab + row * H64 + 8 * c);
    r.b[i] = ld_stream_v(bb + row * H64 + 8 * c);
  }
}

__device__ __forceinline__ void store_pair64(const PairRegs64& r, uint16_t* as, uint16_t* bs, int rows, int tid) {
  const int c = tid & 7;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4*>(as + row * ROW64 + 8 * c) = row < rows ? r.a[i] : z;
    *reinterpret_cast<u32x4*>(bs + row * ROW64 + 8 * c) = row < rows ? r.b[i] : z;
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel_hd64(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, void* __restrict__ dk, void* __restrict__ dvg,
    const float* __restrict__ rstarts, float* __restrict__ ds_in, int Hq, int Hkv, int64_t N, int64_t nblocks,
    int64_t blocks_per_seg, int P) {
  __shared__ BwdSmem64 sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..3, uniform
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int bg = blockIdx.x / P;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;

  const uint16_t* kh = k + int64_t(bg) * N * H64;
  const uint16_t* vh = v + int64_t(bg) * N * H64;
  const uint16_t* qg = q + (int64_t(b) * Hq + int64_t(g) * G) * N * H64;
  const uint16_t* og = dout + (int64_t(b) * Hq + int64_t(g) * G) * N * H64;

  // R columns [16w, 16w+16): tile it holds rows 16it + 4grp + i, column 16w + l16
  const float* r0 = rstarts ? rstarts + (int64_t(bg) * P + seg) * DD64 : nullptr;
  floatx4 racc[4];
  for (int it = 0; it < 4; ++it)
    for (int i = 0; i < 4; ++i) racc[it][i] = r0 ? r0[(16 * it + 4 * grp + i) * H64 + 16 * w + l16] : 0.0f;
  for (int it = 0; it < 4; ++it)
    *reinterpret_cast<bf16x4*>(&sm.rt[(16 * w + l16) * RST64 + 16 * it + 4 * grp]) = to_bf16x4(racc[it]);

  const int per_blk = G + 1;
  int64_t ld_blk = blk1 - 1;
  int ld_r = 0;
  auto load_next = [&](PairRegs64& r) __attribute__((always_inline)) {
    const int rows = int(N - ld_blk * C < C ? N - ld_blk * C : C);
    const uint16_t* a = ld_r == 0 ? kh : qg + int64_t(ld_r - 1) * N * H64;
    const uint16_t* bb = ld_r == 0 ? vh : og + int64_t(ld_r - 1) * N * H64;
    load_pair64(r, a + ld_blk * C * H64, bb + ld_blk * C * H64, rows, tid);
    if (ld_blk > blk0 || ld_r < G) {
      if (++ld_r == per_blk) {
        ld_r = 0;
        --ld_blk;
      }
    }
  };

  const int64_t nitems = (blk1 - blk0) * per_blk;
  PairRegs64 s0, s1;
  if (nitems > 0) {
    load_next(s0);
    load_next(s1);
  }

  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 adv[4], adk[4];  // dV^T / dK^T tiles of columns 16w.. for s-tiles 0..3
  int64_t blk = blk1 - 1;
  int r_in = 0;

  auto step = [&](PairRegs64& cur) __attribute__((always_inline)) {
    const int rows = int(N - blk * C < C ? N - blk * C : C);
    if (r_in == 0) {
      store_pair64(cur, sm.k, sm.v, rows, tid);
      load_next(cur);
      for (int si = 0; si < 4; ++si) {
        adv[si] = z4;
        adk[si] = z4;
      }
      r_in = 1;
      return;
    }
    const int h = r_in - 1;
    store_pair64(cur, sm.q, sm.o, rows, tid);
    __syncthreads();  // K/V, this head's Q/dO and the R copy are in LDS
    load_next(cur);

    if (h == 0) {
      // inter: dV^T[n][s] += sum_i R[i][n] K[s][i];  dK^T[i][s] += sum_n R[i][n] V[s][n]
      for (int p = 0; p < 2; ++p) {
        const bf16x8 ra = ld_lds16(sm.rt + (16 * w + l16) * RST64 + 32 * p + 8 * grp);
        const bf16x8 rb = tr_operand(sm.rt, p, 16 * w, l16, grp, 4, RST64);
        for (int si = 0; si < 4; ++si) {
          const uint16_t* krow = sm.k + (16 * si + l16) * ROW64;
          const uint16_t* vrow = sm.v + (16 * si + l16) * ROW64;
          const bf16x8 bk = ld_lds16(krow + 32 * p + 8 * grp);
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 4 * grp);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 16 + 4 * grp);
          const bf16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          adv[si] = mfma(ra, bk, adv[si]);
          adk[si] = mfma(rb, bv, adk[si]);
        }
      }
    }

    // scores of key tile w for all four query tiles: X^T = Q K^T and Y^T = dO V^T
    {
      const uint16_t* krow = sm.k + (16 * w + l16) * ROW64;
      const uint16_t* vrow = sm.v + (16 * w + l16) * ROW64;
      floatx4 xt[4], yt[4];
      for (int ti = 0; ti < 4; ++ti) {
        xt[ti] = z4;
        yt[ti] = z4;
      }
      for (int ds = 0; ds < 2; ++ds) {
        const bf16x8 bk = ld_lds16(krow + 32 * ds + 8 * grp);
        const bf16x8 bv = ld_lds16(vrow + 32 * ds + 8 * grp);
        for (int ti = 0; ti < 4; ++ti) {
          xt[ti] = mfma(ld_lds16(sm.q + (16 * ti + l16) * ROW64 + 32 * ds + 8 * grp), bk, xt[ti]);
          yt[ti] = mfma(ld_lds16(sm.o + (16 * ti + l16) * ROW64 + 32 * ds + 8 * grp), bv, yt[ti]);
        }
      }
      // entry i of tile ti: t = 16ti + 4grp + i, s = 16w + l16; keep t >= s
      const int lim = 16 * w + l16 - 4 * grp;
      for (int ti = 0; ti < 4; ++ti)
        for (int i = 0; i < 4; ++i)
          if (16 * ti + i < lim) {
            xt[ti][i] = 0.0f;
            yt[ti][i] = 0.0f;
          }
      for (int p = 0; p < 2; ++p) {
        sm.xb[0][4 * p + w][lane] = pack_tiles(xt[2 * p], xt[2 * p + 1]);
        sm.xb[1][4 * p + w][lane] = pack_tiles(yt[2 * p], yt[2 * p + 1]);
      }
    }
    __syncthreads();  // every wave's score packs are in LDS

    // intra (dV, dK columns 16w..) and the state update (R columns 16w..)
    for (int p = 0; p < 2; ++p) {
      const bf16x8 ao = tr_operand(sm.o, p, 16 * w, l16, grp, 4, ROW64);
      const bf16x8 aq = tr_operand(sm.q, p, 16 * w, l16, grp, 4, ROW64);
      for (int si = 0; si < 4; ++si) {
        if (p == 0 && si >= 2) continue;  // tokens 0..31 are all before key tiles 2, 3
        adv[si] = mfma(ao, sm.xb[0][4 * p + si][lane], adv[si]);
        adk[si] = mfma(aq, sm.xb[1][4 * p + si][lane], adk[si]);
      }
      for (int it = 0; it < 4; ++it) racc[it] = mfma(tr_operand(sm.q, p, 16 * it, l16, grp, 4, ROW64), ao, racc[it]);
    }
    __syncthreads();  // Q/dO and the packs may be overwritten

    if (h == G - 1) {
      // dV, dK rows of the block: tile si holds columns 16w + 4grp + {0..3} of row 16si + l16
      for (int si = 0; si < 4; ++si) {
        const int64_t s = blk * C + 16 * si + l16;
        if (s < N) {
          const int64_t off = (int64_t(bg) * N + s) * H64 + 16 * w + 4 * grp;
          store_row4<OUT_F32>(dvg, off, adv[si]);
          store_row4<OUT_F32>(dk, off, adk[si]);
        }
      }
      for (int it = 0; it < 4; ++it)
        *reinterpret_cast<bf16x4*>(&sm.rt[(16 * w + l16) * RST64 + 16 * it + 4 * grp]) = to_bf16x4(racc[it]);
      r_in = 0;
      --blk;
    } else {
      ++r_in;
    }
  };

  for (int64_t n = 0; n < nitems; n += 2) {
    step(s0);
    if (n + 1 < nitems) step(s1);
  }

  if (ds_in != nullptr && seg == 0) {
    float* so = ds_in + int64_t(bg) * DD64;
    for (int it = 0; it < 4; ++it)
      for (int i = 0; i < 4; ++i) so[(16 * it + 4 * grp + i) * H64 + 16 * w + l16] = racc[it][i];
  }
}

// ---------------------------------------------------------------------------
// Head size 64, split like the head-size-128 kernel's gradient waves: four
// waves, each owning one kind of gradient for two key tiles of the block
// (waves 0 and 1: dV^T of key tiles {0, 3} and {1, 2}; waves 2 and 3: dK^T of
// the same pairs), computing the score tiles of its own keys in registers.
// At this head size R (64 x 64, float32) is small enough to live in the same
// waves: 4 tiles each (the dV waves row tile PAIR, all columns; the dK waves
// row tiles 2..3 of column tiles 2 PAIR, 2 PAIR + 1), updated with the
// operands of their intra products.  Every wave does 34 matrix products per
// query head.  Items (16 KiB) pass through two register slots and three LDS
// buffers (one barrier per item); LDS 69 KiB, so two workgroups share a
// compute unit (the host plans two segments per unit at this head size).
// ---------------------------------------------------------------------------
struct __align__(16) BwdSmemH64 {
  uint16_t t[3][2][C * ROW64];  // three item buffers of two [64][64] tiles
  uint16_t rt[H64 * RST64];     // bf16 copy of R, n-major
};

template <int SIDE, int PAIR>
__device__ constexpr int r_row64(int m) { return SIDE == 0 ? PAIR : 2 + m / 2; }
template <int SIDE, int PAIR>
__device__ constexpr int r_col64(int m) { return SIDE == 0 ? m : 2 * PAIR + m % 2; }

template <bool OUT_F32, int SIDE, int PAIR, int NS>
__device__ __forceinline__ void bwd_kv_wave64(const BwdArgs& A, BwdSmemH64& sm) {
  constexpr int KA = PAIR, KB = 3 - PAIR;  // key tiles (KA < 2 <= KB)
  const int tid = threadIdx.x;
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % A.P;
  const int bg = blockIdx.x / A.P;
  const int b = bg / A.Hkv, g = bg % A.Hkv;
  const int G = A.Hq / A.Hkv;
  const int64_t N = A.N;
  const int64_t blk0 = int64_t(seg) * A.blocks_per_seg;
  const int64_t blk1 = blk0 + A.blocks_per_seg < A.nblocks ? blk0 + A.blocks_per_seg : A.nblocks;

  const uint16_t* kh = A.k + int64_t(bg) * N * H64;
  const uint16_t* vh = A.v + int64_t(bg) * N * H64;
  const uint16_t* qg = A.q + (int64_t(b) * A.Hq + int64_t(g) * G) * N * H64;
  const uint16_t* og = A.dout + (int64_t(b) * A.Hq + int64_t(g) * G) * N * H64;

  // R tile m: rows 16 r_row64(m) + 4grp + i, column 16 r_col64(m) + l16
  const float* r0 = A.rstarts ? A.rstarts + (int64_t(bg) * A.P + seg) * DD64 : nullptr;
  floatx4 racc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      racc[m][i] = r0 ? r0[(16 * r_row64<SIDE, PAIR>(m) + 4 * grp + i) * H64 + 16 * r_col64<SIDE, PAIR>(m) + l16]
                      : 0.0f;
  auto write_rt = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<bf16x4*>(
          &sm.rt[(16 * r_col64<SIDE, PAIR>(m) + l16) * RST64 + 16 * r_row64<SIDE, PAIR>(m) + 4 * grp]) =
          to_bf16x4(racc[m]);
  };
  write_rt();

  const int per_blk = G + 1;
  int64_t ld_blk = blk1 - 1;
  int ld_r = 0;
  auto load_next = [&](PairRegs64& r) __attribute__((always_inline)) {
    const int rows = int(N - ld_blk * C < C ? N - ld_blk * C : C);
    const uint16_t* a = ld_r == 0 ? kh : qg + int64_t(ld_r - 1) * N * H64;
    const uint16_t* bb = ld_r == 0 ? vh : og + int64_t(ld_r - 1) * N * H64;
    load_pair64(r, a + ld_blk * C * H64, bb + ld_blk * C * H64, rows, tid);
    if (ld_blk > blk0 || ld_r < G) {
      if (++ld_r == per_blk) {
        ld_r = 0;
        --ld_blk;
      }
    }
  };

  const int64_t nitems = (blk1 - blk0) * per_blk;
  PairRegs64 slot[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (i < nitems) load_next(slot[i]);

  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  // acc[0][t] / acc[1][t]: dV^T (SIDE 0) or dK^T (SIDE 1) of key tile KA / KB,
  // rows 16t + 4grp + i (column of dV or dK), column 16 key + l16 (key)
  floatx4 acc[2][4];
  int64_t blk = blk1 - 1;
  int r_in = 0;
  int kvb = 0, hlast = 1;  // as in bwd_kv_wave: each item goes to the third buffer

  auto step = [&](PairRegs64& cur) __attribute__((always_inline)) {
    const int rows = int(N - blk * C < C ? N - blk * C : C);
    const int nb = 3 - kvb - hlast;
    store_pair64(cur, sm.t[nb][0], sm.t[nb][1], rows, tid);
    __syncthreads();  // the item is in LDS
    load_next(cur);
    if (r_in == 0) {
      // a block's K/V: start the gradients with the inter terms from the bf16
      // copy of R (the state after the later blocks)
      kvb = nb;
      const uint16_t* kv = sm.t[nb][SIDE] + l16 * ROW64 + 8 * grp;  // K rows (SIDE 0) or V rows
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 ba = ld_lds16(kv + 16 * KA * ROW64 + 32 * kk);
        const bf16x8 bb = ld_lds16(kv + 16 * KB * ROW64 + 32 * kk);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 r = SIDE == 0 ? ld_lds16(sm.rt + (16 * t + l16) * RST64 + 32 * kk + 8 * grp)
                                     : tr_operand_lin(sm.rt, 32 * kk, 16 * t, l16, grp, RST64);
          acc[0][t] = mfma(r, ba, kk ? acc[0][t] : z4);
          acc[1][t] = mfma(r, bb, kk ? acc[1][t] : z4);
        }
      }
      r_in = 1;
      return;
    }
    const int h = r_in - 1;
    hlast = nb;
    const uint16_t* srow = sm.t[nb][SIDE];      // score rows: Q (SIDE 0) or dO
    const uint16_t* scol = sm.t[nb][1 - SIDE];  // contraction operands: dO (SIDE 0) or Q
    const uint16_t* kv = sm.t[kvb][SIDE] + l16 * ROW64 + 8 * grp;

    // all score tiles of the head: sc[ti] of key tile KA for query tiles
    // ti = KA..3, sb[u] of KB for query tiles 2 + u; entry i of a tile holds
    // t = 16ti + 4grp + i, key l16
    floatx4 sc[4] = {z4, z4, z4, z4}, sb[2] = {z4, z4};
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      const bf16x8 ba = ld_lds16(kv + 16 * KA * ROW64 + 32 * ds);
      const bf16x8 bb = ld_lds16(kv + 16 * KB * ROW64 + 32 * ds);
#pragma unroll
      for (int ti = KA; ti < 4; ++ti) {
        const bf16x8 a = ld_lds16(srow + (16 * ti + l16) * ROW64 + 32 * ds + 8 * grp);
        sc[ti] = mfma(a, ba, sc[ti]);
        if (ti >= KB) sb[ti - 2] = mfma(a, bb, sb[ti - 2]);
      }
    }
    sc[KA] = causal_mask_t(sc[KA], l16, grp);
    sb[KB - 2] = causal_mask_t(sb[KB - 2], l16, grp);
    const bf16x8 pa[2] = {pack_tiles(sc[0], sc[1]), pack_tiles(sc[2], sc[3])};
    const bf16x8 pb = pack_tiles(sb[0], sb[1]);
    // intra:  dV^T[n][s] += sum_t dO[t][n] X^T[t][s]  (SIDE 0)
    //         dK^T[i][s] += sum_t Q[t][i] Y^T[t][s]   (SIDE 1)
    // and R[i][n] += sum_t Q[t][i] dO[t][n] on this wave's tiles of R
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if constexpr (SIDE == 0) {
        const bf16x8 qa = tr_operand(srow, p, 16 * PAIR, l16, grp, 4, ROW64);  // Q^T, row tile PAIR
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 ot = tr_operand(scol, p, 16 * t, l16, grp, 4, ROW64);  // dO^T, column tile t
          acc[0][t] = mfma(ot, pa[p], acc[0][t]);
          if (p == 1) acc[1][t] = mfma(ot, pb, acc[1][t]);
          racc[t] = mfma(qa, ot, racc[t]);
        }
      } else {
        bf16x8 ob[2];  // dO^T of column tiles 2 PAIR, 2 PAIR + 1
#pragma unroll
        for (int c = 0; c < 2; ++c) ob[c] = tr_operand(srow, p, 16 * (2 * PAIR + c), l16, grp, 4, ROW64);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 qt = tr_operand(scol, p, 16 * t, l16, grp, 4, ROW64);  // Q^T, row tile t
          acc[0][t] = mfma(qt, pa[p], acc[0][t]);
          if (p == 1) acc[1][t] = mfma(qt, pb, acc[1][t]);
          if (t >= 2)
#pragma unroll
            for (int c = 0; c < 2; ++c) racc[2 * (t - 2) + c] = mfma(qt, ob[c], racc[2 * (t - 2) + c]);
        }
      }
    }

    if (h == G - 1) {
      // gradient rows of the block: tile t holds columns 16t + 4grp + {0..3} of a key
      void* out = SIDE == 0 ? A.dvg : A.dk;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t s = blk * C + 16 * (e ? KB : KA) + l16;
        if (s < N) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            store_row4<OUT_F32>(out, (int64_t(bg) * N + s) * H64 + 16 * t + 4 * grp, acc[e][t]);
        }
      }
      write_rt();
      r_in = 0;
      --blk;
    } else {
      ++r_in;
    }
  };

  // whole rounds of NS items in the loop, the remainder after it (as in bwd_kv_wave)
  int64_t n = 0;
  for (; n + NS <= nitems; n += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) step(slot[i]);
  }
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (n + i < nitems) step(slot[i]);

  if (A.ds_in != nullptr && seg == 0) {
    float* so = A.ds_in + int64_t(bg) * DD64;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(16 * r_row64<SIDE, PAIR>(m) + 4 * grp + i) * H64 + 16 * r_col64<SIDE, PAIR>(m) + l16] = racc[m][i];
  }
}

template <bool OUT_F32, int NS>
__global__ __launch_bounds__(256, 2) void bwd_kv_kernel64(BwdArgs args) {
  __shared__ BwdSmemH64 sm;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 0) bwd_kv_wave64<OUT_F32, 0, 0, NS>(args, sm);
  else if (w == 1) bwd_kv_wave64<OUT_F32, 0, 1, NS>(args, sm);
  else if (w == 2) bwd_kv_wave64<OUT_F32, 1, 0, NS>(args, sm);
  else bwd_kv_wave64<OUT_F32, 1, 1, NS>(args, sm);
}

// rstarts[c][j] = ds_out[c] + sum over segments i > j and the G query heads of
// chain c of the pre-pass partials (partial index ((c G + h)(P - 1) + i - 1) R
// + r), in a fixed order (segments from the last, then heads, then parts); E
// elements per state (d dv, a multiple of 256).  The partials are independent
// loads, issued kRScanBatch at a time ahead of the additions.
constexpr int kRScanBatch = 16;

__global__ __launch_bounds__(256) void scan_rstarts(const float* __restrict__ partial, float* __restrict__ rstarts,
                                                    const float* ds_out, int G, int P, int R, int E) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t c = gid / E;
  const int e = int(gid % E);
  const int GR = G * R, n = (P - 1) * GR;  // partials of the chain, in summation order
  float* rc = rstarts + c * P * E + e;
  float run = ds_out ? ds_out[c * E + e] : 0.0f;
  rc[int64_t(P - 1) * E] = run;
  for (int b = 0; b < n; b += kRScanBatch) {
    float x[kRScanBatch];
#pragma unroll
    for (int i = 0; i < kRScanBatch; ++i) {
      // summation step s adds head h, part r of segment j = P - 1 - s / GR
      // (past the end: the last step again, so no load is conditional)
      const int s = b + i < n ? b + i : n - 1, j = P - 1 - s / GR, h = (s / R) % G, r = s % R;
      x[i] = partial[(((c * G + h) * (P - 1) + (j - 1)) * R + r) * E + e];
    }
#pragma unroll
    for (int i = 0; i < kRScanBatch; ++i) {
      const int s = b + i;
      if (s < n) {
        run += x[i];
        if ((s + 1) % GR == 0) rc[int64_t(P - 2 - s / GR) * E] = run;
      }
    }
  }
}

// out[c][n][i] = in[c][i][n] for n x n states (n = 64 or 128), through 32 x 32
// LDS tiles.  Workgroup (n/32)^2 c + t moves tile t of state c.
__global__ __launch_bounds__(256) void transpose_states(const float* __restrict__ in, float* __restrict__ out,
                                                        int n) {
  __shared__ float tile[32][33];
  const int T = n / 32;
  const int64_t c = blockIdx.x / (T * T);
  const int t = blockIdx.x % (T * T);
  const int bx = t % T, by = t / T;
  const int64_t nn = int64_t(n) * n;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int j = ty; j < 32; j += 8) tile[j][tx] = in[c * nn + (by * 32 + j) * n + bx * 32 + tx];
  __syncthreads();
  for (int j = ty; j < 32; j += 8) out[c * nn + (bx * 32 + j) * n + by * 32 + tx] = tile[tx][j];
}

}  // namespace

hipError_t launch_transpose_states(const float* in, float* out, int64_t count, int64_t n, hipStream_t stream) {
  if (n != 64 && n != 128) return hipErrorInvalidValue;
  const int64_t T = n / 32;
  hipLaunchKernelGGL(transpose_states, dim3(unsigned(T * T * count)), dim3(256), 0, stream, in, out, int(n));
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dvg,
                         bool out_f32, const float* ds_out, float* ds_in, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, const BwdPlan& plan, float* workspace_f, hipStream_t stream) {
  const int hd = plan.fwd.hd;
  if (hd != 128 && hd != 64) return hipErrorInvalidValue;
  const int E = hd * hd;
  float* partial = workspace_f;
  float* rstarts = partial + plan.partial_floats;
  const float* rs = ds_out;  // one segment: it starts from ds_out
  if (plan.P > 1) {
    // fused: the dQ pass has written one partial per (chain, query-head
    // subgroup, segment); else the pre-pass writes R per query head
    int scan_g = plan.fwd.subgroups;
    if (!plan.fused) {
      hipError_t e = launch_state_parts(q, dout, partial, B * Hq, N, plan.nblocks, plan.blocks_per_seg,
                                        plan.blocks_per_part, plan.P, plan.R, 1, hd, stream);
      if (e != hipSuccess) return e;
      scan_g = int(Hq / Hkv);
    }
    hipLaunchKernelGGL(scan_rstarts, dim3(unsigned(B * Hkv * E / 256)), dim3(256), 0, stream, partial, rstarts,
                       ds_out, scan_g, plan.P, plan.R, E);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    rs = rstarts;
  }
  const dim3 grid(unsigned(B * Hkv * plan.P));
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* o16 = static_cast<const uint16_t*>(dout);
  const BwdArgs args{q16, k16, v16, o16, dk, dvg, rs, ds_in, int(Hq), int(Hkv), N, plan.nblocks,
                     plan.blocks_per_seg, plan.P};
  if (hd == 64) {
    // one query head per KV head: the column-split kernel, which stores the
    // K/V item without a barrier and runs the inter products with the head
    // (measured 11.8 against 12.3 ms per 1M-token backward at 32 over 32
    // heads); groups of two or more: the key-tile-pair kernel (24.2 against
    // 25.8 ms at 128 over 32 heads)
    if (Hq == Hkv) {
      if (out_f32)
        hipLaunchKernelGGL(bwd_kv_kernel_hd64<true>, grid, dim3(256), 0, stream, q16, k16, v16, o16, dk, dvg, rs,
                           ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
      else
        hipLaunchKernelGGL(bwd_kv_kernel_hd64<false>, grid, dim3(256), 0, stream, q16, k16, v16, o16, dk, dvg, rs,
                           ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
    } else if (out_f32) {
      hipLaunchKernelGGL((bwd_kv_kernel64<true, kSlots>), grid, dim3(256), 0, stream, args);
    } else {
      hipLaunchKernelGGL((bwd_kv_kernel64<false, kSlots>), grid, dim3(256), 0, stream, args);
    }
    return hipGetLastError();
  }
  if (out_f32)
    hipLaunchKernelGGL((bwd_kv_kernel<true, kSlots>), grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<false, kSlots>), grid, dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace la
