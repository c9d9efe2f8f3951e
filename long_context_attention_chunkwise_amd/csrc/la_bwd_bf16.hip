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
// Design for MI355X: one workgroup of eight waves (two per SIMD, so one
// wave's LDS and memory waits overlap the other's products) per (batch, KV
// head, sequence segment); segment j starts from the sum over later segments,
// produced by the forward's pre-pass kernel run on (Q, dO) pairs and a
// reverse scan here.  Wave w owns columns [16w, 16w+16) of dV, dK and the
// state R; the fp32 state stays in VGPRs and is rounded to bf16 once per
// block into an n-major LDS copy for the inter terms.  Query heads are
// processed one at a time through LDS: the K/V pair and each head's (Q, dO)
// pair form one stream of 32 KiB items rotating over two register slots (two
// items in flight).  Products are v_mfma_f32_16x16x32_bf16 with the
// transposed-product layout of the forward kernel: wave w computes the score
// tiles X^T = Q K^T (w < 4) or Y^T = dO V^T (w >= 4) of key tile w % 4 for all
// four query tiles, masks t >= s arithmetically (no branch depends on the
// wave) and publishes them in LDS as bf16 B operands of the token-contracting
// products.
#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

using namespace mfma16;

constexpr int kThreads = 512;  // eight waves, two per SIMD
constexpr int kSlots = 2;      // 32 KiB tile pairs in flight per workgroup
constexpr int DD = D * DV;

__device__ __forceinline__ u32x4 ld_stream_v(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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

template <bool OUT_F32, int NS>
__global__ __launch_bounds__(kThreads, 1) void bwd_kv_kernel8(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, void* __restrict__ dk, void* __restrict__ dvg,
    const float* __restrict__ rstarts, float* __restrict__ ds_in, int Hq, int Hkv, int64_t N,
    int64_t nblocks, int64_t blocks_per_seg, int P) {
  static_assert(NS == 1 || NS == 2, "one or two slots");
  __shared__ BwdSmem sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, uniform
  const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int seg = blockIdx.x % P;
  const int bg = blockIdx.x / P;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int64_t blk0 = int64_t(seg) * blocks_per_seg;
  const int64_t blk1 = blk0 + blocks_per_seg < nblocks ? blk0 + blocks_per_seg : nblocks;

  const uint16_t* kh = k + int64_t(bg) * N * D;
  const uint16_t* vh = v + int64_t(bg) * N * DV;
  const uint16_t* qg = q + (int64_t(b) * Hq + int64_t(g) * G) * N * D;
  const uint16_t* og = dout + (int64_t(b) * Hq + int64_t(g) * G) * N * DV;

  // R columns [16w, 16w+16): tile it holds rows 16it + 4grp + i, column 16w + l16
  const float* r0 = rstarts ? rstarts + (int64_t(bg) * P + seg) * DD : nullptr;
  floatx4 racc[8];
  for (int it = 0; it < 8; ++it)
    for (int i = 0; i < 4; ++i) racc[it][i] = 0.0f;
  if (r0 != nullptr)
    for (int it = 0; it < 8; ++it)
      for (int i = 0; i < 4; ++i) racc[it][i] = r0[(16 * it + 4 * grp + i) * DV + 16 * w + l16];
  for (int it = 0; it < 8; ++it)
    *reinterpret_cast<bf16x4*>(&sm.rt[(16 * w + l16) * ROWST + 16 * it + 4 * grp]) = to_bf16x4(racc[it]);

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
  PairRegs8 s0, s1;
  if (nitems > 0) {
    load_next(s0);
    if constexpr (NS == 2) load_next(s1);
  }

  const floatx4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 adv[4], adk[4];  // dV^T / dK^T tiles of columns 16w.. for s-tiles 0..3
  int64_t blk = blk1 - 1;
  int r_in = 0;
  const bool is_y = w >= 4;   // uniform: this wave's score tiles are Y^T = dO V^T
  const int skey = w & 3;     // its key tile

  auto step = [&](PairRegs8& cur) __attribute__((always_inline)) {
    const int rows = int(N - blk * C < C ? N - blk * C : C);
    if (r_in == 0) {
      store_pair8(cur, sm.k, sm.v, rows, tid);
      load_next(cur);
      for (int si = 0; si < 4; ++si) {
        adv[si] = z4;
        adk[si] = z4;
      }
      r_in = 1;
      return;
    }
    const int h = r_in - 1;
    store_pair8(cur, sm.q, sm.o, rows, tid);
    __syncthreads();  // K/V, this head's Q/dO and the state copy are in LDS
    load_next(cur);

    if (h == 0) {
      // inter: dV^T[n][s] += sum_i R[i][n] K[s][i];  dK^T[i][s] += sum_n R[i][n] V[s][n]
      for (int p = 0; p < 4; ++p) {
        const bf16x8 ra = ld_lds16(sm.rt + (16 * w + l16) * ROWST + 32 * p + 8 * grp);
        const bf16x8 rb = tr_operand(sm.rt, p, 16 * w, l16, grp, 4, ROWST);
        for (int si = 0; si < 4; ++si) {
          const uint16_t* krow = sm.k + (16 * si + l16) * ROWKV;
          const uint16_t* vrow = sm.v + (16 * si + l16) * ROWKV;
          const bf16x8 bk = ld_lds16(krow + 32 * p + 8 * grp);
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 4 * grp);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 32 * p + 16 + 4 * grp);
          const bf16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          adv[si] = mfma(ra, bk, adv[si]);
          adk[si] = mfma(rb, bv, adk[si]);
        }
      }
    }

    // scores of key tile skey for all four query tiles: X^T = Q K^T or Y^T = dO V^T
    {
      const uint16_t* arows = is_y ? sm.o : sm.q;
      const uint16_t* brows = (is_y ? sm.v : sm.k) + (16 * skey + l16) * ROWKV;
      floatx4 xt[4];
      for (int ti = 0; ti < 4; ++ti) xt[ti] = z4;
      for (int ds = 0; ds < 4; ++ds) {
        const bf16x8 bop = ld_lds16(brows + 32 * ds + 8 * grp);
        for (int ti = 0; ti < 4; ++ti)
          xt[ti] = mfma(ld_lds16(arows + (16 * ti + l16) * ROWKV + 32 * ds + 8 * grp), bop, xt[ti]);
      }
      // entry i of tile ti: t = 16ti + 4grp + i, s = 16skey + l16; keep t >= s
      const int lim = 16 * skey + l16 - 4 * grp;
      for (int ti = 0; ti < 4; ++ti)
        for (int i = 0; i < 4; ++i)
          if (16 * ti + i < lim) xt[ti][i] = 0.0f;
      for (int p = 0; p < 2; ++p) sm.xb[is_y ? 1 : 0][4 * p + skey][lane] = pack_tiles(xt[2 * p], xt[2 * p + 1]);
    }
    __syncthreads();  // every wave's score packs are in LDS

    // intra (dV, dK columns 16w..) and the state update (R columns 16w..)
    for (int p = 0; p < 2; ++p) {
      const bf16x8 ao = tr_operand(sm.o, p, 16 * w, l16, grp);
      const bf16x8 aq = tr_operand(sm.q, p, 16 * w, l16, grp);
      for (int si = 0; si < 4; ++si) {
        if (p == 0 && si >= 2) continue;  // tokens 0..31 are all before key tiles 2, 3
        adv[si] = mfma(ao, sm.xb[0][4 * p + si][lane], adv[si]);
        adk[si] = mfma(aq, sm.xb[1][4 * p + si][lane], adk[si]);
      }
      for (int it = 0; it < 8; ++it) racc[it] = mfma(tr_operand(sm.q, p, 16 * it, l16, grp), ao, racc[it]);
    }
    __syncthreads();  // Q/dO and the packs may be overwritten

    if (h == G - 1) {
      // dV, dK rows of the block: tile si holds columns 16w + 4grp + {0..3} of row 16si + l16
      for (int si = 0; si < 4; ++si) {
        const int64_t s = blk * C + 16 * si + l16;
        if (s < N) {
          const int64_t off = (int64_t(bg) * N + s) * DV + 16 * w + 4 * grp;
          store_row4<OUT_F32>(dvg, off, adv[si]);
          store_row4<OUT_F32>(dk, off, adk[si]);
        }
      }
      for (int it = 0; it < 8; ++it)
        *reinterpret_cast<bf16x4*>(&sm.rt[(16 * w + l16) * ROWST + 16 * it + 4 * grp]) = to_bf16x4(racc[it]);
      r_in = 0;
      --blk;
    } else {
      ++r_in;
    }
  };

  for (int64_t n = 0; n < nitems; n += NS) {
    step(s0);
    if constexpr (NS == 2)
      if (n + 1 < nitems) step(s1);
  }

  if (ds_in != nullptr && seg == 0) {
    float* so = ds_in + int64_t(bg) * DD;
    for (int it = 0; it < 8; ++it)
      for (int i = 0; i < 4; ++i) so[(16 * it + 4 * grp + i) * DV + 16 * w + l16] = racc[it][i];
  }
}

// ---------------------------------------------------------------------------
// Head size 64 (d = dv = 64): the same reverse recurrence with four waves, one
// per SIMD.  Wave w owns columns [16w, 16w+16) of dV, dK and R and computes
// both score tiles of key tile w for all four query tiles, X^T = Q K^T and
// Y^T = dO V^T, published as the same bf16 operand packs.  The K/V pair and
// each head's (Q, dO) pair form one stream of 16 KiB items over two register
// slots; LDS: four 64 x 64 tiles (160-byte rows), the bf16 copy of R and the
// packs = 65 KiB, so two workgroups share a compute unit (the host plans two
// segments per unit at this head size).
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

// rstarts[c][j] = ds_out[c] + sum over segments i > j and the G query heads of
// chain c of the pre-pass partials (partial index ((c G + h)(P - 1) + i - 1) R
// + r), in a fixed order; E elements per state (d dv, a multiple of 256).
__global__ __launch_bounds__(256) void scan_rstarts(const float* __restrict__ partial, float* __restrict__ rstarts,
                                                    const float* ds_out, int G, int P, int R, int E) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t c = gid / E;
  const int e = int(gid % E);
  float run = ds_out ? ds_out[c * E + e] : 0.0f;
  for (int j = P - 1; j >= 0; --j) {
    rstarts[(c * P + j) * E + e] = run;
    if (j >= 1)
      for (int h = 0; h < G; ++h)
        for (int r = 0; r < R; ++r) run += partial[(((c * G + h) * (P - 1) + (j - 1)) * R + r) * E + e];
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
    hipError_t e = launch_state_parts(q, dout, partial, B * Hq, N, plan.nblocks, plan.blocks_per_seg,
                                      plan.blocks_per_part, plan.P, plan.R, 1, hd, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_rstarts, dim3(unsigned(B * Hkv * E / 256)), dim3(256), 0, stream, partial, rstarts,
                       ds_out, int(Hq / Hkv), plan.P, plan.R, E);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    rs = rstarts;
  }
  const dim3 grid(unsigned(B * Hkv * plan.P));
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* o16 = static_cast<const uint16_t*>(dout);
  if (hd == 64) {
    if (out_f32)
      hipLaunchKernelGGL(bwd_kv_kernel_hd64<true>, grid, dim3(256), 0, stream, q16, k16, v16, o16, dk, dvg, rs, ds_in,
                         int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
    else
      hipLaunchKernelGGL(bwd_kv_kernel_hd64<false>, grid, dim3(256), 0, stream, q16, k16, v16, o16, dk, dvg, rs,
                         ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
    return hipGetLastError();
  }
  if (out_f32)
    hipLaunchKernelGGL((bwd_kv_kernel8<true, kSlots>), grid, dim3(kThreads), 0, stream, q16, k16, v16, o16, dk, dvg,
                       rs, ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
  else
    hipLaunchKernelGGL((bwd_kv_kernel8<false, kSlots>), grid, dim3(kThreads), 0, stream, q16, k16, v16, o16, dk, dvg,
                       rs, ds_in, int(Hq), int(Hkv), N, plan.nblocks, plan.blocks_per_seg, plan.P);
  return hipGetLastError();
}

}  // namespace la
