// Host side of liblightning.so: argument validation, work planning and
// dispatch to the HIP kernels.  Every check runs before any HIP call, so a
// rejected call touches neither the device nor the stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "la_internal.h"

namespace {

constexpr int64_t kBf16Block = 64;  // tokens per block of the matrix-core path

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t esize(la_dtype t) { return t == LA_F32 ? 4 : 2; }

bool valid_dtype(la_dtype t) { return t == LA_F32 || t == LA_BF16; }

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Block sizes.  The result does not depend on the block size (the chunkwise
// form re-associates the causal sum exactly), so a block that is a multiple
// of 64 tokens is computed as 64-token blocks, the tile both kernel families
// are built for; a shorter block is honoured by the scalar kernels.
constexpr int64_t kMaxBlockArg = int64_t(1) << 20;
int64_t tile_block(int64_t block) { return block % kBf16Block == 0 ? kBf16Block : block; }

// bf16 inputs with d = dv = 128 or 64 and 64-token tiles run on the
// matrix-core kernels, any query-head group size (at 64, groups that are not
// a multiple of four run one or two query heads per four-wave workgroup with
// the other waves idle); every other supported shape (float32 inputs, or bf16
// at other head or block sizes) on the scalar float32-FMA kernels.  The
// forward, the variants and the backward share this rule.
bool mfma_path(la_dtype in_dtype, int64_t d, int64_t dv, int64_t block) {
  return in_dtype == LA_BF16 && d == dv && (d == 128 || d == 64) && tile_block(block) == kBf16Block;
}

// Shape/dtype checks shared by la_forward_ex and la_forward_workspace_bytes.
la_status check_forward_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                              int64_t block, la_dtype in_dtype, la_dtype out_dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N < 0 || d <= 0 || dv <= 0 || block <= 0) return LA_ERR_SHAPE;
  if (Hq % Hkv != 0) return LA_ERR_SHAPE;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return LA_ERR_UNSUPPORTED;
  if (in_dtype == LA_F32 && out_dtype != LA_F32) return LA_ERR_UNSUPPORTED;
  if (block > kMaxBlockArg) return LA_ERR_UNSUPPORTED;
  if (!mfma_path(in_dtype, d, dv, block) && (d > 128 || dv > 128 || dv % 32 != 0 || tile_block(block) > 64))
    return LA_ERR_UNSUPPORTED;
  // Grid dimensions are 32-bit; keep the workgroup counts well inside that,
  // and keep every byte count (B * Hq * N * 128 elements of up to 4 bytes)
  // far from 64-bit overflow.
  // (each factor is bounded before the product, which therefore cannot overflow)
  if (B > (int64_t(1) << 24) || Hq > (int64_t(1) << 24) || B * Hq > (int64_t(1) << 24) ||
      N > (int64_t(1) << 40))
    return LA_ERR_UNSUPPORTED;
  if (N > 0 && B * Hq > (int64_t(1) << 44) / N) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

}  // namespace

namespace la {

Bf16Plan plan_bf16(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus,
                   bool allow_solo) {
  Bf16Plan p;
  const int64_t G = Hq / Hkv;
  p.hd = static_cast<int>(d);
  (void)dv;  // d = dv on the matrix-core path
  p.gw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  p.subgroups = static_cast<int>(G / p.gw);
  // head size 64 with one query head per KV head: one-wave workgroups, four
  // per compute unit (one per SIMD)
  p.solo = allow_solo && d == 64 && G == 1;
  p.nblocks = (N + kBf16Block - 1) / kBf16Block;
  if (p.nblocks == 0) return p;

  const int64_t kv_chains = B * Hkv;
  const int64_t main_chains = kv_chains * p.subgroups;
  // Enough segments for one workgroup per compute unit (four one-wave ones),
  // each at least kMinBlocks long so the pre-pass stays a small fraction of
  // the traffic.
  constexpr int64_t kMinBlocks = 4;
  const int64_t slots = p.solo ? 4 * int64_t(cus) : int64_t(cus);
  int64_t P = 1;
  if (main_chains < slots) P = (slots + main_chains - 1) / main_chains;
  P = std::min(P, std::max<int64_t>(1, p.nblocks / kMinBlocks));
  p.blocks_per_seg = (p.nblocks + P - 1) / P;
  P = (p.nblocks + p.blocks_per_seg - 1) / p.blocks_per_seg;
  p.P = static_cast<int>(P);

  if (P > 1) {
    // Pre-pass parts: as many as fit the chip in one round (two pre-pass
    // workgroups are resident per compute unit at head size 128, three at
    // 64), so no partial last round leaves compute units idle; each part sums
    // at least kMinPartBlocks blocks (a part writes a 64 KiB partial).
    constexpr int64_t kMinPartBlocks = 8;
    const int64_t kPartWgsPerCu = d == 128 ? 2 : 3;
    int64_t R = (kPartWgsPerCu * int64_t(cus)) / (kv_chains * (P - 1));
    R = std::max<int64_t>(1, std::min(R, p.blocks_per_seg / kMinPartBlocks));
    p.blocks_per_part = (p.blocks_per_seg + R - 1) / R;
    R = (p.blocks_per_seg + p.blocks_per_part - 1) / p.blocks_per_part;
    p.R = static_cast<int>(R);
  }
  // Boundaries shifted per KV chain by up to 15 blocks (the four-head kernel,
  // long segments only: the longest segment grows by at most 15 blocks, under
  // 1.5%).  Measured at 1M tokens on the same buffer pairs: at head size 128
  // a pair whose streams collided in the memory system went from 17.9 to
  // 17.0-17.4 ms and no pair got slower; at 64 the mean over four pairs went
  // from 8.77 to 8.66 ms.
  constexpr int64_t kShiftMinBlocks = 1024;
  p.shifted = P > 1 && p.gw == 4 && !p.solo && p.blocks_per_seg >= kShiftMinBlocks &&
              p.nblocks - (P - 1) * p.blocks_per_seg >= 32;
  p.use_starts = (P > 1) || (p.subgroups > 1);
  if (p.use_starts) {
    p.partial_floats = size_t(kv_chains) * size_t(P - 1) * size_t(p.R) * size_t(d * dv);
    p.start_floats = size_t(kv_chains) * size_t(P) * size_t(d * dv);
    p.workspace_bytes = (p.partial_floats + p.start_floats) * sizeof(float);
  }
  return p;
}

VarPlan plan_variant(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus, bool causal,
                     bool norm) {
  VarPlan vp;
  vp.causal = causal;
  vp.norm = norm;
  // causal forms at head size 64 with one query head per KV head run the
  // one-wave kernel, as the plain forward does
  vp.base = plan_bf16(B, Hq, Hkv, N, d, dv, cus, causal);
  Bf16Plan& p = vp.base;
  if (p.nblocks == 0) return vp;
  const size_t chains = size_t(B * Hkv);
  size_t Ppre = size_t(p.P);  // scanned entries per chain
  if (!causal) {
    // the pre-pass sums every segment (into totals: plain boundaries); one
    // part per segment when unsplit
    p.shifted = false;
    if (p.P == 1) {
      p.R = 1;
      p.blocks_per_part = p.blocks_per_seg;
    }
    Ppre = size_t(p.P) + 1;
    // output kernel: independent blocks, one workgroup per compute unit
    const int64_t out_chains = B * Hkv * p.subgroups;
    int64_t P = std::max<int64_t>(1, (cus + out_chains - 1) / out_chains);
    P = std::min(P, p.nblocks);
    vp.bps_out = (p.nblocks + P - 1) / P;
    vp.P_out = static_cast<int>((p.nblocks + vp.bps_out - 1) / vp.bps_out);
  } else if (!p.use_starts) {
    return vp;  // one segment, one subgroup: s_in and z_in are read directly
  }
  vp.partial_floats = chains * (Ppre - 1) * size_t(p.R) * size_t(d * dv);
  vp.start_floats = chains * Ppre * size_t(d * dv);
  if (norm) {
    vp.zpart_floats = chains * (Ppre - 1) * size_t(p.R) * size_t(d);
    vp.zstart_floats = chains * Ppre * size_t(d);
  }
  vp.workspace_bytes = (vp.partial_floats + vp.start_floats + vp.zpart_floats + vp.zstart_floats) * sizeof(float);
  return vp;
}

StatePlan plan_state(int64_t B, int64_t Hkv, int64_t N, int64_t d, int cus) {
  StatePlan p;
  p.hd = static_cast<int>(d);
  p.nblocks = (N + kBf16Block - 1) / kBf16Block;
  if (p.nblocks == 0) return p;
  // Parts: one round of resident pre-pass workgroups (two per compute unit at
  // head size 128, three at 64) over all chains, each part at least
  // kMinPartBlocks blocks.
  constexpr int64_t kMinPartBlocks = 8;
  const int64_t chains = B * Hkv;
  const int64_t slots = (d == 128 ? 2 : 3) * int64_t(cus);
  int64_t R = (slots + chains - 1) / chains;
  R = std::max<int64_t>(1, std::min(R, p.nblocks / kMinPartBlocks));
  p.blocks_per_part = (p.nblocks + R - 1) / R;
  R = (p.nblocks + p.blocks_per_part - 1) / p.blocks_per_part;
  p.R = static_cast<int>(R);
  p.partial_floats = size_t(chains) * size_t(R) * size_t(d * d);
  p.workspace_bytes = p.partial_floats * sizeof(float);
  return p;
}

BwdPlan plan_backward(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus) {
  BwdPlan p;
  // dQ is the forward over (dO, V, K): head sizes swap.
  p.fwd = plan_bf16(B, Hq, Hkv, N, dv, d, cus, true);
  // The dQ pass's segments are the dK/dV kernel's (its per-segment q^T dO sums
  // start the reverse walks): plain boundaries.
  p.fwd.shifted = false;
  p.nblocks = (N + kBf16Block - 1) / kBf16Block;
  if (p.nblocks == 0) return p;

  // dK/dV: one workgroup per (batch, KV head, segment).  At head size 128 it
  // fills a compute unit (eight waves, 122 KiB of LDS); at 64 it takes four
  // waves and 65 KiB, so two run on each unit.
  const int64_t chains = B * Hkv;
  constexpr int64_t kMinBlocks = 4;
  const int64_t slots_kv = (d == 64 ? 2 : 1) * int64_t(cus);
  int64_t P = 1;
  if (chains < slots_kv) P = (slots_kv + chains - 1) / chains;
  P = std::min(P, std::max<int64_t>(1, p.nblocks / kMinBlocks));
  p.blocks_per_seg = (p.nblocks + P - 1) / P;
  P = (p.nblocks + p.blocks_per_seg - 1) / p.blocks_per_seg;
  p.P = static_cast<int>(P);

  // Head size 128 with four query heads per dQ workgroup and the same
  // segments in both passes: the dQ pass sums q^T dO per segment itself, so
  // dO is read once for both (a separate pre-pass reads 7/8 of Q and dO).
  p.fused = P > 1 && d == 128 && p.fwd.hd == 128 && p.fwd.gw == 4 && !p.fwd.solo && p.fwd.P == P &&
            p.fwd.blocks_per_seg == p.blocks_per_seg;
  if (p.fused) {
    p.blocks_per_part = p.blocks_per_seg;
    p.R = 1;
    p.partial_floats = size_t(B * Hkv * p.fwd.subgroups) * size_t(P - 1) * size_t(d * dv);
    p.rstart_floats = size_t(chains) * size_t(P) * size_t(d * dv);
  } else if (P > 1) {
    // Pre-pass over (Q, dO) of every query head and every segment but the
    // first.  Parts per segment: the count with the least (rounds of resident
    // workgroups, two per compute unit at head size 128 and three at 64) x
    // (blocks per part + the cost of its partial, written once and read once
    // by the scan: 4 d dv floats against a block's 64 (d + dv) bf16 values,
    // four blocks at d = dv = 128), i.e. the shortest pre-pass when every part
    // streams at the same rate; ties go to fewer parts.
    constexpr int64_t kMinPartBlocks = 8;
    const int64_t kPartWgsPerCu = d == 128 ? 2 : 3;
    const int64_t kPartialCostBlocks = std::max<int64_t>(1, (4 * d * dv) / (kBf16Block * (d + dv)));
    const int64_t pre_chains = B * Hq * (P - 1);
    const int64_t slots = kPartWgsPerCu * int64_t(cus);
    int64_t best_R = 1, best_cost = -1;
    const int64_t max_R = std::max<int64_t>(1, p.blocks_per_seg / kMinPartBlocks);
    for (int64_t R = 1; R <= max_R; ++R) {
      const int64_t bpp = (p.blocks_per_seg + R - 1) / R;
      const int64_t rounds = (pre_chains * R + slots - 1) / slots;
      const int64_t cost = rounds * (bpp + kPartialCostBlocks);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best_R = R;
      }
    }
    p.blocks_per_part = (p.blocks_per_seg + best_R - 1) / best_R;
    p.R = static_cast<int>((p.blocks_per_seg + p.blocks_per_part - 1) / p.blocks_per_part);
    p.partial_floats = size_t(B * Hq) * size_t(P - 1) * size_t(p.R) * size_t(d * dv);
    p.rstart_floats = size_t(chains) * size_t(P) * size_t(d * dv);
  }
  p.fwd_floats = p.fwd.workspace_bytes / sizeof(float);
  p.sin_t_floats = size_t(chains) * size_t(d * dv);
  p.workspace_bytes = (p.fwd_floats + p.sin_t_floats + p.partial_floats + p.rstart_floats) * sizeof(float);
  return p;
}

}  // namespace la

extern "C" {

const char* la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_NULL: return "a required pointer is NULL";
    case LA_ERR_SHAPE: return "invalid shape (non-positive size or Hq not a multiple of Hkv)";
    case LA_ERR_UNSUPPORTED: return "unsupported head size, block size or dtype combination";
    case LA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LA_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_HIP: return "HIP runtime or launch error";
    case LA_ERR_TOO_LARGE: return "problem needs more workspace than the allocation-free entry point's fixed scratch";
    default: break;
  }
  return "unknown status";
}

size_t la_forward_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                  int64_t block, la_dtype in_dtype) {
  la_dtype out = in_dtype;
  if (check_forward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, out) != LA_OK) return 0;
  if (!mfma_path(in_dtype, d, dv, block) || N == 0) return 0;
  return la::plan_bf16(B, Hq, Hkv, N, d, dv, device_cus(), true).workspace_bytes;
}

}  // extern "C"

namespace {

// Everything la_forward_ex, la_forward_states and la_forward_outputs check,
// in one place.  need_q_o is false for la_forward_states (it reads only k, v).
struct ForwardCall {
  la::Bf16Plan plan;
  size_t ns = 0;        // state bytes
  bool scalar = false;  // the scalar kernels serve this call (no workspace)
};

la_status validate_forward(ForwardCall& fc, const void* q, const void* k, const void* v, const void* o,
                           bool need_q_o, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                           int64_t block, la_dtype in_dtype, la_dtype out_dtype, const float* s_in,
                           const float* s_out, const void* workspace, size_t workspace_bytes,
                           bool check_workspace = true) {
  la_status st = check_forward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype);
  if (st != LA_OK) return st;
  // With N == 0 the token tensors are empty and may be NULL.
  if (N > 0 && (k == nullptr || v == nullptr || (need_q_o && (q == nullptr || o == nullptr)))) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(s_in) || !aligned16(s_out))
    return LA_ERR_ALIGN;

  const size_t ei = esize(in_dtype), eo = esize(out_dtype);
  const size_t nq = size_t(B * Hq * N * d) * ei, nk = size_t(B * Hkv * N * d) * ei;
  const size_t nv = size_t(B * Hkv * N * dv) * ei, no = size_t(B * Hq * N * dv) * eo;
  const size_t ns = size_t(B * Hkv * d * dv) * sizeof(float);
  fc.ns = ns;
  fc.scalar = !mfma_path(in_dtype, d, dv, block);
  // o may be q itself on the four-head matrix-core kernel, where each query
  // head's rows are read and then written by one wave in program order.
  const bool in_place = o != nullptr && o == q;
  if (in_place && !(mfma_path(in_dtype, d, dv, block) && out_dtype == in_dtype && (Hq / Hkv) % 4 == 0))
    return LA_ERR_ALIAS;
  if ((!in_place && overlap(o, no, q, nq)) || overlap(o, no, k, nk) || overlap(o, no, v, nv) ||
      overlap(o, no, s_in, ns))
    return LA_ERR_ALIAS;
  if (s_out != nullptr &&
      (overlap(s_out, ns, q, nq) || overlap(s_out, ns, k, nk) || overlap(s_out, ns, v, nv) ||
       overlap(s_out, ns, o, no) || (s_out != s_in && overlap(s_out, ns, s_in, ns))))
    return LA_ERR_ALIAS;

  if (!fc.scalar && N > 0) {
    fc.plan = la::plan_bf16(B, Hq, Hkv, N, d, dv, device_cus(), true);
    const size_t nw = fc.plan.workspace_bytes;
    if (nw > 0 && check_workspace) {
      if (workspace == nullptr || workspace_bytes < nw) return LA_ERR_WORKSPACE;
      if (!aligned16(workspace)) return LA_ERR_ALIGN;
      if (overlap(workspace, nw, q, nq) || overlap(workspace, nw, k, nk) || overlap(workspace, nw, v, nv) ||
          overlap(workspace, nw, o, no) || overlap(workspace, nw, s_in, ns) || overlap(workspace, nw, s_out, ns))
        return LA_ERR_ALIAS;
    }
  }
  return LA_OK;
}

la_status run_states(const ForwardCall& fc, const void* k, const void* v, int64_t B, int64_t Hkv, int64_t N,
                     la_dtype in_dtype, const float* s_in, void* workspace, hipStream_t hs) {
  (void)in_dtype;
  if (fc.scalar || N == 0 || !fc.plan.use_starts) return LA_OK;
  return la::launch_segment_states(k, v, s_in, B, Hkv, N, fc.plan, workspace, hs) == hipSuccess ? LA_OK
                                                                                                  : LA_ERR_HIP;
}

la_status run_outputs(const ForwardCall& fc, const void* q, const void* k, const void* v, void* o, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                      la_dtype out_dtype, const float* s_in, float* s_out, const void* workspace,
                      hipStream_t hs) {
  hipError_t err = hipSuccess;
  if (N == 0) {
    // No tokens: the final state is the initial state (zeros without s_in).
    if (s_out != nullptr && s_out != s_in) err = la::launch_copy_or_zero(s_out, s_in, fc.ns / sizeof(float), hs);
  } else if (fc.scalar) {
    err = la::launch_fwd_f32(q, k, v, o, in_dtype == LA_BF16, out_dtype == LA_BF16, s_in, s_out, B, Hq, Hkv, N, d,
                             dv, tile_block(block), hs);
  } else {
    err = la::launch_fwd_bf16(q, k, v, o, out_dtype == LA_F32, s_in, s_out, B, Hq, Hkv, N, fc.plan, workspace,
                              hs);
  }
  return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// The state-only passes: s_out[c] = s_in[c] + sum over the Hin / Hkv input
// chains of output chain c and their N tokens of a_t^T b_t, c < B * Hkv; the
// forward's final state (a = k, b = v, Hin = Hkv) or the backward's
// initial-state gradient (a = q, b = dO, Hin = Hq).  The forward's shape rules
// apply with Hin heads over Hkv.
size_t state_only_workspace(int64_t B, int64_t Hin, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                            la_dtype in_dtype) {
  if (check_forward_shape(B, Hin, Hkv, N, d, dv, kBf16Block, in_dtype, in_dtype) != LA_OK) return 0;
  if (!mfma_path(in_dtype, d, dv, kBf16Block) || N == 0) return 0;
  return la::plan_state(B, Hin, N, d, device_cus()).workspace_bytes;
}

la_status run_state_only(const void* a, const void* b, int64_t B, int64_t Hin, int64_t Hkv, int64_t N, int64_t d,
                         int64_t dv, la_dtype in_dtype, const float* s_in, float* s_out, void* workspace,
                         size_t workspace_bytes, la_stream stream) {
  la_status st = check_forward_shape(B, Hin, Hkv, N, d, dv, kBf16Block, in_dtype, in_dtype);
  if (st != LA_OK) return st;
  if (s_out == nullptr || (N > 0 && (a == nullptr || b == nullptr))) return LA_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(s_in) || !aligned16(s_out)) return LA_ERR_ALIGN;
  const size_t ei = esize(in_dtype);
  const size_t na = size_t(B * Hin * N * d) * ei, nb = size_t(B * Hin * N * dv) * ei;
  const size_t ns = size_t(B * Hkv * d * dv) * sizeof(float);
  if (overlap(s_out, ns, a, na) || overlap(s_out, ns, b, nb) || (s_out != s_in && overlap(s_out, ns, s_in, ns)))
    return LA_ERR_ALIAS;
  const bool mfma = mfma_path(in_dtype, d, dv, kBf16Block);
  la::StatePlan plan;
  if (mfma && N > 0) {
    plan = la::plan_state(B, Hin, N, d, device_cus());
    const size_t nw = plan.workspace_bytes;
    if (workspace == nullptr || workspace_bytes < nw) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_ALIGN;
    if (overlap(workspace, nw, a, na) || overlap(workspace, nw, b, nb) || overlap(workspace, nw, s_in, ns) ||
        overlap(workspace, nw, s_out, ns))
      return LA_ERR_ALIAS;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int G = static_cast<int>(Hin / Hkv);
  hipError_t err = hipSuccess;
  if (N == 0) {
    if (s_out != s_in) err = la::launch_copy_or_zero(s_out, s_in, ns / sizeof(float), hs);
  } else if (mfma) {
    err = la::launch_state_total_bf16(a, b, s_in, s_out, B * Hkv, G, N, plan, static_cast<float*>(workspace), hs);
  } else {
    err = la::launch_state_total_f32(a, b, in_dtype == LA_BF16, s_in, s_out, B * Hkv, G, N, d, dv, hs);
  }
  return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

namespace la {

la_status check_forward_args(const void* q, const void* k, const void* v, const void* o, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                             la_dtype out_dtype, const float* s_in, const float* s_out, size_t* workspace_bytes) {
  ForwardCall fc;
  la_status st = validate_forward(fc, q, k, v, o, true, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in,
                                  s_out, nullptr, 0, false);
  *workspace_bytes = (st == LA_OK && !fc.scalar && N > 0) ? fc.plan.workspace_bytes : 0;
  return st;
}

}  // namespace la

extern "C" {

la_status la_forward_ex(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                        la_dtype out_dtype, const float* s_in, float* s_out, void* workspace,
                        size_t workspace_bytes, la_stream stream) {
  ForwardCall fc;
  la_status st = validate_forward(fc, q, k, v, o, true, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in,
                                  s_out, workspace, workspace_bytes);
  if (st != LA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = run_states(fc, k, v, B, Hkv, N, in_dtype, s_in, workspace, hs);
  if (st != LA_OK) return st;
  return run_outputs(fc, q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in, s_out, workspace,
                     hs);
}

la_status la_forward_states(const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                            int64_t d, int64_t dv, int64_t block, la_dtype in_dtype, const float* s_in,
                            void* workspace, size_t workspace_bytes, la_stream stream) {
  ForwardCall fc;
  la_status st = validate_forward(fc, nullptr, k, v, nullptr, false, B, Hq, Hkv, N, d, dv, block, in_dtype,
                                  in_dtype, s_in, nullptr, workspace, workspace_bytes);
  if (st != LA_OK) return st;
  return run_states(fc, k, v, B, Hkv, N, in_dtype, s_in, workspace, static_cast<hipStream_t>(stream));
}

la_status la_forward_outputs(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                             la_dtype out_dtype, const float* s_in, float* s_out, const void* workspace,
                             size_t workspace_bytes, la_stream stream) {
  ForwardCall fc;
  la_status st = validate_forward(fc, q, k, v, o, true, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in,
                                  s_out, workspace, workspace_bytes);
  if (st != LA_OK) return st;
  return run_outputs(fc, q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, s_in, s_out, workspace,
                     static_cast<hipStream_t>(stream));
}

size_t la_forward_state_workspace_bytes(int64_t B, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                        la_dtype in_dtype) {
  return state_only_workspace(B, Hkv, Hkv, N, d, dv, in_dtype);
}

la_status la_forward_state(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                           la_dtype in_dtype, const float* s_in, float* s_out, void* workspace,
                           size_t workspace_bytes, la_stream stream) {
  return run_state_only(k, v, B, Hkv, Hkv, N, d, dv, in_dtype, s_in, s_out, workspace, workspace_bytes, stream);
}

size_t la_backward_state_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                         la_dtype in_dtype) {
  return state_only_workspace(B, Hq, Hkv, N, d, dv, in_dtype);
}

la_status la_backward_state(const void* q, const void* grad_o, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                            int64_t d, int64_t dv, la_dtype in_dtype, const float* grad_s_out, float* grad_s_in,
                            void* workspace, size_t workspace_bytes, la_stream stream) {
  return run_state_only(q, grad_o, B, Hq, Hkv, N, d, dv, in_dtype, grad_s_out, grad_s_in, workspace,
                        workspace_bytes, stream);
}

la_status la_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype, la_dtype out_dtype,
                     la_stream stream) {
  la_status st = check_forward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype);
  if (st != LA_OK) return st;
  size_t ws = 0;
  if (mfma_path(in_dtype, d, dv, block) && N > 0)
    ws = la::plan_bf16(B, Hq, Hkv, N, d, dv, device_cus(), true).workspace_bytes;
  if (ws == 0)
    return la_forward_ex(q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, nullptr, nullptr,
                         nullptr, 0, stream);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* buf = nullptr;
  if (hipMallocAsync(&buf, ws, hs) != hipSuccess) return LA_ERR_HIP;
  st = la_forward_ex(q, k, v, o, B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, nullptr, nullptr, buf, ws,
                     stream);
  if (hipFreeAsync(buf, hs) != hipSuccess && st == LA_OK) st = LA_ERR_HIP;
  return st;
}

la_status la_decode_step(float* S, const void* q, const void* k, const void* v, void* o, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t d, int64_t dv, la_dtype in_dtype, la_dtype out_dtype,
                         la_stream stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || dv <= 0 || Hq % Hkv != 0) return LA_ERR_SHAPE;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return LA_ERR_UNSUPPORTED;
  if (d > 128 || dv > 128 || dv % 4 != 0 || B > (int64_t(1) << 30) || Hkv > (int64_t(1) << 30) ||
      B * Hkv > (int64_t(1) << 30) || Hq / Hkv > 1024)
    return LA_ERR_UNSUPPORTED;
  if (S == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr) return LA_ERR_NULL;
  if (!aligned16(S) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  const size_t ei = esize(in_dtype);
  const size_t ns = size_t(B * Hkv * d * dv) * sizeof(float);
  const size_t nq = size_t(B * Hq * d) * ei, nk = size_t(B * Hkv * d) * ei, nv = size_t(B * Hkv * dv) * ei;
  const size_t no = size_t(B * Hq * dv) * esize(out_dtype);
  if (overlap(S, ns, q, nq) || overlap(S, ns, k, nk) || overlap(S, ns, v, nv) || overlap(S, ns, o, no) ||
      overlap(o, no, q, nq) || overlap(o, no, k, nk) || overlap(o, no, v, nv))
    return LA_ERR_ALIAS;
  hipError_t err = la::launch_decode(S, q, k, v, o, in_dtype == LA_BF16, out_dtype == LA_F32, B, Hq, Hkv, d,
                                     dv, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"

namespace {

la_status check_backward_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                               int64_t block, la_dtype in_dtype, la_dtype grad_dtype) {
  la_status st = check_forward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, grad_dtype);
  if (st != LA_OK) return st;
  // scalar kernels: dK is computed in 32-column slices of d (dv is already a multiple of 32)
  if (!mfma_path(in_dtype, d, dv, block) && d % 32 != 0) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// The backward runs on the matrix cores for the forward's shapes: its dQ pass
// is the forward over (dO, V, K) and its dK/dV kernel is built for head sizes
// 128 (eight waves) and 64 (four waves).
size_t backward_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                          la_dtype in_dtype) {
  if (!mfma_path(in_dtype, d, dv, block)) return la::bwd_f32_workspace_floats(B, Hkv, d, dv) * sizeof(float);
  return la::plan_backward(B, Hq, Hkv, N, d, dv, device_cus()).workspace_bytes;
}

}  // namespace

extern "C" {

size_t la_backward_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                   int64_t block, la_dtype in_dtype) {
  if (check_backward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, in_dtype) != LA_OK || N == 0) return 0;
  return backward_workspace(B, Hq, Hkv, N, d, dv, block, in_dtype);
}

la_status la_backward(const void* q, const void* k, const void* v, const void* grad_o, void* grad_q,
                      void* grad_k, void* grad_v, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      int64_t dv, int64_t block, la_dtype in_dtype, la_dtype grad_dtype, const float* s_in,
                      const float* grad_s_out, float* grad_s_in, void* workspace, size_t workspace_bytes,
                      la_stream stream) {
  la_status st = check_backward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, grad_dtype);
  if (st != LA_OK) return st;
  if (N > 0 && (q == nullptr || k == nullptr || v == nullptr || grad_o == nullptr || grad_q == nullptr ||
                grad_k == nullptr || grad_v == nullptr))
    return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(grad_o) || !aligned16(grad_q) ||
      !aligned16(grad_k) || !aligned16(grad_v) || !aligned16(s_in) || !aligned16(grad_s_out) ||
      !aligned16(grad_s_in) || !aligned16(workspace))
    return LA_ERR_ALIGN;

  const size_t ei = esize(in_dtype), eg = esize(grad_dtype);
  const size_t nq = size_t(B * Hq * N * d) * ei, nk = size_t(B * Hkv * N * d) * ei;
  const size_t nv = size_t(B * Hkv * N * dv) * ei, ndo = size_t(B * Hq * N * dv) * ei;
  const size_t gq = size_t(B * Hq * N * d) * eg, gk = size_t(B * Hkv * N * d) * eg;
  const size_t gv = size_t(B * Hkv * N * dv) * eg;
  const size_t ns = size_t(B * Hkv * d * dv) * sizeof(float);
  struct Range {
    const void* p;
    size_t n;
  };
  const Range inputs[] = {{q, nq}, {k, nk}, {v, nv}, {grad_o, ndo}, {s_in, ns}, {grad_s_out, ns}};
  const Range outputs[] = {{grad_q, gq}, {grad_k, gk}, {grad_v, gv}, {grad_s_in, ns}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& in : inputs) {
      // grad_s_in may be grad_s_out itself (in-place chunk chaining)
      if (i == 3 && in.p == grad_s_out && grad_s_in == grad_s_out) continue;
      if (overlap(outputs[i].p, outputs[i].n, in.p, in.n)) return LA_ERR_ALIAS;
    }
    for (int j = 0; j < i; ++j)
      if (overlap(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n)) return LA_ERR_ALIAS;
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (N == 0) {
    // No tokens: the state gradient passes through unchanged.
    if (grad_s_in == nullptr || grad_s_in == grad_s_out) return LA_OK;
    return la::launch_copy_or_zero(grad_s_in, grad_s_out, ns / sizeof(float), hs) == hipSuccess ? LA_OK
                                                                                                  : LA_ERR_HIP;
  }

  const size_t nw = backward_workspace(B, Hq, Hkv, N, d, dv, block, in_dtype);
  if (workspace == nullptr || workspace_bytes < nw) return LA_ERR_WORKSPACE;
  for (const Range& in : inputs)
    if (overlap(workspace, nw, in.p, in.n)) return LA_ERR_ALIAS;
  for (const Range& out : outputs)
    if (overlap(workspace, nw, out.p, out.n)) return LA_ERR_ALIAS;

  if (!mfma_path(in_dtype, d, dv, block))
    return la::launch_bwd_f32(q, k, v, grad_o, grad_q, grad_k, grad_v, in_dtype == LA_BF16, grad_dtype == LA_BF16,
                              s_in, grad_s_out, grad_s_in, B, Hq, Hkv, N, d, dv, tile_block(block),
                              static_cast<float*>(workspace), hs) == hipSuccess
               ? LA_OK
               : LA_ERR_HIP;

  const la::BwdPlan plan = la::plan_backward(B, Hq, Hkv, N, d, dv, device_cus());
  float* ws = static_cast<float*>(workspace);
  float* ws_fwd = ws;
  float* sin_t = ws_fwd + plan.fwd_floats;
  float* ws_kv = sin_t + plan.sin_t_floats;
  const bool out_f32 = grad_dtype == LA_F32;

  // dQ: the forward over (queries dO, keys V, values K) from s_in^T.
  const float* s_t = nullptr;
  if (s_in != nullptr) {
    if (la::launch_transpose_states(s_in, sin_t, B * Hkv, d, hs) != hipSuccess) return LA_ERR_HIP;
    s_t = sin_t;
  }
  if (plan.fwd.use_starts && la::launch_segment_states(v, k, s_t, B, Hkv, N, plan.fwd, ws_fwd, hs) != hipSuccess)
    return LA_ERR_HIP;
  if (plan.fused) {
    // ... and the per-segment sums of q^T dO that start the reverse recurrence
    if (la::launch_fwd_bf16_rsum(grad_o, v, k, grad_q, out_f32, B, Hq, Hkv, N, plan.fwd, ws_fwd, q, ws_kv, hs) !=
        hipSuccess)
      return LA_ERR_HIP;
  } else if (la::launch_fwd_bf16(grad_o, v, k, grad_q, out_f32, s_t, nullptr, B, Hq, Hkv, N, plan.fwd, ws_fwd,
                                 hs) != hipSuccess) {
    return LA_ERR_HIP;
  }
  // dK, dV, ds_in: the reverse recurrence.
  if (la::launch_bwd_kv(q, k, v, grad_o, grad_k, grad_v, out_f32, grad_s_out, grad_s_in, B, Hq, Hkv, N, plan,
                        ws_kv, hs) != hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

}  // extern "C"

namespace {

la_status check_variant_args(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                             la_dtype in_dtype, la_dtype out_dtype, int causal, int fmap, int normalize, float eps,
                             const float* z_in, const float* z_out) {
  la_status st = check_forward_shape(B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype);
  if (st != LA_OK) return st;
  if ((causal != 0 && causal != 1) || (fmap != LA_FMAP_IDENTITY && fmap != LA_FMAP_RELU) ||
      (normalize != 0 && normalize != 1))
    return LA_ERR_UNSUPPORTED;
  if (normalize) {
    if (!(eps >= 0.0f) || eps > 3.0e38f) return LA_ERR_UNSUPPORTED;  // also rejects NaN
  } else if (z_in != nullptr || z_out != nullptr) {
    return LA_ERR_UNSUPPORTED;
  }
  return LA_OK;
}

}  // namespace

extern "C" {

size_t la_forward_variant_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                          int64_t block, la_dtype in_dtype, int causal, int normalize) {
  if (check_variant_args(B, Hq, Hkv, N, d, dv, block, in_dtype, in_dtype, causal, LA_FMAP_IDENTITY, normalize, 0.0f,
                         nullptr, nullptr) != LA_OK ||
      N == 0 || !mfma_path(in_dtype, d, dv, block))
    return 0;
  return la::plan_variant(B, Hq, Hkv, N, d, dv, device_cus(), causal != 0, normalize != 0).workspace_bytes;
}

la_status la_forward_variant(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                             la_dtype out_dtype, int causal, la_feature_map fmap, int normalize, float eps,
                             const float* s_in, float* s_out, const float* z_in, float* z_out, void* workspace,
                             size_t workspace_bytes, la_stream stream) {
  la_status st = check_variant_args(B, Hq, Hkv, N, d, dv, block, in_dtype, out_dtype, causal, fmap, normalize, eps,
                                    z_in, z_out);
  if (st != LA_OK) return st;
  if (N > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr)) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(s_in) || !aligned16(s_out) ||
      !aligned16(z_in) || !aligned16(z_out) || !aligned16(workspace))
    return LA_ERR_ALIGN;
  const size_t ei = esize(in_dtype), eo = esize(out_dtype);
  const size_t nq = size_t(B * Hq * N * d) * ei, nk = size_t(B * Hkv * N * d) * ei;
  const size_t nv = size_t(B * Hkv * N * dv) * ei, no = size_t(B * Hq * N * dv) * eo;
  const size_t ns = size_t(B * Hkv * d * dv) * sizeof(float), nz = size_t(B * Hkv * d) * sizeof(float);
  struct Range {
    const void* p;
    size_t n;
  };
  const Range inputs[] = {{q, nq}, {k, nk}, {v, nv}, {s_in, ns}, {z_in, nz}};
  const Range outputs[] = {{o, no}, {s_out, ns}, {z_out, nz}};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j) {
      // s_out may be s_in itself and z_out z_in itself (in-place resume)
      if ((i == 1 && j == 3 && s_out == s_in) || (i == 2 && j == 4 && z_out == z_in)) continue;
      if (overlap(outputs[i].p, outputs[i].n, inputs[j].p, inputs[j].n)) return LA_ERR_ALIAS;
    }
    for (int j = 0; j < i; ++j)
      if (overlap(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n)) return LA_ERR_ALIAS;
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (s_out != nullptr && s_out != s_in && la::launch_copy_or_zero(s_out, s_in, ns / sizeof(float), hs) != hipSuccess)
      return LA_ERR_HIP;
    if (z_out != nullptr && z_out != z_in && la::launch_copy_or_zero(z_out, z_in, nz / sizeof(float), hs) != hipSuccess)
      return LA_ERR_HIP;
    return LA_OK;
  }
  if (!mfma_path(in_dtype, d, dv, block))
    return la::launch_fwd_f32_variant(q, k, v, o, in_dtype == LA_BF16, out_dtype == LA_BF16, causal != 0,
                                      fmap == LA_FMAP_RELU, normalize != 0, eps, s_in, s_out, z_in, z_out, B, Hq,
                                      Hkv, N, d, dv, tile_block(block), hs) == hipSuccess
               ? LA_OK
               : LA_ERR_HIP;
  const la::VarPlan vp = la::plan_variant(B, Hq, Hkv, N, d, dv, device_cus(), causal != 0, normalize != 0);
  const size_t nw = vp.workspace_bytes;
  if (nw > 0) {
    if (workspace == nullptr || workspace_bytes < nw) return LA_ERR_WORKSPACE;
    for (const Range& r : inputs)
      if (overlap(workspace, nw, r.p, r.n)) return LA_ERR_ALIAS;
    for (const Range& r : outputs)
      if (overlap(workspace, nw, r.p, r.n)) return LA_ERR_ALIAS;
  }
  return la::launch_variant(q, k, v, o, out_dtype == LA_F32, fmap == LA_FMAP_RELU, s_in, s_out, z_in, z_out, eps, B,
                            Hq, Hkv, N, vp, workspace, hs) == hipSuccess
             ? LA_OK
             : LA_ERR_HIP;
}

}  // extern "C"
