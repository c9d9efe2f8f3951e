// Internal declarations shared by the host dispatcher and the kernel files of
// liblightning.so.  Not part of the public interface (include/la.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "la.h"

namespace la {

// Work split of one bf16 forward call.
//
// The sequence of each (batch, KV head) "chain" is cut into P segments of
// whole 64-token blocks so that B * Hkv * subgroups * P workgroups fill the
// chip.  Segment j starts from s_in + sum over earlier segments of K_b^T V_b
// (exact by associativity).  Those earlier sums are produced by a pre-pass
// that splits every segment but the last into R parts, and a scan that adds
// the parts up in a fixed order.  With `shifted`, every inner boundary of
// chain c moves by a small per-chain number of blocks (the first and last
// segments absorb it), so that the chains' concurrent streams do not all sit
// at the same offsets; the pre-pass and the output kernel use the same
// boundaries.
struct Bf16Plan {
  int64_t nblocks = 0;          // ceil(N / 64)
  int hd = 128;                 // head size d = dv (128; 64 for groups of four query heads)
  int gw = 4;                   // query heads per workgroup (1, 2 or 4)
  bool solo = false;            // one-wave workgroups (head size 64, one query head per KV head)
  int subgroups = 1;            // (Hq / Hkv) / gw workgroups per KV head and segment
  int P = 1;                    // segments per chain
  int R = 1;                    // pre-pass parts per segment
  int64_t blocks_per_seg = 0;
  int64_t blocks_per_part = 0;
  bool use_starts = false;      // segment start states come from the workspace
  bool shifted = false;         // segment boundaries moved per KV chain (seg_shift in la_fwd_bf16.hip)
  size_t partial_floats = 0;    // B*Hkv*(P-1)*R*d*dv
  size_t start_floats = 0;      // B*Hkv*P*d*dv
  size_t workspace_bytes = 0;
};

// allow_solo: the caller runs the output kernels of launch_fwd_bf16 (the
// forward, the backward's dQ pass), which include the one-wave kernel for head
// size 64 with one query head per KV head; the variants plan without it.
Bf16Plan plan_bf16(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus,
                   bool allow_solo = false);

// Scalar (float32 FMA) forward: q, k, v stored as float32 or bf16 (in_bf16),
// o as float32 or bf16 (out_bf16); d up to 128, dv a multiple of 32 up to
// 128, blocks of up to 64 tokens.  It serves float32 inputs, and bf16 inputs
// at shapes the matrix-core kernels are not built for.  No workspace.
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, bool in_bf16, bool out_bf16,
                          const float* s_in, float* s_out, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                          int64_t dv, int64_t block, hipStream_t stream);

// Forward variants on the scalar kernel (same storage types and shapes as
// launch_fwd_f32): phi = ReLU on q and k (relu), division by phi(q_t) . z_t +
// eps (norm, with z_in / z_out the normaliser sums; z_out may be z_in), causal
// or non-causal.  No workspace.
hipError_t launch_fwd_f32_variant(const void* q, const void* k, const void* v, void* o, bool in_bf16,
                                  bool out_bf16, bool causal, bool relu, bool norm, float eps, const float* s_in,
                                  float* s_out, const float* z_in, float* z_out, int64_t B, int64_t Hq,
                                  int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block,
                                  hipStream_t stream);

// Segment start states into the workspace (pre-pass + scan); only when
// plan.use_starts.
hipError_t launch_segment_states(const void* k, const void* v, const float* s_in, int64_t B, int64_t Hkv,
                                 int64_t N, const Bf16Plan& plan, void* workspace, hipStream_t stream);

// Outputs and final state; reads the segment start states from the workspace
// when plan.use_starts, else s_in directly.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, bool out_f32,
                           const float* s_in, float* s_out, int64_t B, int64_t Hq, int64_t Hkv,
                           int64_t N, const Bf16Plan& plan, const void* workspace, hipStream_t stream);

// The backward's dQ pass (launch_fwd_bf16 over queries q = dO, keys V, values
// K) that also writes, for every segment j >= 1 of every (batch, KV head,
// query-head subgroup) chain c, rpart[c (P - 1) + j - 1] = sum over the
// segment and the subgroup's four query heads of x_t^T q_t (x = the forward's
// queries, [B*Hq][N][128] bf16; float32 128 x 128 each).  Head size 128,
// groups of four query heads per workgroup, at least two segments.
hipError_t launch_fwd_bf16_rsum(const void* q, const void* k, const void* v, void* o, bool out_f32,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, const Bf16Plan& plan,
                                const void* workspace, const void* x, float* rpart, hipStream_t stream);

// Pre-pass over `chains` row-major [N][hd] tile pairs (a, b), hd = 64 or 128:
// partial sums of a_b^T b_b over part r of segment j + seg_offset, j < P - 1.
hipError_t launch_state_parts(const void* a, const void* b, float* partial, int64_t chains, int64_t N,
                              int64_t nblocks, int64_t blocks_per_seg, int64_t blocks_per_part, int P, int R,
                              int seg_offset, int hd, hipStream_t stream);

// Forward variants (feature map, non-causal, normalised), bf16 inputs, any
// query-head group size.  Causal: the forward's split, with the
// normaliser sums carried beside the state.  Non-causal: the pre-pass sums
// every segment (the scan's last entry is the total) and the output kernel
// splits each chain into P_out segments of bps_out blocks.
struct VarPlan {
  Bf16Plan base;
  bool causal = true;
  bool norm = false;
  int P_out = 1;
  int64_t bps_out = 0;
  size_t partial_floats = 0;    // B*Hkv*(Ppre-1)*R*d*dv
  size_t start_floats = 0;      // B*Hkv*Ppre*d*dv
  size_t zpart_floats = 0;      // B*Hkv*(Ppre-1)*R*d      (norm)
  size_t zstart_floats = 0;     // B*Hkv*Ppre*d            (norm)
  size_t workspace_bytes = 0;   // all four, in that order
};

VarPlan plan_variant(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus, bool causal,
                     bool norm);

hipError_t launch_variant(const void* q, const void* k, const void* v, void* o, bool out_f32, bool relu,
                          const float* s_in, float* s_out, const float* z_in, float* z_out, float eps, int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t N, const VarPlan& plan, void* workspace,
                          hipStream_t stream);

// State-only pass (la_forward_state) on the matrix cores: each (batch, KV
// head) chain's blocks are summed in R parts of blocks_per_part blocks
// (enough parts to fill the chip), then added up in order with s_in.
struct StatePlan {
  int64_t nblocks = 0;          // ceil(N / 64)
  int64_t blocks_per_part = 0;
  int R = 1;
  int hd = 128;                 // head size d = dv (128 or 64)
  size_t partial_floats = 0;    // B*Hkv*R*d*dv
  size_t workspace_bytes = 0;
};

StatePlan plan_state(int64_t B, int64_t Hkv, int64_t N, int64_t d, int cus);

// s_out[c] = s_in[c] (zeros if NULL) + sum over the G input chains c G ..
// c G + G - 1 and their N tokens of a_t^T b_t, for c < chains: the forward's
// final state (a = k, b = v, G = 1) or the backward's initial-state gradient
// (a = q, b = dO of the G query heads of a KV head).  bf16 inputs at d = dv =
// plan.hd (plan_state over chains * G input chains), through the pre-pass
// kernel; the workspace holds the plan's partials.  s_out may be s_in.
hipError_t launch_state_total_bf16(const void* a, const void* b, const float* s_in, float* s_out, int64_t chains,
                                   int G, int64_t N, const StatePlan& plan, float* workspace, hipStream_t stream);

// The same on float32 FMA for float32 inputs, or bf16 inputs (in_bf16) off the
// matrix-core shape: d and dv up to 128, no workspace.  s_out may be s_in.
hipError_t launch_state_total_f32(const void* a, const void* b, bool in_bf16, const float* s_in, float* s_out,
                                  int64_t chains, int G, int64_t N, int64_t d, int64_t dv, hipStream_t stream);

// Backward work split: dK/dV walk each chain's segments from the end; segment
// j starts from the sum of q^T dO over later segments and the group's heads.
struct BwdPlan {
  Bf16Plan fwd;                 // dQ = forward over (dO, V, K)
  int64_t nblocks = 0;
  int64_t blocks_per_seg = 0;
  int64_t blocks_per_part = 0;
  int P = 1;
  int R = 1;
  // The dQ pass also writes the partials (launch_fwd_bf16_rsum): its segments
  // are these, and there is no separate pre-pass over (Q, dO).
  bool fused = false;
  size_t fwd_floats = 0;        // forward workspace
  size_t sin_t_floats = 0;      // transposed initial state for dQ
  size_t partial_floats = 0;    // B*Hq*(P-1)*R*d*dv; fused: B*Hkv*subgroups*(P-1)*d*dv
  size_t rstart_floats = 0;     // B*Hkv*P*d*dv
  size_t workspace_bytes = 0;   // all four, in that order
};

BwdPlan plan_backward(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus);

// out[c] = in[c]^T for `count` n x n float32 states (n = 64 or 128).
hipError_t launch_transpose_states(const float* in, float* out, int64_t count, int64_t n, hipStream_t stream);

// dK, dV and (if ds_in) the initial-state gradient; the reverse state starts
// from ds_out (zeros if NULL).  workspace_f holds the plan's partials and
// segment start states; with plan.fused the partials are already there (the
// dQ pass wrote them), else the pre-pass over (Q, dO) writes them first.
hipError_t launch_bwd_kv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dvg,
                         bool out_f32, const float* ds_out, float* ds_in, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, const BwdPlan& plan, float* workspace_f, hipStream_t stream);

// Scalar (float32 FMA) backward (inputs and gradients stored as float32 or
// bf16, d and dv multiples of 32 up to 128, blocks of up to 64 tokens): dQ by
// the scalar forward over (dO, V, K) from s_in^T, then dK and dV (and ds_in)
// by the reverse recurrence.  The workspace holds s_in^T
// (bwd_f32_workspace_floats floats).
size_t bwd_f32_workspace_floats(int64_t B, int64_t Hkv, int64_t d, int64_t dv);
hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                          void* dvg, bool in_bf16, bool grad_bf16, const float* s_in, const float* ds_out,
                          float* ds_in, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                          int64_t block, float* workspace, hipStream_t stream);

// Every check la_forward_ex makes except those on the workspace; on LA_OK,
// *workspace_bytes is the workspace the call needs (0 when none).  Touches no
// device memory.
la_status check_forward_args(const void* q, const void* k, const void* v, const void* o, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t N, int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                             la_dtype out_dtype, const float* s_in, const float* s_out, size_t* workspace_bytes);

// dst[i] = src ? src[i] : 0 for i < n.
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream);

hipError_t launch_decode(float* S, const void* q, const void* k, const void* v, void* o,
                         bool in_bf16, bool out_f32, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t d, int64_t dv, hipStream_t stream);

}  // namespace la
