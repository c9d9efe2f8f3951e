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
// the parts up in a fixed order.
struct Bf16Plan {
  int64_t nblocks = 0;          // ceil(N / 64)
  int gw = 4;                   // query heads per workgroup (1, 2 or 4)
  int subgroups = 1;            // (Hq / Hkv) / gw workgroups per KV head and segment
  int P = 1;                    // segments per chain
  int R = 1;                    // pre-pass parts per segment
  int64_t blocks_per_seg = 0;
  int64_t blocks_per_part = 0;
  bool use_starts = false;      // segment start states come from the workspace
  size_t partial_floats = 0;    // B*Hkv*(P-1)*R*d*dv
  size_t start_floats = 0;      // B*Hkv*P*d*dv
  size_t workspace_bytes = 0;
};

Bf16Plan plan_bf16(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv, int cus);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o,
                          const float* s_in, float* s_out, int64_t B, int64_t Hq, int64_t Hkv,
                          int64_t N, int64_t d, int64_t dv, int64_t block, hipStream_t stream);

// Segment start states into the workspace (pre-pass + scan); only when
// plan.use_starts.
hipError_t launch_segment_states(const void* k, const void* v, const float* s_in, int64_t B, int64_t Hkv,
                                 int64_t N, const Bf16Plan& plan, void* workspace, hipStream_t stream);

// Outputs and final state; reads the segment start states from the workspace
// when plan.use_starts, else s_in directly.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, bool out_f32,
                           const float* s_in, float* s_out, int64_t B, int64_t Hq, int64_t Hkv,
                           int64_t N, const Bf16Plan& plan, const void* workspace, hipStream_t stream);

// dst[i] = src ? src[i] : 0 for i < n.
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream);

hipError_t launch_decode(float* S, const void* q, const void* k, const void* v, void* o,
                         bool in_bf16, bool out_f32, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t d, int64_t dv, hipStream_t stream);

}  // namespace la
