/*
 * la.h — C ABI of liblightning.so: causal chunkwise linear attention
 * (Lightning Attention) forward pass, its backward pass, its feature-map,
 * normalised and non-causal variants, state-only passes (the final state and
 * the initial-state gradient alone), and batched single-token decode on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  Page "如何理解MiniMax股价创历史新高？拆解国产大模型技术底座"
 * (vergex.cn), section "Lightning Attention：长上下文为什么突然变得便宜了", chunkwise
 * teaching code: per head, with a running d x dv state S (zero unless s_in is
 * given), each block of `block` tokens produces
 *     O_b = Q_b S + tril(Q_b K_b^T) V_b      (diagonal kept)
 * and only then updates S <- S + K_b^T V_b.  In exact arithmetic this equals
 *     o_t = q_t . s_in + sum_{s <= t} (q_t . k_s) v_s,
 * for every block size (associativity; page "MiniMax-01与Lightning Attention",
 * section 2.2).  Apart from la_forward_variant, no normalisation, scaling or
 * feature map is applied: q and k arrive already feature-mapped.  Query head
 * h reads KV head h / (Hq / Hkv) (grouped-query attention with contiguous
 * groups; same page, section 1.1 table: 128 heads over 32 KV heads).
 *
 * Layouts (all row-major and contiguous, element strides implied by the
 * sizes, every pointer 16-byte aligned):
 *     q [B][Hq][N][d]    k [B][Hkv][N][d]    v [B][Hkv][N][dv]
 *     o [B][Hq][N][dv]   state [B][Hkv][d][dv] (float32)
 * Decode tensors drop the N axis: q [B][Hq][d], k [B][Hkv][d], v [B][Hkv][dv],
 * o [B][Hq][dv].
 *
 * Ownership and errors.  Every buffer is device memory owned by the caller;
 * the library keeps no global mutable state other than the fixed scratch of
 * la_forward_noalloc.  Calls are asynchronous on
 * `stream` (a hipStream_t; NULL is the default stream).  Arguments are
 * validated before anything is launched: on any error status nothing is
 * written and nothing is enqueued.  LA_ERR_HIP reports a failed launch or
 * runtime call; faults during execution surface at the next synchronisation.
 * No C++ exception crosses this interface.
 */
#ifndef LIGHTNING_LA_H
#define LIGHTNING_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL */
  LA_ERR_SHAPE = 2,       /* a size <= 0 (N may be 0 for forward), or Hq % Hkv != 0 */
  LA_ERR_UNSUPPORTED = 3, /* head size, block size or dtype combination not built */
  LA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  LA_ERR_ALIAS = 5,       /* an output overlaps an input */
  LA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than la_forward_workspace_bytes */
  LA_ERR_HIP = 7,         /* HIP runtime or launch error */
  LA_ERR_TOO_LARGE = 8,   /* la_forward_noalloc: the problem needs more than its fixed scratch */
  /* Range sentinels (not statuses): every 32-bit int is a value of the type, so
   * an out-of-range code passed in from C is well defined and reported as such
   * (the same holds for la_dtype and la_feature_map below). */
  LA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  LA_STATUS_RANGE_MAX_ = 2147483647
} la_status;

typedef enum {
  LA_F32 = 0,
  LA_BF16 = 1,
  LA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  LA_DTYPE_RANGE_MAX_ = 2147483647
} la_dtype;

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void* la_stream;

/*
 * Causal forward pass, zero initial state, final state discarded.
 * in_dtype / out_dtype:
 *   LA_F32  -> LA_F32   float32 arithmetic throughout (no reduced precision);
 *                       d in 1..128, dv a multiple of 32 up to 128.
 *   LA_BF16 -> LA_BF16 or LA_F32
 *                       d = dv = 128 or 64 (any Hq / Hkv): bf16
 *                       matrix-core products with float32
 *                       accumulation and a float32 state.  Other shapes within
 *                       the LA_F32 limits: the float32 FMA kernels on the
 *                       exactly widened inputs (a small-problem path, workspace
 *                       size 0).
 * block: 1..64, or any multiple of 64 up to 2^20 tokens (the pages' chunkwise
 * code defaults to 128-token blocks).  A multiple of 64 is computed as 64-token
 * blocks, the tile the kernels are built for: since the chunkwise form is an
 * exact re-association of the causal sum, the result is the same for every
 * block size up to rounding.  A block below 64 is taken as given (float32 FMA
 * kernels only; the matrix-core kernels need a multiple of 64).
 * N may be 0 (then q, k, v and o may be NULL and only s_out is written) and
 * need not be a multiple of block: the last block is shorter.  Temporary
 * workspace (see la_forward_workspace_bytes) is allocated stream-ordered on
 * `stream` and released after use.
 */
la_status la_forward(const void* q, const void* k, const void* v, void* o,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                     int64_t d, int64_t dv, int64_t block,
                     la_dtype in_dtype, la_dtype out_dtype, la_stream stream);

/*
 * la_forward with state carry and caller-owned workspace.
 *   s_in   [B][Hkv][d][dv] float32 initial state, or NULL for zeros.
 *   s_out  [B][Hkv][d][dv] float32 state after token N-1, or NULL.
 *          s_out may equal s_in (in-place resume); any other overlap with an
 *          input is LA_ERR_ALIAS.
 *   o      may be q itself (the output overwrites the queries, saving one
 *          [B][Hq][N][dv] buffer) when in_dtype = out_dtype = LA_BF16,
 *          d = dv = 128 or 64, block a multiple of 64 and Hq / Hkv a
 *          multiple of 4:
 *          there each query row is read before the same output row is
 *          written, by the same wave.  The result equals the out-of-place
 *          one bit for bit.  Any other overlap of o with an input is
 *          LA_ERR_ALIAS (la_forward and la_forward_outputs follow the same
 *          rule).
 *   workspace / workspace_bytes: at least la_forward_workspace_bytes(...)
 *          bytes of device memory (may be NULL when that size is 0).  Its
 *          contents are scratch and need no initialisation.  Concurrent calls
 *          must not share one workspace.
 * Resuming is exact up to rounding: forward_ex over tokens [0, M) with s_out,
 * then over [M, N) with that state as s_in, equals one pass over [0, N).
 */
la_status la_forward_ex(const void* q, const void* k, const void* v, void* o,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                        int64_t d, int64_t dv, int64_t block,
                        la_dtype in_dtype, la_dtype out_dtype,
                        const float* s_in, float* s_out,
                        void* workspace, size_t workspace_bytes,
                        la_stream stream);

/*
 * The two phases of la_forward_ex, for callers that schedule or time them
 * separately (same arguments and validation as la_forward_ex).
 *
 * la_forward_states: the long sequence of each (batch, KV head) is processed
 * as several segments in parallel; this phase writes into `workspace` the
 * state at the start of every segment, s_in + sum over earlier tokens of
 * k_s^T v_s (exact by associativity: page "奧特曼的“溫和奇點”愿景，線性注意力的
 * 勝利？MiniMax-M1技術報告深度解析" (digipub.cc), the A*B*C = A*(B*C) passage).
 * It reads k, v and s_in only.  A no-op when the workspace size is 0.
 *
 * la_forward_outputs: the outputs and s_out, starting every segment from the
 * states la_forward_states left in `workspace`.  The caller must have run
 * la_forward_states with the same sizes, dtype, k, v and s_in on the same
 * stream first (or with an event dependency); the workspace is read only.
 */
la_status la_forward_states(const void* k, const void* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                            int64_t d, int64_t dv, int64_t block, la_dtype in_dtype,
                            const float* s_in, void* workspace, size_t workspace_bytes,
                            la_stream stream);

la_status la_forward_outputs(const void* q, const void* k, const void* v, void* o,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                             int64_t d, int64_t dv, int64_t block,
                             la_dtype in_dtype, la_dtype out_dtype,
                             const float* s_in, float* s_out,
                             const void* workspace, size_t workspace_bytes,
                             la_stream stream);

/*
 * Workspace bytes la_forward_ex needs for this problem on the current device
 * (0 when none).  Returns 0 for invalid arguments as well; la_forward_ex then
 * reports the argument error itself.
 */
size_t la_forward_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                  int64_t d, int64_t dv, int64_t block,
                                  la_dtype in_dtype);

/*
 * State only, no outputs: for every (batch, KV head),
 *     s_out = s_in + sum over the N tokens of k_t^T v_t
 * (s_in zero if NULL): the state the forward pass ends with (its s_out),
 * which is all a later chunk or a decode step needs from these tokens (page
 * "MiniMax-01与Lightning Attention", section 4.1 table: the key-value state is
 * updated incrementally), without reading q or writing o.  It is also the
 * per-shard total that a sequence split over several devices exchanges: with
 * shard totals T_0 .. T_{M-1}, shard j's forward starts from s_in + T_0 + ...
 * + T_{j-1} (associativity; page "奧特曼的“溫和奇點”愿景，線性注意力的勝利？
 * MiniMax-M1技術報告深度解析" (digipub.cc), the A*B*C = A*(B*C) passage).
 *   k [B][Hkv][N][d], v [B][Hkv][N][dv] in in_dtype (NULL allowed when N = 0);
 *   s_in, s_out [B][Hkv][d][dv] float32; s_out may be s_in (in place) and
 *   must not overlap k or v; s_in may be NULL.
 *   Shapes and dtypes as la_forward_ex with Hq = Hkv (bf16 with d = dv = 128
 *   or 64 on the matrix cores; float32, or bf16 at other head sizes, on float32
 *   FMA).  The result does not depend on a block size.
 *   workspace / workspace_bytes: at least la_forward_state_workspace_bytes
 *   bytes (may be NULL when that is 0); scratch, no initialisation needed.
 * Statuses as la_forward_ex (LA_ERR_NULL also for a NULL s_out).
 */
la_status la_forward_state(const void* k, const void* v,
                           int64_t B, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                           la_dtype in_dtype, const float* s_in, float* s_out,
                           void* workspace, size_t workspace_bytes, la_stream stream);

/* Workspace bytes la_forward_state needs on the current device (0 when none
 * or for invalid arguments). */
size_t la_forward_state_workspace_bytes(int64_t B, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                                        la_dtype in_dtype);

/*
 * la_forward_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call) and computes exactly la_forward_ex
 * (same kernels, bit-for-bit the same o and s_out).
 *
 * The segment-state workspace comes from a fixed array in this library's
 * device code, LA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends.  A problem whose
 * la_forward_workspace_bytes exceeds it returns LA_ERR_TOO_LARGE before
 * anything is launched; use la_forward_ex with a caller workspace then.  At
 * head size 128 on a 256-CU part, 128 query heads over 32 KV heads at
 * 1,048,576 tokens need 44 MiB, and up to 1024 (batch, KV head) pairs fit at
 * any sequence length.
 * Every call on one GPU shares that GPU's array and leaves its contents behind
 * (nothing in it needs clearing: each call writes the entries it reads before
 * reading them).  Calls that overlap in time on one GPU (two streams, or two
 * host threads) race on it and must be ordered by the caller.
 * Arguments, layouts, in-place rules and statuses otherwise as la_forward_ex.
 * The first call on a device looks up the array's device address (once per
 * device, with that device current).
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

la_status la_forward_noalloc(const void* q, const void* k, const void* v, void* o,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                             int64_t d, int64_t dv, int64_t block,
                             la_dtype in_dtype, la_dtype out_dtype,
                             const float* s_in, float* s_out, la_stream stream);

/*
 * One decode token for a batch of sequences (page "MiniMax-01与Lightning
 * Attention", section 4.1 table: the key-value state is updated incrementally
 * without keeping the history).  For every (b, KV head g):
 *     S[b][g] <- S[b][g] + k[b][g]^T v[b][g]          (in place, float32)
 * then for each query head h of group g:
 *     o[b][h] = q[b][h] . S[b][g]                     (reads the updated state)
 * so the new token attends to itself, as in the forward pass.
 *   in_dtype  LA_BF16 or LA_F32 (q, k, v); out_dtype LA_F32 or LA_BF16 (o).
 *   d in 1..128, dv a multiple of 4 up to 128, Hq / Hkv up to 1024.
 *   Arithmetic is float32.
 * Each state is read once and written once per call; groups of more than 8
 * query heads per KV head read it once more for every further 8 heads.
 */
la_status la_decode_step(float* S, const void* q, const void* k, const void* v, void* o,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t dv,
                         la_dtype in_dtype, la_dtype out_dtype, la_stream stream);

/*
 * Forward variants: feature map, non-causal form and normalisation.
 *   fmap      LA_FMAP_IDENTITY (q, k used as given) or LA_FMAP_RELU: phi = ReLU
 *             applied to q and k inside the kernels (the feature map of the
 *             LinearAttentionCore code, page "MiniMax-01与Lightning Attention",
 *             section 2.2, without its learned linear layer).
 *   causal    1: o_t sums over s <= t, as la_forward_ex; 0: over every token
 *             of the sequence (LinearAttentionCore: phi(Q) (phi(K)^T V)).
 *   normalize 0: o_t = phi(q_t) . S_t.  1: o_t = phi(q_t) . S_t / (phi(q_t) . z_t + eps),
 *             z_t = z_in + sum of phi(k_s) over the same tokens as S_t (the
 *             kernel-approximation family cited on page "从 Transformer 到
 *             Lightning Attention，从 PPO 到 CISPO", "Transformers are RNNs").
 *             eps >= 0, finite.  A row whose denominator is 0 (eps = 0 and no
 *             positive weight) comes out as the IEEE quotient (NaN or inf).
 *   S_t       = s_in + sum of phi(k_s)^T v_s over the same tokens.
 *   s_in, s_out   as la_forward_ex (s_out = s_in + sum over all tokens).
 *   z_in, z_out   [B][Hkv][d] float32 normaliser sums, or NULL; only with
 *                 normalize = 1 (LA_ERR_UNSUPPORTED otherwise).  z_out may
 *                 equal z_in.
 * in_dtype LA_BF16 (matrix-core kernels at d = dv = 128, block a multiple of
 * 64, and also at d = dv = 64; out_dtype LA_BF16 or LA_F32) or LA_F32 (out_dtype LA_F32).  Other shapes,
 * d up to 128, dv a multiple of 32 up to 128, block as for la_forward, run on
 * the float32 FMA kernels (workspace size 0), for bf16 inputs too.  Any
 * Hq / Hkv.
 * causal = 1, LA_FMAP_IDENTITY, normalize = 0 computes exactly la_forward_ex.
 * Workspace: la_forward_variant_workspace_bytes (may be 0).
 */
typedef enum {
  LA_FMAP_IDENTITY = 0,
  LA_FMAP_RELU = 1,
  LA_FMAP_RANGE_MIN_ = -2147483647 - 1,
  LA_FMAP_RANGE_MAX_ = 2147483647
} la_feature_map;

la_status la_forward_variant(const void* q, const void* k, const void* v, void* o,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                             int64_t d, int64_t dv, int64_t block,
                             la_dtype in_dtype, la_dtype out_dtype,
                             int causal, la_feature_map fmap, int normalize, float eps,
                             const float* s_in, float* s_out,
                             const float* z_in, float* z_out,
                             void* workspace, size_t workspace_bytes, la_stream stream);

size_t la_forward_variant_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                          int64_t d, int64_t dv, int64_t block,
                                          la_dtype in_dtype, int causal, int normalize);

/*
 * Backward pass of la_forward_ex: the gradients of a scalar loss L given
 * grad_o = dL/do and, optionally, grad_s_out = dL/ds_out.  The pages define
 * only the forward; differentiating its exact form (page
 * "如何理解MiniMax股价创历史新高？拆解国产大模型技术底座", section "Lightning
 * Attention", with the grouped heads of page "MiniMax-01与Lightning Attention",
 * section 1.1)
 *     o_t   = q_t . s_in + sum_{s <= t} (q_t . k_s) v_s
 *     s_out = s_in + sum_s k_s^T v_s
 * gives, with h over the query heads of a KV head's group,
 *     dq_t  = grad_o_t . s_in^T + sum_{s <= t} (grad_o_t . v_s) k_s
 *     dk_s  = v_s . grad_s_out^T + sum_h sum_{t >= s} (v_s . grad_o_ht) q_ht
 *     dv_s  = k_s . grad_s_out   + sum_h sum_{t >= s} (k_s . q_ht) grad_o_ht
 *     ds_in = grad_s_out + sum_h sum_t q_ht^T grad_o_ht
 * dq is computed as the forward recurrence over (grad_o, v, k) from s_in^T;
 * dk, dv and ds_in by the same block recurrence run from the last block to
 * the first with a float32 d x dv state that starts at grad_s_out.
 *
 *   q, k, v        the forward's inputs (layouts as above).
 *   grad_o         [B][Hq][N][dv], in_dtype.
 *   in_dtype       LA_BF16: grad_dtype LA_BF16 or LA_F32; matrix-core
 *                  kernels at d = dv = 128 or 64, block a multiple of 64.
 *                  LA_F32:
 *                  grad_dtype LA_F32.  Other shapes, d and dv multiples of 32
 *                  up to 128 and block as for la_forward, run on float32 FMA
 *                  kernels (a small-problem path), for bf16 inputs too.
 *   grad_q, grad_k, grad_v   outputs shaped like q, k, v, in grad_dtype;
 *                  every element is written.
 *   s_in           the forward's initial state, or NULL for zeros (used for dq).
 *   grad_s_out     [B][Hkv][d][dv] float32 gradient on the forward's final
 *                  state, or NULL for zeros.
 *   grad_s_in      [B][Hkv][d][dv] float32 output, or NULL.  May equal
 *                  grad_s_out (in place); no other output may overlap an
 *                  input or another output (LA_ERR_ALIAS).
 *   N may be 0 (then only grad_s_in is written).
 *   workspace / workspace_bytes: at least la_backward_workspace_bytes(...)
 *                  bytes of device memory, scratch, not shared by concurrent
 *                  calls.
 * A sequence processed in chunks with la_forward_ex (state carried from chunk
 * to chunk) is differentiated by calling la_backward on the chunks from the
 * last to the first, each with its own s_in and with the grad_s_in of the
 * chunk after it as grad_s_out.
 */
la_status la_backward(const void* q, const void* k, const void* v, const void* grad_o,
                      void* grad_q, void* grad_k, void* grad_v,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                      int64_t d, int64_t dv, int64_t block,
                      la_dtype in_dtype, la_dtype grad_dtype,
                      const float* s_in, const float* grad_s_out, float* grad_s_in,
                      void* workspace, size_t workspace_bytes, la_stream stream);

/* Workspace bytes la_backward needs on the current device (0 for N = 0 or
 * invalid arguments). */
size_t la_backward_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                   int64_t d, int64_t dv, int64_t block,
                                   la_dtype in_dtype);

/*
 * The initial-state gradient alone, without dq, dk and dv:
 *     grad_s_in = grad_s_out + sum_h sum_t q_ht^T grad_o_ht
 * per (batch, KV head), h over the query heads of its group (grad_s_out zero
 * if NULL): la_backward's grad_s_in, which depends on q and grad_o only.  In
 * a sequence split over devices, shard j's backward takes as grad_s_out the
 * global one plus these sums over the later shards (the mirror of
 * la_forward_state).
 *   q [B][Hq][N][d], grad_o [B][Hq][N][dv] in in_dtype (NULL allowed when
 *   N = 0); grad_s_out, grad_s_in [B][Hkv][d][dv] float32, grad_s_in
 *   required, may be grad_s_out (in place), must not overlap q or grad_o.
 *   Shapes and dtypes as la_forward_state with Hq query heads over Hkv.
 *   workspace / workspace_bytes: at least la_backward_state_workspace_bytes.
 */
la_status la_backward_state(const void* q, const void* grad_o,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t dv,
                            la_dtype in_dtype, const float* grad_s_out, float* grad_s_in,
                            void* workspace, size_t workspace_bytes, la_stream stream);

/* Workspace bytes la_backward_state needs on the current device (0 when none
 * or for invalid arguments). */
size_t la_backward_state_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                         int64_t d, int64_t dv, la_dtype in_dtype);

/* Static, NUL-terminated description of a status code. */
const char* la_status_str(la_status status);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_LA_H */
