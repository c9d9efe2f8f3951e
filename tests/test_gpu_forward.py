"""Forward-pass parity: the HIP path through the C ABI against the fp64 oracle.

Every input is seeded and synthetic (long_context_attention_chunkwise_amd.synth);
the oracle consumes the exact values the kernels consumed (bf16 upcast to
float64).  Sizes here span several 64-token blocks, several sequence
segments and ragged tails; the full-size workloads are checked on slices and
recomputed states in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import long_context_attention_chunkwise_amd as la
import oracle
from long_context_attention_chunkwise_amd import synth
from gpu_util import check_close, check_state, f64, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def qkv(B, Hq, Hkv, N, d, dv, dtype, seed, relu=True, scale_v=False):
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, 64, dtype, relu, scale_v)
    return synth.make_qkv(w, DEV, seed=seed)


def run_case(B, Hq, Hkv, N, d, dv, dtype, out_dtype, seed=0, block=64, s_in=False, relu=True):
    say(f"case B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} {dtype} -> {out_dtype} block={block} s_in={s_in}")
    q, k, v = qkv(B, Hq, Hkv, N, d, dv, dtype, seed, relu=relu, scale_v=(dtype == torch.float32))
    S0 = synth.random_state((B, Hkv, d, dv), DEV, seed=seed + 7, scale=0.5) if s_in else None
    o, S = la.forward(q, k, v, block=block, out_dtype=out_dtype, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), block, None if S0 is None else f64(S0))
    check_close("o", f64(o), ref_o, dtype, out_dtype)
    check_state("state", f64(S), ref_S, dtype)
    return o, S


def test_tiny_f32_matches_brute_force():
    """fp32, B=1, H=1, N=256, d=dv=64, block 64, q,k,v ~ N(0,1)/8, seed 0."""
    need_gpu()
    w = synth.WORKLOADS["tiny_f32"]
    say("case tiny_f32 (1x1x256x64 fp32, seed 0)")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    o = la.forward(q, k, v, block=w.block)
    torch.cuda.synchronize()
    check_close("o vs brute force", f64(o), oracle.brute_force(f64(q), f64(k), f64(v)), torch.float32,
                torch.float32)


@pytest.mark.parametrize("N", [1, 63, 64, 65, 200, 1000])
def test_f32_ragged_gqa_state(N):
    need_gpu()
    run_case(2, 4, 2, N, 48, 64, torch.float32, torch.float32, seed=N, block=64, s_in=True, relu=False)


@pytest.mark.parametrize("block", [1, 16, 37, 64])
def test_f32_block_sizes(block):
    need_gpu()
    run_case(1, 2, 1, 300, 64, 32, torch.float32, torch.float32, seed=3, block=block, relu=False)


def test_mha_4k_bf16():
    """B=2, Hq=Hkv=8, N=4096, d=dv=128, bf16 in, bf16 and fp32 out."""
    need_gpu()
    w = synth.WORKLOADS["mha_4k"]
    say("case mha_4k (2x8x4096x128 bf16, seed 0)")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    for out_dtype in (torch.bfloat16, torch.float32):
        o, S = la.forward(q, k, v, out_dtype=out_dtype, return_state=True)
        torch.cuda.synchronize()
        check_close(f"o ({out_dtype})", f64(o), ref_o, torch.bfloat16, out_dtype)
        check_state("state", f64(S), ref_S, torch.bfloat16)


# Group sizes 1, 2, 4, 8 (two subgroups of 4), 16 (four subgroups) and 3
# (three subgroups of 1); lengths that are not multiples of 64; short and long
# segment splits.
@pytest.mark.parametrize("Hq,Hkv,N", [
    (2, 2, 1), (2, 2, 37), (4, 2, 64), (8, 2, 65), (8, 1, 1000), (3, 1, 777),
    (4, 4, 4095), (8, 2, 3000), (16, 4, 2113), (16, 1, 1500), (4, 1, 64 * 300 + 5),
])
def test_bf16_shapes(Hq, Hkv, N):
    need_gpu()
    run_case(1, Hq, Hkv, N, 128, 128, torch.bfloat16, torch.float32, seed=N + Hq)


@pytest.mark.parametrize("s_in", [False, True])
def test_bf16_bf16_out_and_initial_state(s_in):
    need_gpu()
    run_case(2, 8, 2, 2500, 128, 128, torch.bfloat16, torch.bfloat16, seed=11, s_in=s_in)


def test_bf16_causality_prefix():
    """Outputs of the first T tokens do not depend on later tokens."""
    need_gpu()
    q, k, v = qkv(1, 8, 2, 5000, 128, 128, torch.bfloat16, seed=21)
    full = la.forward(q, k, v, out_dtype=torch.float32)
    T = 1234
    part = la.forward(q[:, :, :T].contiguous(), k[:, :, :T].contiguous(), v[:, :, :T].contiguous(),
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.chunkwise(f64(q[:, :, :T]), f64(k[:, :, :T]), f64(v[:, :, :T]), 64)[0]
    check_close("prefix run", f64(part), ref, torch.bfloat16, torch.float32)
    check_close("full run, first T rows", f64(full[:, :, :T]), ref, torch.bfloat16, torch.float32)
    # changing the future leaves the past untouched (bit for bit: same split)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 3000:] = 0
    v2[:, :, 3000:] *= -1
    full2 = la.forward(q, k2, v2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(full2[:, :, :3000], full[:, :, :3000])


def test_bf16_resume_equals_single_pass():
    need_gpu()
    q, k, v = qkv(2, 4, 2, 3001, 128, 128, torch.bfloat16, seed=31)
    M = 1337
    o_full, S_full = la.forward(q, k, v, out_dtype=torch.float32, return_state=True)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1 = la.forward(sl(q, 0, M), sl(k, 0, M), sl(v, 0, M), out_dtype=torch.float32, return_state=True)
    # resume in place: s_in and s_out are the same buffer
    o2 = la.forward(sl(q, M, 3001), sl(k, M, 3001), sl(v, M, 3001), out_dtype=torch.float32, s_in=S1, s_out=S1)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    check_close("single pass", f64(o_full), ref_o, torch.bfloat16, torch.float32)
    check_close("resumed", f64(torch.cat([o1, o2], dim=2)), ref_o, torch.bfloat16, torch.float32)
    check_state("resumed state (in place)", f64(S1), ref_S, torch.bfloat16)


def test_bf16_deterministic():
    need_gpu()
    q, k, v = qkv(1, 8, 2, 4100, 128, 128, torch.bfloat16, seed=41)
    a, Sa = la.forward(q, k, v, return_state=True)
    b, Sb = la.forward(q, k, v, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(Sa, Sb)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 8, 2, 3001), (2, 8, 1, 1000), (1, 4, 1, 64)])
def test_bf16_in_place_output(B, Hq, Hkv, N):
    """o written over q (group sizes 4 and 8, ragged tail, state carry) equals
    the out-of-place result bit for bit."""
    need_gpu()
    say(f"case in-place B={B} Hq={Hq} Hkv={Hkv} N={N}")
    q, k, v = qkv(B, Hq, Hkv, N, 128, 128, torch.bfloat16, seed=N + Hq)
    S0 = synth.random_state((B, Hkv, 128, 128), DEV, seed=N, scale=0.5)
    o, S = la.forward(q, k, v, s_in=S0, return_state=True)
    qi = q.clone()
    oi, Si = la.forward(qi, k, v, s_in=S0, return_state=True, out=qi)
    torch.cuda.synchronize()
    assert oi.data_ptr() == qi.data_ptr()
    assert torch.equal(oi, o) and torch.equal(Si, S)


def test_bf16_in_place_rejected_off_the_four_head_kernel():
    need_gpu()
    q, k, v = qkv(1, 2, 1, 500, 128, 128, torch.bfloat16, seed=3)
    with pytest.raises(la.LAError, match="LA_ERR_ALIAS"):
        la.forward(q, k, v, out=q)


@pytest.mark.parametrize("B,Hq,Hkv,N,out_dtype,s_in", [
    (1, 8, 2, 3001, torch.bfloat16, True),    # G = 4, several segments, ragged tail
    (2, 16, 2, 777, torch.float32, False),    # G = 8: two query-head subgroups
    (1, 4, 1, 64, torch.bfloat16, False),     # one block
    (1, 4, 1, 20000, torch.float32, True),    # many segments on one chain
    (2, 4, 4, 3001, torch.bfloat16, True),    # G = 1: one-wave workgroups, several segments per head
    (1, 8, 4, 777, torch.float32, False),     # G = 2
    (1, 6, 2, 2000, torch.bfloat16, True),    # G = 3: one query head per workgroup, three subgroups
    (1, 1, 1, 20000, torch.float32, True),    # a single head, many segments (one-wave workgroups)
    (1, 2, 2, 64, torch.float32, True),       # G = 1, one block
    (3, 3, 3, 1, torch.bfloat16, True),       # G = 1, one token
    (1, 32, 32, 5000, torch.bfloat16, False), # G = 1, 32 heads: more heads than one workgroup per SIMD
    (1, 12, 2, 1500, torch.bfloat16, True),   # G = 6: two query heads per workgroup, three subgroups
])
def test_bf16_head_size_64(B, Hq, Hkv, N, out_dtype, s_in):
    """Head size 64 on the matrix cores: the four-wave kernel (four query heads
    per workgroup, or two with the other waves idle), one-wave workgroups for
    one query head per KV head, and their pre-pass."""
    need_gpu()
    if N > 64:
        assert la.workspace_bytes(B, Hq, Hkv, N, 64, 64, 64, torch.bfloat16) > 0   # the matrix-core split
    run_case(B, Hq, Hkv, N, 64, 64, torch.bfloat16, out_dtype, seed=N + Hq, s_in=s_in)


def test_bf16_head_size_64_in_place_and_resume():
    """Head size 64: a 3000-token sequence resumed after 1000 tokens, the
    second chunk written in place over its queries with the state carried in
    place, matches the oracle; the in-place call equals the out-of-place one
    bit for bit."""
    need_gpu()
    q, k, v = qkv(1, 8, 2, 3000, 64, 64, torch.bfloat16, seed=77)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1 = la.forward(sl(q, 0, 1000), sl(k, 0, 1000), sl(v, 0, 1000), return_state=True)
    q2, k2, v2 = sl(q, 1000, 3000), sl(k, 1000, 3000), sl(v, 1000, 3000)
    o2_ref = la.forward(q2, k2, v2, s_in=S1.clone())
    qi = q2.clone()
    o2 = la.forward(qi, k2, v2, s_in=S1, s_out=S1, out=qi)
    torch.cuda.synchronize()
    assert o2.data_ptr() == qi.data_ptr() and torch.equal(o2, o2_ref)
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    check_close("resumed o (second chunk in place)", f64(torch.cat([o1, o2], dim=2)), ref_o, torch.bfloat16,
                torch.bfloat16)
    check_state("resumed state (in place)", f64(S1), ref_S, torch.bfloat16)


def test_bf16_head_size_64_one_head_per_kv_head_in_place_state_and_resume():
    """Head size 64, one query head per KV head (one-wave workgroups): a
    9000-token sequence resumed after 2000 tokens with the state carried in
    place (s_out = s_in), against the oracle, and the single pass."""
    need_gpu()
    q, k, v = qkv(2, 3, 3, 9000, 64, 64, torch.bfloat16, seed=91)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o_full, S_full = la.forward(q, k, v, return_state=True)
    o1, S = la.forward(sl(q, 0, 2000), sl(k, 0, 2000), sl(v, 0, 2000), return_state=True)
    o2 = la.forward(sl(q, 2000, 9000), sl(k, 2000, 9000), sl(v, 2000, 9000), s_in=S, s_out=S)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    check_close("single pass", f64(o_full), ref_o, torch.bfloat16, torch.bfloat16)
    check_state("single pass state", f64(S_full), ref_S, torch.bfloat16)
    check_close("resumed", f64(torch.cat([o1, o2], dim=2)), ref_o, torch.bfloat16, torch.bfloat16)
    check_state("resumed state (in place)", f64(S), ref_S, torch.bfloat16)


def test_empty_sequence_state_passthrough():
    need_gpu()
    for dtype in (torch.bfloat16, torch.float32):
        d = 128 if dtype == torch.bfloat16 else 64
        q = torch.empty((1, 4, 0, d), dtype=dtype, device=DEV)
        k = torch.empty((1, 2, 0, d), dtype=dtype, device=DEV)
        v = torch.empty((1, 2, 0, d), dtype=dtype, device=DEV)
        S0 = synth.random_state((1, 2, d, d), DEV, seed=5)
        o, S = la.forward(q, k, v, s_in=S0, return_state=True)
        _, Sz = la.forward(q, k, v, return_state=True)
        torch.cuda.synchronize()
        assert o.shape == (1, 4, 0, d)
        assert torch.equal(S, S0) and torch.count_nonzero(Sz) == 0


def test_forward_then_decode_equals_forward():
    """Prefill with the forward kernel, then decode token by token: same as
    one forward pass over the whole sequence (outputs and state)."""
    need_gpu()
    q, k, v = qkv(2, 8, 2, 700, 128, 128, torch.bfloat16, seed=51)
    P = 640
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    _, S = la.forward(sl(q, 0, P), sl(k, 0, P), sl(v, 0, P), return_state=True)
    outs = []
    for t in range(P, 700):
        outs.append(la.decode_step(S, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous()))
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    check_close("decoded outputs", np.stack([f64(x) for x in outs], axis=2), ref_o[:, :, P:], torch.bfloat16,
                torch.float32)
    check_state("state after decode", f64(S), ref_S, torch.bfloat16)
