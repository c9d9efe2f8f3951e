"""Backward-pass parity: la_backward through the C ABI against the fp64
oracle's block-wise backward (itself pinned by finite differences in
test_oracle_backward.py).

Inputs are seeded and synthetic: q, k, v from synth.make_qkv (the forward
workloads' distributions), the upstream gradient dO ~ N(0,1) from
synth.make_grad, optional initial state and final-state gradient N(0,1)*0.5.
Sizes span several 64-token blocks, several reverse segments per chain (the
per-segment sums of q^T dO, written by the dQ pass where its segments are the
dK/dV kernel's and by the separate pre-pass over (Q, dO) otherwise, and the
reverse scan), ragged tails, group sizes 1 to 8,
head sizes 128 and 64 and both gradient dtypes; the 1M-token workloads (head
sizes 128 and 64) are checked on their first and last 4096 tokens and on a
window across a segment boundary in the middle, with the states entering each
window computed in float64.
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
BF16 = torch.bfloat16


def inputs(B, Hq, Hkv, N, seed, d=128):
    w = synth.Workload("t", B, Hq, Hkv, N, d, d, 64, BF16, True, False)
    q, k, v = synth.make_qkv(w, DEV, seed=seed)
    do = synth.make_grad((B, Hq, N, d), DEV, seed=seed + 1)
    return q, k, v, do


def check_grads(tag, got, ref, grad_dtype):
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check_close(f"{tag} {name}", f64(g), r, BF16, grad_dtype)
    if len(got) > 3:
        check_state(f"{tag} ds_in", f64(got[3]), ref[3], BF16)


@pytest.mark.parametrize("B,Hq,Hkv,N,grad_dtype,s_in,ds_out", [
    (1, 4, 1, 3000, torch.float32, False, False),     # G = 4, 11 segments, ragged tail
    (2, 8, 2, 777, BF16, True, True),                 # G = 4, bf16 gradients, both state terms
    (1, 2, 2, 100, torch.float32, True, False),       # G = 1, two blocks
    (1, 6, 2, 1000, torch.float32, False, True),      # G = 3 (dQ forward with one head per workgroup)
    (1, 4, 2, 64, BF16, False, False),                # one full block
    (1, 4, 2, 1, torch.float32, True, True),          # one token
    (1, 8, 1, 4100, BF16, False, False),              # G = 8, dQ forward subgroups (sums from the dQ pass)
    (1, 16, 2, 40000, BF16, True, True),              # G = 8, dQ and dK/dV segments differ: the pre-pass
    (1, 24, 3, 19200, BF16, False, True),             # G = 8, three KV heads, dQ segments not whole dK/dV ones
])
def test_backward_matches_oracle(B, Hq, Hkv, N, grad_dtype, s_in, ds_out):
    need_gpu()
    say(f"case backward B={B} Hq={Hq} Hkv={Hkv} N={N} grad={grad_dtype} s_in={s_in} ds_out={ds_out}")
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=N + Hq)
    S0 = synth.random_state((B, Hkv, 128, 128), DEV, seed=N + 11, scale=0.5) if s_in else None
    dS = synth.random_state((B, Hkv, 128, 128), DEV, seed=N + 12, scale=0.5) if ds_out else None
    got = la.backward(q, k, v, do, grad_dtype=grad_dtype, s_in=S0, grad_s_out=dS, return_state_grad=True)
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, None if S0 is None else f64(S0),
                                    None if dS is None else f64(dS))
    check_grads("", got, ref, grad_dtype)


@pytest.mark.parametrize("B,Hq,Hkv,N,grad_dtype,s_in,ds_out", [
    (1, 4, 1, 3000, torch.float32, False, False),     # G = 4, 11 segments, ragged tail
    (2, 8, 2, 777, BF16, True, True),                 # bf16 gradients, both state terms
    (1, 4, 2, 64, BF16, False, False),                # one full block
    (1, 4, 1, 1, torch.float32, True, True),          # one token
    (1, 8, 1, 4100, BF16, False, True),               # G = 8
    (1, 16, 4, 20000, BF16, True, True),              # G = 4, four chains of many segments
    (2, 4, 4, 3000, torch.float32, True, True),       # G = 1 (dQ on one-wave workgroups)
    (1, 2, 2, 70, BF16, True, True),                  # G = 1, two blocks
    (1, 6, 3, 777, BF16, False, True),                # G = 2
    (1, 3, 1, 1000, torch.float32, True, False),      # G = 3
    (1, 8, 2, 65536, BF16, True, True),               # G = 4, two dK/dV segments per dQ segment
])
def test_backward_head_size_64(B, Hq, Hkv, N, grad_dtype, s_in, ds_out):
    """d = dv = 64, any group size: dQ on the forward kernels (four-wave
    workgroups of one, two or four query heads, one-wave workgroups for one
    query head per KV head), dK/dV on the four-wave reverse kernel."""
    need_gpu()
    say(f"case backward d=64 B={B} Hq={Hq} Hkv={Hkv} N={N} grad={grad_dtype} s_in={s_in} ds_out={ds_out}")
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=N + Hq + 64, d=64)
    S0 = synth.random_state((B, Hkv, 64, 64), DEV, seed=N + 13, scale=0.5) if s_in else None
    dS = synth.random_state((B, Hkv, 64, 64), DEV, seed=N + 14, scale=0.5) if ds_out else None
    got = la.backward(q, k, v, do, grad_dtype=grad_dtype, s_in=S0, grad_s_out=dS, return_state_grad=True)
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, None if S0 is None else f64(S0),
                                    None if dS is None else f64(dS))
    check_grads("d=64", got, ref, grad_dtype)


def test_backward_empty_sequence():
    """N = 0: no gradients to write; ds_in equals ds_out (zeros without it)."""
    need_gpu()
    q = torch.empty((1, 4, 0, 128), dtype=BF16, device=DEV)
    k = torch.empty((1, 1, 0, 128), dtype=BF16, device=DEV)
    dS = synth.random_state((1, 1, 128, 128), DEV, seed=5)
    got = la.backward(q, k, k, q, grad_s_out=dS, return_state_grad=True)
    zero = la.backward(q, k, k, q, return_state_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(got[3], dS) and bool((zero[3] == 0).all())


@pytest.mark.parametrize("d", [128, 64])
def test_backward_in_place_state_gradient_and_chunks(d):
    """A 6000-token sequence as two chunks: forward with the state carried,
    then backward from the last chunk to the first with grad_s_in written in
    place over grad_s_out; equals the oracle's whole-sequence gradients."""
    need_gpu()
    B, Hq, Hkv, N, a = 1, 8, 2, 6000, 2500
    say(f"case backward chunks B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} split={a}")
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=31, d=d)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=32, scale=0.5)
    parts = [(0, a), (a, N)]
    S_a = la.forward(q[:, :, :a].contiguous(), k[:, :, :a].contiguous(), v[:, :, :a].contiguous(), s_in=S0,
                     return_state=True)[1]
    dS = torch.zeros((B, Hkv, d, d), dtype=torch.float32, device=DEV)
    grads = {}
    for (lo, hi), s in reversed(list(zip(parts, (S0, S_a)))):
        sl = [x[:, :, lo:hi].contiguous() for x in (q, k, v, do)]
        dq, dk, dv = la.backward(*sl, grad_dtype=torch.float32, s_in=s, grad_s_out=dS, grad_s_in=dS)[:3]
        grads[lo] = (dq, dk, dv)
    torch.cuda.synchronize()
    got = [torch.cat([grads[0][i], grads[a][i]], dim=2) for i in range(3)] + [dS]
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, f64(S0))
    check_grads("chunked", got, ref, torch.float32)


@pytest.mark.parametrize("d", [128, 64])
def test_backward_repeatable(d):
    """Two calls on the same inputs give bitwise-identical gradients (fixed
    reduction orders everywhere)."""
    need_gpu()
    q, k, v, do = inputs(1, 8, 2, 20000, seed=41, d=d)
    a = la.backward(q, k, v, do, return_state_grad=True)
    b = la.backward(q, k, v, do, return_state_grad=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("workload", ["gqa_1m", "gqa_1m_d64"])
def test_backward_gqa_1m_slices(workload):
    """B=1, 128/32 heads, N=1,048,576 (the forward workloads at head sizes 128
    and 64), bf16 gradients.
    For KV groups 0 and 31: dk, dv of the last 4096 tokens (they depend on
    those tokens only), dk, dv, dq of the first 4096 tokens (the reverse state
    entering them is sum over the group's heads of Q^T dO over every later
    token, computed in float64 here), dq of the last 4096 tokens (from the
    forward state of (V, K) before them) and the initial-state gradient; for
    KV group 13, dq, dk, dv of a 4096-token window across a segment boundary
    in the middle of the sequence."""
    need_gpu()
    w = synth.WORKLOADS[workload]
    G = w.Hq // w.Hkv
    N, W = w.N, 4096
    say(f"case backward {workload}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} d={w.d}")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    do = synth.make_grad((w.B, w.Hq, N, w.dv), DEV, seed=1)
    dq, dk, dv, ds = la.backward(q, k, v, do, return_state_grad=True)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert bool(torch.isfinite(x).all())
    for g in (0, 31):
        hs = slice(g * G, (g + 1) * G)
        gs = slice(g, g + 1)
        a = N - W
        # last W tokens: dk, dv from the tokens after them only
        tail = oracle.backward_chunkwise(f64(q[:, hs, a:]), f64(k[:, gs, a:]), f64(v[:, gs, a:]),
                                         f64(do[:, hs, a:]), 64)
        check_close(f"group {g} dk tokens [{a}, {N})", f64(dk[:, gs, a:]), tail[1], BF16, BF16)
        check_close(f"group {g} dv tokens [{a}, {N})", f64(dv[:, gs, a:]), tail[2], BF16, BF16)
        # dq of the last W tokens: forward state of (V, K) over the earlier tokens
        S_vk = oracle.final_state(f64(v[:, gs, :a]), f64(k[:, gs, :a]))
        ref_dq = oracle.chunkwise(f64(do[:, hs, a:]), f64(v[:, gs, a:]), f64(k[:, gs, a:]), 64, S_vk)[0]
        check_close(f"group {g} dq tokens [{a}, {N})", f64(dq[:, hs, a:]), ref_dq, BF16, BF16)
        # first W tokens: the reverse state after them
        R = np.zeros((1, 1, w.d, w.dv))
        for h in range(G):
            qh = f64(q[:, g * G + h, W:])[0]
            doh = f64(do[:, g * G + h, W:])[0]
            R[0, 0] += qh.T @ doh
            del qh, doh
        head = oracle.backward_chunkwise(f64(q[:, hs, :W]), f64(k[:, gs, :W]), f64(v[:, gs, :W]),
                                         f64(do[:, hs, :W]), 64, None, R)
        check_close(f"group {g} dk tokens [0, {W})", f64(dk[:, gs, :W]), head[1], BF16, BF16)
        check_close(f"group {g} dv tokens [0, {W})", f64(dv[:, gs, :W]), head[2], BF16, BF16)
        check_close(f"group {g} dq tokens [0, {W})", f64(dq[:, hs, :W]), head[0], BF16, BF16)
        check_state(f"group {g} ds_in", f64(ds[:, gs]), head[3], BF16)
    # KV group 13: a window across a segment boundary at the middle (8 or 16 segments per chain),
    # from the forward state of (K, V) before it and the reverse state after it, in float64
    g, c = 13, N // 2
    a, b = c - W // 2, c + W // 2
    hs, gs = slice(g * G, (g + 1) * G), slice(g, g + 1)
    S_a = oracle.final_state(f64(k[:, gs, :a]), f64(v[:, gs, :a]))
    R = np.zeros((1, 1, w.d, w.dv))
    for h in range(G):
        qh = f64(q[:, g * G + h, b:])[0]
        doh = f64(do[:, g * G + h, b:])[0]
        R[0, 0] += qh.T @ doh
        del qh, doh
    mid = oracle.backward_chunkwise(f64(q[:, hs, a:b]), f64(k[:, gs, a:b]), f64(v[:, gs, a:b]),
                                    f64(do[:, hs, a:b]), 64, S_a, R)
    for name, x, r in zip(("dq", "dk", "dv"), (dq[:, hs, a:b], dk[:, gs, a:b], dv[:, gs, a:b]), mid[:3]):
        check_close(f"group {g} {name} tokens [{a}, {b})", f64(x), r, BF16, BF16)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dv,block,state", [
    (1, 3, 1, 300, 64, 64, 64, True),      # G = 3, ragged tail, both state terms
    (2, 3, 3, 130, 128, 96, 32, False),    # G = 1, d != dv, 32-token blocks
    (1, 8, 2, 257, 32, 128, 16, True),     # G = 4, 16-token blocks
    (1, 4, 1, 1, 64, 64, 64, True),        # one token
])
def test_backward_f32_matches_oracle(B, Hq, Hkv, N, d, dv, block, state):
    """float32 inputs and gradients (the float32 FMA kernels) against the
    oracle at the float32 bar, 1e-5 of each gradient's RMS."""
    need_gpu()
    say(f"case backward f32 B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} block={block} state={state}")
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, block, torch.float32, False, True)
    q, k, v = synth.make_qkv(w, DEV, seed=N + d)
    do = synth.make_grad((B, Hq, N, dv), DEV, seed=N + d + 1, dtype=torch.float32)
    S0 = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 21, scale=0.5) if state else None
    dS = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 22, scale=0.5) if state else None
    got = la.backward(q, k, v, do, block=block, s_in=S0, grad_s_out=dS, return_state_grad=True)
    torch.cuda.synchronize()
    assert all(g.dtype == torch.float32 for g in got)
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), block, None if S0 is None else f64(S0),
                                    None if dS is None else f64(dS))
    for name, g, r in zip(("dq", "dk", "dv", "ds_in"), got, ref):
        check_close(f"f32 {name}", f64(g), r, torch.float32, torch.float32)


def test_backward_f32_in_place_state_gradient():
    """float32: grad_s_in written over grad_s_out gives the same gradients."""
    need_gpu()
    say("case backward f32 in place ds")
    w = synth.Workload("t", 1, 4, 2, 200, 64, 96, 64, torch.float32, False, True)
    q, k, v = synth.make_qkv(w, DEV, seed=31)
    do = synth.make_grad((1, 4, 200, 96), DEV, seed=32, dtype=torch.float32)
    dS = synth.random_state((1, 2, 64, 96), DEV, seed=33, scale=0.5)
    ref = la.backward(q, k, v, do, grad_s_out=dS, return_state_grad=True)
    buf = dS.clone()
    got = la.backward(q, k, v, do, grad_s_out=buf, grad_s_in=buf)
    torch.cuda.synchronize()
    for a, b in zip(ref[:3], got[:3]):
        assert torch.equal(a, b)
    assert torch.equal(ref[3], buf)
