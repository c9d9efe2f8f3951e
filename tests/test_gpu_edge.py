"""Degenerate inputs and extreme work splits, through the C ABI, against the
fp64 oracle or exact identities.

* Zero queries give exactly zero outputs; zero keys or zero values leave the
  state exactly s_in (float32 adds of zero) and the outputs q . s_in.
* One KV chain of 262,161 tokens: the plan cuts it into ~240 segments (the
  most the pre-pass and scans ever handle); forward and backward are checked
  on the first and last 4096 tokens and on the final state.
* Values scaled by 1000: the same relative bar holds.
* A decode step with zero k and v leaves the state unchanged.
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


def qkv(B, Hq, Hkv, N, d, dtype, seed):
    w = synth.Workload("t", B, Hq, Hkv, N, d, d, 64, dtype, dtype == BF16, dtype == torch.float32)
    return synth.make_qkv(w, DEV, seed=seed)


@pytest.mark.parametrize("dtype,d", [(BF16, 128), (torch.float32, 64)])
def test_zero_inputs(dtype, d):
    need_gpu()
    say(f"case zero inputs {dtype}")
    q, k, v = qkv(1, 8, 2, 2000, d, dtype, seed=3)
    S0 = synth.random_state((1, 2, d, d), DEV, seed=4, scale=0.5)
    zq, zk, zv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    o, S = la.forward(zq, k, v, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0
    check_state("state with zero queries", f64(S), oracle.final_state(f64(k), f64(v)), dtype)
    for name, kk, vv in (("zero keys", zk, v), ("zero values", k, zv)):
        o, S = la.forward(q, kk, vv, out_dtype=torch.float32, s_in=S0, return_state=True)
        torch.cuda.synchronize()
        assert torch.equal(S, S0), name
        check_close(f"o with {name}", f64(o), oracle.chunkwise(f64(q), f64(kk), f64(vv), 64, f64(S0))[0], dtype,
                    torch.float32)


def test_many_segments_forward_and_backward():
    """B=1, Hq=4, Hkv=1, N=262,161: one chain split into ~240 segments."""
    need_gpu()
    B, Hq, Hkv, N, W = 1, 4, 1, 4096 * 64 + 17, 4096
    say(f"case many segments: N={N}")
    q, k, v = qkv(B, Hq, Hkv, N, 128, BF16, seed=7)
    o, S = la.forward(q, k, v, out_dtype=torch.float32, return_state=True)
    do = synth.make_grad((B, Hq, N, 128), DEV, seed=8)
    dq, dk, dv, ds = la.backward(q, k, v, do, grad_dtype=torch.float32, return_state_grad=True)
    torch.cuda.synchronize()
    a = N - W
    qf, kf, vf, dof = f64(q), f64(k), f64(v), f64(do)
    S_a = oracle.final_state(kf[:, :, :a], vf[:, :, :a])
    check_close("o first tokens", f64(o[:, :, :W]), oracle.chunkwise(qf[:, :, :W], kf[:, :, :W], vf[:, :, :W], 64)[0],
                BF16, torch.float32)
    check_close("o last tokens", f64(o[:, :, a:]), oracle.chunkwise(qf[:, :, a:], kf[:, :, a:], vf[:, :, a:], 64,
                                                                     S_a)[0], BF16, torch.float32)
    check_state("final state", f64(S), oracle.final_state(kf, vf), BF16)
    # backward: last tokens depend only on later tokens; first tokens on the reverse state after them
    tail = oracle.backward_chunkwise(qf[:, :, a:], kf[:, :, a:], vf[:, :, a:], dof[:, :, a:], 64)
    check_close("dk last tokens", f64(dk[:, :, a:]), tail[1], BF16, torch.float32)
    check_close("dv last tokens", f64(dv[:, :, a:]), tail[2], BF16, torch.float32)
    R = np.zeros((1, 1, 128, 128))
    for h in range(Hq):
        R[0, 0] += qf[0, h, W:].T @ dof[0, h, W:]
    head = oracle.backward_chunkwise(qf[:, :, :W], kf[:, :, :W], vf[:, :, :W], dof[:, :, :W], 64, None, R)
    check_close("dk first tokens", f64(dk[:, :, :W]), head[1], BF16, torch.float32)
    check_close("dv first tokens", f64(dv[:, :, :W]), head[2], BF16, torch.float32)
    check_close("dq first tokens", f64(dq[:, :, :W]), head[0], BF16, torch.float32)
    check_state("ds_in", f64(ds), head[3], BF16)


def test_large_values():
    """Values scaled by 1000: outputs and state keep the relative bar."""
    need_gpu()
    q, k, v = qkv(1, 8, 2, 3000, 128, BF16, seed=9)
    v = (v.float() * 1000).to(BF16)
    o, S = la.forward(q, k, v, out_dtype=torch.float32, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64)
    check_close("o", f64(o), ref_o, BF16, torch.float32)
    check_state("state", f64(S), ref_S, BF16)


def test_decode_zero_token_keeps_state():
    need_gpu()
    S = synth.random_state((3, 2, 128, 128), DEV, seed=10, scale=0.5)
    S0 = S.clone()
    q = torch.randn((3, 8, 128), device=DEV).to(BF16)
    zk = torch.zeros((3, 2, 128), dtype=BF16, device=DEV)
    o = la.decode_step(S, q, zk, zk)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    check_close("o = q S", f64(o), oracle.decode_step(f64(S0), f64(q), f64(zk), f64(zk))[1], BF16, torch.float32)
