"""GPU checks of the remaining C-ABI entry points and decode variants.

la_forward (allocating), la_forward_states + la_forward_outputs with an
initial state, and la_decode_step across group sizes, head sizes and dtypes,
each against the fp64 oracle or bit-for-bit against la_forward_ex.
"""
import ctypes

import numpy as np
import pytest
import torch

import long_context_attention_chunkwise_amd as la
import oracle
from long_context_attention_chunkwise_amd import synth
from gpu_util import check_close, check_state, f64, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = ctypes.c_void_p


def stream():
    return P(torch.cuda.current_stream().cuda_stream)


def qkv(B, Hq, Hkv, N, d, dv, dtype, seed):
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, 64, dtype, dtype == torch.bfloat16, dtype == torch.float32)
    return synth.make_qkv(w, DEV, seed=seed)


@pytest.mark.parametrize("dtype,Hq,Hkv,N,d,dv", [
    (torch.bfloat16, 8, 2, 3000, 128, 128),
    (torch.float32, 4, 2, 500, 64, 64),
])
def test_la_forward_matches_forward_ex(dtype, Hq, Hkv, N, d, dv):
    """The allocating entry point computes exactly what la_forward_ex does."""
    need_gpu()
    say(f"case la_forward {dtype} Hq={Hq} Hkv={Hkv} N={N}")
    lib = la.load_library()
    q, k, v = qkv(1, Hq, Hkv, N, d, dv, dtype, seed=61)
    code = la.LA_BF16 if dtype == torch.bfloat16 else la.LA_F32
    o = torch.empty((1, Hq, N, dv), dtype=dtype, device=DEV)
    st = lib.la_forward(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), 1, Hq, Hkv, N, d, dv,
                        64, code, code, stream())
    assert st == 0, la.status_str(st)
    ref = la.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    check_close("o", f64(o), oracle.chunkwise(f64(q), f64(k), f64(v), 64)[0], dtype, dtype)


def test_two_phase_entry_points_with_initial_state():
    """la_forward_states then la_forward_outputs (with s_in and s_out) equals
    la_forward_ex bit for bit and the oracle within tolerance."""
    need_gpu()
    lib = la.load_library()
    B, Hq, Hkv, N, d = 2, 8, 2, 5000, 128
    q, k, v = qkv(B, Hq, Hkv, N, d, d, torch.bfloat16, seed=71)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=72, scale=0.3)
    ws_bytes = la.workspace_bytes(B, Hq, Hkv, N, d, d, 64, torch.bfloat16)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=DEV)
    S = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=DEV)
    st = lib.la_forward_states(P(k.data_ptr()), P(v.data_ptr()), B, Hq, Hkv, N, d, d, 64, la.LA_BF16,
                               P(S0.data_ptr()), P(ws.data_ptr()), ws_bytes, stream())
    assert st == 0, la.status_str(st)
    st = lib.la_forward_outputs(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), B, Hq, Hkv, N,
                                d, d, 64, la.LA_BF16, la.LA_F32, P(S0.data_ptr()), P(S.data_ptr()),
                                P(ws.data_ptr()), ws_bytes, stream())
    assert st == 0, la.status_str(st)
    o_ex, S_ex = la.forward(q, k, v, out_dtype=torch.float32, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ex) and torch.equal(S, S_ex)
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64, f64(S0))
    check_close("o", f64(o), ref_o, torch.bfloat16, torch.float32)
    check_state("state", f64(S), ref_S, torch.bfloat16)


def test_rejected_call_writes_nothing():
    """An argument error returns before anything is enqueued."""
    need_gpu()
    lib = la.load_library()
    N = 4096
    q, k, v = qkv(1, 4, 2, N, 128, 128, torch.bfloat16, seed=81)
    o = torch.full((1, 4, N, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    assert la.workspace_bytes(1, 4, 2, N, 128, 128, 64, torch.bfloat16) > 16
    scratch = torch.empty(16, dtype=torch.uint8, device=DEV)
    # workspace too small
    st = lib.la_forward_ex(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), 1, 4, 2, N,
                           128, 128, 64, la.LA_BF16, la.LA_BF16, None, None, P(scratch.data_ptr()), 16, stream())
    assert st == 6
    # output overlapping an input
    st = lib.la_forward_ex(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(q.data_ptr() + 256), 1, 4, 2,
                           N, 128, 128, 64, la.LA_BF16, la.LA_BF16, None, None, None, 0, stream())
    assert st == 5
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


@pytest.mark.parametrize("G,d,dv,in_dtype,out_dtype", [
    (1, 128, 128, torch.bfloat16, torch.float32),
    (2, 128, 128, torch.bfloat16, torch.bfloat16),
    (4, 64, 96, torch.float32, torch.float32),
    (8, 128, 128, torch.bfloat16, torch.float32),
    (3, 100, 36, torch.float32, torch.bfloat16),
    (12, 128, 128, torch.bfloat16, torch.float32),   # groups above 8: chunks of 8 + 4
    (17, 128, 64, torch.bfloat16, torch.bfloat16),   # 8 + 8 + 1
    (32, 64, 64, torch.float32, torch.float32),      # four chunks of 8
])
def test_decode_variants(G, d, dv, in_dtype, out_dtype):
    """20 decode steps on a random initial state against the oracle's decode_step."""
    need_gpu()
    B, Hkv = 5, 3
    Hq = G * Hkv
    say(f"case decode G={G} d={d} dv={dv} {in_dtype}->{out_dtype}")
    S = synth.random_state((B, Hkv, d, dv), DEV, seed=90 + G, scale=0.5)
    Sref = f64(S)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(91)
    outs, refs = [], []
    for _ in range(20):
        q = (torch.randn((B, Hq, d), generator=gen, device=DEV) / np.sqrt(d)).to(in_dtype)
        k = (torch.randn((B, Hkv, d), generator=gen, device=DEV) / np.sqrt(d)).to(in_dtype)
        v = torch.randn((B, Hkv, dv), generator=gen, device=DEV).to(in_dtype)
        outs.append(la.decode_step(S, q, k, v, out_dtype=out_dtype))
        Sref, o_ref = oracle.decode_step(Sref, f64(q), f64(k), f64(v))
        refs.append(o_ref)
    torch.cuda.synchronize()
    check_close("outputs", np.stack([f64(x) for x in outs]), np.stack(refs), in_dtype, out_dtype)
    check_state("state", f64(S), Sref, in_dtype)
