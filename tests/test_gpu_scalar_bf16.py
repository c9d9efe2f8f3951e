"""bf16 inputs at shapes the matrix-core kernels are not built for (head sizes
other than 128 and 64, d != dv, blocks other than 64 tokens) run on the scalar
float32-FMA kernels: forward, variants and backward against the oracle.

The bf16 inputs widen to float32 exactly and the arithmetic is float32, so
float32 outputs are held to the float32 bar (1e-5 of the RMS) and bf16
outputs to that bar plus their own rounding (2^-8 of |ref|).
"""
import pytest
import torch

import long_context_attention_chunkwise_amd as la
import oracle
from long_context_attention_chunkwise_amd import synth
from gpu_util import check_close, check_state, f64, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16, F32 = torch.bfloat16, torch.float32


def inputs(B, Hq, Hkv, N, d, dv, seed, relu_gen=True):
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, 64, BF16, relu_gen, False)
    return synth.make_qkv(w, DEV, seed=seed)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dv,block,out_dtype", [
    (1, 4, 2, 300, 64, 64, 32, F32),     # head size 64 with 32-token blocks
    (2, 2, 2, 257, 96, 32, 64, BF16),    # d != dv, ragged tail, bf16 output
    (1, 8, 2, 200, 128, 128, 32, F32),   # head size 128 with 32-token blocks
])
def test_forward_bf16_scalar(B, Hq, Hkv, N, d, dv, block, out_dtype):
    need_gpu()
    say(f"case scalar bf16 forward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} block={block} out={out_dtype}")
    q, k, v = inputs(B, Hq, Hkv, N, d, dv, seed=N + d)
    S0 = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 1, scale=0.5)
    assert la.workspace_bytes(B, Hq, Hkv, N, d, dv, block, BF16) == 0
    o, S = la.forward(q, k, v, block=block, out_dtype=out_dtype, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), block, f64(S0))
    check_close("o", f64(o), ref_o, F32, out_dtype)
    check_state("S_out", f64(S), ref_S, F32)


def test_variants_bf16_scalar():
    """ReLU-normalised causal and non-causal forms at head size 96."""
    need_gpu()
    say("case scalar bf16 variants d=96")
    q, k, v = inputs(1, 4, 2, 333, 96, 96, seed=7, relu_gen=False)
    S0 = synth.random_state((1, 2, 96, 96), DEV, seed=8, scale=0.5)
    Z0 = synth.random_state((1, 2, 96), DEV, seed=9).abs()
    for causal in (True, False):
        o, S, Z = la.forward_variant(q, k, v, causal=causal, feature_map="relu", normalize=True, eps=1e-6,
                                     out_dtype=F32, s_in=S0, z_in=Z0, return_state=True)
        torch.cuda.synchronize()
        ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=causal, relu=True, normalize=True,
                                             eps=1e-6, s_in=f64(S0), z_in=f64(Z0))
        check_close(f"o causal={causal}", f64(o), ref_o, F32, F32, per_row=True)
        check_state(f"S_out causal={causal}", f64(S), ref_S, F32)
        check_state(f"z_out causal={causal}", f64(Z), ref_z, F32)


@pytest.mark.parametrize("grad_dtype", [F32, BF16])
def test_backward_bf16_scalar(grad_dtype):
    """Gradients at d = 64, dv = 96 with both state terms."""
    need_gpu()
    say(f"case scalar bf16 backward grad={grad_dtype}")
    q, k, v = inputs(1, 4, 2, 250, 64, 96, seed=11)
    do = synth.make_grad((1, 4, 250, 96), DEV, seed=12)
    S0 = synth.random_state((1, 2, 64, 96), DEV, seed=13, scale=0.5)
    dS = synth.random_state((1, 2, 64, 96), DEV, seed=14, scale=0.5)
    got = la.backward(q, k, v, do, grad_dtype=grad_dtype, s_in=S0, grad_s_out=dS, return_state_grad=True)
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, f64(S0), f64(dS))
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check_close(name, f64(g), r, F32, grad_dtype)
    check_state("ds_in", f64(got[3]), ref[3], F32)
