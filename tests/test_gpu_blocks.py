"""Blocks longer than 64 tokens.  The chunkwise form is an exact
re-association of the causal sum (page "MiniMax-01与Lightning Attention",
section 2.2), so the library computes any block that is a multiple of 64 as
64-token blocks.  Checked here: each such call matches the oracle's chunkwise
evaluation at that block size (the pages' chunkwise code defaults to 128) at
the usual bar, and equals the 64-token call bit for bit, for the forward,
variants and backward, bf16 and float32 inputs.
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


def inputs(dtype, d, N, seed):
    w = synth.Workload("t", 1, 4, 1, N, d, d, 64, dtype, True, False)
    return synth.make_qkv(w, DEV, seed=seed)


@pytest.mark.parametrize("dtype,d", [(BF16, 128), (F32, 64)])
@pytest.mark.parametrize("block", [128, 4096])
def test_forward_long_blocks(dtype, d, block):
    need_gpu()
    say(f"case forward block={block} dtype={dtype} d={d}")
    q, k, v = inputs(dtype, d, 3000, seed=block + d)
    S0 = synth.random_state((1, 1, d, d), DEV, seed=5, scale=0.5)
    o, S = la.forward(q, k, v, block=block, s_in=S0, return_state=True)
    o64, S64 = la.forward(q, k, v, block=64, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), block, f64(S0))
    check_close("o", f64(o), ref_o, dtype, dtype)
    check_state("S_out", f64(S), ref_S, dtype)
    assert torch.equal(o, o64) and torch.equal(S, S64)


@pytest.mark.parametrize("dtype,d", [(BF16, 128), (F32, 64)])
def test_variant_and_backward_long_blocks(dtype, d):
    need_gpu()
    say(f"case variant/backward block=128 dtype={dtype} d={d}")
    q, k, v = inputs(dtype, d, 1000, seed=17 + d)
    a = la.forward_variant(q, k, v, feature_map="relu", normalize=True, eps=1e-6, block=128)
    b = la.forward_variant(q, k, v, feature_map="relu", normalize=True, eps=1e-6, block=64)
    do = synth.make_grad((1, 4, 1000, d), DEV, seed=3, dtype=dtype)
    g = la.backward(q, k, v, do, block=128)
    g64 = la.backward(q, k, v, do, block=64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for x, y in zip(g, g64):
        assert torch.equal(x, y)
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 128)
    for name, x, r in zip(("dq", "dk", "dv"), g, ref[:3]):
        check_close(name, f64(x), r, dtype, dtype)
