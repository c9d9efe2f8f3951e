"""Argument checks of the Python binding on the GPU: each malformed call
raises before anything is enqueued, and a preset output is left untouched.
"""
import pytest
import torch

import long_context_attention_chunkwise_amd as la
from long_context_attention_chunkwise_amd import synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def inputs(N=512, Hq=8, Hkv=2):
    w = synth.Workload("t", 1, Hq, Hkv, N, 128, 128, 64, torch.bfloat16, True, False)
    return synth.make_qkv(w, DEV, seed=91)


def test_forward_argument_checks():
    need_gpu()
    say("case binding checks: forward")
    q, k, v = inputs()
    o = torch.full((1, 8, 512, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    bad = [
        (ValueError, dict(q=q.transpose(2, 3).contiguous().transpose(2, 3))),      # non-contiguous q
        (ValueError, dict(k=k.cpu())),                                             # host tensor
        (TypeError, dict(v=v.float())),                                            # mixed dtypes
        (ValueError, dict(v=v[:, :, :256].contiguous())),                          # length mismatch
        (ValueError, dict(s_in=torch.zeros(1, 2, 128, 128, dtype=torch.float64, device=DEV))),  # s_in dtype
        (ValueError, dict(out=torch.empty(1, 8, 512, 128, dtype=torch.float32, device=DEV))),  # out dtype
        (ValueError, dict(workspace=torch.empty(1 << 26, dtype=torch.uint8))),     # host workspace
        (ValueError, dict(workspace=torch.empty(1 << 26, dtype=torch.uint8, device=DEV)[::2])),  # strided
    ]
    for exc, kw in bad:
        args = dict(q=q, k=k, v=v, out=o)
        args.update(kw)
        with pytest.raises(exc):
            la.forward(args.pop("q"), args.pop("k"), args.pop("v"), **args)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
    # a device workspace that is large enough is used as given
    ws = torch.empty(la.workspace_bytes(1, 8, 2, 512, 128, 128) + 64, dtype=torch.uint8, device=DEV)
    ref = la.forward(q, k, v)
    assert torch.equal(la.forward(q, k, v, workspace=ws), ref)


def test_variant_backward_decode_argument_checks():
    need_gpu()
    say("case binding checks: variant, backward, decode")
    q, k, v = inputs()
    with pytest.raises(ValueError):
        la.forward_variant(q, k, v, feature_map="softmax")
    with pytest.raises(ValueError):
        la.forward_variant(q, k, v, normalize=True, z_in=torch.zeros(1, 2, 64, device=DEV))
    with pytest.raises(ValueError):
        la.forward_variant(q, k, v, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    do = synth.make_grad((1, 8, 512, 128), DEV, seed=92)
    with pytest.raises(ValueError):
        la.backward(q, k, v, do[:, :, :500].contiguous())
    with pytest.raises(ValueError):
        la.backward(q, k, v, do, workspace=torch.empty(1 << 26, dtype=torch.uint8))
    S = torch.zeros(2, 2, 128, 128, device=DEV)
    qt = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device=DEV)
    kt = torch.zeros(2, 2, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        la.decode_step(S.double(), qt, kt, kt)
    with pytest.raises(ValueError):
        la.decode_step(S, qt, kt[:, :1].contiguous(), kt)
    with pytest.raises(ValueError):
        la.decode_step(S, qt, kt, kt, out=torch.empty(2, 8, 64, device=DEV))  # out too small
    torch.cuda.synchronize()
    assert bool((S == 0).all())
