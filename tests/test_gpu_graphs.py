"""HIP-graph capture of the library's entry points (what a serving loop
does): la_forward_ex with caller-owned workspace and a loop of
la_decode_step calls are captured once into graphs and replayed several
times, with eager work and synchronisations between the replays; every
replay must equal the eager result bit for bit.  The entry points allocate
nothing and clear memory with kernels, never with memset nodes.
"""
import pytest
import torch

import long_context_attention_chunkwise_amd as la
from long_context_attention_chunkwise_amd import synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_forward_ex_graph_replays():
    need_gpu()
    say("case graph: la_forward_ex, B=1 Hq=8 Hkv=2 N=5000 bf16, s_in and s_out, 4 replays")
    w = synth.Workload("t", 1, 8, 2, 5000, 128, 128, 64, torch.bfloat16, True, False)
    q, k, v = synth.make_qkv(w, DEV, seed=1)
    S0 = synth.random_state((1, 2, 128, 128), DEV, seed=2, scale=0.5)
    ws = torch.empty(max(la.workspace_bytes(1, 8, 2, 5000, 128, 128), 16), dtype=torch.uint8, device=DEV)
    o = torch.empty((1, 8, 5000, 128), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((1, 2, 128, 128), dtype=torch.float32, device=DEV)
    ref_o, ref_S = la.forward(q, k, v, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.forward(q, k, v, s_in=S0, out=o, s_out=S, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.forward(q, k, v, s_in=S0, out=o, s_out=S, workspace=ws)
    for i in range(4):
        o.fill_(0)
        S.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(S, ref_S), f"replay {i}"
        _ = (q.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_decode_loop_graph_replays():
    need_gpu()
    say("case graph: 8 decode steps captured, 3 replays, 64 sequences")
    w = synth.Workload("t", 64, 128, 32, 0, 128, 128, 64, torch.bfloat16, True, False, 8)
    qs, ks, vs = synth.make_decode_steps(w, DEV, seed=3, steps=8)
    S_init = synth.random_state((64, 32, 128, 128), DEV, seed=4, scale=0.1)
    o = torch.empty((8, 64, 128, 128), dtype=torch.float32, device=DEV)

    def run(S):
        for t in range(8):
            la.decode_step(S, qs[t], ks[t], vs[t], out=o[t])

    S_ref = S_init.clone()
    run(S_ref)
    o_ref = o.clone()
    torch.cuda.synchronize()
    S = S_init.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(S)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(S)
    for i in range(3):
        S.copy_(S_init)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref) and torch.equal(o, o_ref), f"replay {i}"
