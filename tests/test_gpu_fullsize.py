"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on outputs and states the fp64 oracle can compute: whole KV groups at
65,536 tokens, head/sequence slices and recomputed final states at 1,048,576
tokens, sampled sequences of the 256-sequence decode workload, and a
4,194,304-token sequence prefilled in 1M-token chunks with the state carried.
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


def group_slice(q, k, v, g, G, a, b):
    return (f64(q[:, g * G:(g + 1) * G, a:b]), f64(k[:, g:g + 1, a:b]), f64(v[:, g:g + 1, a:b]))


def test_gqa_64k_groups_and_states():
    """B=1, 128 query heads over 32 KV heads, N=65,536: three whole KV groups
    (12 query heads, every token), bf16 and fp32 output, and every final state."""
    need_gpu()
    w = synth.WORKLOADS["gqa_64k"]
    G = w.Hq // w.Hkv
    say(f"case gqa_64k: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N}")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    o16, S = la.forward(q, k, v, return_state=True)
    o32 = la.forward(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for g in (0, 17, 31):
        qs, ks, vs = group_slice(q, k, v, g, G, 0, w.N)
        ref, ref_S = oracle.chunkwise(qs, ks, vs, w.block)
        check_close(f"group {g} o (bf16 out)", f64(o16[:, g * G:(g + 1) * G]), ref, torch.bfloat16, torch.bfloat16)
        check_close(f"group {g} o (fp32 out)", f64(o32[:, g * G:(g + 1) * G]), ref, torch.bfloat16, torch.float32)
    check_state("all final states", f64(S), oracle.final_state(f64(k), f64(v)), torch.bfloat16)


@pytest.mark.parametrize("workload", ["gqa_1m", "gqa_1m_d64", "mha_1m_d64"])
def test_gqa_1m_slices_and_states(workload):
    """B=1, 128/32 heads, N=1,048,576, head sizes 128 and 64 (and 32/32 heads
    at 64: one-wave workgroups, 32 segments per head), through
    la_forward_states + la_forward_outputs (the benchmark's step): KV groups
    0, 13 and 31 on the first and last 65,536 tokens and on 8192-token windows
    across the boundaries of segments 0/1 and 3/4; the final state of every
    KV head (each against an fp64 GEMM over all its tokens) and the start state
    of every segment of KV heads 0, 13 and 31 as the pre-pass left it in the
    workspace, at the state bar (with four query heads per KV head the inner
    segment boundaries of KV head g sit ((g mod 16) - 8) * 2 + 1 blocks before
    the multiples of the segment length: heads 0, 13 and 31 cover shifts -15,
    11 and 15); finiteness of every output and bitwise
    repeatability of the whole pass; the final states once more from the
    state-only call (la_forward_state).  For the 128-head-size workload the same
    slices are checked once more with float32 output at the literal 2e-2 RMS.
    About 1-2 minutes per workload, most of it the fp64 state GEMMs on the host."""
    need_gpu()
    w = synth.WORKLOADS[workload]
    G = w.Hq // w.Hkv
    say(f"case {workload}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    import ctypes
    lib = la.load_library()
    P = ctypes.c_void_p
    ws_bytes = la.workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, torch.bfloat16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=DEV)
    sp = P(torch.cuda.current_stream().cuda_stream)

    def run(o, s_out, out_code=la.LA_BF16):
        assert lib.la_forward_states(P(k.data_ptr()), P(v.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block,
                                     la.LA_BF16, None, P(ws.data_ptr()), ws_bytes, sp) == 0
        assert lib.la_forward_outputs(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), w.B,
                                      w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16, out_code, None,
                                      None if s_out is None else P(s_out.data_ptr()), P(ws.data_ptr()), ws_bytes,
                                      sp) == 0

    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device=DEV)
    run(o, S)
    S_only = la.forward_state(k, v)   # the same final state without the outputs
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    W = 65536
    # segments per chain at 1M tokens on 256 compute units, and pre-pass parts per summed segment:
    # 8 segments (four-wave workgroups) in 2 parts at head size 128 and 3 at 64 (two and three pre-pass
    # workgroups per compute unit), 32 in 1 part (one-wave workgroups: head size 64, Hq = Hkv)
    nseg, nparts = (32, 1) if (w.d == 64 and w.Hq == w.Hkv) else (8, 2 if w.d == 128 else 3)
    seg = w.N // nseg
    shifted = G % 4 == 0  # the four-head kernel (not the one-wave one)

    def bound(g, j):
        """First token of segment j of KV head g, as the library places it."""
        if j == 0:
            return 0
        if j == nseg:
            return w.N
        return j * seg - ((((g % 16) - 8) * 2 + 1) * w.block if shifted else 0)

    assert ws_bytes == (w.Hkv * (nseg - 1) * nparts + w.Hkv * nseg) * w.d * w.dv * 4
    # segment start states as the pre-pass and scan left them: [Hkv][segment][d][dv] after the partials
    starts = ws.view(torch.float32)[w.Hkv * (nseg - 1) * nparts * w.d * w.dv:].view(w.Hkv, nseg, w.d, w.dv)

    o2 = torch.empty_like(o)
    run(o2, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    del o2
    o32 = None
    if w.d == 128:
        o32 = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.float32, device=DEV)
        run(o32, None, la.LA_F32)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o32).all())

    def check_slice(g, a, b, s_a):
        qs, ks, vs = group_slice(q, k, v, g, G, a, b)
        ref = oracle.chunkwise(qs, ks, vs, w.block, s_a)[0]
        hs = slice(g * G, (g + 1) * G)
        check_close(f"group {g} tokens [{a}, {b})", f64(o[:, hs, a:b]), ref, torch.bfloat16, torch.bfloat16)
        if o32 is not None:
            check_close(f"group {g} tokens [{a}, {b}) fp32 out", f64(o32[:, hs, a:b]), ref, torch.bfloat16,
                        torch.float32)

    for g in range(w.Hkv):
        ks_all, vs_all = f64(k[:, g:g + 1]), f64(v[:, g:g + 1])
        ref_final = oracle.final_state(ks_all, vs_all)
        check_state(f"group {g} final state", f64(S[:, g:g + 1]), ref_final, torch.bfloat16)
        check_state(f"group {g} final state (state only)", f64(S_only[:, g:g + 1]), ref_final, torch.bfloat16)
        if g not in (0, 13, 31):
            continue
        # start state of every segment (j = 0 is zero: no initial state), the
        # fp64 state of the tokens before it, summed segment by segment
        ref_j = np.zeros((1, 1, w.d, w.dv))
        for j in range(nseg):
            check_state(f"group {g} segment {j} start state", f64(starts[g, j])[None, None], ref_j,
                        torch.bfloat16)
            a, b = bound(g, j), bound(g, j + 1)
            ref_j = oracle.final_state(ks_all[:, :, a:b], vs_all[:, :, a:b], ref_j)
        check_slice(g, 0, W, None)
        # windows across the boundaries of segments 0/1 and 3/4, from the fp64 state before them
        for c in (bound(g, 1), bound(g, 4)):
            a, b = c - 4096, c + 4096
            check_slice(g, a, b, oracle.final_state(ks_all[:, :, :a], vs_all[:, :, :a]))
        a = w.N - W
        check_slice(g, a, w.N, oracle.final_state(ks_all[:, :, :a], vs_all[:, :, :a]))
        del ks_all, vs_all


def test_decode_256_sequences():
    """256 sequences, 128/32 heads, d = dv = 128: state from the forward kernel
    over a seeded 8192-token prefix, then 1000 decode steps.  Checked against
    the oracle: the prefix state of every sequence (an fp64 GEMM over its 8192
    tokens, one sequence at a time); every step's outputs of 16 sampled
    sequences (for 2 of them by the oracle's decode step repeated 1000 times,
    for all 16 by the oracle's causal sum over the 1000 step tokens from the
    prefix state, which the oracle's pins equate with the recurrence); and the
    final state of every sequence (its prefix state plus the sum over the steps
    of k^T v, one sequence at a time).  About a minute, most of it the host's
    fp64 work."""
    need_gpu()
    w = synth.WORKLOADS["decode_256"]
    say(f"case decode_256: B={w.B} Hq={w.Hq} Hkv={w.Hkv} prefix={w.N} steps={w.steps}")
    rng = np.random.default_rng(123)
    seqs = np.sort(rng.choice(w.B, 16, replace=False))
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=DEV)
    batch = 32
    ref_pre = np.empty((w.B, w.Hkv, w.d, w.dv))
    for i in range(0, w.B, batch):
        q, k, v = synth.make_qkv(w, DEV, seed=1000 + i // batch, B=batch)
        la.forward(q, k, v, s_out=S[i:i + batch])
        del q
        for j in range(batch):
            ref_pre[i + j] = oracle.final_state(f64(k[j:j + 1]), f64(v[j:j + 1]))[0]
        del k, v
    torch.cuda.synchronize()
    check_state("prefix states (all 256 sequences)", f64(S), ref_pre, torch.bfloat16)

    qs, ks, vs = synth.make_decode_steps(w, DEV, seed=1, steps=w.steps)
    o = torch.empty((w.B, w.Hq, w.dv), dtype=torch.float32, device=DEV)
    sidx = torch.as_tensor(seqs, device=DEV)
    outs = []
    for t in range(w.steps):
        la.decode_step(S, qs[t], ks[t], vs[t], out=o)
        outs.append(o.index_select(0, sidx))
    torch.cuda.synchronize()
    got = f64(torch.stack(outs, dim=2))                 # [16, Hq, T, dv]
    del outs

    # the 16 sequences' step tokens as sequences of length T: [16, H, T, dim]
    q_s, k_s, v_s = (f64(x.index_select(1, sidx)).transpose(1, 2, 0, 3) for x in (qs, ks, vs))
    pre16 = ref_pre[seqs]
    ref_out = oracle.chunkwise(q_s, k_s, v_s, w.block, pre16)[0]
    check_close("decode outputs (16 sequences x 1000 steps)", got, ref_out, torch.bfloat16, torch.float32)
    # 2 of them by the token recurrence, one oracle decode step after another
    Sref = pre16[:2].copy()
    rec = np.empty((2, w.Hq, w.steps, w.dv))
    for t in range(w.steps):
        Sref, rec[:, :, t] = oracle.decode_step(Sref, q_s[:2, :, t], k_s[:2, :, t], v_s[:2, :, t])
    check_close("decode outputs by the recurrence (2 sequences x 1000 steps)", got[:2], rec, torch.bfloat16,
                torch.float32)
    del q_s, got, ref_out, rec

    # final state of every sequence: prefix state + sum over the steps of k^T v
    ref_final = np.empty_like(ref_pre)
    for b in range(w.B):
        kb = f64(ks[:, b]).transpose(1, 0, 2)[None]    # [1, Hkv, T, d]
        vb = f64(vs[:, b]).transpose(1, 0, 2)[None]
        ref_final[b] = oracle.final_state(kb, vb, ref_pre[b:b + 1])[0]
    check_state("final states (all 256 sequences)", f64(S), ref_final, torch.bfloat16)
    check_state("oracle recurrence vs closed form (2 sequences)", Sref, ref_final[seqs[:2]], torch.float32)


def test_gqa_4m_chunked_prefill():
    """4,194,304 tokens (the pages' longest context) as four 1M-token chunks
    through la_forward_ex with the state carried in place (s_in = s_out).
    Q/K/V/O of the whole sequence (320 GiB) do not fit one GPU; the chunks do.
    Checked for KV groups 0 and 31: the first 4096 tokens of every chunk (each
    starts from the carried state) and the state after every chunk, against
    the oracle's running state."""
    need_gpu()
    w = synth.WORKLOADS["gqa_1m"]
    G = w.Hq // w.Hkv
    chunks = 4
    say(f"case gqa_4m_chunked: {chunks} x {w.N} tokens, Hq={w.Hq} Hkv={w.Hkv}")
    S = torch.zeros((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=DEV)
    ws = torch.empty(la.workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device=DEV)
    groups = (0, 31)
    S_ref = {g: np.zeros((1, 1, w.d, w.dv)) for g in groups}
    W = 4096
    for c in range(chunks):
        q, k, v = synth.make_qkv(w, DEV, seed=100 + c)
        la.forward(q, k, v, s_in=S, s_out=S, out=o, workspace=ws)
        torch.cuda.synchronize()
        for g in groups:
            qs, ks, vs = group_slice(q, k, v, g, G, 0, W)
            check_close(f"chunk {c} group {g} tokens [{c * w.N}, {c * w.N + W})",
                        f64(o[:, g * G:(g + 1) * G, :W]),
                        oracle.chunkwise(qs, ks, vs, w.block, S_ref[g])[0], torch.bfloat16, torch.bfloat16)
            S_ref[g] = oracle.final_state(f64(k[:, g:g + 1]), f64(v[:, g:g + 1]), S_ref[g])
            check_state(f"state after chunk {c} group {g}", f64(S[:, g:g + 1]), S_ref[g], torch.bfloat16)
        del q, k, v
