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
    at 64: one query head per four-wave workgroup), through
    la_forward_states + la_forward_outputs (the benchmark's step): KV groups
    0, 13 and 31 on the first and last 65,536 tokens and on 8192-token windows
    across the boundaries of segments 0/1 and 3/4, their final states,
    finiteness of every output and bitwise repeatability of the whole pass."""
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

    def run(o, s_out):
        assert lib.la_forward_states(P(k.data_ptr()), P(v.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block,
                                     la.LA_BF16, None, P(ws.data_ptr()), ws_bytes, sp) == 0
        assert lib.la_forward_outputs(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), w.B,
                                      w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16, la.LA_BF16, None,
                                      None if s_out is None else P(s_out.data_ptr()), P(ws.data_ptr()), ws_bytes,
                                      sp) == 0

    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device=DEV)
    run(o, S)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    W = 65536
    seg = w.N // 8   # 8 segments per chain at 1M tokens (both head sizes), one workgroup each
    assert ws_bytes == (32 * 7 * 3 + 32 * 8) * w.d * w.dv * 4   # 7 summed segments in 3 parts + 8 starts
    for g in (0, 13, 31):
        ks_all, vs_all = f64(k[:, g:g + 1]), f64(v[:, g:g + 1])
        qs, ks, vs = group_slice(q, k, v, g, G, 0, W)
        check_close(f"group {g} tokens [0, {W})", f64(o[:, g * G:(g + 1) * G, :W]),
                    oracle.chunkwise(qs, ks, vs, w.block)[0], torch.bfloat16, torch.bfloat16)
        # windows across the boundaries of segments 0/1 and 3/4, from the fp64 state before them
        for c in (seg, 4 * seg):
            a, b = c - 4096, c + 4096
            S_a = oracle.final_state(ks_all[:, :, :a], vs_all[:, :, :a])
            qs, ks, vs = group_slice(q, k, v, g, G, a, b)
            check_close(f"group {g} tokens [{a}, {b})", f64(o[:, g * G:(g + 1) * G, a:b]),
                        oracle.chunkwise(qs, ks, vs, w.block, S_a)[0], torch.bfloat16, torch.bfloat16)
        a = w.N - W
        S_a = oracle.final_state(ks_all[:, :, :a], vs_all[:, :, :a])
        qs, ks, vs = group_slice(q, k, v, g, G, a, w.N)
        check_close(f"group {g} tokens [{a}, {w.N})", f64(o[:, g * G:(g + 1) * G, a:]),
                    oracle.chunkwise(qs, ks, vs, w.block, S_a)[0], torch.bfloat16, torch.bfloat16)
        check_state(f"group {g} final state", f64(S[:, g:g + 1]), oracle.final_state(ks_all, vs_all),
                    torch.bfloat16)
        del ks_all, vs_all
    o2 = torch.empty_like(o)
    run(o2, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_decode_256_sequences():
    """256 sequences, 128/32 heads, d = dv = 128: state from the forward kernel
    over a seeded 8192-token prefix, then 1000 decode steps.  Checked against
    the oracle: 16 sampled prefix states; every step's outputs of 2 of those
    sequences (the oracle's token recurrence); the outputs of all 16 at sampled
    steps (the oracle's state before the step in closed form, then its decode
    step); and the final states of the 16."""
    need_gpu()
    w = synth.WORKLOADS["decode_256"]
    G = w.Hq // w.Hkv
    say(f"case decode_256: B={w.B} Hq={w.Hq} Hkv={w.Hkv} prefix={w.N} steps={w.steps}")
    rng = np.random.default_rng(123)
    seqs = np.sort(rng.choice(w.B, 16, replace=False))
    out_seqs = seqs[:2]
    check_steps = [0, 1, 2, 99, 500, 998, 999]
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=DEV)
    batch = 32
    pre_k, pre_v, pre_q = {}, {}, {}
    for i in range(0, w.B, batch):
        q, k, v = synth.make_qkv(w, DEV, seed=1000 + i // batch, B=batch)
        la.forward(q, k, v, s_out=S[i:i + batch])
        for s in seqs:
            if i <= s < i + batch:
                pre_k[s], pre_v[s] = f64(k[s - i:s - i + 1]), f64(v[s - i:s - i + 1])
        del q, k, v
    torch.cuda.synchronize()
    ref_pre = {s: oracle.final_state(pre_k[s], pre_v[s]) for s in seqs}
    check_state("prefix states (16 sequences)", np.concatenate([f64(S[s:s + 1]) for s in seqs]),
                np.concatenate([ref_pre[s] for s in seqs]), torch.bfloat16)

    qs, ks, vs = synth.make_decode_steps(w, DEV, seed=1, steps=w.steps)
    o = torch.empty((w.B, w.Hq, w.dv), dtype=torch.float32, device=DEV)
    idx = torch.as_tensor(out_seqs, device=DEV)
    sidx = torch.as_tensor(seqs, device=DEV)
    outs, sampled = [], {}
    for t in range(w.steps):
        la.decode_step(S, qs[t], ks[t], vs[t], out=o)
        outs.append(o.index_select(0, idx))
        if t in check_steps:
            sampled[t] = o.index_select(0, sidx)
    torch.cuda.synchronize()
    got = np.stack([f64(x) for x in outs])            # [T, 2, Hq, dv]

    q_s, k_s, v_s = (f64(x.index_select(1, sidx)) for x in (qs, ks, vs))   # [T, 16, H, d]
    # outputs of 2 sequences, all steps, by the oracle's token recurrence
    Sref = np.concatenate([ref_pre[s] for s in out_seqs])
    ref_out = np.empty_like(got)
    for t in range(w.steps):
        Sref, ref_out[t] = oracle.decode_step(Sref, q_s[t, :2], k_s[t, :2], v_s[t, :2])
    check_close("decode outputs (2 sequences x 1000 steps)", got, ref_out, torch.bfloat16, torch.float32)
    # outputs of all 16 sequences at sampled steps: state before step t in closed form
    pre16 = np.concatenate([ref_pre[s] for s in seqs])
    for t in check_steps:
        S_before = oracle.final_state(np.transpose(k_s[:t], (1, 2, 0, 3)), np.transpose(v_s[:t], (1, 2, 0, 3)),
                                      pre16)
        _, o_ref = oracle.decode_step(S_before, q_s[t], k_s[t], v_s[t])
        check_close(f"decode outputs (16 sequences, step {t})", f64(sampled[t]), o_ref, torch.bfloat16,
                    torch.float32)
    # final states of 16 sequences: prefix state + sum over steps of k^T v
    ref_final = oracle.final_state(np.transpose(k_s, (1, 2, 0, 3)), np.transpose(v_s, (1, 2, 0, 3)),
                                   np.concatenate([ref_pre[s] for s in seqs]))
    check_state("final states (16 sequences)", f64(S.index_select(0, sidx)), ref_final, torch.bfloat16)
    check_close("oracle recurrence vs closed form (2 sequences)", Sref, ref_final[:2], torch.float32,
                torch.float32)


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
