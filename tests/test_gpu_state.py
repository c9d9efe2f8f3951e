"""la_forward_state (the final state without outputs) and la_backward_state
(the initial-state gradient without dq, dk, dv) against the oracle, and the
sequence split they serve: shard totals computed independently, added up in
order, and each shard's forward started from the sum of the earlier ones, and
each shard's backward from the global grad_s_out plus the later shards' sums,
must reproduce one pass over the whole sequence, forward and backward."""
import pytest
import torch

import long_context_attention_chunkwise_amd as la
import oracle
from long_context_attention_chunkwise_amd import synth
from gpu_util import check_close, check_state, f64, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16 = torch.bfloat16


def kv(B, Hkv, N, d, dv, dtype, seed):
    w = synth.Workload("t", B, Hkv, Hkv, N, d, dv, 64, dtype, dtype == BF16, dtype == torch.float32)
    _, k, v = synth.make_qkv(w, DEV, seed=seed)
    return k, v


@pytest.mark.parametrize("B,Hkv,N,d,dv,dtype,with_s_in,in_place", [
    (2, 3, 3000, 128, 128, BF16, True, False),        # ragged tail, two batches, s_in
    (1, 4, 777, 64, 64, BF16, False, False),          # head size 64
    (1, 2, 1, 128, 128, BF16, True, True),            # one token, in place over s_in
    (1, 2, 64, 128, 128, BF16, False, False),         # one full block
    (1, 1, 200000, 128, 128, BF16, False, False),     # one chain in hundreds of parts
    (1, 2, 1000, 64, 96, torch.float32, True, False), # float32, d != dv
    (2, 1, 300, 128, 128, torch.float32, True, True), # float32, in place
    (1, 2, 500, 96, 64, BF16, False, False),          # bf16 off the matrix-core shape
])
def test_state_matches_oracle(B, Hkv, N, d, dv, dtype, with_s_in, in_place):
    need_gpu()
    say(f"case state B={B} Hkv={Hkv} N={N} d={d} dv={dv} {dtype} s_in={with_s_in} in_place={in_place}")
    k, v = kv(B, Hkv, N, d, dv, dtype, seed=N + d)
    S0 = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 5, scale=0.5) if with_s_in else None
    ref = oracle.final_state(f64(k), f64(v), None if S0 is None else f64(S0))
    if in_place:
        got = la.forward_state(k, v, s_in=S0, out=S0)
        assert got.data_ptr() == S0.data_ptr()
    else:
        got = la.forward_state(k, v, s_in=S0)
    torch.cuda.synchronize()
    check_state("state", f64(got), ref, dtype)
    # the forward's own final state agrees with it
    if not in_place:
        q = torch.zeros((B, Hkv, N, d), dtype=dtype, device=DEV)
        _, S_fwd = la.forward(q, k, v, s_in=S0, return_state=True)
        torch.cuda.synchronize()
        check_state("forward's state", f64(S_fwd), ref, dtype)


def test_state_empty_sequence():
    need_gpu()
    say("case state N=0: s_out = s_in, or zeros")
    k = torch.empty((1, 2, 0, 128), dtype=BF16, device=DEV)
    S0 = synth.random_state((1, 2, 128, 128), DEV, seed=9, scale=0.5)
    assert torch.equal(la.forward_state(k, k, s_in=S0), S0)
    out = torch.full((1, 2, 128, 128), 7.0, device=DEV)
    la.forward_state(k, k, out=out)
    torch.cuda.synchronize()
    assert not bool(out.any())


@pytest.mark.parametrize("d", [128, 64])
def test_sequence_shards_equal_one_pass(d):
    """A 40,000-token sequence (8 query heads over 2 KV heads) split into four
    uneven shards, as a sequence-sharded run over several devices would split
    it: each shard's total state is computed on its own (la_forward_state, no
    initial state), the totals are added in shard order on top of s_in, and
    each shard's forward starts from the sum over the shards before it.  The
    outputs and the final state equal the oracle over the whole sequence."""
    need_gpu()
    B, Hq, Hkv, N = 1, 8, 2, 40000
    cuts = [0, 7000, 19000, 30500, N]
    say(f"case shards d={d} N={N} cuts={cuts}")
    w = synth.Workload("t", B, Hq, Hkv, N, d, d, 64, BF16, True, False)
    q, k, v = synth.make_qkv(w, DEV, seed=21)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=22, scale=0.5)
    shards = [(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    totals = [la.forward_state(sl(k, a, b), sl(v, a, b)) for a, b in shards]   # independent of each other
    outs, s = [], S0.clone()
    for (a, b), T in zip(shards, totals):
        o_j, S_j = la.forward(sl(q, a, b), sl(k, a, b), sl(v, a, b), s_in=s, return_state=True)
        outs.append(o_j)
        s = s + T                                                               # start of the next shard
        check_state(f"shard [{a}, {b}) final state against s + T", f64(S_j), f64(s), BF16)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64, f64(S0))
    check_close("sharded outputs", f64(torch.cat(outs, dim=2)), ref_o, BF16, BF16)
    check_state("sharded final state", f64(s), ref_S, BF16)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dv,dtype,with_ds", [
    (1, 8, 2, 3000, 128, 128, BF16, True),            # four query heads per KV head, ragged
    (2, 4, 4, 777, 64, 64, BF16, False),              # one query head per KV head, head size 64
    (1, 4, 1, 1, 128, 128, BF16, True),               # one token
    (1, 16, 2, 5000, 128, 128, BF16, False),          # eight query heads per KV head
    (1, 6, 2, 1000, 64, 96, torch.float32, True),     # float32, d != dv
    (1, 3, 1, 500, 96, 64, BF16, False),              # bf16 off the matrix-core shape
])
def test_backward_state_matches_oracle(B, Hq, Hkv, N, d, dv, dtype, with_ds):
    need_gpu()
    say(f"case backward state B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} {dtype} grad_s_out={with_ds}")
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, 64, dtype, dtype == BF16, dtype == torch.float32)
    q, k, v = synth.make_qkv(w, DEV, seed=N + 31)
    do = synth.make_grad((B, Hq, N, dv), DEV, seed=N + 32, dtype=dtype)
    dS = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 33, scale=0.5) if with_ds else None
    got = la.backward_state(q, do, Hkv, grad_s_out=dS)
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, None, None if dS is None else f64(dS))[3]
    check_state("grad_s_in", f64(got), ref, dtype)


def test_backward_state_in_place_and_empty():
    need_gpu()
    say("case backward state: in place over grad_s_out; N = 0 passes grad_s_out through")
    w = synth.Workload("t", 1, 8, 2, 2000, 128, 128, 64, BF16, True, False)
    q, k, v = synth.make_qkv(w, DEV, seed=41)
    do = synth.make_grad((1, 8, 2000, 128), DEV, seed=42)
    dS = synth.random_state((1, 2, 128, 128), DEV, seed=43, scale=0.5)
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, None, f64(dS))[3]
    assert la.backward_state(q, do, 2, grad_s_out=dS, out=dS).data_ptr() == dS.data_ptr()
    torch.cuda.synchronize()
    check_state("grad_s_in in place", f64(dS), ref, BF16)
    e = torch.empty((1, 8, 0, 128), dtype=BF16, device=DEV)
    assert torch.equal(la.backward_state(e, e, 2, grad_s_out=dS), dS)


@pytest.mark.parametrize("d", [128, 64])
def test_sequence_shards_backward_equals_one_pass(d):
    """The backward of a 30,000-token sequence (8 query heads over 2 KV heads)
    split into three shards: forward shard totals (la_forward_state) give each
    shard's initial state, backward shard sums (la_backward_state) give each
    shard's grad_s_out (the global one plus the later shards' sums), and each
    shard's la_backward then yields its slice of dq, dk, dv; the first shard's
    grad_s_in is the whole sequence's.  All against the oracle's backward over
    the whole sequence."""
    need_gpu()
    B, Hq, Hkv, N = 1, 8, 2, 30000
    cuts = [0, 9000, 21000, N]
    say(f"case backward shards d={d} N={N} cuts={cuts}")
    w = synth.Workload("t", B, Hq, Hkv, N, d, d, 64, BF16, True, False)
    q, k, v = synth.make_qkv(w, DEV, seed=51)
    do = synth.make_grad((B, Hq, N, d), DEV, seed=52)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=53, scale=0.5)
    dS = synth.random_state((B, Hkv, d, d), DEV, seed=54, scale=0.5)
    shards = [(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    T = [la.forward_state(sl(k, a, b), sl(v, a, b)) for a, b in shards]           # independent
    U = [la.backward_state(sl(q, a, b), sl(do, a, b), Hkv) for a, b in shards]    # independent
    grads, ds_in = [], None
    for j, (a, b) in enumerate(shards):
        s_j = S0 + sum(T[:j], torch.zeros_like(S0))
        g_j = dS + sum(U[j + 1:], torch.zeros_like(dS))
        dq, dk, dv, ds_j = la.backward(sl(q, a, b), sl(k, a, b), sl(v, a, b), sl(do, a, b), s_in=s_j,
                                       grad_s_out=g_j, return_state_grad=True)
        grads.append((dq, dk, dv))
        if j == 0:
            ds_in = ds_j
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, f64(S0), f64(dS))
    for i, name in enumerate(("dq", "dk", "dv")):
        check_close(f"sharded {name}", f64(torch.cat([g[i] for g in grads], dim=2)), ref[i], BF16, BF16)
    check_state("sharded grad_s_in", f64(ds_in), ref[3], BF16)
