"""GPU parity of la_forward_variant (ReLU feature map, non-causal,
normalised) against the fp64 oracle's `variant`.

Tolerance: the forward's bar (2e-2 of the output RMS, + 2^-8|ref| for bf16
output).  Normalised outputs, weighted averages of value rows whose magnitude
shrinks as the averages widen (about 1e-3 of RMS(v) a million tokens in),
take the RMS row by row, so each row is held to the bar at its own scale
(tests/test_parity_bar.py shows that this bar rejects a zero output, flipped
signs and a dropped normaliser term at that range).

Inputs are seeded and synthetic (synth): q, k ~ N(0,1)/sqrt(d) raw (so the
ReLU inside the kernels matters) or ReLU'd by the generator (for the
normalised identity-map case, whose weights must be non-negative); v ~ N(0,1);
initial states N(0,1)*0.5 (normaliser sums |N(0,1)|).  Sizes span several
segments per chain and a ragged last block; the 1M-token workload is checked
on its first and last 4096 tokens with the carried state and normaliser sums
computed in float64.
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


def inputs(B, Hq, Hkv, N, seed, relu_gen=False):
    w = synth.Workload("t", B, Hq, Hkv, N, 128, 128, 64, BF16, relu_gen, False)
    return synth.make_qkv(w, DEV, seed=seed)


CASES = [
    # causal, fmap, normalize, eps, s_in, z_in, out dtype, B, Hq, Hkv, N, generator ReLU
    (1, "relu", 0, 0.0, True, False, BF16, 1, 8, 2, 3000, False),
    (1, "relu", 1, 1e-6, True, True, torch.float32, 1, 8, 2, 3000, False),
    (1, "identity", 1, 0.0, False, False, torch.float32, 2, 4, 1, 1000, True),
    (0, "identity", 0, 0.0, True, False, torch.float32, 1, 8, 2, 2100, False),
    (0, "relu", 1, 1e-3, False, True, BF16, 1, 8, 2, 3000, False),
    (0, "relu", 0, 0.0, False, False, torch.float32, 1, 8, 1, 777, False),   # G = 8: two subgroups
    (1, "relu", 1, 0.0, True, True, torch.float32, 1, 8, 1, 2500, False),    # G = 8, causal
    (1, "relu", 1, 1e-6, True, True, torch.float32, 1, 8, 2, 100, False),    # one segment: s_in/z_in read directly
    (0, "relu", 1, 1e-6, True, True, torch.float32, 1, 8, 2, 1, False),      # one token
    # groups of 1, 2 and 3 query heads (eight-wave causal kernel; non-causal steps of 4/GW blocks)
    (1, "relu", 1, 1e-6, True, True, torch.float32, 2, 8, 8, 3000, False),   # G = 1
    (1, "relu", 0, 0.0, False, False, BF16, 1, 4, 2, 2500, False),           # G = 2
    (1, "identity", 1, 0.0, False, False, torch.float32, 1, 6, 2, 1200, True),  # G = 3
    (0, "identity", 0, 0.0, True, False, BF16, 2, 4, 4, 2900, False),        # G = 1: segments of 2 blocks, steps of 4
    (0, "relu", 0, 0.0, False, False, torch.float32, 1, 4, 2, 777, False),   # G = 2
    (0, "relu", 1, 1e-3, True, True, torch.float32, 1, 6, 2, 1500, False),   # G = 3
    (1, "relu", 1, 1e-6, True, True, torch.float32, 1, 2, 2, 100, False),    # G = 1, one segment: s_in, z_in direct
    (1, "identity", 1, 1e-6, True, True, BF16, 1, 4, 2, 64, True),           # G = 2, one block
]


@pytest.mark.parametrize("causal,fmap,norm,eps,use_s,use_z,out_dtype,B,Hq,Hkv,N,relu_gen", CASES)
def test_variant_matches_oracle(causal, fmap, norm, eps, use_s, use_z, out_dtype, B, Hq, Hkv, N, relu_gen):
    need_gpu()
    say(f"case variant causal={causal} fmap={fmap} norm={norm} eps={eps} s_in={use_s} z_in={use_z} "
        f"out={out_dtype} B={B} Hq={Hq} Hkv={Hkv} N={N}")
    q, k, v = inputs(B, Hq, Hkv, N, seed=N + 7 * Hq + causal, relu_gen=relu_gen)
    S0 = synth.random_state((B, Hkv, 128, 128), DEV, seed=N + 3, scale=0.5) if use_s else None
    Z0 = synth.random_state((B, Hkv, 128), DEV, seed=N + 4).abs() if use_z else None
    o, S, Z = la.forward_variant(q, k, v, causal=bool(causal), feature_map=fmap, normalize=bool(norm), eps=eps,
                                 out_dtype=out_dtype, s_in=S0, z_in=Z0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=bool(causal), relu=(fmap == "relu"),
                                         normalize=bool(norm), eps=eps, s_in=None if S0 is None else f64(S0),
                                         z_in=None if Z0 is None else f64(Z0))
    # normalised outputs are weighted averages of value rows: tolerance in units of RMS(v)
    check_close("o", f64(o), ref_o, BF16, out_dtype, per_row=norm)
    check_state("S_out", f64(S), ref_S, BF16)
    if norm:
        check_state("z_out", f64(Z), ref_z, BF16)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 2), (3, 3)])
def test_plain_variant_is_the_forward(Hq, Hkv):
    """causal, identity map, no normalisation: bit for bit la_forward_ex."""
    need_gpu()
    say(f"case plain variant = forward, Hq={Hq} Hkv={Hkv}")
    q, k, v = inputs(1, Hq, Hkv, 5000, seed=5)
    S0 = synth.random_state((1, Hkv, 128, 128), DEV, seed=6, scale=0.5)
    a, Sa, _ = la.forward_variant(q, k, v, s_in=S0, return_state=True)
    b, Sb = la.forward(q, k, v, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(Sa, Sb)


def test_variant_head_size_64_one_head_per_kv_head_two_batches():
    """Two batch entries of three heads (one query head per KV head) on the
    one-wave kernel: every (batch, head) chain reads its own s_in and z_in and
    writes its own S_out and z_out, over several segments and a ragged tail."""
    need_gpu()
    say("case variant d=64 B=2 Hq=Hkv=3 N=2500 ReLU-normalised")
    w = synth.Workload("t", 2, 3, 3, 2500, 64, 64, 64, BF16, False, False)
    q, k, v = synth.make_qkv(w, DEV, seed=12)
    S0 = synth.random_state((2, 3, 64, 64), DEV, seed=13, scale=0.5)
    Z0 = synth.random_state((2, 3, 64), DEV, seed=14).abs()
    o, S, Z = la.forward_variant(q, k, v, feature_map="relu", normalize=True, eps=1e-6, s_in=S0, z_in=Z0,
                                 return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=True, relu=True, normalize=True, eps=1e-6,
                                         s_in=f64(S0), z_in=f64(Z0))
    check_close("o", f64(o), ref_o, BF16, BF16, per_row=True)
    check_state("S_out", f64(S), ref_S, BF16)
    check_state("z_out", f64(Z), ref_z, BF16)


def test_plain_variant_is_the_forward_head_size_64_one_head_per_kv_head():
    """The same at head size 64 with one query head per KV head, where both
    calls run the one-wave kernel over many segments."""
    need_gpu()
    say("case plain variant = forward, d=64, Hq=Hkv=4, N=9000")
    w = synth.Workload("t", 1, 4, 4, 9000, 64, 64, 64, BF16, False, False)
    q, k, v = synth.make_qkv(w, DEV, seed=8)
    S0 = synth.random_state((1, 4, 64, 64), DEV, seed=9, scale=0.5)
    a, Sa, _ = la.forward_variant(q, k, v, s_in=S0, return_state=True)
    b, Sb = la.forward(q, k, v, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(Sa, Sb)


def test_variants_gqa_1m_slices():
    """The 1M-token GQA workload (raw q, k; phi = ReLU inside): the causal
    normalised variant on the first and last 4096 tokens of KV groups 0 and
    31 with the oracle's carried (S, z), its final (S, z); and the
    non-causal ReLU variant (normalised and not) on the same slices against
    the totals."""
    need_gpu()
    w = synth.WORKLOADS["gqa_1m"]
    G = w.Hq // w.Hkv
    N, W = w.N, 4096
    say(f"case variants gqa_1m: N={N}")
    q, k, v = inputs(w.B, w.Hq, w.Hkv, N, seed=0)
    eps = 1e-6
    o, S, Z = la.forward_variant(q, k, v, causal=True, feature_map="relu", normalize=True, eps=eps,
                                 return_state=True)
    onc = la.forward_variant(q, k, v, causal=False, feature_map="relu", normalize=True, eps=eps)
    onc_plain, S_nc, _ = la.forward_variant(q, k, v, causal=False, feature_map="relu", return_state=True)
    torch.cuda.synchronize()
    for x in (o, onc, onc_plain):
        assert bool(torch.isfinite(x).all())
    a = N - W
    for g in (0, 31):
        hs, gs = slice(g * G, (g + 1) * G), slice(g, g + 1)
        kr = np.maximum(f64(k[:, gs]), 0.0)
        vg = f64(v[:, gs])
        ones = np.ones(kr.shape[:3] + (1,))
        S_a, z_a = oracle.final_state(kr[:, :, :a], vg[:, :, :a]), oracle.final_state(kr[:, :, :a], ones[:, :, :a])[..., 0]
        S_t, z_t = oracle.final_state(kr, vg), oracle.final_state(kr, ones)[..., 0]
        del kr, ones
        for lo, hi, s_in, z_in in ((0, W, None, None), (a, N, S_a, z_a)):
            qs, ks, vs = f64(q[:, hs, lo:hi]), f64(k[:, gs, lo:hi]), vg[:, :, lo:hi]
            ref = oracle.variant(qs, ks, vs, causal=True, relu=True, normalize=True, eps=eps, s_in=s_in, z_in=z_in)
            check_close(f"causal normalised group {g} tokens [{lo}, {hi})", f64(o[:, hs, lo:hi]), ref[0], BF16, BF16,
                        per_row=True)
            # non-causal: zero keys add nothing, the totals come in as the initial state
            zk, zv = np.zeros_like(ks), np.zeros_like(vs)
            ref_nc = oracle.variant(qs, zk, zv, causal=False, relu=True, normalize=True, eps=eps, s_in=S_t, z_in=z_t)
            check_close(f"non-causal normalised group {g} tokens [{lo}, {hi})", f64(onc[:, hs, lo:hi]), ref_nc[0],
                        BF16, BF16, per_row=True)
            ref_np = oracle.variant(qs, zk, zv, causal=False, relu=True, s_in=S_t)
            check_close(f"non-causal group {g} tokens [{lo}, {hi})", f64(onc_plain[:, hs, lo:hi]), ref_np[0], BF16,
                        BF16)
        check_state(f"causal final state group {g}", f64(S[:, gs]), S_t, BF16)
        check_state(f"causal final z group {g}", f64(Z[:, gs]), z_t, BF16)
        check_state(f"non-causal state group {g}", f64(S_nc[:, gs]), S_t, BF16)


def test_variants_mha_1m_d64_slices():
    """The 1M-token workload with one query head per KV head at head size 64
    (32 heads), where the causal ReLU-normalised variant runs the one-wave
    kernel over 32 segments per head: heads 0 and 31 on their first and last
    4096 tokens and on a window across the first segment boundary (token
    32768), each from the oracle's carried (S, z), and their final (S, z)."""
    need_gpu()
    w = synth.WORKLOADS["mha_1m_d64"]
    N, W = w.N, 4096
    say(f"case variants mha_1m_d64: N={N}")
    q, k, v = synth.make_qkv(w, DEV, seed=0)
    eps = 1e-6
    o, S, Z = la.forward_variant(q, k, v, causal=True, feature_map="relu", normalize=True, eps=eps,
                                 return_state=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    for h in (0, 31):
        hs = slice(h, h + 1)
        kr = np.maximum(f64(k[:, hs]), 0.0)
        vh = f64(v[:, hs])
        ones = np.ones(kr.shape[:3] + (1,))
        for lo, hi in ((0, W), (32768 - W // 2, 32768 + W // 2), (N - W, N)):
            s_in = oracle.final_state(kr[:, :, :lo], vh[:, :, :lo]) if lo else None
            z_in = oracle.final_state(kr[:, :, :lo], ones[:, :, :lo])[..., 0] if lo else None
            ref = oracle.variant(f64(q[:, hs, lo:hi]), f64(k[:, hs, lo:hi]), vh[:, :, lo:hi], causal=True, relu=True,
                                 normalize=True, eps=eps, s_in=s_in, z_in=z_in)
            check_close(f"causal normalised head {h} tokens [{lo}, {hi})", f64(o[:, hs, lo:hi]), ref[0], BF16, BF16,
                        per_row=True)
        check_state(f"final state head {h}", f64(S[:, hs]), oracle.final_state(kr, vh), BF16)
        check_state(f"final z head {h}", f64(Z[:, hs]), oracle.final_state(kr, ones)[..., 0], BF16)


F32_CASES = [
    # causal, fmap, normalize, eps, s_in, z_in, B, Hq, Hkv, N, d, dv, block, generator ReLU
    (1, "relu", 1, 1e-6, True, True, 1, 4, 2, 300, 64, 64, 64, False),
    (0, "relu", 1, 1e-3, True, True, 1, 3, 1, 200, 128, 96, 32, False),
    (0, "identity", 0, 0.0, True, False, 2, 2, 2, 150, 32, 32, 64, False),
    (1, "identity", 1, 0.0, False, False, 1, 4, 4, 257, 64, 128, 16, True),
    (1, "relu", 0, 0.0, False, False, 1, 8, 2, 100, 128, 64, 64, False),
]


@pytest.mark.parametrize("causal,fmap,norm,eps,use_s,use_z,B,Hq,Hkv,N,d,dv,block,relu_gen", F32_CASES)
def test_variant_f32_matches_oracle(causal, fmap, norm, eps, use_s, use_z, B, Hq, Hkv, N, d, dv, block, relu_gen):
    """float32 inputs (the float32 FMA kernel with the variant flags) at the
    float32 bar, 1e-5 of the output RMS (of RMS(v) when normalised)."""
    need_gpu()
    say(f"case variant f32 causal={causal} fmap={fmap} norm={norm} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} "
        f"block={block}")
    F32 = torch.float32
    w = synth.Workload("t", B, Hq, Hkv, N, d, dv, block, F32, relu_gen, True)
    q, k, v = synth.make_qkv(w, DEV, seed=N + d + causal)
    S0 = synth.random_state((B, Hkv, d, dv), DEV, seed=N + 5, scale=0.5) if use_s else None
    Z0 = synth.random_state((B, Hkv, d), DEV, seed=N + 6).abs() if use_z else None
    o, S, Z = la.forward_variant(q, k, v, causal=bool(causal), feature_map=fmap, normalize=bool(norm), eps=eps,
                                 block=block, s_in=S0, z_in=Z0, return_state=True)
    torch.cuda.synchronize()
    assert o.dtype == F32
    ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=bool(causal), relu=(fmap == "relu"),
                                         normalize=bool(norm), eps=eps, s_in=None if S0 is None else f64(S0),
                                         z_in=None if Z0 is None else f64(Z0))
    check_close("f32 o", f64(o), ref_o, F32, F32, per_row=norm)
    check_state("f32 S_out", f64(S), ref_S, F32)
    if norm:
        check_state("f32 z_out", f64(Z), ref_z, F32)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_variant_in_place_state_and_normaliser(dtype):
    """s_out written over s_in and z_out over z_in give the results of
    separate buffers (non-causal normalised, the float32 path computes z_out
    after every workgroup has read z_in)."""
    need_gpu()
    say(f"case variant in place S, z {dtype}")
    d = 64 if dtype == torch.float32 else 128
    w = synth.Workload("t", 1, 4, 2, 500, d, d, 64, dtype, False, dtype == torch.float32)
    q, k, v = synth.make_qkv(w, DEV, seed=41)
    S0 = synth.random_state((1, 2, d, d), DEV, seed=42, scale=0.5)
    Z0 = synth.random_state((1, 2, d), DEV, seed=43).abs()
    ref = la.forward_variant(q, k, v, causal=False, feature_map="relu", normalize=True, eps=1e-6, s_in=S0, z_in=Z0,
                             return_state=True)
    S, Z = S0.clone(), Z0.clone()
    o = la.forward_variant(q, k, v, causal=False, feature_map="relu", normalize=True, eps=1e-6, s_in=S, z_in=Z,
                           s_out=S, z_out=Z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(Z, ref[2])


@pytest.mark.parametrize("causal,fmap,norm,eps,out_dtype,Hq,Hkv,N", [
    (True, "relu", True, 1e-6, torch.float32, 8, 2, 3000),   # G = 4, several segments
    (True, "identity", False, 0.0, BF16, 8, 1, 1000),         # G = 8: two query-head subgroups
    (True, "relu", False, 0.0, BF16, 4, 1, 100),              # two blocks
    (False, "relu", True, 1e-6, torch.float32, 8, 2, 3000),  # non-causal: totals over 3000 tokens
    (False, "identity", False, 0.0, BF16, 8, 1, 1000),        # G = 8
    (False, "relu", False, 0.0, BF16, 4, 1, 100),             # two blocks, ragged
    (False, "relu", True, 1e-6, BF16, 4, 1, 1),               # one token
    (True, "relu", True, 1e-6, torch.float32, 4, 4, 3000),   # G = 1: one-wave workgroups, ten segments
    (True, "relu", True, 1e-6, BF16, 2, 2, 20000),            # G = 1, 79 segments per head
    (True, "relu", True, 1e-6, BF16, 2, 2, 1),                # G = 1, one token (z_in read directly)
    (True, "relu", False, 0.0, BF16, 4, 4, 1000),             # G = 1, ReLU without normalisation
    (False, "relu", True, 1e-6, torch.float32, 4, 4, 3000),  # G = 1, non-causal
    (True, "identity", False, 0.0, BF16, 6, 3, 1000),         # G = 2
    (False, "identity", False, 0.0, BF16, 6, 2, 1000),        # G = 3, non-causal
    (False, "relu", True, 1e-6, torch.float32, 4, 2, 2000),  # G = 2, non-causal (steps of two blocks)
])
def test_variant_head_size_64(causal, fmap, norm, eps, out_dtype, Hq, Hkv, N):
    """Variants at head size 64, any group size: causal ones on the four-wave
    forward kernel (on one-wave workgroups for one query head per KV head),
    the non-causal one on its own kernel, both after the pre-pass with the
    variant flags."""
    need_gpu()
    say(f"case variant d=64 causal={causal} fmap={fmap} norm={norm} out={out_dtype} Hq={Hq} Hkv={Hkv} N={N}")
    w = synth.Workload("t", 1, Hq, Hkv, N, 64, 64, 64, BF16, False, False)
    q, k, v = synth.make_qkv(w, DEV, seed=N + Hq)
    S0 = synth.random_state((1, Hkv, 64, 64), DEV, seed=N + 3, scale=0.5)
    Z0 = synth.random_state((1, Hkv, 64), DEV, seed=N + 4).abs() if norm else None
    if N > 256:
        lib = la.load_library()
        assert lib.la_forward_variant_workspace_bytes(1, Hq, Hkv, N, 64, 64, 64, la.LA_BF16, int(causal),
                                                      int(norm)) > 0
    o, S, Z = la.forward_variant(q, k, v, causal=causal, feature_map=fmap, normalize=norm, eps=eps,
                                 out_dtype=out_dtype, s_in=S0, z_in=Z0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=causal, relu=(fmap == "relu"),
                                         normalize=norm, eps=eps, s_in=f64(S0),
                                         z_in=None if Z0 is None else f64(Z0))
    check_close("o", f64(o), ref_o, BF16, out_dtype, per_row=norm)
    check_state("S_out", f64(S), ref_S, BF16)
    if norm:
        check_state("z_out", f64(Z), ref_z, BF16)
