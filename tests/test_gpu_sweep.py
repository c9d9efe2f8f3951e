"""Seeded sweep of problem shapes against the fp64 oracle: forward, variants and
backward on the matrix-core path at shapes drawn from one fixed-seed generator.

The hand-picked cases of the other GPU tests cover each kernel and plan branch
once; this sweep draws further shapes that stress the host planner (segment
count P, blocks per segment, pre-pass parts, query-head subgroups): odd numbers
of KV heads (1, 2, 3, 5, 7), batch sizes 1 to 3, group sizes 1 to 8, both head
sizes (64 and 128), lengths spread from one token to ~16K with a bias towards
one token either side of a block or segment boundary, bf16 and float32
outputs, with or without an initial state.  The draw is made once on the CPU
(numpy default_rng with a fixed seed), so every run checks the same cases.

Bars are those of the other parity tests: outputs and gradients within 2e-2 of
the reference RMS (+ 2^-8 |ref| for bf16 storage; row by row for normalised
outputs), states within 2e-4 of their RMS.  Inputs: synth.make_qkv (q, k
ReLU'd N(0,1)/sqrt(d), v ~ N(0,1)), upstream gradient N(0,1), initial states
N(0,1)*0.5.  Each case prints its shape before it runs.
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
SEED = 20261204
MAX_ROWS = 60_000  # B * Hq * N per case: keeps each oracle call to about a second


def _length(rng, blocks_per_seg_hint):
    """A sequence length: uniform, or one token either side of a multiple of
    64 tokens or of a likely segment length."""
    kind = rng.integers(0, 3)
    if kind == 0:
        return int(rng.integers(1, 16_000))
    unit = 64 if kind == 1 else 64 * blocks_per_seg_hint
    n = unit * int(rng.integers(1, max(2, 16_000 // unit)))
    return max(1, n + int(rng.choice([-1, 0, 1])))


def _draw(kind, count):
    rng = np.random.default_rng(SEED + {"fwd": 0, "var": 1, "bwd": 2}[kind])
    cases = []
    while len(cases) < count:
        B = int(rng.choice([1, 1, 2, 3]))
        Hkv = int(rng.choice([1, 2, 3, 5, 7]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        d = int(rng.choice([64, 128]))
        N = _length(rng, int(rng.choice([2, 4, 8, 16])))
        if B * Hkv * G * N > MAX_ROWS:
            N = max(1, MAX_ROWS // (B * Hkv * G))
        out = [BF16, torch.float32][int(rng.integers(0, 2))]
        s_in = bool(rng.integers(0, 2))
        extra = {}
        if kind == "var":
            # every combination of the three flags in turn
            i = len(cases)
            extra = {"causal": bool(i & 1), "relu": bool(i & 2), "norm": bool(i & 4)}
        elif kind == "bwd":
            extra = {"ds_out": bool(len(cases) & 1)}
        cases.append((B, G * Hkv, Hkv, N, d, out, s_in, extra))
    return cases


def _ids(cases):
    return [f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-d{c[4]}-{'bf16' if c[5] == BF16 else 'f32'}"
            f"{'-s' if c[6] else ''}" + "".join(f"-{k}{int(v)}" for k, v in c[7].items()) for c in cases]


def _inputs(B, Hq, Hkv, N, d, seed, relu_gen=True):
    w = synth.Workload("sweep", B, Hq, Hkv, N, d, d, 64, BF16, relu_gen, False)
    return synth.make_qkv(w, DEV, seed=seed)


FWD = _draw("fwd", 16)
VAR = _draw("var", 8)
BWD = _draw("bwd", 8)


@pytest.mark.parametrize("case", FWD, ids=_ids(FWD))
def test_sweep_forward(case):
    need_gpu()
    B, Hq, Hkv, N, d, out, s_in, _ = case
    say(f"case sweep forward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} out={out} s_in={s_in}")
    seed = (N * 31 + Hq * 7 + d) % 100_000
    q, k, v = _inputs(B, Hq, Hkv, N, d, seed)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=seed + 1, scale=0.5) if s_in else None
    o, S = la.forward(q, k, v, out_dtype=out, s_in=S0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.chunkwise(f64(q), f64(k), f64(v), 64, None if S0 is None else f64(S0))
    check_close("o", f64(o), ref_o, BF16, out)
    check_state("state", f64(S), ref_S, BF16)


@pytest.mark.parametrize("case", VAR, ids=_ids(VAR))
def test_sweep_variant(case):
    need_gpu()
    B, Hq, Hkv, N, d, out, s_in, ex = case
    causal, relu, norm = ex["causal"], ex["relu"], ex["norm"]
    say(f"case sweep variant B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} out={out} s_in={s_in} causal={causal} "
        f"relu={relu} norm={norm}")
    seed = (N * 17 + Hq * 5 + d + 3) % 100_000
    # raw N(0,1) q, k when ReLU is applied inside; ReLU'd by the generator when
    # the identity map is normalised (its weights must be non-negative)
    q, k, v = _inputs(B, Hq, Hkv, N, d, seed, relu_gen=not relu)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=seed + 1, scale=0.5) if s_in else None
    Z0 = synth.random_state((B, Hkv, d), DEV, seed=seed + 2).abs() if (s_in and norm) else None
    eps = 1e-6 if norm else 0.0
    o, S, Z = la.forward_variant(q, k, v, causal=causal, feature_map="relu" if relu else "identity",
                                 normalize=norm, eps=eps, out_dtype=out, s_in=S0, z_in=Z0, return_state=True)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_z = oracle.variant(f64(q), f64(k), f64(v), causal=causal, relu=relu, normalize=norm,
                                         eps=eps, s_in=None if S0 is None else f64(S0),
                                         z_in=None if Z0 is None else f64(Z0))
    check_close("o", f64(o), ref_o, BF16, out, per_row=norm)
    check_state("S_out", f64(S), ref_S, BF16)
    if norm:
        check_state("z_out", f64(Z), ref_z, BF16)


@pytest.mark.parametrize("case", BWD, ids=_ids(BWD))
def test_sweep_backward(case):
    need_gpu()
    B, Hq, Hkv, N, d, out, s_in, ex = case
    say(f"case sweep backward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} grad={out} s_in={s_in} ds_out={ex['ds_out']}")
    seed = (N * 13 + Hq * 3 + d + 5) % 100_000
    q, k, v = _inputs(B, Hq, Hkv, N, d, seed)
    do = synth.make_grad((B, Hq, N, d), DEV, seed=seed + 1)
    S0 = synth.random_state((B, Hkv, d, d), DEV, seed=seed + 2, scale=0.5) if s_in else None
    dS = synth.random_state((B, Hkv, d, d), DEV, seed=seed + 3, scale=0.5) if ex["ds_out"] else None
    got = la.backward(q, k, v, do, grad_dtype=out, s_in=S0, grad_s_out=dS, return_state_grad=True)
    torch.cuda.synchronize()
    ref = oracle.backward_chunkwise(f64(q), f64(k), f64(v), f64(do), 64, None if S0 is None else f64(S0),
                                    None if dS is None else f64(dS))
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check_close(name, f64(g), r, BF16, out)
    check_state("ds_in", f64(got[3]), ref[3], BF16)
