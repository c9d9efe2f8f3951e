"""Pins for the oracle's forward variants (feature map, non-causal, normalised).

Each pin reaches `oracle.variant` from something it does not share code with:
the hand-worked examples in tests/golden/variant_examples.json, the already
pinned causal and non-causal functions (special cases), the token-by-token
recurrence of the normalised form (S and z updated per token, then read),
closed forms for constant values and one-hot features, the convex-hull
property of a normalised average with non-negative weights, and resuming from
carried (S, z).  Planted mistakes in a copy each fail at least one pin.
"""
import json
import os

import numpy as np
import pytest

import oracle

# Rows whose weights are all zero divide 0 by 0 when eps = 0 (NaN); the pins
# skip those rows, and the mutants may divide by zero on purpose.
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "variant_examples.json")


def close(a, b, tol=1e-10):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) <= tol * max(1.0, float(np.max(np.abs(b))))


def rand(rng, B=2, Hq=4, Hkv=2, N=9, d=3, dv=2):
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, dv)))


def token_recurrence(q, k, v, relu, normalize, eps, s_in=None, z_in=None):
    """The RNN form: per token S += phi(k)^T v, z += phi(k), then read."""
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    G = Hq // Hkv
    f = (lambda x: np.maximum(x, 0.0)) if relu else (lambda x: x)
    o = np.zeros((B, Hq, N, dv))
    for b in range(B):
        for g in range(Hkv):
            S = np.zeros((d, dv)) if s_in is None else s_in[b, g].copy()
            z = np.zeros(d) if z_in is None else z_in[b, g].copy()
            for t in range(N):
                kt = f(k[b, g, t])
                S += np.outer(kt, v[b, g, t])
                z += kt
                for h in range(g * G, (g + 1) * G):
                    qt = f(q[b, h, t])
                    num = qt @ S
                    o[b, h, t] = num / (qt @ z + eps) if normalize else num
    return o


def pin_golden(fn):
    ok = True
    for c in json.load(open(GOLDEN))["cases"]:
        q = np.array(c["q"], float)[None, None]
        k = np.array(c["k"], float)[None, None]
        v = np.array(c["v"], float)[None, None]
        o = fn(q, k, v, causal=c["causal"], relu=c["relu"], normalize=c["normalize"], eps=c["eps"])[0]
        ok &= close(o[0, 0], np.array(c["o"], float))
    return bool(ok)


def pin_special_cases(fn):
    rng = np.random.default_rng(30)
    q, k, v = rand(rng)
    s_in = rng.standard_normal((2, 2, 3, 2))
    ok = close(fn(q, k, v, s_in=s_in)[0], oracle.brute_force(q, k, v, s_in))
    ok &= close(fn(q, k, v, s_in=s_in)[1], oracle.final_state(k, v, s_in))
    ok &= close(fn(q, k, v, causal=False)[0], oracle.noncausal(q, k, v))
    ok &= close(fn(q, k, v, relu=True)[0], oracle.brute_force(np.maximum(q, 0), np.maximum(k, 0), v))
    return bool(ok)


def pin_recurrence(fn):
    rng = np.random.default_rng(31)
    q, k, v = rand(rng, N=11)
    s_in = np.abs(rng.standard_normal((2, 2, 3, 2)))
    z_in = np.abs(rng.standard_normal((2, 2, 3)))
    qpos = np.abs(q) + 0.1  # every denominator > 0, so eps = 0 is exact
    ok = True
    for qq, relu, norm, eps in ((qpos, True, True, 0.0), (q, True, True, 0.5), (q, False, False, 0.0),
                                (q, True, False, 0.0)):
        got = fn(qq, k, v, relu=relu, normalize=norm, eps=eps, s_in=s_in, z_in=z_in)[0]
        ok &= close(got, token_recurrence(qq, k, v, relu, norm, eps, s_in, z_in), 1e-9)
    return bool(ok)


def pin_noncausal_is_last_row(fn):
    """Non-causal output of query t = causal output of the last token when
    that token's query is q_t (it then sees every key)."""
    rng = np.random.default_rng(32)
    q, k, v = rand(rng, B=1, N=7)
    full = fn(q, k, v, causal=False, relu=True, normalize=True, eps=0.25)[0]
    ok = True
    for t in range(7):
        q2 = q.copy()
        q2[:, :, -1] = q[:, :, t]
        ok &= close(fn(q2, k, v, causal=True, relu=True, normalize=True, eps=0.25)[0][:, :, -1], full[:, :, t])
    return bool(ok)


def pin_closed_forms(fn):
    rng = np.random.default_rng(33)
    ok = True
    # constant values: a normalised average of identical vectors is that vector
    q, k, _ = rand(rng, N=10)
    q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    c = rng.standard_normal(2)
    v = np.broadcast_to(c, (2, 2, 10, 2)).copy()
    for causal in (True, False):
        ok &= close(fn(q, k, v, causal=causal, relu=True, normalize=True)[0], np.broadcast_to(c, (2, 4, 10, 2)))
    # one-hot features: phi(q_t) = e0, phi(k_s) = e0 for s in A else e1 ->
    # o_t = mean of v_s over s in A, s <= t (a running mean)
    N = 12
    A = np.array([0, 2, 3, 7, 11])
    q = np.zeros((1, 1, N, 2))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, 2))
    k[..., 1] = 1.0
    k[0, 0, A] = [1.0, 0.0]
    v = rng.standard_normal((1, 1, N, 3))
    o = fn(q, k, v, causal=True, relu=True, normalize=True)[0][0, 0]
    for t in range(N):
        sel = A[A <= t]
        if len(sel):
            ok &= close(o[t], v[0, 0, sel].mean(axis=0))
    return bool(ok)


def pin_convex_hull(fn):
    rng = np.random.default_rng(34)
    q, k, v = rand(rng, N=15)
    o = fn(q, k, v, causal=True, relu=True, normalize=True)[0]
    qk = np.maximum(q, 0), np.maximum(k, 0)
    ok = True
    for b in range(2):
        for h in range(4):
            g = h // 2
            for t in range(15):
                w = qk[1][b, g, :t + 1] @ qk[0][b, h, t]
                if w.sum() <= 1e-12:
                    continue
                lo = v[b, g, :t + 1][w > 0].min(axis=0) - 1e-12
                hi = v[b, g, :t + 1][w > 0].max(axis=0) + 1e-12
                ok &= bool(np.all(o[b, h, t] >= lo) and np.all(o[b, h, t] <= hi))
    return bool(ok)


def pin_resume(fn):
    rng = np.random.default_rng(35)
    q, k, v = rand(rng, N=13)
    whole = fn(q, k, v, relu=True, normalize=True, eps=0.1)
    a = 5
    first = fn(q[:, :, :a], k[:, :, :a], v[:, :, :a], relu=True, normalize=True, eps=0.1)
    second = fn(q[:, :, a:], k[:, :, a:], v[:, :, a:], relu=True, normalize=True, eps=0.1, s_in=first[1],
                z_in=first[2])
    ok = close(np.concatenate([first[0], second[0]], axis=2), whole[0])
    ok &= close(second[1], whole[1]) and close(second[2], whole[2])
    return bool(ok)


PINS = [pin_golden, pin_special_cases, pin_recurrence, pin_noncausal_is_last_row, pin_closed_forms,
        pin_convex_hull, pin_resume]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_variant_pins(pin):
    assert pin(oracle.variant)


def mutant(mode):
    """Copies of the variant with one planted mistake."""
    def fn(q, k, v, causal=True, relu=False, normalize=False, eps=0.0, s_in=None, z_in=None):
        B, Hq, N, d = q.shape
        Hkv, dv = k.shape[1], v.shape[3]
        G = Hq // Hkv
        if relu:
            q, k = np.maximum(q, 0), np.maximum(k, 0)
            if mode == "relu_on_v":
                v = np.maximum(v, 0)
        keep = np.tril(np.ones((N, N))) if causal else np.ones((N, N))
        o = np.zeros((B, Hq, N, dv))
        for b in range(B):
            for h in range(Hq):
                g = h // G
                W = q[b, h] @ k[b, g].T
                den = (W if mode == "den_all_tokens" else W * keep).sum(axis=1)
                W = W * keep
                num = W @ v[b, g]
                if s_in is not None:
                    num = num + q[b, h] @ s_in[b, g]
                if z_in is not None and mode != "z_in_ignored":
                    den = den + q[b, h] @ z_in[b, g]
                e = 0.0 if mode == "eps_ignored" else eps
                o[b, h] = num / (den + e)[:, None] if normalize else num
        S = np.swapaxes(k, -1, -2) @ v + (0 if s_in is None else s_in)
        z = k.sum(axis=2) + (0 if z_in is None else z_in)
        return o, S, z
    return fn


@pytest.mark.parametrize("mode", ["den_all_tokens", "relu_on_v", "eps_ignored", "z_in_ignored"])
def test_variant_mutants_are_caught(mode):
    failed = [p.__name__ for p in PINS if not p(mutant(mode))]
    assert failed, f"mutant {mode} passed every pin"
    assert all(p(mutant("none")) for p in PINS)
