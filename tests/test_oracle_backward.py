"""Pins for the oracle's backward pass.

The gradients are checked against central finite differences of the forward
oracle (itself pinned in test_oracle.py).  The output is linear in every
single input entry, so a central difference is exact up to rounding and the
check is tight.  Planted mistakes in copies of the block-wise backward (the
diagonal dropped, one head instead of the group's sum, the state updated
before it is read, the initial state's term missing) each fail a pin.
"""
import numpy as np
import pytest

import oracle


def rand_problem(rng, B=1, Hq=4, Hkv=2, N=7, d=3, dv=2):
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, dv))
    do = rng.standard_normal((B, Hq, N, dv))
    s_in = rng.standard_normal((B, Hkv, d, dv))
    return q, k, v, do, s_in


def finite_difference_grads(q, k, v, do, s_in, block=3, eps=0.5, ds_out=None):
    """d/dx of L = sum(o * dO) (+ sum(S_out * ds_out)) by central differences
    of the forward oracle."""
    def loss(qq, kk, vv, ss):
        o, S = oracle.chunkwise(qq, kk, vv, block, ss)
        total = float(np.sum(o * do))
        if ds_out is not None:
            total += float(np.sum(S * ds_out))
        return total

    grads = []
    args = [q, k, v, s_in]
    for idx in range(4):
        x = args[idx]
        g = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[idx][pos] += eps
            minus[idx][pos] -= eps
            g[pos] = (loss(*plus) - loss(*minus)) / (2 * eps)
        grads.append(g)
    return grads


def close(a, b, tol=1e-9):
    return float(np.max(np.abs(a - b))) <= tol * max(1.0, float(np.max(np.abs(b))))


def pin_finite_differences(bwd):
    rng = np.random.default_rng(20)
    ok = True
    for shape in ({}, {"Hq": 2, "Hkv": 2, "N": 5}, {"Hq": 3, "Hkv": 1, "N": 8, "d": 2, "dv": 3}):
        q, k, v, do, s_in = rand_problem(rng, **shape)
        ref = finite_difference_grads(q, k, v, do, s_in)
        got = bwd(q, k, v, do, s_in)
        ok &= all(close(g, r) for g, r in zip(got, ref))
    return bool(ok)


def pin_brute_force(bwd):
    rng = np.random.default_rng(21)
    q, k, v, do, s_in = rand_problem(rng, B=2, Hq=4, Hkv=2, N=11, d=4, dv=3)
    ref = oracle.backward_brute_force(q, k, v, do, s_in)
    return all(close(g, r) for g, r in zip(bwd(q, k, v, do, s_in), ref))


def pin_zero_and_linear_in_do(bwd):
    rng = np.random.default_rng(22)
    q, k, v, do, s_in = rand_problem(rng)
    zero = bwd(q, k, v, np.zeros_like(do), s_in)
    ok = all(float(np.max(np.abs(z))) == 0.0 for z in zero)
    do2 = rng.standard_normal(do.shape)
    a, b, c = bwd(q, k, v, do, s_in), bwd(q, k, v, do2, s_in), bwd(q, k, v, 2 * do - 3 * do2, s_in)
    ok &= all(close(z, 2 * x - 3 * y) for x, y, z in zip(a, b, c))
    return bool(ok)


def chunk_impl(block):
    return lambda q, k, v, do, s_in: oracle.backward_chunkwise(q, k, v, do, block, s_in)


BACKWARD_PINS = [pin_finite_differences, pin_brute_force, pin_zero_and_linear_in_do]


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=[p.__name__ for p in BACKWARD_PINS])
@pytest.mark.parametrize("block", [1, 2, 3, 64])
def test_backward_chunkwise_pins(pin, block):
    assert pin(chunk_impl(block))


def test_backward_brute_force_matches_finite_differences():
    assert pin_finite_differences(lambda *a: oracle.backward_brute_force(*a))


def test_backward_without_initial_state():
    rng = np.random.default_rng(23)
    q, k, v, do, _ = rand_problem(rng, N=9)
    a = oracle.backward_chunkwise(q, k, v, do, 4)
    b = oracle.backward_chunkwise(q, k, v, do, 4, np.zeros((1, 2, 3, 2)))
    assert all(close(x, y) for x, y in zip(a, b))


def test_dq_is_the_forward_on_do_v_k():
    """dQ is the causal forward with queries dO, keys V, values K (no s_in)."""
    rng = np.random.default_rng(24)
    q, k, v, do, _ = rand_problem(rng, N=10, d=3, dv=3)
    dq = oracle.backward_chunkwise(q, k, v, do, 4)[0]
    assert close(dq, oracle.brute_force(do, v, k))


def test_final_state_gradient_matches_finite_differences():
    """A gradient ds_out on the final state: every output of both backward
    forms against central differences of L = sum(o dO) + sum(S_out ds_out)."""
    rng = np.random.default_rng(25)
    for shape in ({}, {"Hq": 3, "Hkv": 1, "N": 8, "d": 2, "dv": 3}):
        q, k, v, do, s_in = rand_problem(rng, **shape)
        ds_out = rng.standard_normal(s_in.shape)
        ref = finite_difference_grads(q, k, v, do, s_in, ds_out=ds_out)
        for got in (oracle.backward_brute_force(q, k, v, do, s_in, ds_out),
                    oracle.backward_chunkwise(q, k, v, do, 3, s_in, ds_out),
                    oracle.backward_chunkwise(q, k, v, do, 64, s_in, ds_out)):
            assert all(close(g, r) for g, r in zip(got, ref))
        # without the ds_out term the gradients differ
        plain = oracle.backward_chunkwise(q, k, v, do, 3, s_in)
        assert not close(plain[1], ref[1]) and not close(plain[3], ref[3])


def test_chunked_backward_equals_whole_sequence():
    """Splitting a sequence in two chunks (the second starts from the first's
    final state) and back-propagating the second chunk's ds_in into the first
    as its ds_out gives the whole sequence's gradients."""
    rng = np.random.default_rng(26)
    q, k, v, do, s_in = rand_problem(rng, B=2, Hq=4, Hkv=2, N=13, d=3, dv=4)
    whole = oracle.backward_chunkwise(q, k, v, do, 4, s_in)
    a = 6
    S_a = oracle.final_state(k[:, :, :a], v[:, :, :a], s_in)
    dq2, dk2, dv2, ds2 = oracle.backward_chunkwise(q[:, :, a:], k[:, :, a:], v[:, :, a:], do[:, :, a:], 4, S_a)
    dq1, dk1, dv1, ds1 = oracle.backward_chunkwise(q[:, :, :a], k[:, :, :a], v[:, :, :a], do[:, :, :a], 4, s_in,
                                                   ds2)
    assert close(np.concatenate([dq1, dq2], axis=2), whole[0])
    assert close(np.concatenate([dk1, dk2], axis=2), whole[1])
    assert close(np.concatenate([dv1, dv2], axis=2), whole[2])
    assert close(ds1, whole[3])


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def mutant(mode, block=3):
    def bwd(q, k, v, do, s_in):
        B, Hq, N, d = q.shape
        Hkv, dv = k.shape[1], v.shape[3]
        G = Hq // Hkv
        s_t = None if (s_in is None or mode == "no_s_in_term") else np.swapaxes(s_in, -1, -2)
        dq, _ = oracle.chunkwise(do, v, k, block, s_t)
        R = np.zeros((B, Hkv, d, dv))
        dk, dvv = np.zeros_like(k), np.zeros_like(v)
        for a in reversed(range(0, N, block)):
            e = min(a + block, N)
            kb, vb = k[:, :, a:e], v[:, :, a:e]
            c = e - a
            keep = np.arange(c)[None, :] >= np.arange(c)[:, None] + (1 if mode == "strict" else 0)
            upd = np.zeros_like(R)
            heads = [0] if mode == "one_head" else range(G)
            for j in heads:
                qh = q[:, [g * G + j for g in range(Hkv)], a:e]
                doh = do[:, [g * G + j for g in range(Hkv)], a:e]
                upd = upd + np.matmul(np.swapaxes(qh, -1, -2), doh)
            if mode == "update_first":
                R = R + upd
            dvb, dkb = np.matmul(kb, R), np.matmul(vb, np.swapaxes(R, -1, -2))
            for j in heads:
                qh = q[:, [g * G + j for g in range(Hkv)], a:e]
                doh = do[:, [g * G + j for g in range(Hkv)], a:e]
                dvb = dvb + np.matmul(np.matmul(kb, np.swapaxes(qh, -1, -2)) * keep, doh)
                dkb = dkb + np.matmul(np.matmul(vb, np.swapaxes(doh, -1, -2)) * keep, qh)
            dvv[:, :, a:e], dk[:, :, a:e] = dvb, dkb
            if mode != "update_first":
                R = R + upd
        return dq, dk, dvv, R
    return bwd


@pytest.mark.parametrize("mode", ["strict", "one_head", "update_first", "no_s_in_term"])
def test_backward_mutants_are_caught(mode):
    failed = [p.__name__ for p in BACKWARD_PINS if not p(mutant(mode))]
    assert failed, f"mutant {mode} passed every pin"
    assert all(p(mutant("none")) for p in BACKWARD_PINS)
