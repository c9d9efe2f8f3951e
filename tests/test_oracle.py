"""Pins for the fp64 oracle, checked against things other than the oracle itself.

Each check below is written so that a plausible mistake in the oracle (the
diagonal dropped, the state read after the block's own update, a wrong GQA
mapping, a transposed state, a lost inter-block term, a wrong initial state)
fails at least one of them; test_mutants_are_caught plants those mistakes in
copies of the oracle and confirms it.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_inputs(rng, B, Hq, Hkv, N, d, dv, relu=True):
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, dv))
    if relu:
        q, k = np.maximum(q, 0), np.maximum(k, 0)
    return q / np.sqrt(d), k / np.sqrt(d), v


def loop_sum(q, k, v, s_in=None):
    """The definition with Python loops only (no matrix routines)."""
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Hq, N, dv))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in range(N):
                for s in range(t + 1):
                    w = sum(float(q[b, h, t, i]) * float(k[b, g, s, i]) for i in range(d))
                    for j in range(dv):
                        o[b, h, t, j] += w * float(v[b, g, s, j])
                if s_in is not None:
                    for j in range(dv):
                        o[b, h, t, j] += sum(float(q[b, h, t, i]) * float(s_in[b, g, i, j]) for i in range(d))
    return o


# ---------------------------------------------------------------------------
# Pin checks, parametrised by implementation so mutants can be run through them.
# Each returns True when the implementation passes.
# ---------------------------------------------------------------------------

def _close(a, b, rtol=1e-11):
    scale = max(1.0, float(np.max(np.abs(b))) if np.size(b) else 1.0)
    return np.size(a) == np.size(b) and float(np.max(np.abs(np.asarray(a) - np.asarray(b)), initial=0.0)) <= rtol * scale


def pin_hand_examples(impl):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
        s_in = np.array(c["s_in"], dtype=np.float64) if "s_in" in c else None
        for blk in (1, 2, 3):
            o, S = impl["chunkwise"](q, k, v, blk, s_in)
            if not (np.array_equal(o, np.array(c["o"], dtype=np.float64))
                    and np.array_equal(S, np.array(c["state"], dtype=np.float64))):
                return False
        if not np.array_equal(impl["brute_force"](q, k, v, s_in), np.array(c["o"], dtype=np.float64)):
            return False
        o, S = impl["recurrent"](q, k, v, s_in)
        if not (np.array_equal(o, np.array(c["o"], dtype=np.float64))
                and np.array_equal(S, np.array(c["state"], dtype=np.float64))):
            return False
    for c in json.load(open(GOLDEN))["decode"]:
        S_new, o = impl["decode_step"](*(np.array(c[x], dtype=np.float64) for x in ("S", "q", "k", "v")))
        if not (np.array_equal(S_new, np.array(c["S_new"], dtype=np.float64))
                and np.array_equal(o, np.array(c["o"], dtype=np.float64))):
            return False
    return True


def pin_loop_sum(impl):
    rng = np.random.default_rng(1)
    q, k, v = rand_inputs(rng, 1, 4, 2, 11, 3, 2, relu=False)
    s_in = rng.standard_normal((1, 2, 3, 2))
    ref = loop_sum(q, k, v, s_in)
    ok = _close(impl["brute_force"](q, k, v, s_in), ref)
    for blk in (1, 4, 11):
        ok &= _close(impl["chunkwise"](q, k, v, blk, s_in)[0], ref)
    ok &= _close(impl["recurrent"](q, k, v, s_in)[0], ref)
    return bool(ok)


def pin_cumsum(impl):
    """Closed form: q_t = k_s = c with |c| = 1 makes o_t the prefix sum of v."""
    rng = np.random.default_rng(2)
    N, d, dv = 37, 5, 3
    c = rng.standard_normal(d)
    c /= np.linalg.norm(c)
    q = np.broadcast_to(c, (1, 1, N, d)).copy()
    v = rng.standard_normal((1, 1, N, dv))
    ref = np.cumsum(v, axis=2)
    ok = True
    for blk in (1, 4, 8, 37):
        ok &= _close(impl["chunkwise"](q, q, v, blk)[0], ref)
    ok &= _close(impl["recurrent"](q, q, v)[0], ref)
    return bool(ok)


def pin_onehot(impl):
    """Closed form: q_t = e_{t mod d}, k_s = e_{s mod d} picks s <= t with s = t (mod d)."""
    rng = np.random.default_rng(3)
    N, d, dv = 23, 4, 2
    eye = np.eye(d)
    q = eye[np.arange(N) % d][None, None]
    k = eye[(np.arange(N) * 1) % d][None, None]
    v = rng.standard_normal((1, 1, N, dv))
    ref = np.zeros((1, 1, N, dv))
    for t in range(N):
        ref[0, 0, t] = v[0, 0, [s for s in range(t + 1) if s % d == t % d]].sum(axis=0)
    ok = True
    for blk in (1, 3, 5, 23):
        ok &= _close(impl["chunkwise"](q, k, v, blk)[0], ref)
    return bool(ok)


def pin_block_invariance(impl):
    rng = np.random.default_rng(4)
    q, k, v = rand_inputs(rng, 2, 4, 2, 50, 6, 5)
    ref = impl["brute_force"](q, k, v)
    ok = True
    for blk in (1, 2, 3, 7, 16, 49, 50, 64):
        ok &= _close(impl["chunkwise"](q, k, v, blk)[0], ref)
    return bool(ok)


def pin_causality(impl):
    rng = np.random.default_rng(5)
    q, k, v = rand_inputs(rng, 1, 2, 1, 40, 4, 3)
    full = impl["chunkwise"](q, k, v, 8)[0]
    ok = True
    for T in (1, 8, 13, 39):
        part = impl["chunkwise"](q[:, :, :T], k[:, :, :T], v[:, :, :T], 8)[0]
        ok &= np.array_equal(part, full[:, :, :T])
    # future tokens must not change the past: perturb the tail
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    k2[:, :, 20:] += 1.0
    v2[:, :, 20:] -= 2.0
    ok &= _close(impl["chunkwise"](q2, k2, v2, 8)[0][:, :, :20], full[:, :, :20])
    return bool(ok)


def pin_state_is_gemm(impl):
    rng = np.random.default_rng(6)
    q, k, v = rand_inputs(rng, 2, 2, 2, 33, 5, 4)
    ref = np.einsum("bhnd,bhne->bhde", k, v)  # library contraction
    ok = _close(impl["chunkwise"](q, k, v, 4)[1], ref)
    ok &= _close(impl["recurrent"](q, k, v)[1], ref)
    ok &= _close(impl["final_state"](k, v), ref)
    return bool(ok)


def pin_last_row_noncausal(impl):
    rng = np.random.default_rng(7)
    q, k, v = rand_inputs(rng, 1, 3, 3, 29, 4, 6)
    o = impl["chunkwise"](q, k, v, 5)[0]
    # last row of the causal output sees every key: q_{N-1} (K^T V)
    kv = np.stack([[k[0, h].T @ v[0, h] for h in range(3)]])
    ref = np.stack([[q[0, h, -1] @ kv[0, h] for h in range(3)]])
    ok = _close(o[:, :, -1], ref)
    ok &= _close(impl["noncausal"](q, k, v)[:, :, -1], ref)
    ok &= _close(impl["noncausal"](q, k, v)[:, :, 0], np.stack([[q[0, h, 0] @ kv[0, h] for h in range(3)]]))
    return bool(ok)


def pin_linearity(impl):
    rng = np.random.default_rng(8)
    q, k, v1 = rand_inputs(rng, 1, 2, 1, 21, 4, 3)
    v2 = rng.standard_normal(v1.shape)
    f = lambda qq, vv: impl["chunkwise"](qq, k, vv, 4)[0]
    ok = _close(f(q, 2.5 * v1 - 0.5 * v2), 2.5 * f(q, v1) - 0.5 * f(q, v2))
    ok &= _close(f(-3.0 * q, v1), -3.0 * f(q, v1))
    return bool(ok)


def pin_gqa_vs_mha(impl):
    rng = np.random.default_rng(9)
    B, Hq, Hkv = 2, 8, 2
    q, k, v = rand_inputs(rng, B, Hq, Hkv, 19, 4, 3)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    ok = _close(impl["chunkwise"](q, k, v, 4)[0], impl["chunkwise"](q, kr, vr, 4)[0])
    # per-head check against single-head runs on the expected KV head
    o = impl["chunkwise"](q, k, v, 4)[0]
    for h in range(Hq):
        g = h // (Hq // Hkv)
        ok &= _close(o[:, h:h + 1], impl["brute_force"](q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1]))
    return bool(ok)


def pin_decode_vs_forward(impl):
    rng = np.random.default_rng(10)
    q, k, v = rand_inputs(rng, 2, 4, 2, 30, 5, 4)
    P = 22
    o_pre, S = impl["chunkwise"](q[:, :, :P], k[:, :, :P], v[:, :, :P], 8)
    ok = True
    o_full = impl["brute_force"](q, k, v)
    ok &= _close(o_pre, o_full[:, :, :P])
    for t in range(P, 30):
        S, o_t = impl["decode_step"](S, q[:, :, t], k[:, :, t], v[:, :, t])
        ok &= _close(o_t, o_full[:, :, t])
    ok &= _close(S, np.einsum("bhnd,bhne->bhde", k, v))
    return bool(ok)


def pin_resume(impl):
    rng = np.random.default_rng(11)
    q, k, v = rand_inputs(rng, 1, 2, 2, 45, 4, 4)
    o_full, S_full = impl["chunkwise"](q, k, v, 8)
    M = 19
    o1, S1 = impl["chunkwise"](q[:, :, :M], k[:, :, :M], v[:, :, :M], 8)
    o2, S2 = impl["chunkwise"](q[:, :, M:], k[:, :, M:], v[:, :, M:], 8, S1)
    ok = _close(np.concatenate([o1, o2], axis=2), o_full) and _close(S2, S_full)
    ok &= _close(impl["brute_force"](q[:, :, M:], k[:, :, M:], v[:, :, M:], S1), o2)
    return bool(ok)


PINS = [pin_hand_examples, pin_loop_sum, pin_cumsum, pin_onehot, pin_block_invariance,
        pin_causality, pin_state_is_gemm, pin_last_row_noncausal, pin_linearity,
        pin_gqa_vs_mha, pin_decode_vs_forward, pin_resume]

ORACLE = {name: getattr(oracle, name) for name in
          ("brute_force", "chunkwise", "recurrent", "decode_step", "final_state", "noncausal")}


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(ORACLE)


def test_kv_group_contiguous():
    assert [oracle.kv_group(h, 128, 32) for h in (0, 3, 4, 127)] == [0, 0, 1, 31]
    assert [oracle.kv_group(h, 8, 8) for h in range(8)] == list(range(8))
    with pytest.raises(ValueError):
        oracle.kv_group(0, 6, 4)


def test_ragged_and_empty_edges():
    rng = np.random.default_rng(12)
    q, k, v = rand_inputs(rng, 1, 1, 1, 1, 3, 2)
    assert _close(oracle.chunkwise(q, k, v, 64)[0], (q[0, 0, 0] @ k[0, 0, 0]) * v)
    z = np.zeros((1, 1, 0, 3))
    o, S = oracle.chunkwise(z, z, np.zeros((1, 1, 0, 2)), 4)
    assert o.shape == (1, 1, 0, 2) and np.array_equal(S, np.zeros((1, 1, 3, 2)))


def test_tile_update_then_read_is_not_causal():
    """The xennon tiling box updates S with the whole tile before reading it;
    with tiles wider than one token that lets a row see later keys.  The oracle
    must differ from that order (and match it at one-token tiles)."""
    rng = np.random.default_rng(13)
    q, k, v = rand_inputs(rng, 1, 1, 1, 16, 4, 3)

    def update_then_read(tile):
        S = np.zeros((4, 3))
        o = np.zeros((16, 3))
        for a in range(0, 16, tile):
            S = S + k[0, 0, a:a + tile].T @ v[0, 0, a:a + tile]
            o[a:a + tile] = q[0, 0, a:a + tile] @ S
        return o

    ref = oracle.chunkwise(q, k, v, 4)[0][0, 0]
    assert not _close(update_then_read(4), ref, rtol=1e-3)
    assert _close(update_then_read(1), ref)


# ---------------------------------------------------------------------------
# Planted mistakes: every mutant must fail at least one pin.
# ---------------------------------------------------------------------------

def _mutant_chunkwise(mode):
    """A copy of the oracle's chunkwise form with one mistake planted."""
    def chunkwise(q, k, v, block, s_in=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, N, d = q.shape
        Hkv, dv = k.shape[1], v.shape[3]
        G = Hq // Hkv
        nb = -(-N // block)
        L = nb * block
        pad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (L - N, x.shape[3]))], axis=2)
        if mode == "gqa_modulo":   # query head h reads KV head h % Hkv
            kq = pad(k)[:, [h % Hkv for h in range(Hq)]].reshape(B, Hq, nb, block, d)
            vq = pad(v)[:, [h % Hkv for h in range(Hq)]].reshape(B, Hq, nb, block, dv)
        else:
            kq = pad(np.repeat(k, G, axis=1)).reshape(B, Hq, nb, block, d)
            vq = pad(np.repeat(v, G, axis=1)).reshape(B, Hq, nb, block, dv)
        Qb = pad(q).reshape(B, Hq, nb, block, d)
        T = np.matmul(np.swapaxes(kq, -1, -2), vq)
        if mode == "update_first":   # start states include the block's own keys
            starts = np.cumsum(T, axis=2)
        else:
            starts = np.zeros_like(T)
            if nb > 1:
                starts[:, :, 1:] = np.cumsum(T[:, :, :-1], axis=2)
        if s_in is not None and mode != "s_in_ignored":
            starts = starts + np.repeat(np.asarray(s_in, dtype=np.float64), G, axis=1)[:, :, None]
        if mode == "transposed_state" and d == dv:
            starts = np.swapaxes(starts, -1, -2)
        keep = np.tril(np.ones((block, block)), -1 if mode == "strict_tril" else 0)
        inter = 0 if mode == "no_inter" else np.matmul(Qb, starts)
        intra = np.matmul(np.matmul(Qb, np.swapaxes(kq, -1, -2)) * keep, vq)
        o = (inter + intra).reshape(B, Hq, L, dv)[:, :, :N]
        S = np.matmul(np.swapaxes(k, -1, -2), v)
        if s_in is not None and mode != "s_in_ignored":
            S = S + np.asarray(s_in, dtype=np.float64)
        return o, S
    return chunkwise


MUTANTS = ["update_first", "strict_tril", "gqa_modulo", "no_inter", "transposed_state", "s_in_ignored"]


@pytest.mark.parametrize("mode", MUTANTS)
def test_mutants_are_caught(mode):
    impl = dict(ORACLE)
    impl["chunkwise"] = _mutant_chunkwise(mode)
    failed = [p.__name__ for p in PINS if not p(impl)]
    assert failed, f"mutant {mode} passed every pin"
