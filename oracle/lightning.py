"""fp64 CPU oracle for the causal Lightning Attention forward pass and decode step.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module.  It shares no code with the HIP path: it
imports NumPy and nothing else, and every function below is a plain
transcription of the mathematics it cites, in float64.

Sources (page title, then the passage):

* "如何理解MiniMax股价创历史新高？拆解国产大模型技术底座" (vergex.cn), section
  "Lightning Attention：长上下文为什么突然变得便宜了", the chunkwise teaching
  code: a running d x dv state starts at zero; for each block the output is the
  block's queries times the state plus the lower-triangular (diagonal included)
  in-block score matrix times the block's values; only then is K_b^T V_b added
  to the state.  The page omits normalisation and stabilisation, so the oracle
  has none.
* "MiniMax-01与Lightning Attention" (metaphor-xennon.pages.dev), section 2.2:
  linear attention drops softmax and uses associativity, phi(Q) (phi(K)^T V);
  its LinearAttentionCore is the non-causal form (one global K^T V).
  Section 4.1 table: the key-value state is updated incrementally and the full
  history is not kept (streaming decode).  Section 1.1 table: 128 attention
  heads over 32 KV heads (grouped-query attention).
* "奧特曼的“溫和奇點”愿景，線性注意力的勝利？MiniMax-M1技術報告深度解析"
  (digipub.cc), the associativity passage: A*B*C = A*(B*C).
* "从 Transformer 到 Lightning Attention，从 PPO 到 CISPO" (space.minimaxi.com),
  the "Transformers are RNNs" entry: softmax approximated by a kernel feature
  map (the family of the normalised variant in `variant`).

Readings where the pages are silent (each pinned in tests/test_oracle.py):

* no normalisation, no 1/sqrt(d) scaling and no feature map inside the
  operator: inputs arrive already feature-mapped and scaled;
* the causal mask keeps s <= t (the teaching code's tril keeps the diagonal);
* the state is read before the block's own update (teaching code order);
* query head h reads KV head g(h) = h // (Hq // Hkv) (contiguous groups);
* an optional initial state s_in adds q_t . s_in to every output row;
* decode updates the state with the new token first, then reads it, so the
  current token attends to itself as in the forward pass.

Every function is pinned by tests that do not re-type its formula: a
hand-worked example, closed forms, brute force over Python loops, block-size
invariance, causality, the final state against a library GEMM, the non-causal
special case, linearity, GQA against repeated-head MHA, and recurrent/decode
against the block form (tests/test_oracle.py); the backward pass against
central finite differences of the forward (tests/test_oracle_backward.py);
the variants against their special cases, closed forms and the token-by-token
recurrence (tests/test_oracle_variants.py).
No function here is parity unpinned.

Layouts: q [B, Hq, N, d], k [B, Hkv, N, d], v [B, Hkv, N, dv],
o [B, Hq, N, dv], state [B, Hkv, d, dv].  Decode drops the N axis.
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_group(h, Hq, Hkv):
    """KV head read by query head h: contiguous groups of Hq // Hkv heads."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _heads_to_groups(Hq, Hkv):
    return np.array([kv_group(h, Hq, Hkv) for h in range(Hq)], dtype=np.int64)


def _check(q, k, v, s_in):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, dim]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape[:3] != (B, Hkv, N):
        raise ValueError("shape mismatch between q, k, v")
    if s_in is not None and s_in.shape != (B, Hkv, d, v.shape[3]):
        raise ValueError("s_in must be [B, Hkv, d, dv]")
    return B, Hq, Hkv, N, d, v.shape[3]


def brute_force(q, k, v, s_in=None):
    """Textbook causal sum: o_t = sum_{s<=t} (q_t . k_s) v_s (+ q_t . s_in).

    Builds the full N x N score matrix per head, zeroes entries with s > t and
    multiplies by V.  Quadratic in N: for small inputs only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s_in = None if s_in is None else _f64(s_in)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    o = np.zeros((B, Hq, N, dv))
    for b in range(B):
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            scores = q[b, h] @ k[b, g].T                  # [N, N], entry (t, s)
            scores = scores * (np.arange(N)[None, :] <= np.arange(N)[:, None])
            o[b, h] = scores @ v[b, g]
            if s_in is not None:
                o[b, h] += q[b, h] @ s_in[b, g]
    return o


def final_state(k, v, s_in=None):
    """State after all tokens: s_in + K^T V per (batch, KV head)."""
    k, v = _f64(k), _f64(v)
    S = np.matmul(np.swapaxes(k, -1, -2), v)
    if s_in is not None:
        S = S + _f64(s_in)
    return S


def chunkwise(q, k, v, block, s_in=None):
    """Chunkwise (block) evaluation of the causal sum, from its algebra.

    Cut the tokens into blocks of `block` (the last one may be shorter).  By
    associativity the causal sum splits, for a query t in block b, into the
    keys of earlier blocks and the keys of block b up to t:
        o_t = q_t . S_b + sum_{s in b, s <= t} (q_t . k_s) v_s,
        S_b = s_in + sum_{i < b} K_i^T V_i     (exclusive prefix sum)
    Every block's contribution K_i^T V_i is formed first, the start states
    are their exclusive running sum, and then each block's output is its
    inter term Q_b S_b plus its masked in-block term (Q_b K_b^T, entries with
    s <= t kept, diagonal included) times V_b.  The final state is s_in plus
    the sum over every block.  Returns (o, S_final).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s_in = None if s_in is None else _f64(s_in)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    if block < 1:
        raise ValueError("block must be >= 1")
    G = Hq // Hkv
    nb = -(-N // block)
    L = nb * block
    # Zero rows pad the last block: a zero key or value adds nothing to any
    # sum, and the rows of zero queries are dropped from the output.
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (L - N, x.shape[3]))], axis=2)
    # Query head j of KV head g is head g * G + j (kv_group: contiguous
    # groups), so [B, Hq] splits into [B, Hkv, G].
    Qb = pad(q).reshape(B, Hkv, G, nb, block, d)
    Kb = pad(k).reshape(B, Hkv, nb, block, d)
    Vb = pad(v).reshape(B, Hkv, nb, block, dv)
    T = np.matmul(np.swapaxes(Kb, -1, -2), Vb)                # [B, Hkv, nb, d, dv]
    before = np.zeros_like(T)
    if nb > 1:
        before[:, :, 1:] = np.cumsum(T[:, :, :-1], axis=2)    # sum over blocks i < b
    starts = before if s_in is None else before + s_in[:, :, None]
    inter = np.matmul(Qb, starts[:, :, None])                 # [B, Hkv, G, nb, block, dv]
    keep = np.tril(np.ones((block, block)))                   # s <= t, diagonal kept
    scores = np.matmul(Qb, np.swapaxes(Kb, -1, -2)[:, :, None]) * keep
    intra = np.matmul(scores, Vb[:, :, None])
    o = (inter + intra).reshape(B, Hq, L, dv)[:, :, :N]
    S = T.sum(axis=2) if s_in is None else s_in + T.sum(axis=2)
    return o, S


def recurrent(q, k, v, s_in=None):
    """Token-by-token form: S <- S + k_t^T v_t, then o_t = q_t S.

    This is the tiling box of the xennon page run with one-token tiles
    (update, then read), which is causal and keeps the diagonal.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s_in = None if s_in is None else _f64(s_in)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    S = np.zeros((B, Hkv, d, dv)) if s_in is None else s_in.copy()
    o = np.zeros((B, Hq, N, dv))
    for t in range(N):
        S, o[:, :, t] = decode_step(S, q[:, :, t], k[:, :, t], v[:, :, t])
    return o, S


def decode_step(S, q, k, v):
    """One decode token for every (batch, KV head) state.

    S [B, Hkv, d, dv]; q [B, Hq, d]; k [B, Hkv, d]; v [B, Hkv, dv].
    Rank-one update first (S + k^T v), then each query head in the group
    reads the updated state.  Returns (S_new, o) with o [B, Hq, dv].
    """
    S, q, k, v = _f64(S), _f64(q), _f64(k), _f64(v)
    B, Hkv, d, dv = S.shape
    Hq = q.shape[1]
    if q.shape != (B, Hq, d) or k.shape != (B, Hkv, d) or v.shape != (B, Hkv, dv):
        raise ValueError("decode shapes do not match the state")
    S_new = S + k[:, :, :, None] * v[:, :, None, :]
    gidx = _heads_to_groups(Hq, Hkv)
    o = np.matmul(q[:, :, None, :], S_new[:, gidx])[:, :, 0, :]
    return S_new, o


def noncausal(q, k, v):
    """Non-causal linear attention (LinearAttentionCore): q_t (K^T V) for every t."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, None)
    gidx = _heads_to_groups(Hq, Hkv)
    kv = final_state(k, v)
    return np.matmul(q, kv[:, gidx])


# ---------------------------------------------------------------------------
# Variants of the forward (feature map, non-causal, normalised).
#
# The LinearAttentionCore code ("MiniMax-01与Lightning Attention", section
# 2.2) applies a feature map phi (a linear layer and a ReLU; the learned layer
# is not part of the operator, the ReLU is) to Q and K and computes the
# non-causal phi(Q) (phi(K)^T V).  The kernel-approximation family it belongs
# to ("从 Transformer 到 Lightning Attention，从 PPO 到 CISPO", the
# "Transformers are RNNs" entry) divides each output by the same weights summed
# without the values, phi(q_t) . sum_s phi(k_s); the teaching code of the
# vergex page leaves that normalisation (and its stabilisation) out.  Reading
# taken here: the denominator runs over the same tokens as the numerator, and
# eps is added to it (eps = 0 divides exactly).
# ---------------------------------------------------------------------------

def variant(q, k, v, causal=True, relu=False, normalize=False, eps=0.0, s_in=None, z_in=None):
    """Forward variants written from the N x N weight matrix.

    phi = ReLU (relu=True) or the identity, applied to q and k.  With
    W[t, s] = phi(q_t) . phi(k_s), kept for s <= t when causal:
        numerator_t   = sum_s W[t, s] v_s + phi(q_t) . s_in
        denominator_t = sum_s W[t, s]     + phi(q_t) . z_in
        o_t = numerator_t                         (normalize=False)
        o_t = numerator_t / (denominator_t + eps) (normalize=True)
    Returns (o, S_out, z_out) with S_out = s_in + sum_s phi(k_s)^T v_s and
    z_out = z_in + sum_s phi(k_s) per (batch, KV head); z_in is [B, Hkv, d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s_in = None if s_in is None else _f64(s_in)
    z_in = None if z_in is None else _f64(z_in)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    if z_in is not None and z_in.shape != (B, Hkv, d):
        raise ValueError("z_in must be [B, Hkv, d]")
    if relu:
        q, k = np.maximum(q, 0.0), np.maximum(k, 0.0)
    keep = np.tril(np.ones((N, N))) if causal else np.ones((N, N))
    o = np.zeros((B, Hq, N, dv))
    for b in range(B):
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            W = (q[b, h] @ k[b, g].T) * keep                            # [t, s]
            num = W @ v[b, g]
            den = W.sum(axis=1)
            if s_in is not None:
                num = num + q[b, h] @ s_in[b, g]
            if z_in is not None:
                den = den + q[b, h] @ z_in[b, g]
            o[b, h] = num / (den + eps)[:, None] if normalize else num
    S = np.matmul(np.swapaxes(k, -1, -2), v)
    if s_in is not None:
        S = S + s_in
    z = k.sum(axis=2)
    if z_in is not None:
        z = z + z_in
    return o, S, z


# ---------------------------------------------------------------------------
# Backward pass (gradients of a scalar loss L given dO = dL/do).
#
# The pages give no backward; it follows from the forward definition by
# matrix calculus.  With M = tril(Q K^T) per query head (diagonal kept) and
# O = M V + Q s_in:
#     dQ = tril(dO V^T) K + dO s_in^T
#     dK = sum over the group's query heads of tril(dO V^T)^T Q
#     dV = sum over the group's query heads of M^T dO
#     ds_in = sum over the group's query heads of Q^T dO
# A gradient ds_out on the final state S_out = s_in + K^T V (fed back by the
# next chunk of a sequence processed in chunks) adds V ds_out^T to dK,
# K ds_out to dV and ds_out to ds_in.
# backward_brute_force writes exactly that; backward_chunkwise evaluates the
# same gradients block by block: dQ is the causal forward recurrence applied
# to (dO, V, K) with initial state s_in^T, and dK, dV run backwards over the
# blocks with a state R = sum over later tokens and the group's heads of
# q_t^T dO_t (d x dv):
#     dV_b = K_b R + sum_h triu(K_b Q_hb^T) dO_hb
#     dK_b = V_b R^T + sum_h triu(V_b dO_hb^T) Q_hb
#     R   <- R + sum_h Q_hb^T dO_hb          (after the block)
# starting from R = ds_out (zeros by default) and ending at R = ds_in,
# where triu keeps query positions t >= key position s.  Pinned in
# tests/test_oracle_backward.py by central finite differences of the forward.
# ---------------------------------------------------------------------------

def _check_do(q, v, do):
    if do.shape != (q.shape[0], q.shape[1], q.shape[2], v.shape[3]):
        raise ValueError("dO must be [B, Hq, N, dv]")


def _check_ds_out(ds_out, B, Hkv, d, dv):
    if ds_out is not None and ds_out.shape != (B, Hkv, d, dv):
        raise ValueError("ds_out must be [B, Hkv, d, dv]")


def backward_brute_force(q, k, v, do, s_in=None, ds_out=None):
    """Gradients from the N x N masked score matrix.  Returns (dq, dk, dv, ds_in)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    s_in = None if s_in is None else _f64(s_in)
    ds_out = None if ds_out is None else _f64(ds_out)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    _check_do(q, v, do)
    _check_ds_out(ds_out, B, Hkv, d, dv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    ds = np.zeros((B, Hkv, d, dv))
    if ds_out is not None:
        dk += np.matmul(v, np.swapaxes(ds_out, -1, -2))
        dvv += np.matmul(k, ds_out)
        ds += ds_out
    mask = np.arange(N)[None, :] <= np.arange(N)[:, None]          # (t, s): s <= t
    for b in range(B):
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            m = (q[b, h] @ k[b, g].T) * mask                         # [t, s]
            dm = (do[b, h] @ v[b, g].T) * mask                       # dL/dM, [t, s]
            dq[b, h] = dm @ k[b, g]
            if s_in is not None:
                dq[b, h] += do[b, h] @ s_in[b, g].T
            dk[b, g] += dm.T @ q[b, h]
            dvv[b, g] += m.T @ do[b, h]
            ds[b, g] += q[b, h].T @ do[b, h]
    return dq, dk, dvv, ds


def backward_chunkwise(q, k, v, do, block, s_in=None, ds_out=None):
    """Gradients by the block recurrences (forward for dQ, reverse for dK, dV).
    Returns (dq, dk, dv, ds_in)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    s_in = None if s_in is None else _f64(s_in)
    ds_out = None if ds_out is None else _f64(ds_out)
    B, Hq, Hkv, N, d, dv = _check(q, k, v, s_in)
    _check_do(q, v, do)
    _check_ds_out(ds_out, B, Hkv, d, dv)
    if block < 1:
        raise ValueError("block must be >= 1")
    # dQ: causal recurrence on (queries dO, keys V, values K), state s_in^T.
    s_t = None if s_in is None else np.swapaxes(s_in, -1, -2)
    dq, _ = chunkwise(do, v, k, block, s_t)
    # dK, dV: reverse recurrence, state summed over each group's query heads.
    G = Hq // Hkv
    R = np.zeros((B, Hkv, d, dv)) if ds_out is None else ds_out.copy()
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    starts = list(range(0, N, block))
    for a in reversed(starts):
        e = min(a + block, N)
        kb, vb = k[:, :, a:e], v[:, :, a:e]                            # [B, Hkv, c, *]
        c = e - a
        keep = np.arange(c)[None, :] >= np.arange(c)[:, None]           # (s, t): t >= s
        dvb = np.matmul(kb, R)
        dkb = np.matmul(vb, np.swapaxes(R, -1, -2))
        upd = np.zeros_like(R)
        for j in range(G):
            qh = q[:, [g * G + j for g in range(Hkv)], a:e]            # head j of every group
            doh = do[:, [g * G + j for g in range(Hkv)], a:e]
            x = np.matmul(kb, np.swapaxes(qh, -1, -2)) * keep           # [s, t]
            y = np.matmul(vb, np.swapaxes(doh, -1, -2)) * keep
            dvb = dvb + np.matmul(x, doh)
            dkb = dkb + np.matmul(y, qh)
            upd = upd + np.matmul(np.swapaxes(qh, -1, -2), doh)
        dvv[:, :, a:e] = dvb
        dk[:, :, a:e] = dkb
        R = R + upd
    return dq, dk, dvv, R
