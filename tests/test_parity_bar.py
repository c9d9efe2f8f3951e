"""The parity bar must be able to fail.

Negative controls on the CPU for the bar the GPU tests apply (gpu_util.check_close):
the normalised forward variant (o_t = phi(q_t) . S_t / (phi(q_t) . z_t + eps), the
"Transformers are RNNs" family cited on page "从 Transformer 到 Lightning Attention，
从 PPO 到 CISPO") measured row by row, and states measured against their own bar.
Each case takes the oracle's output as the reference, then checks that a correct
answer perturbed at the kernels' own error level passes while plausible wrong
answers fail:

* an all-zero output;
* the sign of the last rows flipped;
* the output of the oracle with the carried normaliser sum z_in dropped (a
  mistake planted in the oracle's inputs, on the CPU).

Two regimes: a short sequence, and the tail of a million-token sequence, where
the carried state and normaliser sum of 1,048,576 - 256 earlier tokens
(drawn in closed form from the same distributions: S_ij a sum of that many
k_si v_sj terms, z_i a sum of that many k_si) make every output about 1e-3 of
the value RMS in size, the regime in which a bar in units of RMS(v) would pass a
zero output.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16_IN, TOL_STATE, check_close, check_state

BF16 = torch.bfloat16


def relu_inputs(rng, Hq, Hkv, N, d):
    q = rng.standard_normal((1, Hq, N, d)) / np.sqrt(d)
    k = rng.standard_normal((1, Hkv, N, d)) / np.sqrt(d)
    v = rng.standard_normal((1, Hkv, N, d))
    return q, k, v


def long_prefix_state(rng, Hkv, d, T):
    """State and normaliser sum after T earlier tokens with k = ReLU(N(0,1))/sqrt(d),
    v ~ N(0,1): S_ij is a sum of T independent k_si v_sj (mean 0, variance
    T E[k^2]) and z_i a sum of T values of k_si (mean T E[k], variance T Var k)."""
    ek = 1.0 / np.sqrt(2.0 * np.pi) / np.sqrt(d)           # E[ReLU(x)] / sqrt(d)
    ek2 = 0.5 / d                                            # E[ReLU(x)^2] / d
    S = rng.standard_normal((1, Hkv, d, d)) * np.sqrt(T * ek2)
    z = T * ek + rng.standard_normal((1, Hkv, d)) * np.sqrt(T * (ek2 - ek * ek))
    return S, z


CASES = [
    # name, causal, prefix tokens carried in (0: s_in, z_in small random)
    ("causal short", True, 0),
    ("non-causal short", False, 0),
    ("causal 1M tail", True, 1048576 - 256),
    ("non-causal 1M tail", False, 1048576 - 256),
]


@pytest.mark.parametrize("name,causal,prefix", CASES, ids=[c[0] for c in CASES])
def test_normalised_bar_rejects_wrong_outputs(name, causal, prefix):
    rng = np.random.default_rng(17)
    Hq, Hkv, N, d = 4, 1, 256, 32
    q, k, v = relu_inputs(rng, Hq, Hkv, N, d)
    if prefix:
        s_in, z_in = long_prefix_state(rng, Hkv, d, prefix)
    else:
        s_in = 0.5 * rng.standard_normal((1, Hkv, d, d))
        z_in = np.abs(rng.standard_normal((1, Hkv, d)))
    eps = 1e-6
    ref = oracle.variant(q, k, v, causal=causal, relu=True, normalize=True, eps=eps, s_in=s_in, z_in=z_in)[0]
    if prefix:
        # the regime the bar is for: outputs far below RMS(v)
        assert np.sqrt(np.mean(ref ** 2)) < 3e-3 * np.sqrt(np.mean(v ** 2))

    # a correct answer with relative errors at the bf16 kernels' level passes
    noisy = ref * (1.0 + 2.0 ** -9 * rng.uniform(-1.0, 1.0, ref.shape))
    check_close(f"{name}: near-exact", noisy, ref, BF16, BF16, per_row=True)
    check_close(f"{name}: near-exact, fp32 out", noisy, ref, BF16, torch.float32, per_row=True)

    wrong = {
        "zero output": np.zeros_like(ref),
        "last rows negated": np.concatenate([ref[:, :, :-16], -ref[:, :, -16:]], axis=2),
        "z_in dropped": oracle.variant(q, k, v, causal=causal, relu=True, normalize=True, eps=eps, s_in=s_in)[0],
    }
    for what, got in wrong.items():
        for out_dtype in (BF16, torch.float32):
            with pytest.raises(AssertionError):
                check_close(f"{name}: {what}", got, ref, BF16, out_dtype, per_row=True)


def test_rms_v_unit_would_pass_a_zero_output():
    """Why the unit changed: at the 1M tail, 2e-2 RMS(v) exceeds every output."""
    rng = np.random.default_rng(18)
    q, k, v = relu_inputs(rng, 4, 1, 256, 32)
    s_in, z_in = long_prefix_state(rng, 1, 32, 1048576 - 256)
    ref = oracle.variant(q, k, v, causal=True, relu=True, normalize=True, eps=1e-6, s_in=s_in, z_in=z_in)[0]
    assert np.max(np.abs(ref)) < TOL_BF16_IN * np.sqrt(np.mean(v ** 2))


def test_state_bar_rejects_a_token_counted_twice_or_dropped():
    """Final states of bf16 inputs are float32 sums of exact products, so they take
    a tighter bar than the outputs (TOL_STATE of the state RMS).  At 1M tokens one
    token counted twice, or dropped, at a segment boundary moves the state's
    largest entries by about 1e-2 of its RMS: that passes the output bar and must
    fail the state bar."""
    rng = np.random.default_rng(19)
    d, T = 32, 1048576
    S, _ = long_prefix_state(rng, 1, d, T)
    kt = np.maximum(rng.standard_normal(d), 0.0) / np.sqrt(d)
    vt = rng.standard_normal(d)
    one = np.outer(kt, vt)[None, None]
    assert TOL_STATE <= 2e-4
    for got in (S + one, S - one):
        check_close("state off by one token, output bar", got, S, BF16, torch.float32)
        with pytest.raises(AssertionError):
            check_state("state off by one token", got, S, BF16)
    # float32 rounding of a sum of T terms stays inside it
    noisy = S * (1.0 + 1e-6 * rng.uniform(-1.0, 1.0, S.shape))
    check_state("state with float32-level error", noisy, S, BF16)
