"""Helpers shared by the GPU parity tests: tolerances and oracle comparison."""
import sys

import numpy as np
import torch

# Tolerance on max |gpu - oracle| in units of the oracle output's RMS over the
# compared tensor or slice: 1e-5 for float32 inputs, 2e-2 for bf16 inputs with
# float32 accumulation.  When the output itself is stored in bf16, each element
# may additionally carry its own round-to-nearest-even error, at most 2^-8 of
# its magnitude (bf16 keeps 8 significant bits).
TOL_F32_IN = 1e-5
TOL_BF16_IN = 2e-2
BF16_UNIT_ROUNDOFF = 2.0 ** -8
# States (and normaliser sums, and the backward's state gradient) of bf16 inputs
# are float32 sums of products that are exact in float32 (8-bit by 8-bit
# significands), so their only error is float32 accumulation: they take this bar
# in units of the reference state's RMS instead of the outputs' 2e-2.  Measured
# on MI355X: at most 4.4e-5 (a 4M-token sequence in 1M chunks) and 6.5e-5 (the
# state gradient summed over four query heads of 1M tokens); one token dropped or
# counted twice moves a million-token state's largest entries by about 1e-2.
TOL_STATE = 2e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    """Exact float64 copy of a device tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rms(x):
    return float(np.sqrt(np.mean(np.square(x)))) if x.size else 0.0


def check_close(name, got, ref, in_dtype, out_dtype, per_row=False, tol=None):
    """Assert the parity bar; returns max|err|/RMS(ref) (the literal metric).

    The unit of the tolerance is RMS(ref) over the compared tensor or slice.
    With per_row, it is the RMS of each row of ref (over its last axis) for the
    elements of that row: a normalised output is a weighted average of value
    rows whose magnitude shrinks like the inverse square root of the number
    of tokens averaged, while a kernel's relative error does not, so every
    row is held to the bar at its own scale.  `tol` overrides the input
    dtype's tolerance (TOL_STATE for states)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if per_row:
        r = np.sqrt(np.mean(np.square(ref), axis=-1, keepdims=True)) if ref.size else np.zeros(ref.shape[:-1] + (1,))
    else:
        r = np.asarray(rms(ref))
    err = np.abs(got - ref)
    if tol is None:
        tol = TOL_F32_IN if in_dtype == torch.float32 else TOL_BF16_IN
    bound = tol * r
    if out_dtype == torch.bfloat16:
        bound = bound + BF16_UNIT_ROUNDOFF * np.abs(ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(r > 0, err / np.where(r > 0, r, 1.0), np.where(err > 0, np.inf, 0.0))
    literal = float(rel.max()) if rel.size else 0.0
    worst = float(np.max(err - bound)) if err.size else 0.0
    unit = "row RMS" if per_row else "RMS"
    say(f"  {name}: max|err|/{unit} = {literal:.3e} (tol {tol:g}{' + 2^-8|ref|' if out_dtype == torch.bfloat16 else ''}),"
        f" {'min row RMS' if per_row else 'RMS'} = {float(np.min(r)) if np.size(r) else 0.0:.4g}, n = {ref.size}")
    assert worst <= 0.0, f"{name}: error exceeds bound by {worst:.3e} (max|err|/{unit} {literal:.3e})"
    return literal


def check_state(name, got, ref, in_dtype):
    """A float32 state against the state bar (the float32-input bar when the
    inputs are float32, which is tighter)."""
    tol = TOL_F32_IN if in_dtype == torch.float32 else TOL_STATE
    return check_close(name, got, ref, in_dtype, torch.float32, tol=tol)


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
