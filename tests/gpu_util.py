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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    """Exact float64 copy of a device tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rms(x):
    return float(np.sqrt(np.mean(np.square(x)))) if x.size else 0.0


def check_close(name, got, ref, in_dtype, out_dtype, scale=None):
    """Assert the parity bar; returns max|err|/RMS(ref) (the literal metric).

    `scale` replaces RMS(ref) as the unit of the tolerance where the output's
    own RMS is not its natural scale: a normalised output is a weighted
    average of value rows, so its errors scale with RMS(v) while its RMS
    shrinks as the averages widen."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    r = rms(ref) if scale is None else float(scale)
    err = np.abs(got - ref)
    tol = TOL_F32_IN if in_dtype == torch.float32 else TOL_BF16_IN
    bound = tol * r
    if out_dtype == torch.bfloat16:
        bound = bound + BF16_UNIT_ROUNDOFF * np.abs(ref)
    literal = float(err.max() / r) if r > 0 else float(err.max())
    worst = float(np.max(err - bound)) if err.size else 0.0
    unit = "RMS" if scale is None else "scale"
    say(f"  {name}: max|err|/{unit} = {literal:.3e} (tol {tol:g}{' + 2^-8|ref|' if out_dtype == torch.bfloat16 else ''}),"
        f" {unit} = {r:.4g}, n = {ref.size}")
    assert worst <= 0.0, f"{name}: error exceeds bound by {worst:.3e} (max|err|/RMS {literal:.3e})"
    return literal


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
