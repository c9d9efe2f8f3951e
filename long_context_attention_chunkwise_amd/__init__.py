"""Causal chunkwise linear attention (Lightning Attention) for AMD MI355X.

The computation lives in liblightning.so (C ABI in include/la.h, HIP kernels
for gfx950 under csrc/).  This package is its thin Python binding; torch is
used for device memory and streams only.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LA_BF16,
    LA_F32,
    LAError,
    backward,
    backward_state,
    backward_workspace_bytes,
    decode_step,
    forward,
    forward_noalloc,
    forward_state,
    forward_variant,
    load_library,
    status_str,
    workspace_bytes,
)
