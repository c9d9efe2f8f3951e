"""Plain fp64 CPU oracle for causal chunkwise linear attention (Lightning Attention).

Test infrastructure only: tests, the smoke check and the benchmark's CPU-baseline
leg may import it.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here.
"""
from .lightning import (  # noqa: F401
    kv_group,
    brute_force,
    chunkwise,
    recurrent,
    decode_step,
    final_state,
    noncausal,
    variant,
    backward_brute_force,
    backward_chunkwise,
)
