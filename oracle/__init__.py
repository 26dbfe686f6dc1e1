"""fp64 CPU oracle of PISA block-sparse attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. The HIP product path never does.
"""
from .pisa import (  # noqa: F401
    attention, block_ranges, block_stats, captured_mass, dense_attention,
    pisa_reference, route, spectral_norm,
)
