"""PISA piecewise block-sparse attention on AMD CDNA4 (gfx950).

The compute path lives in libparo.so (hand-written HIP kernels behind the C
ABI of include/paro.h); this package only marshals torch tensors into it.
"""
from .paro import (  # noqa: F401
    BLOCK, ParoError, ParoProblem, alloc_stats, attention, keep_to_k, lib, num_blocks,
    pisa_attention, precompute, problem, route, workspace_bytes,
)
