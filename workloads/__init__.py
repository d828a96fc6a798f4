"""Seeded synthetic inputs for the FwPKM chunk step.

This package holds shapes and random draws only: none of the method's
arithmetic lives here.  Both the CPU oracle's tests and the GPU path's
tests and benchmark take their inputs from it, so the two sides see the
same fp32 arrays.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .generate import (
    ChunkInputs,
    InitialTables,
    LayerWeights,
    chunk_inputs,
    draw_normal,
    draw_queries,
    draw_targets,
    draw_tokens,
    initial_tables,
    layer_weights,
)

__all__ = [
    "CONFIGS",
    "WorkloadConfig",
    "get_config",
    "ChunkInputs",
    "InitialTables",
    "LayerWeights",
    "chunk_inputs",
    "draw_normal",
    "draw_queries",
    "draw_targets",
    "draw_tokens",
    "initial_tables",
    "layer_weights",
]
