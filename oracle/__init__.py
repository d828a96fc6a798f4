"""Plain CPU oracle of the FwPKM chunked read-then-write step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only the tests, the package smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path.
"""

from .fwpkm_oracle import (  # noqa: F401
    DOT,
    IDW,
    NEAR_TIE_REL,
    UnitChunkResult,
    addressing_gradients,
    apply_updates,
    cartesian_best,
    chunk_gradients,
    dot_scores,
    forward_chunk,
    near_tie,
    read_unit,
    score_weights,
    split_query,
    sq_distances,
    best_k,
    unit_chunk,
)
