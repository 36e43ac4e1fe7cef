"""CPU oracle for exact batched Lloyd's K-Means (fp64 NumPy).

TEST INFRASTRUCTURE ONLY. Nothing but the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package. It shares no code,
constant or helper with the HIP library and imports nothing from it; the
library never calls it.

Parity status of every function is stated in ``oracle.kmeans``'s header.
"""
from .kmeans import (  # noqa: F401
    round_to_dtype,
    centroid_sqnorms,
    sq_distances,
    assign,
    update,
    objective,
    lloyd,
    AssignResult,
    UpdateResult,
    LloydResult,
)
