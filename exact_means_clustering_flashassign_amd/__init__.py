"""Exact batched Lloyd's K-Means on MI355X: FlashAssign + sort-inverse update.

All computation runs in the hand-written HIP kernels of ``libfkmeans.so``
(C ABI in ``include/fkmeans.h``); this package only marshals arguments.
"""
from ._binding import (  # noqa: F401
    BASELINE_LIB_PATH,
    FK_BF16,
    FK_F16,
    FK_F32,
    FKError,
    LIB_PATH,
    dtype_code,
    fk_assign,
    fk_lloyd,
    fk_lloyd_host,
    fk_norms,
    fk_status_string,
    fk_trace_begin,
    fk_trace_end,
    fk_update,
    fk_update_noalloc,
    fk_update_partial,
    FK_NOALLOC_SCRATCH_BYTES,
    fk_version,
    fk_workspace_size,
    fk_workspace_size_host,
    fkb_assign_materialized,
    fkb_mfma_peak,
    fkb_update_atomic,
    fkb_wall_clock_khz,
    load,
    load_baseline,
    torch_dtype,
    workspace,
)
from .api import FlashKMeans, batch_kmeans_Euclid, random_init  # noqa: F401,E402
