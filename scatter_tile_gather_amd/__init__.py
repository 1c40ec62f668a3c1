"""Bounds-checked tile movement for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libstg.so (C ABI in include/stg.h); this
package is its ctypes binding (same function names) plus the seeded synthetic
input generators used by the tests and the benchmark.
"""
from . import inputs  # noqa: F401
from ._binding import (  # noqa: F401
    LIB_PATH,
    Prepared,
    STATIC_SCRATCH_BYTES,
    StgError,
    exported_names,
    gemm_bounded,
    gemm_scaled,
    gemm_scaled_workspace,
    load_library,
    prepare,
    ragged_tile_load,
    ragged_tile_store,
    ragged_tile_schedule,
    stg_tile_grid,
    stg_trace_enable,
    stg_trace_read,
    stg_version,
    tile_copy_bounded,
    tile_copy_windows,
    tile_gather,
    tile_gather_backward,
    tile_gather_backward_static,
    tile_gather_backward_workspace,
    tile_gather_masked,
    tile_scatter_masked,
    tile_store_clipped,
    tile_store_windows,
)
