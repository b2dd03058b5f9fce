"""MI355X-native ring / tree collectives over N rank buffers on one GPU.

The collectives live in a C-ABI shared library (``libar.so``: HIP kernels for
gfx950 plus the C ABI declared in ``include/ar.h``); this package is a thin
ctypes binding with the same names.  The library is loaded on first use; if
it has not been built the call raises.
"""

from .binding import (  # noqa: F401
    ArError,
    RankBuffers,
    allgather,
    allreduce,
    allreduce_choice,
    alltoall,
    broadcast,
    chunk_range,
    chunk_size,
    counters,
    debug_fail_launch,
    expected_bytes,
    expected_steps,
    gather,
    get_cost_model,
    get_impl,
    lib,
    launch_plan,
    predict_time,
    raw_call,
    reduce,
    reduce_scatter,
    reset_counters,
    ring_allreduce,
    scatter,
    set_cost_model,
    set_impl,
    tree_allreduce,
)
