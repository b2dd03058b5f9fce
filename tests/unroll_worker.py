"""Worker for test_unroll_override_is_bit_identical (not collected by pytest).

The library reads AR_TUNE_UNROLL once per process, so each forced value runs
in a process of its own: this script checks the fan-out copy (AllGather,
Broadcast), whose pack grouping the variable forces, and the fused ring fold
(ReduceScatter, ring AllReduce, which must not depend on it) against the
oracle, every element, on ragged shapes whose default pack grouping differs
from the forced one.  Exit status 0 when every result matches.
"""

import os
import sys
import zlib

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import test_gpu_parity as tp  # noqa: E402  (helpers shared with the parity tests)
from tree_allreduce_algorithms_amd import workloads  # noqa: E402

SHAPES = [(2, 4_099), (5, 30_011), (8, 100_003), (16, 16 * 2048 + 5), (64, 20_011)]
COLLECTIVES = ("ring_allreduce", "reduce_scatter", "allgather", "broadcast")


def main():
    forced = os.environ.get("AR_TUNE_UNROLL")
    print(f"[unroll-worker] AR_TUNE_UNROLL={forced}", flush=True)
    for n, t in SHAPES:
        for dtype, dist, op in (("float32", "normal", "sum"), ("bfloat16", "uniform_pm1", "sum"),
                                ("int32", "int_uniform", "max")):
            seed = zlib.crc32(f"unroll-{n}-{t}-{dtype}".encode()) % 100_000
            x = workloads.host_inputs(n, t, dtype, dist, seed=seed, params=tp._params(dist, n))
            for coll in COLLECTIVES:
                tp.compare_collective(coll, x, dtype, op if coll in ("ring_allreduce", "reduce_scatter")
                                      else "sum", root=n // 2, impls=("fused",))
    print("[unroll-worker] all results match", flush=True)


if __name__ == "__main__":
    main()
