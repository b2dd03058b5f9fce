"""CPU tests of the C ABI (no GPU work is launched).

* libar.so loads and exports every function include/ar.h declares;
* the chunk layout and the logical byte / step counts the library reports
  equal the oracle's literal counters (the oracle simulates the schedule, the
  library derives the same schedule in C++: independent code);
* argument errors come back as AR_ERROR_INVALID_ARGUMENT before any HIP call;
* no-op calls (count 0, one rank) succeed and update only the step counter.

Only calls that fail validation or are no-ops are made here, so no kernel is
ever launched and fake device addresses are never dereferenced.
"""

import ctypes
import os
import re
import subprocess
import sys
import threading

import numpy as np
import pytest

import oracle
import tree_allreduce_algorithms_amd as ar
from tree_allreduce_algorithms_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    yield


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared_functions()
    assert len(names) >= 16, names
    handle = ctypes.CDLL(binding.LIB_PATH)
    for name in names:
        assert hasattr(handle, name), f"{name} missing from libar.so"
    assert sorted(binding.SIGNATURES) == names
    assert ar.lib().ar_version() == 1


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 63, 64])
@pytest.mark.parametrize("t", [0, 1, 5, 63, 64, 65, 1000, 16_777_217, 300_000_000])
def test_chunk_layout_matches_oracle(n, t):
    assert ar.chunk_size(n, t) == -(-t // n)
    layout = oracle.chunk_layout(n, t)
    for c in sorted({0, n // 2, n - 1}):
        assert ar.chunk_range(n, t, c) == layout[c]


ORACLE_CALLS = {
    "ring_allreduce": lambda x, root: oracle.ring_allreduce(x, "sum", "int32"),
    "reduce_scatter": lambda x, root: oracle.ring_reduce_scatter(x, "sum", "int32"),
    "allgather": lambda x, root: oracle.ring_allgather(x, "int32"),
    "broadcast": lambda x, root: oracle.broadcast(x, root, "int32"),
    "tree_allreduce": lambda x, root: oracle.tree_allreduce(x, "sum", "int32"),
    "reduce": lambda x, root: oracle.reduce(x, root, "sum", "int32"),
    "scatter": lambda x, root: oracle.scatter(x, root, "int32"),
    "gather": lambda x, root: oracle.gather(x, root, "int32"),
    "alltoall": lambda x, root: oracle.alltoall(x, "int32"),
}


@pytest.mark.parametrize("coll", sorted(ORACLE_CALLS))
@pytest.mark.parametrize("n,t", [(1, 10), (2, 9), (3, 7), (4, 1024), (5, 23), (8, 1000),
                                 (8, 3), (16, 37), (64, 130), (64, 1000), (6, 0)])
@pytest.mark.parametrize("dtype", ["int32", "bfloat16", "bfloat16_acc32"])
def test_expected_bytes_and_steps_match_oracle(coll, n, t, dtype):
    root = (n - 1) // 2
    if coll == "alltoall" and t % n:
        with pytest.raises(ar.ArError):
            ar.expected_bytes(coll, n, t, dtype)
        return
    x = [np.zeros(t, np.int32) for _ in range(n)]
    res = ORACLE_CALLS[coll](x, root)
    scale = oracle.ITEMSIZE[dtype]
    sent, recv = ar.expected_bytes(coll, n, t, dtype, root=root)
    assert sent == [int(v) // 4 * scale for v in res.sent]
    assert recv == [int(v) // 4 * scale for v in res.recv]
    assert ar.expected_steps(coll, n) == res.steps


def test_headline_byte_counts():
    """2T(N-1)/N per rank for the ring (Collectives from scratch, cost table) at
    N = 8, T = 300,000,000 float32; T(N-1)/N for ReduceScatter and AllGather."""
    sent, recv = ar.expected_bytes("ring_allreduce", 8, 300_000_000, "float32")
    assert sent == recv == [2 * 300_000_000 * 7 // 8 * 4] * 8
    sent, _ = ar.expected_bytes("reduce_scatter", 64, 16_777_217, "float32")
    assert sent[0] == 66_060_288 and sent[63] == 66_060_540
    assert sum(sent) == 63 * 16_777_217 * 4


# --- validation ---------------------------------------------------------------

FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation or is a no-op


def _call(name, ptrs, count=16, dtype="float32", op="sum", root=0):
    return binding.raw_call(name, ptrs, count, dtype, op=op, root=root, stream=0)


def _fake(n, stride=1 << 20, offset=0):
    return [FAKE + offset + r * stride for r in range(n)]


ALL = ["ring_allreduce", "reduce_scatter", "allgather", "broadcast", "tree_allreduce", "reduce",
       "scatter", "gather", "alltoall"]
ROOTED = ("broadcast", "reduce", "scatter", "gather")


@pytest.mark.parametrize("name", ALL)
def test_invalid_arguments(name):
    inv = binding.INVALID_ARGUMENT
    assert _call(name, []) == inv                                   # nranks 0
    assert _call(name, _fake(65)) == inv                            # nranks > 64
    assert _call(name, _fake(3)[:2] + [0]) == inv                   # NULL entry
    assert _call(name, _fake(4, offset=2)) == inv                   # not 4-byte aligned
    assert _call(name, _fake(4, stride=32), count=16) == inv        # ranges overlap
    assert _call(name, [FAKE] * 2) == inv                           # same buffer twice
    assert _call(name, _fake(4), count=(1 << 63)) == inv            # byte size overflows
    lib = ar.lib()
    pp, keep = binding._ptr_array(_fake(4))
    assert getattr(lib, "ar_" + name) is not None
    if name in ("ring_allreduce", "reduce_scatter", "tree_allreduce"):
        fn = getattr(lib, "ar_" + name)
        assert fn(pp, 4, 16, 7, 0, None) == inv                     # unknown dtype
        assert fn(pp, 4, 16, 1, 9, None) == inv                     # unknown op
        assert fn(None, 4, 16, 1, 0, None) == inv                   # NULL bufs
    if name in ("broadcast", "scatter", "gather"):
        fn = getattr(lib, "ar_" + name)
        assert fn(pp, 4, 16, 1, 4, None) == inv                     # root out of range
        assert fn(pp, 4, 16, 1, -1, None) == inv
    if name == "alltoall":
        assert lib.ar_alltoall(pp, 4, 18, 1, None) == inv           # 4 does not divide 18
    if name == "reduce":
        assert lib.ar_reduce(pp, 4, 16, 1, 0, 4, None) == inv       # root out of range
        assert lib.ar_reduce(pp, 4, 16, 1, 0, -1, None) == inv
        assert lib.ar_reduce(pp, 4, 16, 1, 9, 0, None) == inv       # unknown op
        assert lib.ar_reduce(pp, 4, 16, 7, 0, 0, None) == inv       # unknown dtype
    del keep


# An armed launch-failure injection fails a call's first launch before
# anything reaches the HIP runtime, so these calls need no GPU either.
HIP_ERROR_LAUNCH_FAILURE = 719   # hipErrorLaunchFailure in HIP's runtime API


@pytest.mark.parametrize("impl", ["fused", "step"])
@pytest.mark.parametrize("name", ALL + ["allreduce"])
def test_injected_launch_failure_is_reported(name, impl):
    """ar_debug_fail_launch(1): the call's first launch reports
    hipErrorLaunchFailure, so the call returns AR_ERROR_HIP, keeps the error
    for ar_last_hip_error() on its own thread only, and leaves the counters
    as they were."""
    lib = ar.lib()
    old = ar.get_impl()
    try:
        ar.set_impl(impl)
        ar.reset_counters()
        ar.debug_fail_launch(1)
        assert _call(name, _fake(4), count=64, root=1) == binding.HIP_ERROR
        assert lib.ar_last_hip_error() == HIP_ERROR_LAUNCH_FAILURE
        assert ar.counters(4) == ([0] * 4, [0] * 4, 0)
        seen = []
        th = threading.Thread(target=lambda: seen.append(lib.ar_last_hip_error()))
        th.start()
        th.join()
        assert seen == [0]
        with pytest.raises(ar.ArError, match=f"hipError_t {HIP_ERROR_LAUNCH_FAILURE}"):
            ar.debug_fail_launch(1)
            binding._check(_call(name, _fake(4), count=64, root=1), name)
    finally:
        ar.debug_fail_launch(0)
        ar.set_impl(old)


_DEBUG_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import tree_allreduce_algorithms_amd as ar
from tree_allreduce_algorithms_amd import binding
names = ["ring_allreduce", "reduce_scatter", "allgather", "broadcast", "tree_allreduce", "reduce",
         "scatter", "gather", "alltoall", "allreduce"]
bad, calls = [], 0
for impl in ("fused", "step"):
    ar.set_impl(impl)
    for n, t in ((2, 5), (5, 23), (12, 1000), (17, 5_921_371), (64, 16_777_217)):
        ptrs = [0x7F0000000000 + r * (1 << 27) for r in range(n)]
        for name in names:
            count = t - t % n if name == "alltoall" else t
            ar.debug_fail_launch(1)
            status = binding.raw_call(name, ptrs, count, "float32", op="sum", root=n - 1)
            calls += 1
            if status != binding.HIP_ERROR:
                bad.append((impl, n, t, name, status))
ar.debug_fail_launch(0)
print("BAD", bad) if bad else print("OK", calls)
"""


def test_debug_mode_checks_each_schedule_before_enqueuing():
    """With AR_DEBUG=1 at load, a call with work builds the schedule it
    follows and checks it (schedule_violation, pinned by the sanitized host
    check) before its first launch, aborting on a violation.  The library's
    schedules pass for every collective and implementation at 2 to 64 ranks,
    ragged sizes included, and each call goes on to its launch (here an
    injected failure, so no GPU is needed)."""
    proc = subprocess.run([sys.executable, "-c", _DEBUG_SCRIPT, ROOT], capture_output=True,
                          text=True, timeout=300, env={**os.environ, "AR_DEBUG": "1"})
    assert proc.returncode == 0, proc.stderr[-3000:]
    assert proc.stdout.split() == ["OK", "100"], proc.stdout[-3000:]


def test_launch_failure_injection_spares_argument_errors_and_no_ops():
    """Calls that fail validation or are no-ops make no launch: they return
    as without the injection, which stays armed for the next launch."""
    lib = ar.lib()
    try:
        assert lib.ar_debug_fail_launch(-1) == binding.INVALID_ARGUMENT
        assert lib.ar_debug_fail_launch(1) == binding.SUCCESS
        assert _call("ring_allreduce", _fake(4, offset=2)) == binding.INVALID_ARGUMENT
        assert _call("ring_allreduce", _fake(4), count=0) == binding.SUCCESS
        assert _call("ring_allreduce", _fake(1), count=64) == binding.SUCCESS
        assert _call("ring_allreduce", _fake(4), count=64) == binding.HIP_ERROR
    finally:
        assert lib.ar_debug_fail_launch(0) == binding.SUCCESS


def test_bfloat16_needs_only_2_byte_alignment_to_validate():
    # odd addresses fail for every dtype; 2-byte offsets fail for 4-byte types
    assert _call("allgather", _fake(2, offset=1), dtype="bfloat16") == binding.INVALID_ARGUMENT
    assert _call("allgather", _fake(2, offset=2), dtype="int32") == binding.INVALID_ARGUMENT


@pytest.mark.parametrize("name", ALL)
def test_noop_calls_succeed_and_count_steps(name):
    ar.reset_counters()
    assert _call(name, _fake(4), count=0) == binding.SUCCESS
    assert _call(name, _fake(1), count=1000) == binding.SUCCESS
    sent, recv, steps = ar.counters(4)
    assert sent == recv == [0, 0, 0, 0]
    assert steps == ar.expected_steps(name, 4)
    ar.reset_counters()
    assert ar.counters(4)[2] == 0


def test_impl_switch_and_status_strings():
    old = ar.get_impl()
    try:
        ar.set_impl("step")
        assert ar.get_impl() == "step"
        ar.set_impl("fused")
        assert ar.get_impl() == "fused"
        assert ar.lib().ar_set_impl(5) == binding.INVALID_ARGUMENT
    finally:
        ar.set_impl(old)
    lib = ar.lib()
    assert lib.ar_status_string(0) == b"success"
    assert lib.ar_status_string(1) == b"invalid argument"
    # no AR_ERROR_HIP on a fresh thread (the value is kept per thread)
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.ar_last_hip_error()))
    th.start()
    th.join()
    assert seen == [0]


def test_host_helpers_reject_bad_arguments():
    lib = ar.lib()
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.ar_chunk_range(0, 10, 0, ctypes.byref(lo), ctypes.byref(hi)) == 1
    assert lib.ar_chunk_range(4, 10, 4, ctypes.byref(lo), ctypes.byref(hi)) == 1
    assert lib.ar_chunk_range(4, 10, 0, None, ctypes.byref(hi)) == 1
    buf = (ctypes.c_uint64 * 64)()
    assert lib.ar_expected_bytes(9, 4, 10, 1, 0, buf, buf) == 1
    assert lib.ar_expected_bytes(3, 4, 10, 1, 4, buf, buf) == 1
    assert lib.ar_expected_steps(0, 0) == -1 and lib.ar_expected_steps(0, 65) == -1
    assert lib.ar_counters_read(65, None, None) == 1
    assert lib.ar_chunk_size(0, 10) == 0


# --- cost model and the size-based ring/tree choice -----------------------------

def _oracle_hbm_bytes(coll, impl, n, t, dtype):
    """HBM bytes of one call from the oracle's literal schedule: the fused
    kernels move each input once and each output once; the step-by-step
    implementation moves 3 bytes per element of every reduce transfer and 2
    per element of every copy transfer."""
    s = 2 if dtype == "bfloat16" else 4
    if n == 1:
        return 0
    if coll == "reduce":                 # one fused implementation
        return (n + 1) * t * s
    if coll == "alltoall":               # every off-diagonal block read and written once
        return 2 * n * (n - 1) * (t // n) * s
    if impl == "fused" and coll not in ("scatter", "gather"):
        if coll in ("ring_allreduce", "tree_allreduce") and _split(n, t, s):
            return (2 * n + 1) * t * s     # fold into one rank per element (N+1) T s, then fan-out N T s
        return {"ring_allreduce": 2 * n * t, "tree_allreduce": 2 * n * t,
                "reduce_scatter": (n + 1) * t, "allgather": n * t, "broadcast": n * t}[coll] * s
    x = [np.zeros(t, np.int32) for _ in range(n)]
    moved = int(sum(ORACLE_CALLS[coll](x, 0).sent)) // 4       # elements transferred
    reduced = {"ring_allreduce": moved // 2, "tree_allreduce": moved // 2,
               "reduce_scatter": moved}.get(coll, 0)
    return (3 * reduced + 2 * (moved - reduced)) * s


def _split(n, t, s):
    """The fused AllReduces run in two launches from 12 ranks and 384 MiB of
    inputs up (the documented rule of ar.h): the ring as ReduceScatter then
    AllGather, the double tree as its folds into the two roots then their
    fan-out."""
    return n >= 12 and n * t * s >= 384 << 20


@pytest.mark.parametrize("coll", sorted(ORACLE_CALLS))
@pytest.mark.parametrize("impl", ["fused", "step"])
@pytest.mark.parametrize("n,t,dtype", [(4, 256, "float32"), (8, 100_003, "bfloat16"),
                                       (64, 1_000_003, "float32"), (2, 7, "int32")])
def test_predicted_time_is_the_documented_formula(coll, impl, n, t, dtype):
    alpha, gbps = ar.get_cost_model(coll, impl)
    launches = 1 if impl == "fused" or coll in ("reduce", "alltoall") else ar.expected_steps(coll, n)
    if impl == "fused" and coll in ("ring_allreduce", "tree_allreduce") and \
            _split(n, t, 2 if dtype == "bfloat16" else 4):
        launches = 2
    if n == 1:
        launches = 0
    want = launches * alpha + _oracle_hbm_bytes(coll, impl, n, t, dtype) / (gbps * 1e3)
    assert ar.predict_time(coll, impl, n, t, dtype) == pytest.approx(want, rel=1e-12)


@pytest.mark.parametrize("coll", sorted(ORACLE_CALLS))
@pytest.mark.parametrize("impl", ["fused", "step"])
@pytest.mark.parametrize("n,t,dtype", [(4, 256, "float32"), (8, 100_003, "bfloat16"),
                                       (64, 1_000_003, "float32"), (2, 7, "int32"),
                                       (17, 5_921_371, "float32"), (40, 16_777_259, "bfloat16"),
                                       (1, 1000, "float32")])
def test_launch_plan_is_the_documented_rule(coll, impl, n, t, dtype):
    """ar_launch_plan: one launch moving the algorithmic bytes for the fused
    kernels (two launches and (2N+1) T s for the split AllReduces), one launch
    per schedule step for the literal schedules, the oracle's step bytes;
    nothing for one rank."""
    s = 2 if dtype == "bfloat16" else 4
    launches, nbytes = ar.launch_plan(coll, impl, n, t, dtype)
    if n == 1:
        assert (launches, nbytes) == (0, 0)
        return
    if impl == "fused" or coll in ("reduce", "alltoall"):
        want = 1
    else:
        want = ar.expected_steps(coll, n)
    if impl == "fused" and coll in ("ring_allreduce", "tree_allreduce") and _split(n, t, s):
        want = 2
    assert launches == want
    assert nbytes == _oracle_hbm_bytes(coll, impl, n, t, dtype)


def test_launch_plan_float32_partials_run_fused():
    """bfloat16 with float32 partials runs its reductions fused under either
    setting, so the step setting plans the fused kernel for them."""
    n, t = 8, 1_000_000
    for coll in ("ring_allreduce", "reduce_scatter", "tree_allreduce"):
        assert ar.launch_plan(coll, "step", n, t, "bfloat16_acc32") == \
            ar.launch_plan(coll, "fused", n, t, "bfloat16_acc32") == (1, ar.launch_plan(coll, "fused", n, t, "bfloat16")[1])
    assert ar.launch_plan("allgather", "step", n, t, "bfloat16_acc32")[0] == n - 1


def test_launch_plan_arguments_are_validated():
    lib = ar.lib()
    n, b = ctypes.c_int(), ctypes.c_uint64()
    assert lib.ar_launch_plan(9, 0, 4, 10, 1, ctypes.byref(n), ctypes.byref(b)) == binding.INVALID_ARGUMENT
    assert lib.ar_launch_plan(0, 2, 4, 10, 1, ctypes.byref(n), ctypes.byref(b)) == binding.INVALID_ARGUMENT
    assert lib.ar_launch_plan(0, 0, 65, 10, 1, ctypes.byref(n), ctypes.byref(b)) == binding.INVALID_ARGUMENT
    assert lib.ar_launch_plan(0, 0, 4, 10, 9, ctypes.byref(n), ctypes.byref(b)) == binding.INVALID_ARGUMENT
    assert lib.ar_launch_plan(0, 0, 4, 10, 1, None, ctypes.byref(b)) == binding.INVALID_ARGUMENT
    assert lib.ar_launch_plan(0, 0, 4, 10, 1, ctypes.byref(n), None) == binding.INVALID_ARGUMENT


@pytest.mark.parametrize("coll", ["ring_allreduce", "tree_allreduce"])
@pytest.mark.parametrize("n,t,dtype", [(64, 1_572_864, "float32"), (64, 1_572_863, "float32"),
                                       (32, 100_000_000, "float32"), (17, 5_921_371, "float32"),
                                       (17, 5_921_370, "float32"), (16, 100_000_000, "float32"),
                                       (12, 8_388_608, "float32"), (12, 8_388_607, "float32"),
                                       (11, 100_000_000, "float32"),
                                       (64, 1_048_576, "float32"), (64, 16_777_217, "float32"),
                                       (20, 10_066_330, "bfloat16"), (20, 10_066_329, "bfloat16"),
                                       (33, 4_194_304, "bfloat16")])
def test_fused_allreduce_split_is_modelled(coll, n, t, dtype):
    """From 12 ranks and 384 MiB of inputs the fused AllReduces are two
    launches moving (2N+1) T s bytes; below either bound one launch of 2N T s."""
    s = 2 if dtype == "bfloat16" else 4
    alpha, gbps = ar.get_cost_model(coll, "fused")
    split = _split(n, t, s)
    assert split == (n >= 12 and n * t * s >= 402_653_184)
    launches, nbytes = (2, (2 * n + 1) * t * s) if split else (1, 2 * n * t * s)
    want = launches * alpha + nbytes / (gbps * 1e3)
    assert ar.predict_time(coll, "fused", n, t, dtype) == pytest.approx(want, rel=1e-12)


def test_allreduce_choice_switches_at_the_model_crossover():
    """With the step implementation on one GPU ring and tree move the same
    HBM bytes (5 (N-1) T s), so the tree (2 ceil(log2 N) launches) beats the
    ring (2 (N-1) launches) unless its bandwidth is lower.  Give the tree a
    lower bandwidth: it must win below the analytic crossover size and lose
    above it."""
    saved = {(c, i): ar.get_cost_model(c, i) for c in ("ring_allreduce", "tree_allreduce")
             for i in ("fused", "step")}
    old = ar.get_impl()
    try:
        ar.set_impl("step")
        ar.set_cost_model("ring_allreduce", "step", 4.0, 6000.0)
        ar.set_cost_model("tree_allreduce", "step", 4.0, 5000.0)
        n, s = 8, 4
        # ring 14 a + 35 T s / 6000e3 = tree 6 a + 35 T s / 5000e3  ->  T*
        t_star = (14 - 6) * 4.0 / (35 * s / 5000e3 - 35 * s / 6000e3)
        below, above = int(t_star * 0.9), int(t_star * 1.1)
        assert ar.allreduce_choice(n, below, "float32") == "tree_allreduce"
        assert ar.allreduce_choice(n, above, "float32") == "ring_allreduce"
        # equal predictions pick the ring
        ar.set_cost_model("tree_allreduce", "step", 4.0 * 14 / 6, 6000.0)
        assert ar.allreduce_choice(n, 1000, "float32") == "ring_allreduce"
        ar.set_impl("fused")
        ar.set_cost_model("ring_allreduce", "fused", 3.0, 6000.0)
        ar.set_cost_model("tree_allreduce", "fused", 2.0, 5000.0)
        assert ar.allreduce_choice(4, 256, "float32") == "tree_allreduce"
        assert ar.allreduce_choice(4, 1 << 26, "float32") == "ring_allreduce"
    finally:
        for (c, i), (a, g) in saved.items():
            ar.set_cost_model(c, i, a, g)
        ar.set_impl(old)


def test_default_model_ties_the_fused_ring_and_tree():
    """The shipped coefficients give the fused ring and the fused double tree
    one shared fit (same launches, same bytes, split alike), so every size
    predicts a tie and the size-based choice runs the ring; under the step
    implementation the tree wins small messages (fewer launches) and the ring
    large ones."""
    assert ar.get_cost_model("ring_allreduce", "fused") == ar.get_cost_model("tree_allreduce", "fused")
    old = ar.get_impl()
    try:
        ar.set_impl("fused")
        for t in (1, 256, 262_144, 4_194_304, 67_108_864, 300_000_000):
            for n in (2, 4, 8, 17, 32, 64):
                assert ar.predict_time("ring_allreduce", "fused", n, t, "float32") == \
                    ar.predict_time("tree_allreduce", "fused", n, t, "float32")
                assert ar.allreduce_choice(n, t, "float32") == "ring_allreduce"
        ar.set_impl("step")
        assert ar.allreduce_choice(4, 4_194_304, "float32") == "tree_allreduce"
        assert ar.allreduce_choice(4, 67_108_864, "float32") == "ring_allreduce"
    finally:
        ar.set_impl(old)


def test_cost_model_arguments_are_validated():
    lib = ar.lib()
    assert lib.ar_set_cost_model(9, 0, 1.0, 1.0) == binding.INVALID_ARGUMENT
    assert lib.ar_set_cost_model(0, 3, 1.0, 1.0) == binding.INVALID_ARGUMENT
    assert lib.ar_set_cost_model(0, 0, -1.0, 1.0) == binding.INVALID_ARGUMENT
    assert lib.ar_set_cost_model(0, 0, 1.0, 0.0) == binding.INVALID_ARGUMENT
    assert lib.ar_set_cost_model(0, 0, float("nan"), 1.0) == binding.INVALID_ARGUMENT
    out = ctypes.c_int()
    assert lib.ar_allreduce_choice(0, 10, 1, ctypes.byref(out)) == binding.INVALID_ARGUMENT
    assert lib.ar_allreduce_choice(4, 10, 9, ctypes.byref(out)) == binding.INVALID_ARGUMENT
    assert lib.ar_allreduce_choice(4, 10, 1, None) == binding.INVALID_ARGUMENT
    us = ctypes.c_double()
    assert lib.ar_predict_time(0, 0, 65, 10, 1, ctypes.byref(us)) == binding.INVALID_ARGUMENT
    assert _call("allreduce", _fake(65)) == binding.INVALID_ARGUMENT
    assert _call("allreduce", _fake(4, offset=2)) == binding.INVALID_ARGUMENT
    assert _call("allreduce", _fake(4), count=0) == binding.SUCCESS
    assert _call("ring_allreduce", [0, 0, 0], count=0) == binding.SUCCESS   # empty tensors


def test_costfit_recovers_known_coefficients():
    from tree_allreduce_algorithms_amd import costfit
    truth = {("ring_allreduce", "step"): (3.7, 6100.0), ("tree_allreduce", "fused"): (2.5, 5600.0)}
    records = []
    for (coll, impl), (alpha, gbps) in truth.items():
        for launches, nbytes in ((6, 15_360), (6, 15_728_640), (6, 251_658_240), (6, 4.0e9),
                                 (1, 8_192), (1, 2.1e9)):
            if impl == "fused":
                launches = 1
            us = launches * alpha + nbytes / (gbps * 1e3)
            records.append({"config": {"collective": coll, "impl": impl,
                                       "timing": "events, Infinity Cache flushed"},
                            "roofline": {"launches_per_step": launches,
                                         "algorithmic_bytes_per_call": nbytes,
                                         "event_ms_mean": us / 1e3}})
    got = costfit.fit(records)
    for key, (alpha, gbps) in truth.items():
        assert got[key][0] == pytest.approx(alpha, rel=1e-9)
        assert got[key][1] == pytest.approx(gbps, rel=1e-9)


def test_costfit_pools_the_fused_ring_and_tree():
    """The fused ring and tree AllReduce points are fitted together: both get
    the pooled least-squares coefficients, so the model ties them (and the
    size-based choice runs the ring); the step pairs stay separate."""
    from tree_allreduce_algorithms_amd import costfit
    truth = {("ring_allreduce", "fused"): (6.0, 6000.0), ("tree_allreduce", "fused"): (6.0, 6000.0),
             ("tree_allreduce", "step"): (3.0, 5000.0)}
    records = []
    for (coll, impl), (alpha, gbps) in truth.items():
        for nbytes in (8_192, 8.4e6, 1.3e8, 2.1e9):
            launches = 1 if impl == "fused" else 4
            us = launches * alpha + nbytes / (gbps * 1e3)
            records.append({"config": {"collective": coll, "impl": impl,
                                       "timing": "events, Infinity Cache flushed"},
                            "roofline": {"launches_per_step": launches,
                                         "algorithmic_bytes_per_call": nbytes,
                                         "event_ms_mean": us / 1e3 * (1.02 if coll == "tree_allreduce" else 1.0)}})
    got = costfit.fit(records)
    assert got[("ring_allreduce", "fused")] == got[("tree_allreduce", "fused")]
    assert got[("tree_allreduce", "step")][1] == pytest.approx(5000.0 / 1.02, rel=1e-9)
    sep = costfit.fit(records, pool_fused_allreduce=False)
    assert sep[("ring_allreduce", "fused")] != sep[("tree_allreduce", "fused")]
