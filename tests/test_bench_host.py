"""Host-side checks of bench.py (no GPU needed).

* More than one GPU is refused with a message, before any GPU work.
* The algorithmic HBM bytes the bench divides by kernel time equal what the
  semantics of each collective force any implementation to move: every input
  that some defined output depends on must be read once (except a value that
  simply stays in place), every defined output that differs from its input
  must be written once.  Both counts are
  found by perturbing inputs of the oracle on tiny int32 cases.
* The profile summaries the bench reads parse, and every suite row names a
  known workload and collective.
"""

import glob
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from tree_allreduce_algorithms_amd import workloads  # noqa: E402

DT = "int32"


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU only" in proc.stderr
    assert proc.stdout == ""


def test_call_count_cap_is_enforced():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "40"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2 and "--steps must stay" in proc.stderr


def _run(coll, x, root):
    fn = {
        "ring_allreduce": lambda: oracle.ring_allreduce(x, "sum", DT),
        "tree_allreduce": lambda: oracle.tree_allreduce(x, "sum", DT),
        "reduce_scatter": lambda: oracle.ring_reduce_scatter(x, "sum", DT),
        "allgather": lambda: oracle.ring_allgather(x, DT),
        "broadcast": lambda: oracle.broadcast(x, root, DT),
        "reduce": lambda: oracle.reduce(x, root, "sum", DT),
        "scatter": lambda: oracle.scatter(x, root, DT),
        "gather": lambda: oracle.gather(x, root, DT),
        "alltoall": lambda: oracle.alltoall(x, DT),
    }[coll]
    return np.stack(fn().bufs)


def _defined(coll, n, t, root):
    """Mask of the output positions the collective defines (the rest keep
    unspecified or untouched values)."""
    owned = oracle.chunk_layout(n, t)
    m = np.zeros((n, t), dtype=bool)
    if coll == "reduce_scatter":
        for r, (lo, hi) in enumerate(owned):
            m[r, lo:hi] = True
    elif coll in ("reduce", "gather"):
        m[root, :] = True
    elif coll == "scatter":
        for r, (lo, hi) in enumerate(owned):
            m[r, lo:hi] = True
    else:
        m[:, :] = True
    return m


def _forced_bytes(coll, n, t, root):
    rng = np.random.default_rng(n * 1000 + t * 10 + root)
    # wide values, so that no output equals its input by coincidence
    x = [rng.integers(-(1 << 30), 1 << 30, size=t, dtype=np.int32) for _ in range(n)]
    base = _run(coll, x, root)
    defined = _defined(coll, n, t, root)
    reads = 0
    for r in range(n):
        for i in range(t):
            y = [a.copy() for a in x]
            y[r][i] += 7
            changed = (_run(coll, y, root) != base) & defined
            # an input that only its own position passes through unchanged
            # (a value that stays where it is) needs no access
            own_only = changed[r, i] and np.count_nonzero(changed) == 1 and \
                _run(coll, y, root)[r, i] == y[r][i] and base[r, i] == x[r][i]
            if np.any(changed) and not own_only:
                reads += 1
    writes = int(np.count_nonzero((base != np.stack(x)) & defined))
    return (reads + writes) * 4


CASES = [(2, 5, 0), (3, 7, 2), (4, 10, 1), (4, 4, 3), (5, 13, 4), (5, 3, 4), (5, 11, 0)]


@pytest.mark.parametrize("coll", ["ring_allreduce", "tree_allreduce", "reduce_scatter",
                                  "allgather", "broadcast", "reduce", "scatter", "gather",
                                  "alltoall"])
@pytest.mark.parametrize("n,t,root", CASES)
def test_algorithmic_bytes_are_the_forced_traffic(coll, n, t, root):
    if coll == "alltoall":
        t -= t % n
        if t == 0:
            pytest.skip("AllToAll needs T >= N")
    assert bench.algorithmic_bytes(coll, n, t, 4, root) == _forced_bytes(coll, n, t, root)


def test_profile_summaries_parse():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md")))
    assert paths, "no traffic summaries committed"
    for p in paths:
        text = open(p).read()
        assert re.search(r"^kernel_source_sha256:\s*[0-9a-f]{64}\s*$", text, re.M), p
        m = re.search(r"^hbm_bytes_per_(launch|call):\s*(\d+)\s*$", text, re.M)
        assert m and int(m.group(2)) > 0, p
    trace = glob.glob(os.path.join(ROOT, "profiles", "*_trace.md"))
    assert trace, "no kernel-trace summary committed"


def test_traffic_lookup_reads_the_matching_key():
    """A single-launch line reads bytes per launch, a multi-launch (step)
    line bytes per call; a missing profile gives None."""
    if bench.traffic_from_profile("large_grad_fp32", "ring_allreduce", "fused") is not None:
        assert bench.traffic_from_profile("large_grad_fp32", "ring_allreduce", "fused",
                                          per_call=True) is None
    if bench.traffic_from_profile("large_grad_fp32", "ring_allreduce", "step", per_call=True):
        assert bench.traffic_from_profile("large_grad_fp32", "ring_allreduce", "step") is None
    assert bench.traffic_from_profile("no_such_workload", "ring_allreduce", "fused") is None
    # bfloat16 with float32 partials is a kernel of its own, with a summary of its own
    hop = bench.traffic_from_profile("large_grad_bf16", "ring_allreduce", "fused")
    acc = bench.traffic_from_profile("large_grad_bf16", "ring_allreduce", "fused",
                                     accumulate="float32")
    if hop is not None and acc is not None:
        assert hop != acc


def test_suite_rows_are_valid():
    for wname, coll, impl, extra in bench.SUITE:
        assert wname in workloads.WORKLOADS, wname
        assert coll in bench.COLLECTIVES, coll
        assert impl in ("fused", "step")
        args = bench.parse(["--workload", wname, "--collective", coll, "--impl", impl] + extra)
        assert args.steps <= bench.MAX_CALLS


@pytest.mark.parametrize("coll", ["ring_allreduce", "reduce_scatter", "tree_allreduce", "alltoall"])
def test_checker_finds_planted_mismatch_and_all_cores_pass_runs(coll):
    """The bench's windowed checker (host arrays in, host arrays out) reports no
    mismatch on the oracle's own output, exactly one after one output element
    is changed, and its all-cores timing pass runs over the same windows."""
    w = workloads.Workload("tiny", 4, 1000, "float32", "normal", 9, {"std": 1.0})
    x = workloads.host_inputs(w.nranks, w.count, w.dtype, w.dist, w.seed, w.params)
    fn = bench._oracle_fn(coll, w, 0, w.dtype)
    got = [b.copy() for b in fn(x, 0).bufs]
    secs, compared, bad = bench.run_checker(coll, x, got, w, 0, 256)
    assert bad == 0 and compared > 0 and secs >= 0
    got[1][0 if coll != "reduce_scatter" else 250] += 1.0
    assert bench.run_checker(coll, x, got, w, 0, 256)[2] == 1
    assert bench.time_checker_all_cores(coll, x, w, 0, 256, w.dtype, 3) >= 0


def test_kernel_hash_ignores_comments_only():
    """A profile stays valid across comment edits, and only those: the hash
    covers the device code with comments and blank lines removed, string
    and character literals kept as written."""
    code = 'int a = 1; // note\n/* block\n comment */\nconst char* s = "// not a comment";\n\nchar c = \'/\';\n'
    assert bench._code_only(code) == 'int a = 1;\nconst char* s = "// not a comment";\nchar c = \'/\';'
    assert bench._code_only("x = 1;  // a\n") == bench._code_only("x = 1;  // b\n")
    assert bench._code_only("x = 1;\n") != bench._code_only("x = 2;\n")


def test_kernel_hash_follows_includes(tmp_path):
    """The hash covers a kernel's source and the headers it includes,
    directly or through one another; a header no kernel includes (host-only
    code) leaves it unchanged."""
    (tmp_path / "a_kernels.hip").write_text('#include "common.hpp"\nint k;\n')
    (tmp_path / "common.hpp").write_text('#include "deep.hpp"\n#include <vector>\nint c;\n')
    (tmp_path / "deep.hpp").write_text("int d;\n")
    (tmp_path / "host_only.hpp").write_text("int h;\n")
    h0 = bench.kernel_source_hash(None, csrc=str(tmp_path))
    (tmp_path / "host_only.hpp").write_text("int h2;\n")
    assert bench.kernel_source_hash(None, csrc=str(tmp_path)) == h0
    (tmp_path / "deep.hpp").write_text("int d2;\n")
    assert bench.kernel_source_hash(None, csrc=str(tmp_path)) != h0


def test_committed_profiles_match_the_current_kernels():
    """Every profile summary records the hash of the device code it was taken
    on; each must match the current sources (its kernel's, or all of them for
    a summary over several kernels), so no committed figure describes code
    that has since changed."""
    keys = [None] + sorted(bench.KERNEL_FILE)
    current = {k: bench.kernel_source_hash(k) for k in keys}
    stale = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        found = re.findall(r"kernel_source_sha256(?: \((\w+)\))?:\s*([0-9a-f]{64})", text)
        assert found, f"{os.path.basename(path)} records no source hash"
        for key, sha in found:
            ok = sha == current.get(key) if key else sha in current.values()
            if not ok:
                stale.append((os.path.basename(path), key))
    assert not stale, stale
