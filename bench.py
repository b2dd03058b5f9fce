"""Benchmark: ring AllReduce of N=8 float32 rank buffers of 1.2 GB each on one
MI355X, through the C ABI of libar.so.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]
                    [--workload large_grad_fp32] [--collective ring_allreduce]
                    [--impl fused|step] [--flush-mall] [--accumulate float32]
                    [--no-cpu-baseline] [--no-parity] [--suite FILE.jsonl]

One "step" is one collective call over the whole workload (every rank buffer
already resident in HBM).  W untimed calls, then K timed calls bracketed by
torch.cuda.synchronize(); HIP events recorded on the stream the library
launches on bracket each call (or, for calls under 1 GiB of traffic run
back to back, the whole group of K calls, whose event time is then spread
evenly over them).  Rank 0 prints one JSON line.

The collectives work in place, so step k+1 reduces step k's output: after an
AllReduce every rank holds the sum, and each further call multiplies the
magnitude by about N.  The workloads' inputs stay finite for more than 35
calls, so W + K is capped there; the kernels have no value-dependent control
flow.

value: algorithm bandwidth, T * itemsize / (wall time per call), in GB/s
(1 GB = 1e9 bytes).  roofline: the dominant kernel's algorithmic HBM bytes per
launch (2 * N * T * itemsize for a fused AllReduce: every input read once,
every output written once) over its average event-timed duration, against the
8 TB/s HBM peak; `traffic` is the HBM bytes per launch that rocprofv3's
FETCH_SIZE / WRITE_SIZE counters measured for the same kernel source (from the
committed summary under profiles/), else null.

After timing, one more call runs on freshly drawn inputs.  The library's
per-rank byte counters for that call go into the line next to their closed
forms (for the ring AllReduce: 2 T (N-1)/N bytes per rank, the cost table of
"Collectives from scratch").  Its whole output is compared, window by window,
with the CPU checker (a literal NumPy simulation of the schedule,
single-threaded) on the same inputs; the checker's time over all windows is
the cpu_baseline, and the same windows spread over one host thread per
affinity core give its all-cores time.  With --flush-mall a
1 GiB buffer is overwritten before every timed call (outside the events) so
that workloads smaller than the 256 MB Infinity Cache are read from HBM;
value then comes from the event times.

--suite FILE runs every configuration of the workload table (fused and
step-by-step implementations, ring and tree, each size of the sweep) and
appends one JSON line per run to FILE; the headline line is printed last.
"""

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring AllReduce algbw GB/s and % of HBM peak, N=8 fp32 1.2 GB/rank"
HBM_PEAK_GBPS = 8000.0
DTYPE_TAG = {"float32": "f32", "bfloat16": "bf16", "int32": "i32"}
MAX_CALLS = 35
COLLECTIVES = ["ring_allreduce", "reduce_scatter", "allgather", "broadcast", "tree_allreduce",
               "allreduce", "reduce", "scatter", "gather", "alltoall"]
def kernel_name(collective, impl, n, launches=1):
    """The kernel that dominates one call (16-byte aligned rank buffers): the
    folds run through LDS-staged tiles for every N >= 2; a fused AllReduce of
    two launches is its fold then the fan-out."""
    if collective in ("ring_allreduce", "tree_allreduce") and impl == "fused" and launches == 2:
        fold = "ring_stage_kernel" if collective == "ring_allreduce" else "tree_stage_kernel"
        return fold + " + fanout_group_kernel"
    if collective in ("ring_allreduce", "reduce_scatter") and impl == "fused":
        return "ring_stage_kernel"
    if collective == "tree_allreduce" and impl == "fused" or collective == "reduce":
        return "tree_stage_kernel"
    if collective in ("allgather", "broadcast") and impl == "fused":
        return "fanout_group_kernel"
    if collective == "alltoall":
        return "alltoall_kernel"
    return "step_kernel"


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large_grad_fp32")
    p.add_argument("--collective", default="ring_allreduce", choices=COLLECTIVES)
    p.add_argument("--impl", default="fused", choices=["fused", "step"])
    p.add_argument("--root", type=int, default=0, help="root of the rooted collectives")
    p.add_argument("--accumulate", default=None, choices=[None, "float32"],
                   help="bfloat16 workloads: reductions carry float32 partials, round once")
    p.add_argument("--flush-mall", action="store_true")
    p.add_argument("--cpu-window", type=int, default=1 << 24,
                   help="elements per rank per window of the CPU checker")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU checker (and with it the output comparison)")
    p.add_argument("--no-parity", action="store_true", help="alias of --no-cpu-baseline")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="also run one device-to-device copy of this many MiB "
                        "(the reference kernel for the PMC byte counters)")
    p.add_argument("--suite", default=None, metavar="FILE",
                   help="run every configuration, append JSON lines to FILE")
    p.add_argument("--jsonl", default=None, help="append the JSON line to this file too")
    return p.parse_args(argv)


KERNEL_FILE = {  # kernel -> the source file that defines it
    "ring_stage_kernel": "ring_kernels.hip", "ring_fold_kernel": "ring_kernels.hip",
    "tree_stage_kernel": "tree_kernels.hip", "tree_fold_kernel": "tree_kernels.hip",
    "fanout_group_kernel": "copy_kernels.hip", "fanout_kernel": "copy_kernels.hip",
    "alltoall_kernel": "copy_kernels.hip",
    "step_kernel": "step_kernels.hip",
}


def _code_only(text):
    """C/C++ source text with comments removed and blank lines dropped, so
    that a change to comments alone keeps a profile valid."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                    # string or char literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line.strip())


def _local_includes(code):
    return re.findall(r'^\s*#\s*include\s+"([^"]+)"', code, re.M)


def kernel_source_hash(kernel=None, csrc=None):
    """sha256 over the device code a kernel is built from (comments and blank
    lines removed): its own source file (every .hip file when kernel is None)
    plus the headers of the same directory that it includes, directly or
    through one another, in name order."""
    csrc = csrc or os.path.join(ROOT, "tree_allreduce_algorithms_amd", "csrc")
    own = KERNEL_FILE.get(kernel)
    code = {}

    def read(name):
        if name not in code:
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                code[name] = _code_only(f.read())
            for inc in _local_includes(code[name]):
                if os.path.exists(os.path.join(csrc, inc)):
                    read(inc)

    for name in sorted(os.listdir(csrc)):
        if name.endswith(".hip") and (own is None or name == own):
            read(name)
    h = hashlib.sha256()
    for name in sorted(code):
        h.update(name.encode() + b"\0" + code[name].encode())
    return h.hexdigest()


def traffic_from_profile(workload, collective, impl, per_call=False, accumulate=None, kernel=None):
    """HBM bytes per launch (per call for a multi-launch implementation, with
    per_call) from the committed PMC summary of this implementation and
    workload (and accumulator: bfloat16 with float32 partials is a kernel of
    its own), if it was taken on the current kernel source; None otherwise."""
    suffix = "_float32_partials" if accumulate else ""
    path = os.path.join(ROOT, "profiles", f"traffic_{collective}_{impl}_{workload}{suffix}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    key = "hbm_bytes_per_call" if per_call else "hbm_bytes_per_launch"
    sha = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    val = re.search(rf"^{key}:\s*([0-9]+)\s*$", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_hash(kernel):
        return None
    return int(val.group(1))


def algorithmic_bytes(collective, n, t, isz, root=0):
    """HBM bytes the fused implementation must move per call."""
    c = -(-t // n)                                   # chunk size (ragged tail, maybe empty chunks)
    root_chunk = max(0, min(t, (root + 1) * c) - min(t, root * c))
    return {
        "ring_allreduce": 2 * n * t * isz,     # read N inputs, write N outputs
        "tree_allreduce": 2 * n * t * isz,
        "reduce_scatter": (n + 1) * t * isz,   # read N, write the owner's chunk
        "allgather": n * t * isz,              # read each chunk once, write N-1 copies
        "broadcast": n * t * isz,
        "reduce": (n + 1) * t * isz,           # read N, write the root's buffer
        # every non-root rank's chunk, read once and written once
        "scatter": 2 * (t - root_chunk) * isz if n > 1 else 0,
        "gather": 2 * (t - root_chunk) * isz if n > 1 else 0,
        "alltoall": 2 * (n - 1) * t * isz,     # every off-diagonal block read and written once
    }[collective]


def step_bytes(collective, n, t, isz, root=0):
    """HBM bytes of the literal schedule: 3 per element of a reduce transfer
    (read both sides, write one), 2 per element of a copy transfer."""
    import tree_allreduce_algorithms_amd as ar
    sent, _ = ar.expected_bytes(collective, n, t, "bfloat16" if isz == 2 else "int32", root=root)
    moved = sum(sent) // isz                     # elements transferred over all steps
    # share of those elements moved by reduce (rather than copy) transfers
    if collective in ("reduce", "alltoall"):     # one implementation
        return algorithmic_bytes(collective, n, t, isz, root)
    reduce_share = {"ring_allreduce": (1, 2), "tree_allreduce": (1, 2),
                    "reduce_scatter": (1, 1)}.get(collective, (0, 1))
    reduced = moved * reduce_share[0] // reduce_share[1]
    return (3 * reduced + 2 * (moved - reduced)) * isz


def _oracle_fn(collective, w, root, odt):
    import oracle
    t = w.count
    return {
        "ring_allreduce": lambda x, a: oracle.ring_allreduce(x, "sum", odt, a, t),
        "tree_allreduce": lambda x, a: oracle.tree_allreduce(x, "sum", odt, 2, a, t),
        "reduce_scatter": lambda x, a: oracle.ring_reduce_scatter(x, "sum", odt, a, t),
        "allgather": lambda x, a: oracle.ring_allgather(x, odt, a, t),
        "broadcast": lambda x, a: oracle.broadcast(x, root, odt, a, t),
        "reduce": lambda x, a: oracle.reduce(x, root, "sum", odt, a, t),
        "scatter": lambda x, a: oracle.scatter(x, root, odt, a, t),
        "gather": lambda x, a: oracle.gather(x, root, odt, a, t),
        "alltoall": lambda x, a: oracle.alltoall(x, odt),
    }[collective]


def host_copy(tensors, dtype):
    """Whole device buffers as host NumPy arrays (bfloat16 as uint16 bits)."""
    import numpy as np
    import torch
    if dtype == "bfloat16":
        return [x.view(torch.int16).cpu().numpy().view(np.uint16) for x in tensors]
    return [x.cpu().numpy() for x in tensors]


def run_checker(collective, pristine, got, w, root, window, odt=None):
    """Run the CPU checker over every window of the workload on the host
    arrays `pristine` (the inputs), single-threaded, and compare with the
    device output `got` (host arrays); returns (seconds in the checker,
    compared elements, mismatching elements)."""
    import numpy as np
    import oracle

    n, t = w.nranks, w.count
    fn = _oracle_fn(collective, w, root, odt or w.dtype)
    owned = oracle.chunk_layout(n, t)
    if collective == "alltoall":
        window = t   # an output element comes from another position: whole buffers
    secs, compared, bad = 0.0, 0, 0
    for a in range(0, t, window):
        b = min(t, a + window)
        xin = [p[a:b] for p in pristine]
        t0 = time.perf_counter()
        want = fn(xin, a).bufs
        secs += time.perf_counter() - t0
        for r in range(n):
            g = got[r][a:b]
            if collective == "reduce_scatter":
                lo, hi = max(owned[r][0], a) - a, min(owned[r][1], b) - a
                if lo >= hi:
                    continue
                g, ww = g[lo:hi], want[r][lo:hi]
            else:
                ww = want[r]
            compared += g.size
            bad += int(np.count_nonzero(g != ww))
    return secs, compared, bad


def time_checker_all_cores(collective, pristine, w, root, window, odt, workers):
    """The same windowed CPU checker, its windows spread over `workers` host
    threads (NumPy releases the GIL inside its array operations); returns the
    wall time over all windows.  Results are not compared again: the
    single-threaded pass already did that on the same inputs."""
    from concurrent.futures import ThreadPoolExecutor

    t = w.count
    fn = _oracle_fn(collective, w, root, odt or w.dtype)
    if collective == "alltoall":
        window = t
    starts = list(range(0, t, window))

    def one(a):
        fn([p[a:min(t, a + window)] for p in pristine], a)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(one, starts))
    return time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_one(args):
    import torch

    import tree_allreduce_algorithms_amd as ar
    from tree_allreduce_algorithms_amd import workloads

    w = workloads.WORKLOADS[args.workload]
    n, t, isz = w.nranks, w.count, w.itemsize
    dev = torch.device("cuda:0")
    ar.set_impl(args.impl)
    print(f"[bench] workload={w.name} N={n} T={t} dtype={w.dtype} collective={args.collective} "
          f"impl={args.impl} flush={args.flush_mall}", file=sys.stderr, flush=True)

    def draw():
        return [workloads.device_rank(w.dist, w.dtype, t, w.seed, r, dev, w.params)
                for r in range(n)]

    bufs = draw()
    torch.cuda.synchronize()
    if args.accumulate and w.dtype != "bfloat16":
        raise SystemExit("--accumulate float32 applies to bfloat16 workloads")
    acc = args.accumulate
    odt = "bfloat16_acc32" if acc else w.dtype     # library / oracle dtype name
    # "allreduce" runs the ring or the tree by the library's cost model
    ran = (ar.allreduce_choice(n, t, odt) if args.collective == "allreduce"
           else args.collective)
    # every call goes through a prepared handle: one library call, arguments
    # checked once (the host cost of the free functions is paid at setup)
    method = {
        "allreduce": lambda rb: rb.allreduce(),
        "ring_allreduce": lambda rb: rb.ring_allreduce(),
        "tree_allreduce": lambda rb: rb.tree_allreduce(),
        "reduce_scatter": lambda rb: rb.reduce_scatter(),
        "allgather": lambda rb: rb.allgather(),
        "broadcast": lambda rb: rb.broadcast(root=args.root),
        "reduce": lambda rb: rb.reduce(root=args.root),
        "scatter": lambda rb: rb.scatter(root=args.root),
        "gather": lambda rb: rb.gather(root=args.root),
        "alltoall": lambda rb: rb.alltoall(),
    }[args.collective]
    handles = {}

    def call(b):
        # the entry keeps `b` alive, so its id cannot be reused by another list
        key = id(b)
        if key not in handles:
            handles[key] = (b, ar.RankBuffers(b, accumulate=acc))
        return method(handles[key][1])

    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush_mall else None
    # Events bracket every call when the Infinity Cache is flushed between
    # calls (the flush must stay outside them) or when a call moves enough
    # bytes that recording two events (a few microseconds of host time each)
    # is noise.  Small calls back to back are bracketed as one group of K
    # calls instead: per-call events would make the host loop, and with it
    # the wall time, several times slower than the calls themselves.
    per_call_events = args.flush_mall or algorithmic_bytes(args.collective if args.collective
                                                           != "allreduce" else "ring_allreduce",
                                                           n, t, isz, args.root) >= (1 << 30)
    nev = args.steps if per_call_events else 1
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    # a reduction multiplies the values' magnitude by up to N per call: with
    # more calls than MAX_CALLS in all, the inputs are put back after the
    # warm-up (a device copy, so the GPU stays busy)
    restore = (args.warmup + args.steps > MAX_CALLS
               and args.collective in ("ring_allreduce", "tree_allreduce", "allreduce",
                                       "reduce_scatter", "reduce"))
    saved = [b.clone() for b in bufs] if restore else None

    # collect garbage now (earlier runs free large host arrays) and keep the
    # collector out of the timed loop, which small workloads make host-bound;
    # done before the warm-up, so that the timed calls follow it without the
    # GPU falling idle (after an idle pause the GPU's clocks take some tens of
    # milliseconds of load to settle, which short calls would otherwise time)
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        call(bufs)
    if saved is not None:
        for b, v in zip(bufs, saved):
            b.copy_(v)
        del saved
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if per_call_events:
        for i in range(args.steps):
            if flush_buf is not None:
                flush_buf.fill_(float(i))
            starts[i].record(stream)
            call(bufs)
            ends[i].record(stream)
    else:
        starts[0].record(stream)
        for i in range(args.steps):
            call(bufs)
        ends[0].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    if per_call_events:
        event_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    else:   # the group's GPU time spread evenly over its calls
        event_ms = [starts[0].elapsed_time(ends[0]) / args.steps] * args.steps
    finite = bool(all(torch.isfinite(b).all().item() for b in bufs))
    del flush_buf

    launch_ms = sum(event_ms) / len(event_ms)
    per_call_s = (launch_ms * 1e-3) if args.flush_mall else wall / args.steps
    alg = algorithmic_bytes(ran, n, t, isz, args.root)
    # Reduce and AllToAll have one implementation; with float32 partials the
    # reductions run fused under either implementation
    fused = (args.impl == "fused" or ran in ("reduce", "alltoall")
             or (acc is not None and ran in ("ring_allreduce", "reduce_scatter", "tree_allreduce")))
    # what the library runs: its launches, and for the two-launch AllReduces
    # of many ranks the (2N+1) T s bytes they move
    launches, impl_bytes = ar.launch_plan(ran, args.impl, n, t, odt)
    if fused:
        moved = impl_bytes if launches > 1 else alg
    else:
        moved = step_bytes(ran, n, t, isz, args.root)
    achieved = moved / (launch_ms * 1e-3) / 1e9
    kernel = kernel_name(ran, "fused" if fused else args.impl, n, launches)
    traffic = traffic_from_profile(w.name, args.collective, args.impl, per_call=launches > 1,
                                   accumulate=acc, kernel=None if launches > 1 else kernel)

    result = {
        "metric": METRIC,
        "value": round(t * isz / per_call_s / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_call_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAG[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "collective": args.collective, "ran": ran,
                   "impl": args.impl, "accumulate": acc or w.dtype,
                   "nranks": n, "count_per_rank": t, "rank_bytes": t * isz,
                   "distribution": w.dist, "params": w.params, "seed": w.seed,
                   "timing": "events, Infinity Cache flushed before each call"
                   if args.flush_mall else "wall clock over the K calls"},
        "pct_of_hbm_peak": round(100.0 * alg / per_call_s / 1e9 / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "algorithmic_bytes_per_launch": moved if launches == 1 else None,
            "algorithmic_bytes_per_call": moved,
            "launches_per_step": launches,
            "events": "one pair per call" if per_call_events else
                      f"one pair around all {args.steps} calls (small calls back to back)",
            "event_ms_mean": round(launch_ms, 4),
            "event_ms_median": round(sorted(event_ms)[len(event_ms) // 2], 4),
            "event_ms_min": round(min(event_ms), 4),
            "event_ms_p90": round(sorted(event_ms)[min(len(event_ms) - 1,
                                                       int(0.9 * len(event_ms)))], 4),
            "event_ms_max": round(max(event_ms), 4),
        },
        "outputs_finite": finite,
        "device": torch.cuda.get_device_name(dev),
    }

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        torch.cuda.synchronize()
        ce0.record(stream)
        dst.copy_(src)
        ce1.record(stream)
        torch.cuda.synchronize()
        ms = ce0.elapsed_time(ce1)
        result["copy_calibration"] = {"bytes_read": nbytes, "bytes_written": nbytes,
                                      "ms": round(ms, 4),
                                      "gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
        del src, dst

    del bufs
    handles.clear()
    torch.cuda.empty_cache()
    if not (args.no_cpu_baseline or args.no_parity):
        print("[bench] checking one call on fresh inputs against the CPU checker",
              file=sys.stderr, flush=True)
        pristine = draw()
        got = [p.clone() for p in pristine]
        ar.reset_counters()
        call(got)
        torch.cuda.synchronize()
        sent, recv, steps = ar.counters(n)
        want_sent, want_recv = ar.expected_bytes(ran, n, t, odt, root=args.root)
        result["counters"] = {
            "sent": sent, "recv": recv, "steps": steps,
            "closed_form_sent": want_sent, "closed_form_recv": want_recv,
            "expected_steps": ar.expected_steps(ran, n),
            "match": sent == want_sent and recv == want_recv and steps == ar.expected_steps(ran, n),
        }
        if ran == "ring_allreduce" and t % n == 0:
            # the cost table's ring row: 2 T (N-1) / N bytes sent and received per rank
            law = 2 * t * (n - 1) // n * isz
            result["counters"]["ring_law_bytes_per_rank"] = law
            result["counters"]["ring_law_holds"] = all(v == law for v in sent + recv)
        host_in = host_copy(pristine, w.dtype)
        host_out = host_copy(got, w.dtype)
        del pristine, got
        handles.clear()
        torch.cuda.empty_cache()
        secs, compared, bad = run_checker(ran, host_in, host_out, w, args.root, args.cpu_window, odt)
        del host_out
        workers = len(os.sched_getaffinity(0))
        secs_all = time_checker_all_cores(ran, host_in, w, args.root, args.cpu_window, odt, workers)
        del host_in
        windows = -(-t // args.cpu_window)
        result["parity"] = {"compared_elements": compared, "mismatches": bad,
                            "bit_exact": bad == 0}
        result["cpu_baseline"] = {
            "value": round(t * isz / secs / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"the whole workload: {ran} of N={n} ranks x T={t} "
                      f"{w.dtype} elements, run as {windows} windows of up to "
                      f"{args.cpu_window} elements per rank (literal NumPy simulation of "
                      f"the schedule, one thread), {secs:.2f} s",
            "seconds": round(secs, 3),
            "all_cores": {
                "value": round(t * isz / secs_all / 1e9, 4),
                "unit": "GB/s",
                "cores": workers,
                "seconds": round(secs_all, 3),
                "sample": f"the same {windows} windows spread over {workers} host threads "
                          f"(one per affinity core), wall time",
            },
            "cpu_model": cpu_model(),
            "os_cpu_count": os.cpu_count(),
            "affinity_cores": workers,
        }
    return result


# Warm-up calls per row: enough for about 20-30 ms of load before the timed
# calls, so that they run at the GPU's settled clocks (short calls after an
# idle pause measured up to 25 % slower for the first 10-20 calls).
SUITE = [
    # workload, collective, impl, extra flags
    ("large_grad_fp32", "ring_allreduce", "step", []),
    ("large_grad_fp32", "tree_allreduce", "fused", ["--warmup", "8"]),
    ("large_grad_bf16", "ring_allreduce", "fused", ["--warmup", "15"]),
    ("large_grad_bf16", "ring_allreduce", "step", ["--warmup", "8"]),
    ("large_grad_bf16", "ring_allreduce", "fused", ["--accumulate", "float32", "--warmup", "15"]),
    ("ddp_bucket", "ring_allreduce", "fused", ["--warmup", "300"]),
    ("ddp_bucket", "ring_allreduce", "fused", ["--flush-mall", "--warmup", "30"]),
    ("ddp_bucket", "ring_allreduce", "step", ["--flush-mall", "--warmup", "30"]),
    ("zero_n64", "reduce_scatter", "fused", ["--warmup", "40"]),
    ("zero_n64", "allgather", "fused", ["--warmup", "40"]),
    ("zero_n64", "broadcast", "fused", ["--warmup", "40"]),
    ("zero_n64", "reduce_scatter", "step", ["--warmup", "15"]),
    ("zero_n64", "allgather", "step", ["--warmup", "20"]),
    ("zero_n64", "broadcast", "step", ["--warmup", "20"]),
    ("zero_n64", "reduce", "fused", ["--warmup", "40"]),
    ("zero_n64", "scatter", "fused", ["--warmup", "600"]),
    ("zero_n64", "gather", "fused", ["--warmup", "600"]),
    ("zero_n64", "ring_allreduce", "fused", ["--warmup", "20"]),
    ("zero_n64", "tree_allreduce", "fused", ["--warmup", "20"]),
    # the same with the Infinity Cache flushed before each call: a copy's
    # source (one rank's worth, 67 MB here) otherwise stays in that cache
    # from one back-to-back call to the next
    ("zero_n64", "reduce_scatter", "fused", ["--flush-mall", "--warmup", "40"]),
    ("zero_n64", "allgather", "fused", ["--flush-mall", "--warmup", "40"]),
    ("zero_n64", "broadcast", "fused", ["--flush-mall", "--warmup", "40"]),
    ("zero_n64", "ring_allreduce", "fused", ["--flush-mall", "--warmup", "20"]),
    ("zero_n64", "tree_allreduce", "fused", ["--flush-mall", "--warmup", "20"]),
    ("large_grad_fp32", "reduce", "fused", ["--warmup", "15"]),
    ("large_grad_fp32", "allgather", "fused", ["--warmup", "15"]),
    ("large_grad_fp32", "broadcast", "fused", ["--warmup", "15"]),
    ("moe_alltoall", "alltoall", "fused", ["--warmup", "80"]),
    ("moe_alltoall", "alltoall", "fused", ["--flush-mall", "--warmup", "80"]),
    ("small_int32", "ring_allreduce", "fused", ["--steps", "30", "--warmup", "30"]),
    ("small_int32", "reduce_scatter", "fused", ["--steps", "30", "--warmup", "30"]),
    ("small_int32", "allgather", "fused", ["--steps", "30", "--warmup", "30"]),
    ("small_int32", "ring_allreduce", "step", ["--steps", "30", "--warmup", "30"]),
] + [
    # message-size sweep: every size event-timed with the Infinity Cache flushed,
    # so that the events hold GPU time only (the cost model is fitted to these)
    (f"sweep_{t}", coll, impl, ["--steps", "30", "--flush-mall", "--warmup", "30"])
    for t in (256, 262_144, 4_194_304, 67_108_864)
    for coll in ("ring_allreduce", "tree_allreduce", "allreduce")
    for impl in ("fused", "step")
]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the N logical ranks are N buffers in one GPU's HBM; no figure "
              f"across several GPUs is produced.", file=sys.stderr)
        sys.exit(2)
    if args.steps > MAX_CALLS:
        print(f"--steps must stay <= {MAX_CALLS} (values grow by up to N per call)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tree_allreduce_algorithms_amd as ar
    from tree_allreduce_algorithms_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ar.lib()
    torch.cuda.set_device(0)

    failed = False
    if args.suite:
        base = ["--warmup", "3"]
        for wname, coll, impl, extra in SUITE:
            sub = parse(base + ["--workload", wname, "--collective", coll, "--impl", impl] + extra)
            res = run_one(sub)
            failed |= not res.get("parity", {}).get("bit_exact", True)
            failed |= not res.get("counters", {}).get("match", True)
            with open(args.suite, "a") as f:
                f.write(json.dumps(res) + "\n")
            print(f"[suite] {wname} {coll} {impl} {' '.join(extra)}: "
                  f"{res['roofline']['event_ms_mean']} ms/call, "
                  f"{res['roofline']['achieved']} GB/s, parity "
                  f"{res.get('parity', {}).get('bit_exact')}", file=sys.stderr, flush=True)

    result = run_one(args)
    failed |= not result.get("parity", {}).get("bit_exact", True)
    line = json.dumps(result)
    print(line, flush=True)
    for path in filter(None, (args.jsonl, args.suite)):
        with open(path, "a") as f:
            f.write(line + "\n")
    failed |= not result.get("counters", {}).get("match", True)
    failed |= not result.get("counters", {}).get("ring_law_holds", True)
    if failed:
        print("[bench] the device output differs from the CPU checker, or the byte counters "
              "differ from their closed forms", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
