"""ctypes binding of libar.so: the same calls as include/ar.h, plus torch glue.

Argument marshalling only -- every collective runs in the library's HIP
kernels.  The library is loaded on first use from this package's directory;
if it is missing the call raises instead of falling back to anything else.
"""

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libar.so")

MAX_RANKS = 64

SUCCESS, INVALID_ARGUMENT, UNSUPPORTED, HIP_ERROR = 0, 1, 2, 3
DTYPES = {"int32": 0, "float32": 1, "bfloat16": 2, "bfloat16_acc32": 3}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
COLLECTIVES = {"ring_allreduce": 0, "reduce_scatter": 1, "allgather": 2, "broadcast": 3,
               "tree_allreduce": 4, "reduce": 5, "scatter": 6, "gather": 7, "alltoall": 8}
IMPLS = {"fused": 0, "step": 1}

# name -> (restype, argtypes), in the order include/ar.h declares them
_VP, _I, _SZ, _U64P = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint64)
_PP = ctypes.POINTER(ctypes.c_void_p)
SIGNATURES = {
    "ar_ring_allreduce": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_reduce_scatter": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_allgather": (_I, [_PP, _I, _SZ, _I, _VP]),
    "ar_broadcast": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_tree_allreduce": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_reduce": (_I, [_PP, _I, _SZ, _I, _I, _I, _VP]),
    "ar_scatter": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_gather": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_alltoall": (_I, [_PP, _I, _SZ, _I, _VP]),
    "ar_allreduce": (_I, [_PP, _I, _SZ, _I, _I, _VP]),
    "ar_allreduce_choice": (_I, [_I, _SZ, _I, ctypes.POINTER(_I)]),
    "ar_launch_plan": (_I, [_I, _I, _I, _SZ, _I, ctypes.POINTER(_I), _U64P]),
    "ar_predict_time": (_I, [_I, _I, _I, _SZ, _I, ctypes.POINTER(ctypes.c_double)]),
    "ar_set_cost_model": (_I, [_I, _I, ctypes.c_double, ctypes.c_double]),
    "ar_get_cost_model": (_I, [_I, _I, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]),
    "ar_chunk_size": (_SZ, [_I, _SZ]),
    "ar_chunk_range": (_I, [_I, _SZ, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "ar_expected_bytes": (_I, [_I, _I, _SZ, _I, _I, _U64P, _U64P]),
    "ar_expected_steps": (_I, [_I, _I]),
    "ar_counters_read": (_I, [_I, _U64P, _U64P]),
    "ar_counters_steps": (ctypes.c_uint64, []),
    "ar_counters_reset": (None, []),
    "ar_set_impl": (_I, [_I]),
    "ar_get_impl": (_I, []),
    "ar_status_string": (ctypes.c_char_p, [_I]),
    "ar_last_hip_error": (_I, []),
    "ar_version": (_I, []),
    "ar_debug_fail_launch": (_I, [_I]),
}

_lib = None
_lock = threading.Lock()


class ArError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = ""
        if status == HIP_ERROR:
            detail = f" (hipError_t {lib().ar_last_hip_error()})"
        msg = lib().ar_status_string(status).decode()
        super().__init__(f"{where}: {msg}{detail}")


def lib():
    """The loaded libar.so (loads it on first call; raises if it is not built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built; run "
                        "`python -m tree_allreduce_algorithms_amd.build_lib` first")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(status, where):
    if status != SUCCESS:
        raise ArError(status, where)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])
    return ctypes.cast(arr, _PP), arr


# --- raw pointer calls (device addresses as ints) ----------------------------

def raw_call(name, ptrs, count, dtype, op=None, root=None, stream=0):
    """Call one collective on device pointers; returns the status code."""
    pp, keep = _ptr_array(ptrs)
    n = len(ptrs)
    fn = getattr(lib(), "ar_" + name)
    dt = DTYPES[dtype]
    if name in ("ring_allreduce", "reduce_scatter", "tree_allreduce", "allreduce"):
        status = fn(pp, n, count, dt, OPS[op], stream)
    elif name in ("allgather", "alltoall"):
        status = fn(pp, n, count, dt, stream)
    elif name in ("broadcast", "scatter", "gather"):
        status = fn(pp, n, count, dt, root, stream)
    elif name == "reduce":
        status = fn(pp, n, count, dt, OPS[op], root, stream)
    else:
        raise ValueError(name)
    del keep
    return status


# --- torch glue ---------------------------------------------------------------

def _torch_dtype_name(t):
    import torch
    names = {torch.int32: "int32", torch.float32: "float32", torch.bfloat16: "bfloat16"}
    if t.dtype not in names:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return names[t.dtype]


def _prep(tensors):
    import torch
    tensors = list(tensors)
    if not tensors:
        raise ValueError("need at least one rank tensor")
    if len(tensors) > MAX_RANKS:
        raise ValueError(f"at most {MAX_RANKS} ranks")
    t0 = tensors[0]
    if not isinstance(t0, torch.Tensor) or not t0.is_cuda:
        raise TypeError("rank buffers must be GPU tensors")
    dev, dt, numel = t0.get_device(), t0.dtype, t0.numel()
    for t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("rank buffers must be GPU tensors")
        if t.get_device() != dev or t.dtype != dt or t.numel() != numel:
            raise ValueError("rank buffers must share device, dtype and size")
        if not t.is_contiguous():
            raise ValueError("rank buffers must be contiguous")
    return tensors, _torch_dtype_name(t0), numel


def _stream_handle(tensors, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(tensors[0].device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


class _on_device:
    """Makes `dev` the current device for a launch when it is not already.

    The library launches on the stream it is given; the null stream (handle
    0, torch's default stream) is the current device's, so the tensors'
    device must be current.  The check costs well under a microsecond when
    nothing needs to change."""

    __slots__ = ("dev", "prev")

    def __init__(self, dev):
        self.dev, self.prev = dev, None

    def __enter__(self):
        import torch
        cur = torch.cuda.current_device()
        if cur != self.dev:
            self.prev = cur
            torch.cuda.set_device(self.dev)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            import torch
            torch.cuda.set_device(self.prev)
        return False


def _collective(name, tensors, op=None, root=None, stream=None, accumulate=None):
    tensors, dtype, count = _prep(tensors)
    if accumulate not in (None, dtype):
        if accumulate != "float32" or dtype != "bfloat16":
            raise ValueError(f"accumulate={accumulate!r} is only offered as 'float32' for "
                             f"bfloat16 buffers (got {dtype})")
        dtype = "bfloat16_acc32"
    with _on_device(tensors[0].get_device()):
        status = raw_call(name, [t.data_ptr() for t in tensors], count, dtype, op=op,
                          root=root, stream=_stream_handle(tensors, stream))
    _check(status, name)
    return tensors


# accumulate="float32" (bfloat16 buffers only): the reduction carries float32
# partials from hop to hop in the schedule's order and rounds to bfloat16 once
# (AR_BFLOAT16_ACC32); by default every hop rounds to the buffers' dtype.

def ring_allreduce(tensors, op="sum", stream=None, accumulate=None):
    """Ring AllReduce in place over the rank tensors (see ar_ring_allreduce)."""
    return _collective("ring_allreduce", tensors, op=op, stream=stream, accumulate=accumulate)


def reduce_scatter(tensors, op="sum", stream=None, accumulate=None):
    """Ring ReduceScatter in place: chunk r of tensors[r] ends fully reduced."""
    return _collective("reduce_scatter", tensors, op=op, stream=stream, accumulate=accumulate)


def allgather(tensors, stream=None):
    """Ring AllGather in place: chunk r of tensors[r] is copied to every rank."""
    return _collective("allgather", tensors, stream=stream)


def broadcast(tensors, root=0, stream=None):
    """Broadcast tensors[root] into every rank tensor."""
    return _collective("broadcast", tensors, root=root, stream=stream)


def tree_allreduce(tensors, op="sum", stream=None, accumulate=None):
    """Double-binary-tree AllReduce in place (see ar_tree_allreduce)."""
    return _collective("tree_allreduce", tensors, op=op, stream=stream, accumulate=accumulate)


def reduce(tensors, op="sum", root=0, stream=None, accumulate=None):
    """Reduce in place into tensors[root]; the other tensors keep their data."""
    return _collective("reduce", tensors, op=op, root=root, stream=stream, accumulate=accumulate)


def scatter(tensors, root=0, stream=None):
    """Scatter: chunk c of tensors[root] is copied into chunk c of tensors[c]."""
    return _collective("scatter", tensors, root=root, stream=stream)


def gather(tensors, root=0, stream=None):
    """Gather: chunk c of tensors[c] is copied into chunk c of tensors[root]."""
    return _collective("gather", tensors, root=root, stream=stream)


def alltoall(tensors, stream=None):
    """AllToAll in place: block j of tensors[i] <-> block i of tensors[j]."""
    return _collective("alltoall", tensors, stream=stream)


def allreduce(tensors, op="sum", stream=None, accumulate=None):
    """AllReduce in place by the ring or the double tree, whichever the cost
    model predicts faster for this size (see ar_allreduce)."""
    return _collective("allreduce", tensors, op=op, stream=stream, accumulate=accumulate)


class RankBuffers:
    """A fixed set of N rank tensors, checked once.

    Every collective on it is then one call into the library with the
    pointer array, dtype and stream prepared here, which keeps the host cost
    of a call to a few microseconds for the small messages where it matters.
    The object holds references to the tensors; their storage must not be
    reallocated while it is in use.  ``stream`` (a torch stream or a raw
    hipStream_t handle) defaults to the current stream at construction; each
    call may pass another.  Calls run with the tensors' device current.
    ``accumulate='float32'`` (bfloat16 tensors only) selects float32 partials
    for the reductions.
    """

    def __init__(self, tensors, stream=None, accumulate=None):
        self.tensors, dtype, self.count = _prep(tensors)
        self.n = len(self.tensors)
        if accumulate not in (None, dtype):
            if accumulate != "float32" or dtype != "bfloat16":
                raise ValueError(f"accumulate={accumulate!r} is only offered as 'float32' for "
                                 f"bfloat16 buffers (got {dtype})")
        self.dtype = dtype
        self._copy_dt = DTYPES[dtype]
        self._red_dt = DTYPES["bfloat16_acc32" if accumulate == "float32" else dtype]
        self._pp, self._keep = _ptr_array([t.data_ptr() for t in self.tensors])
        self._stream = _stream_handle(self.tensors, stream)
        import torch
        self._dev = self.tensors[0].get_device()
        self._current_device = torch.cuda.current_device
        lib_ = lib()
        self._fn = {name: getattr(lib_, "ar_" + name) for name in COLLECTIVES}
        self._fn["allreduce"] = lib_.ar_allreduce

    def _s(self, stream):
        if stream is None:
            return self._stream
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)

    def _call(self, name, *args):
        fn = self._fn[name]
        if self._current_device() == self._dev:
            status = fn(self._pp, self.n, self.count, *args)
        else:
            with _on_device(self._dev):
                status = fn(self._pp, self.n, self.count, *args)
        if status != SUCCESS:
            raise ArError(status, name)
        return self.tensors

    def ring_allreduce(self, op="sum", stream=None):
        return self._call("ring_allreduce", self._red_dt, OPS[op], self._s(stream))

    def reduce_scatter(self, op="sum", stream=None):
        return self._call("reduce_scatter", self._red_dt, OPS[op], self._s(stream))

    def allgather(self, stream=None):
        return self._call("allgather", self._copy_dt, self._s(stream))

    def broadcast(self, root=0, stream=None):
        return self._call("broadcast", self._copy_dt, root, self._s(stream))

    def tree_allreduce(self, op="sum", stream=None):
        return self._call("tree_allreduce", self._red_dt, OPS[op], self._s(stream))

    def allreduce(self, op="sum", stream=None):
        return self._call("allreduce", self._red_dt, OPS[op], self._s(stream))

    def reduce(self, op="sum", root=0, stream=None):
        return self._call("reduce", self._red_dt, OPS[op], root, self._s(stream))

    def scatter(self, root=0, stream=None):
        return self._call("scatter", self._copy_dt, root, self._s(stream))

    def gather(self, root=0, stream=None):
        return self._call("gather", self._copy_dt, root, self._s(stream))

    def alltoall(self, stream=None):
        return self._call("alltoall", self._copy_dt, self._s(stream))


# --- host-only helpers --------------------------------------------------------

def allreduce_choice(nranks, count, dtype):
    """'ring_allreduce' or 'tree_allreduce': what allreduce() would run."""
    out = ctypes.c_int()
    _check(lib().ar_allreduce_choice(nranks, count, DTYPES[dtype], ctypes.byref(out)),
           "allreduce_choice")
    return {v: k for k, v in COLLECTIVES.items()}[out.value]


def launch_plan(collective, impl, nranks, count, dtype):
    """(kernel launches, HBM bytes) of one call as the library runs it."""
    n, b = ctypes.c_int(), ctypes.c_uint64()
    _check(lib().ar_launch_plan(COLLECTIVES[collective], IMPLS[impl], nranks, count,
                                DTYPES[dtype], ctypes.byref(n), ctypes.byref(b)), "launch_plan")
    return n.value, b.value


def predict_time(collective, impl, nranks, count, dtype):
    """Cost-model prediction of one call, in microseconds."""
    us = ctypes.c_double()
    _check(lib().ar_predict_time(COLLECTIVES[collective], IMPLS[impl], nranks, count,
                                 DTYPES[dtype], ctypes.byref(us)), "predict_time")
    return us.value


def get_cost_model(collective, impl):
    """(alpha_us per launch, GB/s of HBM traffic) for this collective and impl."""
    a, g = ctypes.c_double(), ctypes.c_double()
    _check(lib().ar_get_cost_model(COLLECTIVES[collective], IMPLS[impl], ctypes.byref(a),
                                   ctypes.byref(g)), "get_cost_model")
    return a.value, g.value


def set_cost_model(collective, impl, alpha_us, gbps):
    _check(lib().ar_set_cost_model(COLLECTIVES[collective], IMPLS[impl], float(alpha_us),
                                   float(gbps)), "set_cost_model")


def chunk_size(nranks, count):
    return lib().ar_chunk_size(nranks, count)


def chunk_range(nranks, count, chunk):
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().ar_chunk_range(nranks, count, chunk, ctypes.byref(lo), ctypes.byref(hi)),
           "chunk_range")
    return lo.value, hi.value


def expected_bytes(collective, nranks, count, dtype, root=0):
    sent = (ctypes.c_uint64 * max(1, nranks))()
    recv = (ctypes.c_uint64 * max(1, nranks))()
    _check(lib().ar_expected_bytes(COLLECTIVES[collective], nranks, count, DTYPES[dtype], root,
                                   sent, recv), "expected_bytes")
    return list(sent)[:nranks], list(recv)[:nranks]


def expected_steps(collective, nranks):
    return lib().ar_expected_steps(COLLECTIVES[collective], nranks)


def counters(nranks):
    sent = (ctypes.c_uint64 * max(1, nranks))()
    recv = (ctypes.c_uint64 * max(1, nranks))()
    _check(lib().ar_counters_read(nranks, sent, recv), "counters")
    return list(sent)[:nranks], list(recv)[:nranks], lib().ar_counters_steps()


def reset_counters():
    lib().ar_counters_reset()


def set_impl(impl):
    _check(lib().ar_set_impl(IMPLS[impl]), "set_impl")


def debug_fail_launch(k):
    """Make the k-th kernel launch from now (k >= 1) fail with
    hipErrorLaunchFailure instead of being enqueued; 0 disarms.  For tests
    of the AR_ERROR_HIP path (the call raises ArError)."""
    _check(lib().ar_debug_fail_launch(int(k)), "debug_fail_launch")


def get_impl():
    return {v: k for k, v in IMPLS.items()}[lib().ar_get_impl()]
