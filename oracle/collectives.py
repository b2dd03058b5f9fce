"""Literal step-by-step simulation of ring ReduceScatter / AllGather /
AllReduce, the binomial double-tree AllReduce and Broadcast.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions shared by every function here:

* ``x`` is a list of N one-dimensional NumPy arrays of equal length T, one per
  logical rank, stored as ``oracle.STORAGE[dtype]`` (bfloat16 as uint16 bits).
  Inputs are never modified; each function works on copies and returns a
  ``Result`` holding the final rank arrays, the bytes each rank sent and
  received, and the number of schedule steps.
* Chunk layout (the pages split the tensor into N equal chunks -- Lecture 09,
  section 4.2; Chapter 4, section 4.3.1; Collectives from scratch, two-pass
  ring -- and Lecture 09's lab 1 demands that N divide T).  Where N does not
  divide T this oracle takes C = ceil(T/N) and chunk c = [c*C, min(T,(c+1)*C)),
  so only trailing chunks are short and a chunk may be empty when T < N.
* A step is a map from the state before it to the state after it: what every
  rank receives in a step is read from the state before that step, and only
  then do the receivers update their buffers (in a real ring all ranks send
  and receive at once).
* Byte counters count logical inter-rank bytes: every transfer of k elements
  adds k*itemsize to the sender's ``sent`` and the receiver's ``recv``.
* Windowed runs: every element's result depends only on the N values at its
  index and on the chunk (or tree segment) that index belongs to.  Passing
  ``window_start`` and ``total`` runs the same literal schedule on arrays that
  hold only the elements [window_start, window_start + len) of a T = ``total``
  element problem; chunk and segment bounds come from the global layout and
  the counters count only the bytes inside the window.
"""

from dataclasses import dataclass

import numpy as np

from .numerics import ITEMSIZE, STORAGE, bf16_to_f32, combine, f32_to_bf16_rne

ACC32 = "bfloat16_acc32"


@dataclass
class Result:
    bufs: list
    sent: np.ndarray
    recv: np.ndarray
    steps: int


def ceil_log2(n):
    """Smallest L with 2**L >= n (0 for n <= 1): the depth of a binomial tree."""
    return (int(n) - 1).bit_length() if n > 1 else 0


def chunk_layout(nranks, total):
    """Global [lo, hi) bounds of the N ring chunks of a T-element buffer."""
    if nranks < 1:
        raise ValueError("nranks must be >= 1")
    size = -(-total // nranks)
    return [(min(c * size, total), min((c + 1) * size, total)) for c in range(nranks)]


# --- schedule primitives -----------------------------------------------------
# Each is a one-liner kept as its own function so that the tests can plant a
# mistake in exactly one of them and check that the pins notice.

def ring_next(r, n):
    """Ring edge: every rank sends only to its right neighbour (Lecture 09,
    section 4.2; Collectives from scratch, two-pass ring)."""
    return (r + 1) % n


def rs_send_chunk(r, t, n):
    """ReduceScatter step t = 0..N-2: rank r forwards chunk (r - t - 1) mod N.

    Collectives from scratch (two-pass ring) has rank r send chunk (r - s) mod N
    at step s and end owning the complete chunk r.  That ownership holds when
    s counts from 1, i.e. s = t + 1.  Lecture 09 lab 1 and Chapter 4's
    pseudo-code use the 0-based (r - t), which is the same ring with every rank
    label shifted by one (checked in the tests).
    """
    return (r - t - 1) % n


def ag_send_chunk(r, t, n):
    """AllGather step t = 0..N-2: rank r forwards chunk (r - t) mod N, its own
    completed chunk at t = 0, then what it received in the previous step."""
    return (r - t) % n


def rooted_rank(role, root, n):
    """Rank playing ``role`` in a tree rooted at ``root``: roles are ranks
    counted from the root, (rank - root) mod N (Broadcast, Reduce)."""
    return (role + root) % n


def tree_rank(tree, role, n):
    """Rank playing ``role`` in tree 0 (identity) or tree 1 (mirror N-1-role).

    Lecture 09 section 5.2 and Chapter 4 section 4.3.2 describe two trees that
    each reduce and broadcast half of the data; the pages give no shape.  The
    reading here is two binomial trees, the second on mirrored roles, so that
    for even N every rank is a leaf in at least one of them.
    """
    return role if tree == 0 else n - 1 - role


# --- helpers -----------------------------------------------------------------

def _setup(x, dtype, window_start, total):
    if dtype not in STORAGE:
        raise ValueError(f"unknown dtype {dtype!r}")
    n = len(x)
    if n < 1:
        raise ValueError("need at least one rank")
    length = len(x[0])
    if any(len(a) != length for a in x):
        raise ValueError("all rank buffers must have the same length")
    if total is None:
        total = length
    if window_start < 0 or window_start + length > total:
        raise ValueError("window does not fit in the global buffer")
    bufs = [np.array(a, dtype=STORAGE[dtype], copy=True) for a in x]
    sent = np.zeros(n, dtype=np.uint64)
    recv = np.zeros(n, dtype=np.uint64)
    return n, length, total, bufs, sent, recv


def _local(lo, hi, window_start, length):
    """Slice of the window arrays that holds global elements [lo, hi)."""
    a = min(max(lo - window_start, 0), length)
    b = min(max(hi - window_start, 0), length)
    return slice(a, max(a, b))


def _count(sent, recv, src, dst, nelem, dtype):
    nbytes = np.uint64(nelem * ITEMSIZE[dtype])
    sent[src] += nbytes
    recv[dst] += nbytes


def _float32_partials(x, run):
    """bfloat16 buffers whose reductions carry float32 partials: every rank is
    widened to float32 (exact), the float32 schedule runs unchanged (same
    steps, same order, each hop one float32 operation), and every buffer is
    rounded back to bfloat16 once, to nearest even.  A buffer the schedule
    does not write comes back with its bits (a widened bfloat16 rounds to
    itself; a signalling NaN would come back quiet).  Counters count the
    stored 2-byte elements."""
    res = run([bf16_to_f32(a) for a in x])
    bufs = [f32_to_bf16_rne(b) for b in res.bufs]
    return Result(bufs, res.sent // np.uint64(2), res.recv // np.uint64(2), res.steps)


# --- ring --------------------------------------------------------------------

def _ring_pass(bufs, sent, recv, span, dtype, steps, chunk_sent, merge):
    """Run ``steps`` ring steps.  One step maps the state before it to the
    state after it: rank d's inbox is filled from the pre-step state, with the
    chunk ``chunk_sent(r, t, n)`` of every rank r whose ring successor is d
    (exactly one on a ring), and only then does every rank merge its inbox
    into its own buffer at that chunk: ``merge(own, incoming)``."""
    n = len(bufs)
    senders = [[r for r in range(n) if ring_next(r, n) == d] for d in range(n)]
    for t in range(steps):
        inbox = [[(r, chunk_sent(r, t, n)) for r in senders[d]] for d in range(n)]
        inbox = [[(r, c, bufs[r][span[c]].copy()) for r, c in box] for box in inbox]
        for d, box in enumerate(inbox):
            for r, c, incoming in box:
                bufs[d][span[c]] = merge(bufs[d][span[c]], incoming)
                _count(sent, recv, r, d, incoming.size, dtype)
    return steps


def _ring_reduce_scatter_steps(bufs, sent, recv, span, op, dtype):
    """N-1 steps; the receiver stores own (+) incoming (Lecture 09 section
    4.3; Chapter 4 section 4.3.1)."""
    steps = len(bufs) - 1 if len(bufs) > 1 else 0
    return _ring_pass(bufs, sent, recv, span, dtype, steps, rs_send_chunk,
                      lambda own, incoming: combine(own, incoming, op, dtype))


def _ring_allgather_steps(bufs, sent, recv, span, dtype):
    """N-1 steps; the receiver overwrites its copy of the chunk (Lecture 09
    section 4.3)."""
    steps = len(bufs) - 1 if len(bufs) > 1 else 0
    return _ring_pass(bufs, sent, recv, span, dtype, steps, ag_send_chunk,
                      lambda own, incoming: incoming)


def _ring_spans(n, total, window_start, length):
    return [_local(lo, hi, window_start, length) for lo, hi in chunk_layout(n, total)]


def ring_reduce_scatter(x, op, dtype, window_start=0, total=None):
    """Ring ReduceScatter: N-1 steps; afterwards rank r's chunk r holds the
    reduction of chunk r over all ranks, folded in ring order (starting at rank
    r+1, ending at rank r).  Other chunks hold partial results."""
    if dtype == ACC32:
        return _float32_partials(
            x, lambda w: ring_reduce_scatter(w, op, "float32", window_start, total))
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    steps = _ring_reduce_scatter_steps(
        bufs, sent, recv, _ring_spans(n, total, window_start, length), op, dtype)
    return Result(bufs, sent, recv, steps)


def ring_allgather(x, dtype, window_start=0, total=None):
    """Ring AllGather: rank r contributes chunk r of its buffer; after N-1
    overwrite steps every rank holds every rank's chunk in place."""
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    steps = _ring_allgather_steps(
        bufs, sent, recv, _ring_spans(n, total, window_start, length), dtype)
    return Result(bufs, sent, recv, steps)


def ring_allreduce(x, op, dtype, window_start=0, total=None):
    """Ring AllReduce = ReduceScatter then AllGather on the same buffers
    (Lecture 09 sections 3.9 and 4.3; Collectives from scratch, two-pass ring):
    2(N-1) steps, every rank ends with the same reduction."""
    if dtype == ACC32:
        return _float32_partials(
            x, lambda w: ring_allreduce(w, op, "float32", window_start, total))
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    span = _ring_spans(n, total, window_start, length)
    steps = _ring_reduce_scatter_steps(bufs, sent, recv, span, op, dtype)
    steps += _ring_allgather_steps(bufs, sent, recv, span, dtype)
    return Result(bufs, sent, recv, steps)


# --- trees -------------------------------------------------------------------

def _tree_segments(trees, total):
    if trees == 1:
        return [(0, 0, total)]
    if trees == 2:
        half = -(-total // 2)
        return [(0, 0, half), (1, half, total)]
    raise ValueError("trees must be 1 or 2")


def tree_allreduce(x, op, dtype, trees=2, window_start=0, total=None):
    """Binomial-tree AllReduce: ceil(log2 N) reduce rounds toward role 0, then
    the same number of broadcast rounds back down (Lecture 09 section 5.2;
    Chapter 4 section 4.3.2; Collectives from scratch, cost table: 2 log2 N
    steps).

    Reduce round k (k = 0, 1, ...): every role q with q mod 2^(k+1) == 0 and
    q + 2^k < N receives the segment of role q + 2^k and stores
    ``own (+) received``.  Broadcast round k (k = L-1 .. 0): role q + 2^k
    receives role q's segment and overwrites.

    ``trees=2`` (the double tree): tree 0 handles elements [0, ceil(T/2)) with
    role == rank, tree 1 handles the rest with role == N-1-rank; both run their
    rounds in the same steps.  ``trees=1``: one tree over all T elements.
    """
    if dtype == ACC32:
        return _float32_partials(
            x, lambda w: tree_allreduce(w, op, "float32", trees, window_start, total))
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    segs = [(tree, _local(lo, hi, window_start, length))
            for tree, lo, hi in _tree_segments(trees, total)]
    depth = ceil_log2(n)
    for k in range(depth):
        stride = 1 << k
        packets = []
        for tree, seg in segs:
            for q in range(0, n, 2 * stride):
                if q + stride < n:
                    src = tree_rank(tree, q + stride, n)
                    dst = tree_rank(tree, q, n)
                    packets.append((src, dst, seg, bufs[src][seg].copy()))
        for src, dst, seg, payload in packets:
            bufs[dst][seg] = combine(bufs[dst][seg], payload, op, dtype)
            _count(sent, recv, src, dst, payload.size, dtype)
    for k in reversed(range(depth)):
        stride = 1 << k
        packets = []
        for tree, seg in segs:
            for q in range(0, n, 2 * stride):
                if q + stride < n:
                    src = tree_rank(tree, q, n)
                    dst = tree_rank(tree, q + stride, n)
                    packets.append((src, dst, seg, bufs[src][seg].copy()))
        for src, dst, seg, payload in packets:
            bufs[dst][seg] = payload
            _count(sent, recv, src, dst, payload.size, dtype)
    return Result(bufs, sent, recv, 2 * depth)


def broadcast(x, root, dtype, window_start=0, total=None):
    """Broadcast of the root's buffer along a binomial tree on roles
    (r - root) mod N: ceil(log2 N) overwrite rounds (Lecture 09 section 3.1;
    Collectives from scratch, cost table: T bytes, log2 N tree)."""
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    if not 0 <= root < n:
        raise ValueError("root out of range")
    depth = ceil_log2(n)
    whole = slice(0, length)
    for k in reversed(range(depth)):
        stride = 1 << k
        packets = []
        for q in range(0, n, 2 * stride):
            if q + stride < n:
                src = rooted_rank(q, root, n)
                dst = rooted_rank(q + stride, root, n)
                packets.append((src, dst, bufs[src][whole].copy()))
        for src, dst, payload in packets:
            bufs[dst][whole] = payload
            _count(sent, recv, src, dst, payload.size, dtype)
    return Result(bufs, sent, recv, depth)


# --- rooted primitives: Reduce, Scatter, Gather --------------------------------

def reduce(x, root, op, dtype, window_start=0, total=None):
    """Reduce to ``root`` (Lecture 09, section 3.4): the root ends with the
    reduction of every rank's buffer and every other rank keeps its data.

    Order: the reduce rounds of a binomial tree on roles (rank - root) mod N,
    the same rounds the tree AllReduce runs (Lecture 09 section 5.2; cost
    table of "Collectives from scratch": log2 N tree steps).  Every rank works
    on a copy of its buffer (the receive buffer of a real rank); round k
    (k = 0, 1, ...): role q with q mod 2^(k+1) == 0 and q + 2^k < N receives
    the working copy of role q + 2^k and stores own (+) received.  At the end
    the root's buffer takes the root's working copy; the other buffers are
    unchanged, as section 3.4 requires.
    """
    if dtype == ACC32:
        return _float32_partials(
            x, lambda w: reduce(w, root, op, "float32", window_start, total))
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    if not 0 <= root < n:
        raise ValueError("root out of range")
    work = [b.copy() for b in bufs]
    depth = ceil_log2(n)
    for k in range(depth):
        stride = 1 << k
        packets = []
        for q in range(0, n, 2 * stride):
            if q + stride < n:
                src = rooted_rank(q + stride, root, n)
                dst = rooted_rank(q, root, n)
                packets.append((src, dst, work[src].copy()))
        for src, dst, payload in packets:
            work[dst] = combine(work[dst], payload, op, dtype)
            _count(sent, recv, src, dst, payload.size, dtype)
    bufs[root] = work[root]
    return Result(bufs, sent, recv, depth)


def scatter(x, root, dtype, window_start=0, total=None):
    """Scatter from ``root`` (Lecture 09, section 3.2): the root's buffer is
    cut into the N ring chunks and chunk c goes to rank c, in place of rank
    c's chunk c.  One step of N-1 direct transfers; every other element of
    every buffer (the root's whole buffer included) is unchanged."""
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    if not 0 <= root < n:
        raise ValueError("root out of range")
    span = _ring_spans(n, total, window_start, length)
    packets = [(c, bufs[root][span[c]].copy()) for c in range(n) if c != root]
    for c, payload in packets:
        bufs[c][span[c]] = payload
        _count(sent, recv, root, c, payload.size, dtype)
    return Result(bufs, sent, recv, 1 if n > 1 else 0)


def gather(x, root, dtype, window_start=0, total=None):
    """Gather to ``root`` (Lecture 09, section 3.3): rank c's chunk c lands in
    chunk c of the root's buffer, so the root holds every rank's shard in
    rank order.  One step of N-1 direct transfers; the other ranks keep
    their data."""
    n, length, total, bufs, sent, recv = _setup(x, dtype, window_start, total)
    if not 0 <= root < n:
        raise ValueError("root out of range")
    span = _ring_spans(n, total, window_start, length)
    packets = [(c, bufs[c][span[c]].copy()) for c in range(n) if c != root]
    for c, payload in packets:
        bufs[root][span[c]] = payload
        _count(sent, recv, c, root, payload.size, dtype)
    return Result(bufs, sent, recv, 1 if n > 1 else 0)


# --- AllToAll ---------------------------------------------------------------------

def alltoall_slot(src, dst):
    """Block of rank ``dst`` that receives rank ``src``'s block ``dst``: block
    ``src`` (the cross-rank transpose, recv[dst][src] = send[src][dst], of
    Lecture 09 section 3.8 and lab 4 in section 7.4)."""
    return src


def alltoall(x, dtype):
    """AllToAll (Lecture 09, section 3.8; lab 4, section 7.4): every rank's
    buffer is N equal blocks of T/N elements; block j of rank i is meant for
    rank j, which receives it in block i.  One step: every rank first copies
    out the N-1 blocks it sends (the snapshot), then every block is
    delivered; a rank's own block (j == i) stays in place.  N must divide T.
    Whole buffers only: an output element comes from another position of
    another rank, so the windowed mode of the other functions does not apply.
    """
    n, length, total, bufs, sent, recv = _setup(x, dtype, 0, None)
    if length % n:
        raise ValueError("AllToAll needs N to divide T")
    size = length // n
    block = lambda b: slice(b * size, (b + 1) * size)
    packets = [(i, j, bufs[i][block(j)].copy()) for i in range(n) for j in range(n) if i != j]
    for i, j, payload in packets:
        bufs[j][block(alltoall_slot(i, j))] = payload
        _count(sent, recv, i, j, payload.size, dtype)
    return Result(bufs, sent, recv, 1 if n > 1 else 0)
