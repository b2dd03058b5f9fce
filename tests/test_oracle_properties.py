"""Property-based pins of the oracle (hypothesis; CPU only).

Random small problems (N up to 9 ranks, T up to 40 elements, ragged and
empty chunks included, every op and root) against facts that do not depend
on the oracle's own code:

* int32 results equal a brute-force elementwise reduction over the ranks
  (two's-complement wrap for SUM and PROD; MAX and MIN exactly), for the
  ring, both tree shapes and the rooted Reduce.
* For every dtype: an AllReduce leaves every rank bit-identical; the owned
  chunk of a ReduceScatter equals the AllReduce there; AllGather after
  ReduceScatter equals AllReduce (the pages' decomposition); a Broadcast
  copies the root; Scatter and Gather move exactly the non-root chunks;
  AllToAll is the block transpose and its own inverse.
* The byte counters: what is sent equals what is received, and for the ring
  AllReduce every element crosses N-1 links in each pass.
* A windowed run equals the same elements of the full run.
"""

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None)
OPS = ("sum", "prod", "max", "min")
DTYPES = ("int32", "float32", "bfloat16")


def draw_inputs(draw, dtype, n, t):
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        # wide values: SUM and PROD wrap around
        return [rng.integers(-(1 << 31), 1 << 31, size=t, dtype=np.int64).astype(np.int32)
                for _ in range(n)]
    vals = [rng.standard_normal(t).astype(np.float32) for _ in range(n)]
    if dtype == "float32":
        return vals
    return [oracle.f32_to_bf16_rne(v) for v in vals]


def brute_int32(x, op):
    a = np.stack([v.astype(np.int64) for v in x])
    if op == "sum":
        r = a.sum(axis=0)
    elif op == "prod":
        r = np.ones(a.shape[1], dtype=object)
        for row in a:
            r = [(p * int(v)) % (1 << 32) for p, v in zip(r, row)]
        r = np.array(r, dtype=np.int64)
    elif op == "max":
        r = a.max(axis=0)
    else:
        r = a.min(axis=0)
    return (np.asarray(r, dtype=np.int64) % (1 << 32)).astype(np.uint32).view(np.int32)


@st.composite
def problems(draw, dtypes=DTYPES):
    n = draw(st.integers(1, 9))
    t = draw(st.integers(0, 40))
    dtype = draw(st.sampled_from(dtypes))
    op = draw(st.sampled_from(OPS))
    root = draw(st.integers(0, n - 1))
    return n, t, dtype, op, root, draw_inputs(draw, dtype, n, t)


@SETTINGS
@given(problems(dtypes=("int32",)), st.sampled_from(["ring", "tree1", "tree2", "reduce"]))
def test_int32_results_equal_brute_force(p, algo):
    n, t, dtype, op, root, x = p
    want = brute_int32(x, op) if t else np.zeros(0, np.int32)
    if algo == "ring":
        res = oracle.ring_allreduce(x, op, dtype)
    elif algo == "reduce":
        res = oracle.reduce(x, root, op, dtype)
        assert np.array_equal(res.bufs[root], want)
        for r in range(n):
            if r != root:
                assert np.array_equal(res.bufs[r], x[r])
        return
    else:
        res = oracle.tree_allreduce(x, op, dtype, trees=1 if algo == "tree1" else 2)
    for b in res.bufs:
        assert np.array_equal(b, want)


@SETTINGS
@given(problems())
def test_ring_decomposition_and_identical_ranks(p):
    n, t, dtype, op, root, x = p
    ar = oracle.ring_allreduce(x, op, dtype)
    for b in ar.bufs[1:]:
        assert np.array_equal(b.view(np.uint8), ar.bufs[0].view(np.uint8))
    rs = oracle.ring_reduce_scatter(x, op, dtype)
    for r, (lo, hi) in enumerate(oracle.chunk_layout(n, t)):
        assert np.array_equal(rs.bufs[r][lo:hi].view(np.uint8), ar.bufs[0][lo:hi].view(np.uint8))
    ag = oracle.ring_allgather(rs.bufs, dtype)
    for r in range(n):
        assert np.array_equal(ag.bufs[r].view(np.uint8), ar.bufs[r].view(np.uint8))


@SETTINGS
@given(problems(), st.sampled_from([1, 2]))
def test_tree_leaves_every_rank_identical(p, trees):
    n, t, dtype, op, root, x = p
    res = oracle.tree_allreduce(x, op, dtype, trees=trees)
    for b in res.bufs[1:]:
        assert np.array_equal(b.view(np.uint8), res.bufs[0].view(np.uint8))


@SETTINGS
@given(problems())
def test_copies_move_exactly_their_elements(p):
    n, t, dtype, op, root, x = p
    u8 = lambda a: a.view(np.uint8)  # noqa: E731
    bc = oracle.broadcast(x, root, dtype)
    for b in bc.bufs:
        assert np.array_equal(u8(b), u8(x[root]))
    owned = oracle.chunk_layout(n, t)
    sc = oracle.scatter(x, root, dtype)
    ga = oracle.gather(x, root, dtype)
    for r in range(n):
        lo, hi = owned[r]
        want_sc = x[r].copy()
        want_sc[lo:hi] = x[root][lo:hi]
        assert np.array_equal(u8(sc.bufs[r]), u8(want_sc))
        if r != root:
            assert np.array_equal(u8(ga.bufs[r]), u8(x[r]))
    want_ga = x[root].copy()
    for c, (lo, hi) in enumerate(owned):
        want_ga[lo:hi] = x[c][lo:hi]
    assert np.array_equal(u8(ga.bufs[root]), u8(want_ga))


@SETTINGS
@given(st.integers(1, 8), st.integers(0, 5), st.sampled_from(DTYPES), st.data())
def test_alltoall_is_the_block_transpose_and_an_involution(n, b, dtype, data):
    x = draw_inputs(data.draw, dtype, n, n * b)
    y = oracle.alltoall(x, dtype).bufs
    for d in range(n):
        for s in range(n):
            assert np.array_equal(y[d][s * b:(s + 1) * b].view(np.uint8),
                                  x[s][d * b:(d + 1) * b].view(np.uint8))
    z = oracle.alltoall(y, dtype).bufs
    for r in range(n):
        assert np.array_equal(z[r].view(np.uint8), x[r].view(np.uint8))


@SETTINGS
@given(problems())
def test_byte_counters_balance(p):
    n, t, dtype, op, root, x = p
    s = oracle.ITEMSIZE[dtype]
    ar = oracle.ring_allreduce(x, op, dtype)
    assert int(ar.sent.sum()) == int(ar.recv.sum()) == (2 * (n - 1) * t * s if n > 1 else 0)
    for res in (oracle.tree_allreduce(x, op, dtype), oracle.broadcast(x, root, dtype),
                oracle.reduce(x, root, op, dtype), oracle.scatter(x, root, dtype),
                oracle.gather(x, root, dtype)):
        assert int(res.sent.sum()) == int(res.recv.sum())


@SETTINGS
@given(problems(dtypes=("float32", "bfloat16")), st.data())
def test_windowed_run_equals_full_run(p, data):
    n, t, dtype, op, root, x = p
    if t == 0:
        return
    a = data.draw(st.integers(0, t - 1))
    b = data.draw(st.integers(a + 1, t))
    full = oracle.ring_allreduce(x, op, dtype).bufs
    win = oracle.ring_allreduce([v[a:b] for v in x], op, dtype, window_start=a, total=t).bufs
    for r in range(n):
        assert np.array_equal(win[r].view(np.uint8), full[r][a:b].view(np.uint8))
