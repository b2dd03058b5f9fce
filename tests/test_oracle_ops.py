"""Pins for the oracle's PROD, MAX and MIN operators on float32 and bfloat16.

Lecture 09, section 3.4 lists the reduction operators SUM, MAX, MIN and PROD.
SUM is pinned elsewhere (brute force for int32, closed forms of the fold
order, math.fsum bounds).  Here:

* MAX and MIN have one correct answer whatever the order, as long as no NaN
  and no +0/-0 tie is involved: the maximum (minimum) over the rank axis,
  which NumPy computes directly.  Every rank after ring and tree AllReduce,
  every owned chunk after ReduceScatter and the root after Reduce must equal
  it, for float32, for bfloat16 (widened by torch) and for bfloat16 buffers
  with float32 partials.
* PROD depends on the order in floating point, so it is pinned by the fold
  order written per element: the ring's (chunk c starts at rank c+1 and ends
  at rank c) and the binomial tree's pairing, each hop one float32 multiply,
  rounded to bfloat16 by torch after every hop (per-hop bfloat16) or once at
  the end (float32 partials).
* tests/golden/op_examples.json: hand-derived cases where the order decides
  whether a product overflows, and where the owner's signed zero survives a
  MAX/MIN tie.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SHAPES = [(2, 9), (3, 10), (4, 1024), (5, 23), (8, 1000), (16, 300), (64, 200), (7, 5), (11, 1),
          (13, 169)]


def _torch_widen(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def _torch_round(f):
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _signed_values(n, t, seed, dtype, spread=3):
    """Nonzero values of both signs over several orders of magnitude (no NaN,
    no zero, so no +0/-0 tie), stored as the oracle stores ``dtype``."""
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        v = rng.standard_normal(t) * 10.0 ** rng.integers(-spread, spread + 1, size=t)
        v[v == 0] = 1.0
        v = v.astype(np.float32)
        xs.append(_torch_round(v) if dtype != "float32" else v)
    return xs


def _extreme(xs, op, dtype):
    """Order-free MAX / MIN over the rank axis, returned in storage form (the
    selected input's own bits)."""
    wide = np.stack([_torch_widen(a) if dtype != "float32" else a for a in xs])
    pick = np.argmax(wide, axis=0) if op == "max" else np.argmin(wide, axis=0)
    return np.take_along_axis(np.stack(xs), pick[None, :], axis=0)[0]


MAXMIN_DTYPES = ["float32", "bfloat16", "bfloat16_acc32"]


@pytest.mark.parametrize("n,t", SHAPES)
@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("dtype", MAXMIN_DTYPES)
def test_max_min_brute_force_every_collective(n, t, op, dtype):
    x = _signed_values(n, t, 100 * n + t + (op == "min"), dtype)
    want = _extreme(x, op, dtype)
    for name, res in (("ring", oracle.ring_allreduce(x, op, dtype)),
                      ("tree", oracle.tree_allreduce(x, op, dtype)),
                      ("one tree", oracle.tree_allreduce(x, op, dtype, trees=1))):
        for r in range(n):
            np.testing.assert_array_equal(res.bufs[r].view(np.uint8), want.view(np.uint8),
                                          err_msg=f"{name} rank {r}")
    rs = oracle.ring_reduce_scatter(x, op, dtype)
    for r, (lo, hi) in enumerate(oracle.chunk_layout(n, t)):
        np.testing.assert_array_equal(rs.bufs[r][lo:hi].view(np.uint8), want[lo:hi].view(np.uint8))
    for root in sorted({0, n - 1, n // 2}):
        red = oracle.reduce(x, root, op, dtype)
        np.testing.assert_array_equal(red.bufs[root].view(np.uint8), want.view(np.uint8))


def _near_one(n, t, seed, dtype):
    """Products stay in range: magnitudes 2^u, u uniform in [-2, 2), both signs."""
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        v = (np.exp2(rng.uniform(-2, 2, size=t)) * rng.choice([-1.0, 1.0], size=t)).astype(np.float32)
        xs.append(_torch_round(v) if dtype != "float32" else v)
    return xs


def _mul(dtype):
    """One hop of PROD as the pinned reading states it: a float32 multiply,
    rounded to bfloat16 by torch for per-hop bfloat16.  Values are float32
    arrays here (bfloat16 inputs already widened)."""
    if dtype == "bfloat16":
        return lambda local, incoming: _torch_widen(_torch_round(local * incoming))
    return lambda local, incoming: (local * incoming).astype(np.float32)


def _ring_prod_closed_form(wide, mul):
    n, t = len(wide), len(wide[0])
    size = -(-t // n)
    out = np.empty(t, dtype=np.float32)
    for c in range(n):
        lo, hi = min(c * size, t), min((c + 1) * size, t)
        acc = wide[(c + 1) % n][lo:hi]
        for k in range(2, n + 1):
            acc = mul(wide[(c + k) % n][lo:hi], acc)
        out[lo:hi] = acc
    return out


def _binomial(vals, mul):
    n = len(vals)

    def block(q, k):
        if k == 0:
            return vals[q]
        half = 1 << (k - 1)
        low = block(q, k - 1)
        return mul(low, block(q + half, k - 1)) if q + half < n else low

    return block(0, oracle.ceil_log2(n))


def _to_storage(f, dtype):
    return f.astype(np.float32) if dtype == "float32" else _torch_round(f)


@pytest.mark.parametrize("n,t", SHAPES)
@pytest.mark.parametrize("dtype", MAXMIN_DTYPES)
def test_prod_fold_order_closed_forms(n, t, dtype):
    x = _near_one(n, t, 500 + n * t, dtype)
    wide = [a if dtype == "float32" else _torch_widen(a) for a in x]
    mul = _mul(dtype)
    ring = _to_storage(_ring_prod_closed_form(wide, mul), dtype)
    res = oracle.ring_allreduce(x, "prod", dtype)
    for r in range(n):
        np.testing.assert_array_equal(res.bufs[r], ring, err_msg=f"ring rank {r}")
    rs = oracle.ring_reduce_scatter(x, "prod", dtype)
    for r, (lo, hi) in enumerate(oracle.chunk_layout(n, t)):
        np.testing.assert_array_equal(rs.bufs[r][lo:hi], ring[lo:hi])
    h = -(-t // 2)
    tree = np.empty(t, dtype=np.float32)
    tree[:h] = _binomial([w[:h] for w in wide], mul)
    tree[h:] = _binomial([wide[n - 1 - q][h:] for q in range(n)], mul)
    tree = _to_storage(tree, dtype)
    tr = oracle.tree_allreduce(x, "prod", dtype)
    for r in range(n):
        np.testing.assert_array_equal(tr.bufs[r], tree, err_msg=f"tree rank {r}")
    root = n // 3
    red = oracle.reduce(x, root, "prod", dtype)
    want = _to_storage(_binomial([wide[(q + root) % n] for q in range(n)], mul), dtype)
    np.testing.assert_array_equal(red.bufs[root], want)


def test_prod_order_is_visible():
    """The closed forms above would not notice an order change if every order
    gave the same bits: on these inputs the ring and the tree differ."""
    x = _near_one(8, 4096, 3, "float32")
    ring = oracle.ring_allreduce(x, "prod", "float32").bufs[0]
    tree = oracle.tree_allreduce(x, "prod", "float32").bufs[0]
    assert np.count_nonzero(ring != tree) > 100


def _load_op_examples():
    with open(os.path.join(GOLDEN, "op_examples.json")) as f:
        return json.load(f)["cases"]


def _bits(rows, dtype):
    st = np.uint32 if dtype == "float32" else np.uint16
    arr = [np.array([int(h, 16) for h in row], dtype=st) for row in rows]
    return [a.view(np.float32) for a in arr] if dtype == "float32" else arr


@pytest.mark.filterwarnings("ignore:overflow encountered")
@pytest.mark.parametrize("case", _load_op_examples(), ids=lambda c: c["name"])
def test_op_golden_cases(case):
    dtype = case["dtype"]
    x = _bits(case["inputs_bits"], dtype)
    fn = oracle.ring_allreduce if case["collective"] == "ring_allreduce" else oracle.tree_allreduce
    res = fn(x, case["op"], dtype)
    for r, want in enumerate(_bits(case["expected_bits"], dtype)):
        np.testing.assert_array_equal(res.bufs[r].view(np.uint8), want.view(np.uint8),
                                      err_msg=f"rank {r}")
