"""Plant one mistake at a time in the oracle (on the CPU) and check that the
pins notice.  A pin set that a dropped term, a wrong index or a wrong
direction survives would not be worth trusting.
"""

import json
import os

import numpy as np
import pytest

import oracle
import oracle.collectives as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints(n, t, seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(-100, 100, size=t, endpoint=True, dtype=np.int32) for _ in range(n)]


def _pins_hold():
    """A compact run of the pins: int32 brute force for AllReduce, ownership
    after ReduceScatter, AllGather, ragged byte counts, the order goldens."""
    for n, t in [(4, 1024), (5, 23), (8, 1000), (3, 7), (4, 12)]:
        x = _ints(n, t, n + t)
        want = (np.stack(x).astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        ar = oracle.ring_allreduce(x, "sum", "int32")
        if any(not np.array_equal(b, want) for b in ar.bufs):
            return False
        size = -(-t // n)
        rs = oracle.ring_reduce_scatter(x, "sum", "int32")
        for r in range(n):
            lo, hi = min(r * size, t), min((r + 1) * size, t)
            if not np.array_equal(rs.bufs[r][lo:hi], want[lo:hi]):
                return False
            if rs.sent[r] != (t - (hi - lo)) * 4:
                return False
        tr = oracle.tree_allreduce(x, "sum", "int32")
        if any(not np.array_equal(b, want) for b in tr.bufs):
            return False
        root = n - 1
        red = oracle.reduce(x, root, "sum", "int32")
        if not np.array_equal(red.bufs[root], want) or int(red.sent[root]) != 0:
            return False
        if t % n == 0:
            a2a = oracle.alltoall(x, "int32")
            b = t // n
            if not np.array_equal(a2a.bufs[1][:b], x[0][b:2 * b]):
                return False
        bc = oracle.broadcast(x, root, "int32")
        if any(not np.array_equal(b, x[root]) for b in bc.bufs) or int(bc.recv[root]) != 0:
            return False
    # double-tree order on an odd T: the binomial recursion on each half
    # (roles = ranks below ceil(T/2), mirrored roles above)
    rng = np.random.default_rng(77)
    for n, t in [(5, 11), (8, 9)]:
        x = [rng.standard_normal(t).astype(np.float32) for _ in range(n)]

        def fold(vals):
            def block(q, k):
                if k == 0:
                    return vals[q]
                half = 1 << (k - 1)
                low = block(q, k - 1)
                return low + block(q + half, k - 1) if q + half < len(vals) else low
            return block(0, oracle.ceil_log2(len(vals)))

        h = -(-t // 2)
        want = np.concatenate([fold([v[:h] for v in x]), fold([x[n - 1 - q][h:] for q in range(n)])])
        if any(not np.array_equal(b, want) for b in oracle.tree_allreduce(x, "sum", "float32").bufs):
            return False
    with open(os.path.join(GOLDEN, "order_examples.json")) as f:
        for case in json.load(f)["cases"]:
            x = [np.array(v, dtype=np.float32) for v in case["inputs"]]
            fn = oracle.ring_allreduce if case["collective"] == "ring_allreduce" else oracle.tree_allreduce
            res = fn(x, "sum", "float32")
            if any(not np.array_equal(b, np.array(w, np.float32))
                   for b, w in zip(res.bufs, case["expected"])):
                return False
    return True


def test_unmutated_oracle_passes():
    assert _pins_hold()


MUTATIONS = {
    "reduce_scatter_zero_based_send": ("rs_send_chunk", lambda r, t, n: (r - t) % n),
    "reduce_scatter_wrong_direction": ("rs_send_chunk", lambda r, t, n: (r + t + 1) % n),
    "allgather_sends_unfinished_chunk": ("ag_send_chunk", lambda r, t, n: (r - t + 1) % n),
    "ring_skips_a_neighbour": ("ring_next", lambda r, n: (r + 2) % n),
    "ring_turns_left": ("ring_next", lambda r, n: (r - 1) % n),
    "tree_one_not_mirrored": ("tree_rank", lambda tree, role, n: role),
    "double_tree_split_at_floor": (
        "_tree_segments",
        lambda trees, total: [(0, 0, total)] if trees == 1 else [(0, 0, total // 2), (1, total // 2, total)]),
    "rooted_tree_ignores_root": ("rooted_rank", lambda role, root, n: role),
    "alltoall_keeps_block_index": ("alltoall_slot", lambda src, dst: dst),
    "receiver_overwrites_instead_of_adding": (
        "combine", lambda local, incoming, op, dtype: np.array(incoming, copy=True)),
    "receiver_drops_incoming": ("combine", lambda local, incoming, op, dtype: np.array(local, copy=True)),
    "floor_chunk_layout_tail_in_last": (
        "chunk_layout",
        lambda n, t: [(c * (t // n), (c + 1) * (t // n) if c < n - 1 else t) for c in range(n)]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oc, attr, fn)
    assert not _pins_hold(), f"mutation {name} survived every pin"


# --- bfloat16 rounding: a wrong rounding rule must fail the rounding pins ------

def _truncate(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _half_up(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16).astype(np.uint16)


def _half_odd(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    odd = (u >> 16) & 1
    return ((u + 0x7FFF + (1 - odd)) >> 16).astype(np.uint16)


def _bf16_pins_hold():
    """The rounding golden cases (tests/golden/bf16_rounding.json, IEEE ties)
    and a bfloat16 per-hop AllReduce whose partials hit ties."""
    with open(os.path.join(GOLDEN, "bf16_rounding.json")) as f:
        cases = json.load(f)["cases"]
    bits = np.array([int(c["f32_bits"], 16) for c in cases], dtype=np.uint32)
    want = np.array([int(c["bf16_bits"], 16) for c in cases], dtype=np.uint16)
    if not np.array_equal(oracle.f32_to_bf16_rne(bits.view(np.float32)), want):
        return False
    # A per-hop bfloat16 AllReduce whose partials land on ties.  N = 3, T = 3
    # (one element per chunk); rank 0 holds 1 + 2^-7, ranks 1 and 2 hold 2^-8.
    # Chunk 0 folds ranks 1, 2, 0: 2^-8 + 2^-8 = 2^-7, then 1 + 2^-6, exact.
    # Chunk 1 folds ranks 2, 0, 1: (1 + 2^-7) + 2^-8 = 1 + 3*2^-8 is a tie that
    # rounds up to 1 + 2^-6 (even mantissa 0000010), then + 2^-8 = 1 + 5*2^-8,
    # a tie that rounds down to 1 + 2^-6.  Chunk 2 folds ranks 0, 1, 2: the
    # same two ties.  With ties to even every rank ends with 1 + 2^-6 (0x3F82)
    # everywhere; truncation, half-up and half-to-odd each give another value.
    x = [np.full(3, 0x3F81, np.uint16), np.full(3, 0x3B80, np.uint16), np.full(3, 0x3B80, np.uint16)]
    res = oracle.ring_allreduce(x, "sum", "bfloat16")
    return all(np.array_equal(b, np.full(3, 0x3F82, np.uint16)) for b in res.bufs)


def test_unmutated_rounding_passes():
    assert _bf16_pins_hold()


@pytest.mark.parametrize("rule", [_truncate, _half_up, _half_odd], ids=["truncate", "half_up", "half_to_odd"])
def test_wrong_bf16_rounding_is_caught(rule, monkeypatch):
    import oracle.numerics as on
    monkeypatch.setattr(on, "f32_to_bf16_rne", rule)
    monkeypatch.setattr(oracle, "f32_to_bf16_rne", rule)
    assert not _bf16_pins_hold(), f"rounding rule {rule.__name__} survived the pins"


# --- PROD / MAX / MIN on float32 and bfloat16: planted operator mistakes ---------

import oracle.numerics as on  # noqa: E402

_COMBINE = on.combine


def _op_pins_hold():
    """A compact run of the operator pins of test_oracle_ops.py: MAX/MIN brute
    force over the rank axis (float32, bfloat16), the ring and tree PROD fold
    closed forms (float32, per-hop bfloat16), and the hand-derived op goldens."""
    import test_oracle_ops as ops
    with np.errstate(over="ignore"):
        for dtype in ("float32", "bfloat16"):
            for n, t in [(4, 64), (5, 23), (8, 40)]:
                for op in ("max", "min"):
                    x = ops._signed_values(n, t, 7 * n + t, dtype)
                    want = ops._extreme(x, op, dtype)
                    for res in (oracle.ring_allreduce(x, op, dtype), oracle.tree_allreduce(x, op, dtype)):
                        if any(not np.array_equal(b.view(np.uint8), want.view(np.uint8)) for b in res.bufs):
                            return False
                x = ops._near_one(n, t, 11 * n + t, dtype)
                wide = [a if dtype == "float32" else ops._torch_widen(a) for a in x]
                want = ops._to_storage(ops._ring_prod_closed_form(wide, ops._mul(dtype)), dtype)
                if any(not np.array_equal(b, want) for b in oracle.ring_allreduce(x, "prod", dtype).bufs):
                    return False
        for case in ops._load_op_examples():
            x = ops._bits(case["inputs_bits"], case["dtype"])
            fn = oracle.ring_allreduce if case["collective"] == "ring_allreduce" else oracle.tree_allreduce
            res = fn(x, case["op"], case["dtype"])
            for b, want in zip(res.bufs, ops._bits(case["expected_bits"], case["dtype"])):
                if not np.array_equal(b.view(np.uint8), want.view(np.uint8)):
                    return False
    return True


def _swap_max_min(local, incoming, op, dtype):
    if dtype == "float32" and op in ("max", "min"):
        op = "min" if op == "max" else "max"
    return _COMBINE(local, incoming, op, dtype)


def _bf16_max_on_raw_bits(local, incoming, op, dtype):
    if dtype == "bfloat16" and op == "max":
        a = np.asarray(local, dtype=np.uint16)
        b = np.asarray(incoming, dtype=np.uint16)
        return np.where(b > a, b, a).astype(np.uint16)
    return _COMBINE(local, incoming, op, dtype)


def _f32_prod_as_sum(local, incoming, op, dtype):
    if dtype == "float32" and op == "prod":
        return _COMBINE(local, incoming, "sum", dtype)
    return _COMBINE(local, incoming, op, dtype)


def _bf16_min_on_raw_bits(local, incoming, op, dtype):
    if dtype == "bfloat16" and op == "min":
        a = np.asarray(local, dtype=np.uint16)
        b = np.asarray(incoming, dtype=np.uint16)
        return np.where(b < a, b, a).astype(np.uint16)
    return _COMBINE(local, incoming, op, dtype)


def _max_takes_incoming_on_ties(local, incoming, op, dtype):
    if dtype == "float32" and op == "max":
        a = np.asarray(local, dtype=np.float32)
        b = np.asarray(incoming, dtype=np.float32)
        return np.where(b >= a, b, a).astype(np.float32)
    return _COMBINE(local, incoming, op, dtype)


def _bf16_prod_truncates(local, incoming, op, dtype):
    if dtype == "bfloat16" and op == "prod":
        prod = on.bf16_to_f32(local) * on.bf16_to_f32(incoming)
        return (np.ascontiguousarray(prod, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return _COMBINE(local, incoming, op, dtype)


OP_MUTATIONS = {
    "float32_max_min_swapped": _swap_max_min,
    "bfloat16_max_on_raw_bits": _bf16_max_on_raw_bits,
    "bfloat16_min_on_raw_bits": _bf16_min_on_raw_bits,
    "float32_prod_as_sum": _f32_prod_as_sum,
    "float32_max_takes_incoming_on_ties": _max_takes_incoming_on_ties,
    "bfloat16_prod_truncates": _bf16_prod_truncates,
}


def test_unmutated_operators_pass():
    assert _op_pins_hold()


@pytest.mark.parametrize("name", sorted(OP_MUTATIONS))
def test_planted_operator_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(oc, "combine", OP_MUTATIONS[name])
    assert not _op_pins_hold(), f"mutation {name} survived the operator pins"
