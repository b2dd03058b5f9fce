"""Fit the library's cost model to measured calls (host only, NumPy).

The model is the single-GPU form of the pages' alpha-beta model ("第09讲"
Lecture 09, sections 1.3 and 7.3: time = alpha per message step + bytes over
bandwidth).  On one GPU a step is a kernel launch and the bandwidth is HBM's:

    microseconds(call) = launches * alpha_us + hbm_bytes / (gbps * 1e3)

with launches = 1 for the fused kernels and one per schedule step for the
step-by-step implementation, and hbm_bytes the bytes that implementation
moves (``ar_predict_time`` in include/ar.h).  ``fit`` takes bench.py JSON
records (one per measured configuration) and returns, per (collective,
implementation), the least-squares (alpha_us, gbps).  ``apply`` loads them
into the library so that ``allreduce`` picks ring or tree with them.

    python -m tree_allreduce_algorithms_amd.costfit suite.jsonl
"""

import json
import sys

import numpy as np


def records_from_jsonl(path):
    with open(path) as f:
        return [json.loads(line) for line in f if line.strip()]


def points(records, cache_state="flushed"):
    """(collective, impl) -> list of (launches, hbm_bytes, microseconds).

    Only records whose timing is event based with the Infinity Cache flushed
    before every call are used by default: their events hold GPU time only,
    while back-to-back calls on small buffers are bound by the host."""
    out = {}
    for rec in records:
        cfg, roof = rec["config"], rec["roofline"]
        flushed = "flushed" in cfg.get("timing", "")
        if cache_state == "flushed" and not flushed:
            continue
        coll = cfg.get("ran", cfg["collective"])
        key = (coll, cfg["impl"])
        out.setdefault(key, []).append(
            (roof["launches_per_step"], roof["algorithmic_bytes_per_call"],
             roof["event_ms_mean"] * 1e3))
    return out


def fit_one(pts):
    """Least-squares alpha_us >= 0 and gbps > 0 for one (collective, impl)."""
    a = np.array([[float(n), float(b) / 1e3] for n, b, _ in pts])   # bytes/1e3 -> us at 1 GB/s
    y = np.array([t for _, _, t in pts], dtype=float)
    coef, *_ = np.linalg.lstsq(a, y, rcond=None)
    alpha, inv = float(coef[0]), float(coef[1])
    if alpha < 0.0:                       # refit through the origin
        alpha = 0.0
        inv = float(np.dot(a[:, 1], y) / np.dot(a[:, 1], a[:, 1]))
    if inv <= 0.0:
        raise ValueError("measurements do not determine a positive bandwidth")
    return alpha, 1.0 / inv


# On one GPU the fused ring and the fused double tree are one launch each that
# read N inputs and write N outputs per element: the same work in a different
# fold order.  Measured over the message-size sweep they are within 1-2 % of
# each other at every size, inside the run-to-run spread, so their points are
# fitted together and both get the same coefficients.  The model then predicts
# equal times and ar_allreduce runs the ring (the tie rule); only the step
# implementation, whose launch counts differ (2(N-1) against 2 ceil(log2 N)),
# has a real crossover.
POOLED = (("ring_allreduce", "fused"), ("tree_allreduce", "fused"))


def fit(records, cache_state="flushed", pool_fused_allreduce=True):
    """(collective, impl) -> (alpha_us, gbps) for every pair with >= 2 points;
    with pool_fused_allreduce the fused ring and tree AllReduce share one fit
    over their pooled points."""
    pts = points(records, cache_state)
    if pool_fused_allreduce and all(k in pts for k in POOLED):
        pooled = pts[POOLED[0]] + pts[POOLED[1]]
        for k in POOLED:
            pts[k] = pooled
    return {k: fit_one(v) for k, v in pts.items() if len(v) >= 2}


def apply(coeffs):
    """Load fitted coefficients into the library (``ar_set_cost_model``)."""
    from . import binding
    for (coll, impl), (alpha, gbps) in coeffs.items():
        if coll in binding.COLLECTIVES and impl in binding.IMPLS:
            binding.set_cost_model(coll, impl, alpha, gbps)


def main(argv):
    if len(argv) != 2:
        print(__doc__)
        return 2
    coeffs = fit(records_from_jsonl(argv[1]))
    for (coll, impl), (alpha, gbps) in sorted(coeffs.items()):
        print(f"{coll:16s} {impl:6s} alpha_us={alpha:8.3f} gbps={gbps:9.1f}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
