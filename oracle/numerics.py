"""Element arithmetic of one ring hop: ``local (+) incoming``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages apply the reduction at the receiver as an in-place update of its own
chunk with the chunk it has just received: Lecture 09, section 7.1 (lab 1)
updates the receiver's chunk with ``+=``, and Chapter 4, section 4.3.1 does the
same in its ReduceScatter loop.  Lecture 09, section 3.4 lists the reduction
operators SUM, MAX, MIN and PROD.  The pages never fix the rounding, so the
readings here are:

* int32: two's-complement wrap-around (SUM, PROD); MAX/MIN on signed values.
* float32: one IEEE-754 binary32 operation with round-to-nearest-even, the
  rounding NumPy's float32 ufuncs perform; subnormals are kept.
* bfloat16 (stored as uint16 bit patterns): widen both operands to float32,
  apply the operation in float32, round back to bfloat16 to nearest-even after
  every hop, because in a literal ring the partial sum lives in a bfloat16
  rank buffer between hops.
* MAX keeps the local value unless the incoming one compares strictly greater;
  MIN unless strictly smaller.  That fixes which zero survives a +0/-0 tie and
  that a NaN on the incoming side never wins.
* bfloat16_acc32: bfloat16 buffers whose reductions carry float32 partials
  from hop to hop and round once at the end (the "bf16 with fp32
  accumulation" variant).  It is not a per-hop rule, so ``combine`` refuses
  it; the collectives widen to float32, run the float32 schedule and round
  (``collectives._float32_partials``).
"""

import numpy as np

DTYPES = ("int32", "float32", "bfloat16", "bfloat16_acc32")
OPS = ("sum", "prod", "max", "min")
ITEMSIZE = {"int32": 4, "float32": 4, "bfloat16": 2, "bfloat16_acc32": 2}
STORAGE = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16,
           "bfloat16_acc32": np.uint16}


def bf16_to_f32(bits):
    """Widen bfloat16 bit patterns (uint16) to float32: the bfloat16 bits are
    the top half of the binary32 word, the low half is zero."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """Round float32 values to bfloat16 bit patterns, to nearest, ties to even.

    Textbook integer form: add 0x7FFF plus the lowest kept bit to the binary32
    word and keep the top 16 bits.  A carry out of the mantissa bumps the
    exponent, which also turns values above the largest bfloat16 into
    infinity.  NaN keeps its sign and top payload bits and gets the quiet bit
    (0x0040) set, so it can never round into an infinity.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return np.where(is_nan, quiet, rounded)


def _wrap_int32(wide):
    return (wide & 0xFFFFFFFF).astype(np.uint32).view(np.int32)


def combine(local, incoming, op, dtype):
    """Return ``local (+) incoming`` elementwise, as the receiving rank stores it."""
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}")
    if dtype == "int32":
        a = np.asarray(local, dtype=np.int32)
        b = np.asarray(incoming, dtype=np.int32)
        if op == "sum":
            return _wrap_int32(a.astype(np.int64) + b.astype(np.int64))
        if op == "prod":
            return _wrap_int32(a.astype(np.int64) * b.astype(np.int64))
        if op == "max":
            return np.where(b > a, b, a).astype(np.int32)
        return np.where(b < a, b, a).astype(np.int32)
    if dtype == "float32":
        a = np.asarray(local, dtype=np.float32)
        b = np.asarray(incoming, dtype=np.float32)
        if op == "sum":
            return a + b
        if op == "prod":
            return a * b
        if op == "max":
            return np.where(b > a, b, a).astype(np.float32)
        return np.where(b < a, b, a).astype(np.float32)
    if dtype == "bfloat16":
        abits = np.asarray(local, dtype=np.uint16)
        bbits = np.asarray(incoming, dtype=np.uint16)
        a = bf16_to_f32(abits)
        b = bf16_to_f32(bbits)
        if op == "sum":
            return f32_to_bf16_rne(a + b)
        if op == "prod":
            return f32_to_bf16_rne(a * b)
        if op == "max":
            return np.where(b > a, bbits, abits).astype(np.uint16)
        return np.where(b < a, bbits, abits).astype(np.uint16)
    if dtype == "bfloat16_acc32":
        raise ValueError("bfloat16_acc32 has no per-hop rule: its partials are float32")
    raise ValueError(f"unknown dtype {dtype!r}")
