"""Pins for the oracle's per-hop arithmetic (``oracle.numerics``).

The per-hop operation is ``local (+) incoming`` at the receiver (Lecture 09
section 7.1 lab 1; Chapter 4 section 4.3.1).  Pins: hand-derived bfloat16
rounding cases (tests/golden/bf16_rounding.json), torch's CPU float32->bfloat16
conversion and bfloat16 addition (library routines), two's-complement facts and
IEEE subnormal facts.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_golden_cases():
    with open(os.path.join(GOLDEN, "bf16_rounding.json")) as f:
        cases = json.load(f)["cases"]
    bits = np.array([int(c["f32_bits"], 16) for c in cases], dtype=np.uint32)
    want = np.array([int(c["bf16_bits"], 16) for c in cases], dtype=np.uint16)
    got = oracle.f32_to_bf16_rne(bits.view(np.float32))
    for c, g, w in zip(cases, got, want):
        assert g == w, f"{c['what']}: got {g:#06x} want {w:#06x}"


def test_bf16_rounding_matches_torch_on_random_finite_values():
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    finite = np.isfinite(f)
    f = f[finite]
    # add exact ties and near-ties, which random bit patterns rarely hit
    hi = rng.integers(0, 0x7F7F, size=20_000, dtype=np.uint32) << np.uint32(16)
    for low in (0x8000, 0x7FFF, 0x8001):
        f = np.concatenate([f, (hi | np.uint32(low)).view(np.float32)])
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(f), _torch_bf16_bits(f))


def test_bf16_widening_is_exact():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(bits)
    finite = np.isfinite(f)
    # widening then rounding back is the identity on every non-NaN pattern
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(f[finite]), bits[finite])
    # and agrees with torch's widening
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32)
    np.testing.assert_array_equal(f[finite].view(np.uint32), t.numpy()[finite].view(np.uint32))


@pytest.mark.parametrize("op", ["sum", "prod"])
def test_bf16_combine_matches_torch(op):
    rng = np.random.default_rng(7)
    a32 = (rng.standard_normal(50_000) * 10.0 ** rng.integers(-8, 8, 50_000)).astype(np.float32)
    b32 = (rng.standard_normal(50_000) * 10.0 ** rng.integers(-8, 8, 50_000)).astype(np.float32)
    a = _torch_bf16_bits(a32)
    b = _torch_bf16_bits(b32)
    ta = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    want = (ta + tb) if op == "sum" else (ta * tb)
    got = oracle.combine(a, b, op, "bfloat16")
    np.testing.assert_array_equal(got, want.view(torch.int16).numpy().view(np.uint16))


def test_int32_wraps_twos_complement():
    a = np.array([2**31 - 1, -2**31, 65536, -1], dtype=np.int32)
    b = np.array([1, -1, 65536, -1], dtype=np.int32)
    np.testing.assert_array_equal(oracle.combine(a, b, "sum", "int32"),
                                  np.array([-2**31, 2**31 - 1, 131072, -2], dtype=np.int32))
    # 65536 * 65536 = 2^32 wraps to 0; (-1)*(-1) = 1
    np.testing.assert_array_equal(oracle.combine(a, b, "prod", "int32"),
                                  np.array([2**31 - 1, -2**31, 0, 1], dtype=np.int32))


def test_float32_subnormals_are_kept():
    tiny = np.array([1], dtype=np.uint32).view(np.float32)     # 2^-149
    got = oracle.combine(tiny, tiny, "sum", "float32")
    assert got.view(np.uint32)[0] == 2                          # 2^-148, exact


def test_max_min_keep_local_on_ties_and_nan():
    pz = np.array([0.0], dtype=np.float32)
    nz = np.array([-0.0], dtype=np.float32)
    nan = np.array([np.nan], dtype=np.float32)
    one = np.array([1.0], dtype=np.float32)
    assert np.signbit(oracle.combine(nz, pz, "max", "float32"))[0]          # local -0 kept
    assert not np.signbit(oracle.combine(pz, nz, "min", "float32"))[0]      # local +0 kept
    assert oracle.combine(one, nan, "max", "float32")[0] == 1.0             # NaN incoming loses
    assert np.isnan(oracle.combine(nan, one, "max", "float32"))[0]          # NaN local stays
    a = np.array([-5, 7], dtype=np.int32)
    b = np.array([3, -9], dtype=np.int32)
    np.testing.assert_array_equal(oracle.combine(a, b, "max", "int32"), [3, 7])
    np.testing.assert_array_equal(oracle.combine(a, b, "min", "int32"), [-5, -9])


def test_float32_sum_is_single_rounding():
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: ties to even gives 1;
    # 1 + 3*2^-24 ties between 1 + 2^-23 and 1 + 2^-22: gives 1 + 2^-22.
    one = np.float32(1.0)
    got = oracle.combine(np.array([one, one], dtype=np.float32),
                         np.array([2.0**-24, 3 * 2.0**-24], dtype=np.float32), "sum", "float32")
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2.0**-22], dtype=np.float32))
