"""Pins for the oracle's element formats (E2M1 codes, E4M3 block scales).

Each check compares the oracle with something other than itself: the value
table and rounding intervals written by hand from the format's definition
(tests/golden), and torch's float8_e4m3fn casts as a library routine.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from _golden import e2m1_rne_intervals, e2m1_values, e4m3_examples


def test_e2m1_decode_matches_value_table():
    table = e2m1_values()
    assert len(table) == 16
    for code, v in table.items():
        got = O.e2m1_decode(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), code


def _interval_code(m, intervals):
    for lo, hi, lc, hc, code in intervals:
        above = m >= lo if lc else m > lo
        below = m <= hi if hc else m < hi
        if above and below:
            return code
    raise AssertionError(m)


def _probe_values():
    """All finite non-negative bf16 values, plus fp32 values within 64 ulps of
    every rounding boundary and of every grid point."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    vals = [bits.view(np.float32)]
    anchors = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for a in anchors:
        b = np.array([a], dtype=np.float32).view(np.uint32)[0]
        vals.append((b + np.arange(-64, 65, dtype=np.int64)).astype(np.uint32).view(np.float32))
    v = np.concatenate(vals)
    return v[np.isfinite(v)]


def test_e2m1_rne_matches_interval_table():
    intervals = e2m1_rne_intervals()
    for m in _probe_values()[::7]:
        want = _interval_code(float(m), intervals)
        assert O.e2m1_encode_rne(m) == want, float(m)
        assert O.e2m1_encode_rne(-m) == want | 8, float(m)


def test_e2m1_rne_every_midpoint_by_hand():
    # Each midpoint of neighbouring grid values goes to the even code.
    for m, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        assert O.e2m1_encode_rne(m) == code
    assert O.e2m1_encode_rne(1e30) == 7
    assert O.e2m1_encode_rne(-0.0) == 8
    assert O.e2m1_encode_rne(0.0) == 0


def test_e4m3_decode_matches_torch_float8():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = O.e4m3_decode(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], c


def test_e4m3_encode_matches_torch_cast_below_464():
    # torch's fp32 -> float8_e4m3fn cast is round-to-nearest-even; below 464 it
    # agrees with the saturating reading (at 464 and up torch gives NaN).
    bits = np.arange(0, 0x43E8, dtype=np.uint32) << 16  # bf16 values < 464
    v = bits.view(np.float32)
    rng = np.random.default_rng(0)
    v = np.concatenate([v, (rng.random(20000) * 463.0).astype(np.float32),
                        (rng.random(20000) * 2.0 ** -6).astype(np.float32)])
    v = v[v < 464.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(x) for x in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_hand_examples():
    for v, code in e4m3_examples():
        assert O.e4m3_encode(v) == code, (v, hex(code))


def test_e4m3_encode_saturates():
    for v in [448.0, 464.0, 480.0, 1e10, 3.4e38]:
        assert O.e4m3_encode(v) == 0x7E
