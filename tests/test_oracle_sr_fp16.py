"""Pins for the oracle's fp32 -> fp16 stochastic rounding (the SSM-state cache
recipe: FP16 with Philox<5> stochastic rounding, Super report summary 4.3).

Checked against: numpy's float16 (every finite fp16 value round-trips; the
result is always one of the two fp16 neighbours of x that numpy's
round-to-nearest picks from), exact unbiasedness over all 65536 random
slots, hand-worked examples in the normal and subnormal ranges, the readings
at the edges (saturation, NaN, signed zero), and the Philox slot of each
element taken straight from the oracle's Philox4x32."""
import numpy as np
import pytest

import oracle as O


def _f16_value(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def test_every_finite_fp16_round_trips():
    h = np.arange(0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float32)
    for u in (0, 1, 32768, 65535):
        for s in (1.0, -1.0):
            x = (v * np.float32(s)).astype(np.float32)
            got = np.array([O.sr_fp16_one(xi, u) for xi in x[::37]], dtype=np.uint16)
            want = h[::37] | (np.uint16(0x8000) if s < 0 else np.uint16(0))
            assert np.array_equal(got, want)


def test_result_is_a_neighbour_from_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 4, 3000),
                        rng.uniform(-2 ** -14, 2 ** -14, 1000)]).astype(np.float32)
    for xi in x:
        r = np.float16(xi)  # numpy: round to nearest even
        if float(r) == float(xi):
            nb = {float(r)}
        elif float(r) < float(xi):
            nb = {float(r), float(np.nextafter(r, np.float16(np.inf)))}
        else:
            nb = {float(np.nextafter(r, np.float16(-np.inf))), float(r)}
        for u in (0, 12345, 65535):
            assert _f16_value(O.sr_fp16_one(xi, u)) in nb, (xi, u)


@pytest.mark.parametrize("x", [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -13, 3 * 2.0 ** -26, 123.456,
                               -0.000123, 65000.5, 2.0 ** -20 + 2.0 ** -30])
def test_unbiased_over_all_slots(x):
    """Over the 65536 equally likely slots the mean is lo + (hi - lo) *
    ceil(65536 f) / 65536 exactly, f the fraction of the way from lo to hi."""
    x = float(np.float32(x))
    vals = np.array([_f16_value(O.sr_fp16_one(x, u)) for u in range(65536)])
    a = abs(x)
    lo = max(v for v in np.unique(np.abs(vals)) if v <= a)
    hi = min(v for v in np.unique(np.abs(vals)) if v >= a)
    if lo == hi:
        assert np.all(np.abs(vals) == a)
        return
    f = (a - lo) / (hi - lo)
    ups = np.count_nonzero(np.abs(vals) == hi)
    assert ups == int(np.ceil(65536 * f))
    mean = np.abs(vals).mean()
    assert abs(mean - a) <= (hi - lo) / 65536


def test_hand_examples():
    # halfway between fp16 1.0 (0x3C00) and 1.0 + 2^-10 (0x3C01): up iff u < 32768
    assert O.sr_fp16_one(1.0 + 2.0 ** -11, 32767) == 0x3C01
    assert O.sr_fp16_one(1.0 + 2.0 ** -11, 32768) == 0x3C00
    # three quarters of the subnormal step 2^-24 above 0: up iff u < 49152
    assert O.sr_fp16_one(3 * 2.0 ** -26, 49151) == 0x0001
    assert O.sr_fp16_one(3 * 2.0 ** -26, 49152) == 0x0000
    # just below the smallest normal 2^-14: rounds up into it (0x0400) or down to 0x03FF
    x = float(np.float32(2.0 ** -14 - 2.0 ** -30))  # fp32 spacing here is 2^-38
    assert x < 2.0 ** -14
    assert O.sr_fp16_one(x, 0) == 0x0400 and O.sr_fp16_one(x, 65535) == 0x03FF


def test_edges():
    assert O.sr_fp16_one(65504.0, 0) == 0x7BFF
    assert O.sr_fp16_one(65519.0, 0) == 0x7BFF and O.sr_fp16_one(1e30, 0) == 0x7BFF
    assert O.sr_fp16_one(float("-inf"), 0) == 0xFBFF
    assert O.sr_fp16_one(float("nan"), 0) & 0x7FFF == 0x7E00
    assert O.sr_fp16_one(-0.0, 0) == 0x8000 and O.sr_fp16_one(0.0, 0) == 0x0000
    # an fp32 subnormal is a fraction 2^-125 of the fp16 step: up only for u = 0
    assert O.sr_fp16_one(-(2.0 ** -149), 0) == 0x8001
    assert O.sr_fp16_one(-(2.0 ** -149), 1) == 0x8000


def test_element_i_uses_slot_i_mod_8_of_call_i_div_8():
    """x = 1 + 2^-11 everywhere rounds up exactly when its slot is < 32768."""
    seed, offset, n = 0x1234_5678_9ABC, 77, 40
    y = O.sr_fp16(np.full(n, 1.0 + 2.0 ** -11, dtype=np.float32), seed, offset, rounds=5)
    for i in range(n):
        call = i // 8
        out = O.philox4x32([call & 0xFFFFFFFF, call >> 32, offset & 0xFFFFFFFF, offset >> 32],
                           [seed & 0xFFFFFFFF, seed >> 32], 5)
        w = int(out[(i % 8) // 2])
        u = (w >> 16) if i % 2 else (w & 0xFFFF)
        assert y[i] == (0x3C01 if u < 32768 else 0x3C00), i
