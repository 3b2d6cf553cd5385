"""Pins for the oracle's 16-point randomized Hadamard transform and its
stochastic rounding.

RHT: against scipy's Hadamard matrix (library routine), orthogonality
H H^T = 16 I, norm preservation in exact arithmetic and a worked example.
SR: the pages' property that stochastic rounding is unbiased, checked exactly
by enumerating every 16-bit random slot; outputs are always a neighbouring
grid value and grid values never move.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O
from _golden import e2m1_values

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _rht_matrix(mask):
    cols = []
    for j in range(16):
        e = np.zeros(16, dtype=np.float32)
        e[j] = 1.0
        cols.append(O.rht16_vec(e, mask))
    return np.stack(cols, axis=1).astype(np.float64)


def test_rht_is_quarter_hadamard_times_signs():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    for mask in [0, 1, 0x8000, 0xFFFF, 0xA5C3, 0x1234]:
        s = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        assert np.array_equal(_rht_matrix(mask), 0.25 * H @ np.diag(s))


def test_hadamard_orthogonality_exact():
    for mask in [0, 0xBEEF]:
        Q = _rht_matrix(mask) * 4.0  # integer +-1 entries
        assert np.array_equal(Q @ Q.T, 16.0 * np.eye(16))
        Qs = _rht_matrix(mask)
        assert np.array_equal(Qs.T @ Qs, np.eye(16))


def test_rht_worked_example_e0():
    e0 = np.zeros(16, dtype=np.float32)
    e0[0] = 1.0
    assert np.array_equal(O.rht16_vec(e0, 0), np.full(16, 0.25, dtype=np.float32))


def test_rht_preserves_norm_and_inverts():
    rng = np.random.default_rng(1)
    for _ in range(50):
        x = rng.standard_normal(16).astype(np.float32)
        mask = int(rng.integers(0, 65536))
        y = O.rht16_vec(x, mask).astype(np.float64)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x.astype(np.float64))) < 1e-5
        # Q^T = diag(s) H / 4 undoes it
        s = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        back = s * (scipy.linalg.hadamard(16) @ y) / 4.0
        assert np.allclose(back, x, atol=1e-5)


def test_rht_tensor_row_and_col_axes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32, 48)).astype(np.float32)
    mask = 0x5A5A
    Q = _rht_matrix(mask)
    yr = O.rht16(x, "row", mask)
    for r in range(32):
        for c0 in range(0, 48, 16):
            assert np.allclose(yr[r, c0:c0 + 16], Q @ x[r, c0:c0 + 16], atol=1e-6)
    yc = O.rht16(x, "col", mask)
    for c in range(48):
        for r0 in range(0, 32, 16):
            assert np.allclose(yc[r0:r0 + 16, c], Q @ x[r0:r0 + 16, c], atol=1e-6)


def _sr_all_u(y):
    table = e2m1_values()
    return [table[O.e2m1_encode_sr(y, u)] for u in range(65536)]


@pytest.mark.parametrize("y", [0.1, 0.3, 0.74, 1.2, 1.9, 2.2, 2.75, 3.1, 4.5, 5.99, -0.6, -4.4,
                               1.0000001, 0.0001])
def test_sr_unbiased_to_2pow16_of_a_step(y):
    y = float(np.float32(y))
    outs = _sr_all_u(y)
    m = abs(y)
    lo = max(g for g in GRID if g <= m)
    hi = min(g for g in GRID if g > m)
    # only the two neighbours appear
    assert set(abs(o) for o in outs) <= {lo, hi}
    mean = sum(Fraction(o) for o in outs) / 65536
    assert abs(mean - Fraction(y)) < Fraction(hi - lo) / 65536


def test_sr_grid_values_do_not_move():
    for g in GRID:
        for s in (1.0, -1.0):
            v = s * g
            assert len(set(_sr_all_u(v))) == 1


def test_sr_saturates():
    assert all(abs(v) == 6.0 for v in _sr_all_u(7.5)[::97])


def test_rtne_is_biased_where_sr_is_not():
    # The pages' motivation for SR: RTNE's expected error is not zero.  For
    # values uniformly spread between 1.0 and 1.25, RTNE always returns 1.
    ys = np.linspace(1.01, 1.24, 12, dtype=np.float32)
    table = e2m1_values()
    bias_rne = np.mean([table[O.e2m1_encode_rne(y)] - y for y in ys])
    bias_sr = np.mean([np.mean(_sr_all_u(float(y))) - y for y in ys])
    assert bias_rne < -0.05
    assert abs(bias_sr) < 1e-4
