"""Pins for the oracle's fp64 GEMM reference.

Checked against a brute-force dequantize-then-matmul written independently of
the oracle's decode: E2M1 values from the hand-written table, E4M3 scales
through torch's float8_e4m3fn cast, and numpy's fp64 matmul as the library
routine.  Also: the layouts NT / NN / TN give identical results on the same
logical operands, and the magnitude sum D bounds |R|.
"""
import numpy as np
import pytest
import torch

import oracle as O
from _golden import e2m1_values

E2M1 = np.array([e2m1_values()[c] for c in range(16)], dtype=np.float64)


def _e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _decode(q, rows, cols):
    """Independent decode of a stored operand to fp64 (without g)."""
    c = q["codes"]
    codes = np.stack([c & 0xF, c >> 4], axis=-1).reshape(rows, cols)
    vals = E2M1[codes]
    s = _e4m3(q["scales"])
    if q["block"] == "row":
        sc = np.repeat(s, 16, axis=1)
    elif q["block"] == "col":
        sc = np.repeat(s, 16, axis=0)
    else:
        sc = np.repeat(np.repeat(s, 16, axis=0), 16, axis=1)
    return vals * sc


def _q(x, block, **kw):
    q = O.quantize(x, block, **kw)
    q["block"] = block
    return q


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_matches_bruteforce(layout):
    rng = np.random.default_rng(20)
    M, N, K = 48, 32, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)  # logical B^T [N][K]
    if layout == "NT":
        A = _q(a, "row"); B = _q(b, "2d")
        Ad = _decode(A, M, K); Bd = _decode(B, N, K).T
    elif layout == "NN":
        A = _q(a, "row"); B = _q(np.ascontiguousarray(b.T), "2d")
        Ad = _decode(A, M, K); Bd = _decode(B, K, N)
    else:
        A = _q(np.ascontiguousarray(a.T), "col", rounding=O.SR, seed=3, rht_mask=0x1234)
        B = _q(np.ascontiguousarray(b.T), "col", rht_mask=0x1234)
        Ad = _decode(A, K, M).T; Bd = _decode(B, K, N)
    R, D = O.gemm_full(layout[0], layout[1], M, N, K, A, B)
    want = float(A["g"]) * float(B["g"]) * (Ad @ Bd)
    wantD = float(A["g"]) * float(B["g"]) * (np.abs(Ad) @ np.abs(Bd))
    assert np.allclose(R, want, rtol=0, atol=1e-12 * wantD.max())
    assert np.allclose(D, wantD, rtol=1e-12)
    assert np.all(np.abs(R) <= D * (1 + 1e-12))
    # sampled entries agree with the full matrix
    ii = rng.integers(0, M, 30); jj = rng.integers(0, N, 30)
    Re, De = O.gemm_entries(layout[0], layout[1], M, N, K, A, B, ii, jj)
    assert np.array_equal(Re, R[ii, jj]) and np.array_equal(De, D[ii, jj])


def test_gemm_exact_special_case():
    # Operands drawn on the E2M1 grid with block max 6 everywhere and a tensor
    # amax of 6*448: every block scale is 448, g = 1 and products are exact
    # multiples of 448^2/4; the fp64 reference must be exact.
    rng = np.random.default_rng(21)
    M, N, K = 32, 32, 128
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    a = grid[rng.integers(0, 8, (M, K))] * np.where(rng.random((M, K)) < .5, -1, 1)
    b = grid[rng.integers(0, 8, (N, K))] * np.where(rng.random((N, K)) < .5, -1, 1)
    a[:, ::16] = 6.0
    b[:, ::16] = 6.0
    a = (a * 448).astype(np.float32); b = (b * 448).astype(np.float32)
    A = _q(a, "row"); B = _q(b, "row")
    assert A["g"] == 1.0 and B["g"] == 1.0
    assert (A["scales"] == 0x7E).all() and (B["scales"] == 0x7E).all()
    R, _ = O.gemm_full("N", "T", M, N, K, A, B)
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.array_equal(R, exact)


def test_layout_errors():
    A = _q(np.ones((16, 32), dtype=np.float32), "row")
    with pytest.raises(ValueError):
        O.gemm_entries("T", "T", 32, 16, 16, A, A, [0], [0])
    with pytest.raises(ValueError):  # ROW blocks cannot serve a K-by-rows operand
        O.gemm_entries("T", "N", 32, 32, 16, A, A, [0], [0])


# ---- the parity metric itself ------------------------------------------------------------------
def test_rel_err_hand_cases():
    """max |C - R| / D on hand-made values: exact agreement is 0, a known
    relative offset is recovered, D = 0 demands C = 0, and the maximum over
    entries is what is reported."""
    R = np.array([1.0, -2.0, 0.5, 0.0])
    D = np.array([3.0, 2.0, 8.0, 0.0])
    assert O.gemm_rel_err(R.copy(), R, D) == 0.0
    e = O.gemm_rel_err(R + 2e-3 * D, R, D)
    assert abs(e - 2e-3) < 1e-15
    bad = R.copy()
    bad[3] = 1e-30  # the D = 0 entry must be exactly 0
    assert O.gemm_rel_err(bad, R, D) == np.inf
    one = R.copy()
    one[2] += 0.5 * D[2]  # one entry off by half its D
    assert O.gemm_rel_err(one, R, D) == 0.5
    assert O.gemm_rel_err(np.zeros(0), np.zeros(0), np.zeros(0)) == 0.0


def test_rel_err_flags_a_dropped_block():
    """A product computed independently (numpy fp32 matmul of the decoded
    operands) passes the 1e-3 bar; the same product missing one 16-k block of
    the contraction, or with one operand's block scale off by one code, fails
    it."""
    rng = np.random.default_rng(22)
    M, N, K = 32, 48, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = _q(a, "row"); B = _q(b, "2d")
    R, D = O.gemm_full("N", "T", M, N, K, A, B)
    Ad = _decode(A, M, K).astype(np.float32)
    Bd = _decode(B, N, K).astype(np.float32)
    g = np.float32(A["g"]) * np.float32(B["g"])
    good = (Ad @ Bd.T) * g
    assert O.gemm_rel_err(good, R, D) <= 1e-3
    dropped = (Ad[:, 16:] @ Bd[:, 16:].T) * g
    assert O.gemm_rel_err(dropped, R, D) > 1e-3
    A2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in A.items()}
    A2["scales"][5, 3] = A2["scales"][5, 3] + 1
    off = (_decode(A2, M, K).astype(np.float32) @ Bd.T) * g
    assert O.gemm_rel_err(off, R, D) > 1e-3


def test_thread_count_does_not_change_the_reference():
    """set_threads only splits the outputs over threads: one thread and all
    of them give the same R and D, bit for bit (the CPU baseline times both)."""
    rng = np.random.default_rng(77)
    a = rng.standard_normal((48, 256)).astype(np.float32)
    b = rng.standard_normal((64, 256)).astype(np.float32)
    A, B = _q(a, "row"), _q(b, "2d")
    ii = np.repeat(np.arange(48), 64)
    jj = np.tile(np.arange(64), 48)
    before = O.set_threads(0)
    try:
        assert O.set_threads(1) == 1
        R1, D1 = O.gemm_entries("N", "T", 48, 64, 256, A, B, ii, jj)
        O.set_threads(max(before, 2))
        Rn, Dn = O.gemm_entries("N", "T", 48, 64, 256, A, B, ii, jj)
    finally:
        O.set_threads(before)
    assert np.array_equal(R1, Rn) and np.array_equal(D1, Dn)
    Rf, Df = O.gemm_full("N", "T", 48, 64, 256, A, B)
    assert np.array_equal(R1, Rf.reshape(-1)) and np.array_equal(D1, Df.reshape(-1))
