"""Pins for the oracle's tensor quantizers and dequantizer.

Checked against: a worked example computed by hand (tests/golden), the
closed form of the per-tensor scales, invariants that hold for any input
(the amax element takes the top code under the top block scale; COL equals
the transpose of ROW, random bits included; windows equal the full call;
the fused transform equals transform-then-quantize), the round-to-nearest
error bound, exact round trips of representable tensors, and zero-code counts
of tensors whose zero codes are known by construction.
"""
import numpy as np
import pytest

import oracle as O
from _golden import e2m1_values, quant_example

E2M1 = e2m1_values()


def _codes_unpacked(codes):
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))


def test_worked_example_row():
    ex = quant_example("quant_unit_scale_row.txt")
    q = O.quantize(ex["input"][None, :], "row")
    assert np.array_equal(q["codes"][0], ex["codes"])
    assert np.array_equal(q["scales"][0], ex["scales"])
    assert q["amax"] == ex["amax"] and q["g"] == ex["g"]


def test_worked_example_col_and_2d():
    ex = quant_example("quant_unit_scale_row.txt")
    col = ex["input"].reshape(32, 1)
    x = np.zeros((32, 2), dtype=np.float32)
    x[:, 0] = ex["input"]
    q = O.quantize(x, "col")
    cu = _codes_unpacked(q["codes"])
    want = _codes_unpacked(ex["codes"][None, :])[0]
    assert np.array_equal(cu[:, 0], want)
    assert np.array_equal(q["scales"][:, 0], ex["scales"])
    # 2D: a 16x16 tile holding the amax and a tile whose max is 6.
    x2 = np.zeros((16, 32), dtype=np.float32)
    x2[0, 0] = 2688.0
    x2[:, 16:] = np.resize(ex["input"][16:], (16, 16))
    q2 = O.quantize(x2, "2d")
    assert np.array_equal(q2["scales"], np.array([[0x7E, 0x38]], dtype=np.uint8))
    c2 = _codes_unpacked(q2["codes"])
    assert np.array_equal(c2[0, 16:], want[16:])


def test_global_scales_closed_form():
    for a in [1.0, 2688.0, 448.0, 3.75, 1e-20, 1e20]:
        S, k, g = O.global_scales(a)
        assert S == np.float32(2688.0) / np.float32(a)
        assert k == S / np.float32(6.0)
        assert g == np.float32(a) / np.float32(2688.0)
    assert O.global_scales(0.0) == (1.0, np.float32(1.0) / np.float32(6.0), 0.0)
    S, _, _ = O.global_scales(1e-40)
    assert S == np.finfo(np.float32).max


def test_unit_k_trick_block_scales_are_e4m3_of_block_max():
    # A = 448 gives S = 6, k = 1, so each block scale is E4M3(block max).
    rng = np.random.default_rng(3)
    mx = np.concatenate([[448.0], rng.random(63) * 448.0]).astype(np.float32)
    x = np.zeros((64, 16), dtype=np.float32)
    x[:, 5] = mx
    q = O.quantize(x, "row")
    import torch
    ref = torch.from_numpy(mx).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q["scales"][:, 0], ref)


@pytest.mark.parametrize("block", ["row", "col", "2d"])
def test_amax_element_gets_top_code_and_scale(block):
    rng = np.random.default_rng(4)
    for t in range(5):
        x = (rng.standard_normal((64, 64)) * 10 ** rng.uniform(-6, 6)).astype(np.float32)
        i, j = rng.integers(0, 64, 2)
        x[i, j] = -np.abs(x).max() * 1.5
        q = O.quantize(x, block)
        cu = _codes_unpacked(q["codes"])
        assert cu[i, j] == 0xF
        sc = q["scales"]
        s = sc[i, j // 16] if block == "row" else sc[i // 16, j] if block == "col" else sc[i // 16, j // 16]
        assert s == 0x7E


def _rne_error_ok(x, xh, q, block):
    """|x - x_hat| <= half a grid step at x's magnitude, times d*g, with slack
    for the two fp32 roundings of the encode and decode."""
    rows, cols = x.shape
    for r in range(rows):
        for c in range(cols):
            if block == "row":
                s = q["scales"][r, c // 16]
            elif block == "col":
                s = q["scales"][r // 16, c]
            else:
                s = q["scales"][r // 16, c // 16]
            d = O.e4m3_decode(s) * float(q["g"])
            if d == 0:
                assert xh[r, c] == 0
                continue
            m = abs(x[r, c]) / d
            step = 0.5 if m < 2 else 1.0 if m < 4 else 2.0
            bound = (step / 2) * d if m <= 6 else (abs(x[r, c]) - 6 * d)
            assert abs(x[r, c] - xh[r, c]) <= bound * (1 + 1e-5) + 1e-6 * abs(x[r, c]), (r, c)


@pytest.mark.parametrize("block", ["row", "col", "2d"])
def test_rne_error_bound(block):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    x[3, :] *= 1e-3
    q = O.quantize(x, block)
    xh = O.dequantize(q["codes"], q["scales"], q["g"], block)
    _rne_error_ok(x, xh, q, block)


def test_representable_tensor_round_trips():
    # Blocks built as (E2M1 value) * (E4M3 value) with one block at 2688
    # (S = 1, g = 1) round-trip exactly through quantize + dequantize.
    rng = np.random.default_rng(6)
    grid = np.array([E2M1[c] for c in range(16)], dtype=np.float32)
    x = np.zeros((8, 64), dtype=np.float32)
    e4 = [0.015625, 0.125, 0.875, 1.0, 1.125, 3.5, 13.0, 240.0]
    for r in range(8):
        for b in range(4):
            codes = rng.integers(0, 16, 16)
            codes[rng.integers(0, 16)] = 7  # block max = 6 * scale
            x[r, 16 * b:16 * b + 16] = grid[codes] * np.float32(e4[(r + b) % 8])
    x[0, 0:16] = 0
    x[0, 0] = 2688.0
    q = O.quantize(x, "row")
    assert q["g"] == 1.0
    xh = O.dequantize(q["codes"], q["scales"], q["g"], "row")
    assert np.array_equal(xh, x)


@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
def test_col_equals_transposed_row(rounding):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((48, 32)).astype(np.float32)
    qc = O.quantize(x, "col", rounding=rounding, seed=11, offset=3)
    qr = O.quantize(np.ascontiguousarray(x.T), "row", rounding=rounding, seed=11, offset=3)
    assert np.array_equal(_codes_unpacked(qc["codes"]), _codes_unpacked(qr["codes"]).T)
    assert np.array_equal(qc["scales"], qr["scales"].T)


def test_row_window_equals_full_call():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    full = O.quantize(x, "row", rounding=O.SR, seed=5)
    part = O.quantize(x, "row", rounding=O.SR, seed=5, amax=full["amax"], row_begin=16, row_end=48)
    assert np.array_equal(part["codes"][16:48], full["codes"][16:48])
    assert np.array_equal(part["scales"][16:48], full["scales"][16:48])
    assert not part["codes"][:16].any()


@pytest.mark.parametrize("block", ["row", "col"])
def test_fused_rht_equals_transform_then_quantize(block):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    mask = 0x6C3A
    fused = O.quantize(x, block, rounding=O.SR, seed=1, rht_mask=mask)
    y = O.rht16(x, block, mask)
    two = O.quantize(y, block, rounding=O.SR, seed=1)
    for k in ("codes", "scales"):
        assert np.array_equal(fused[k], two[k])
    assert fused["amax"] == np.abs(y).max()


def test_batched_2d_slices_are_independent():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((3, 32, 48)) * np.array([1, 100, 1e-3])[:, None, None]).astype(np.float32)
    qb = O.quantize(w, "2d")
    for s in range(3):
        q = O.quantize(w[s], "2d")
        assert np.array_equal(qb["codes"][s], q["codes"])
        assert np.array_equal(qb["scales"][s], q["scales"])
        assert qb["g"][s] == q["g"]


def test_zero_tensor_and_negative_zero():
    x = np.zeros((16, 32), dtype=np.float32)
    x[1, 3] = -0.0
    q = O.quantize(x, "row")
    assert q["amax"] == 0 and q["g"] == 0
    cu = _codes_unpacked(q["codes"])
    assert cu[1, 3] == 8 and cu.sum() == 8
    assert not q["scales"].any()


def test_bf16_input_matches_fp32_of_same_values():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: exact bf16 values
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    a = O.quantize(bits, "row")
    b = O.quantize(xf, "row")
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_shape_errors():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((16, 24), dtype=np.float32), "row")
    with pytest.raises(ValueError):
        O.quantize(np.zeros((24, 32), dtype=np.float32), "col")
    with pytest.raises(ValueError):
        O.quantize(np.zeros((16, 32), dtype=np.float32), "2d", rounding=O.SR)


@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
def test_zero_codes_row_and_col_count_exact_zeros(rounding):
    """Exact zeros always encode to magnitude 0 (their fraction is 0, so
    stochastic rounding never rounds them up); every other element equals its
    block's max in magnitude and takes a nonzero code.  So the count is the
    number of exact zeros, whatever the random bits."""
    rng = np.random.default_rng(21)
    rows, cols = 64, 96
    x = np.where(rng.random((rows, cols)) < 0.3, 0.0,
                 np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0)).astype(np.float32)
    # one block of each kind entirely zero, one with a lone nonzero element
    x[0, :16] = 0.0
    x[16:32, 5] = 0.0
    x[2, 16:32] = 0.0
    x[2, 20] = 3.0  # a lone nonzero element: its block's max
    zeros = int(np.count_nonzero(x == 0.0))
    for block in ("row", "col"):
        # make every nonzero element of a block equal the block max in
        # magnitude (zeros stay zeros)
        y = x.copy()
        if block == "row":
            b = y.reshape(rows, cols // 16, 16)
        else:
            b = y.reshape(rows // 16, 16, cols).transpose(0, 2, 1)
        m = np.abs(b).max(axis=-1, keepdims=True)
        b[...] = np.sign(b) * m
        q = O.quantize(y, block, rounding=rounding, seed=5)
        assert O.zero_codes(q["codes"]) == zeros, block


def test_zero_codes_col_with_transform():
    """With the 16-point transform a block with one nonzero value v becomes
    +-v/4 in all 16 places (every Hadamard column is +-1), all at the block
    max: no zero codes.  An all-zero block stays zero: 16 zero codes."""
    rows, cols = 64, 64
    x = np.zeros((rows, cols), dtype=np.float32)
    rng = np.random.default_rng(3)
    zero_blocks = 0
    for gb in range(rows // 16):
        for c in range(cols):
            if rng.random() < 0.4:
                zero_blocks += 1
            else:
                x[16 * gb + rng.integers(16), c] = np.float32(rng.choice([-2.0, 0.5, 7.0]))
    for rounding in (O.RNE, O.SR):
        q = O.quantize(x, "col", rounding=rounding, seed=9, rht_mask=0xB6D1)
        assert O.zero_codes(q["codes"]) == 16 * zero_blocks


def test_zero_codes_counts_both_nibbles():
    codes = np.array([[0x00, 0x88, 0x80, 0x17, 0x9F]], dtype=np.uint8)
    # nibbles: 0,0 | 8,8 | 0,8 | 7,1 | F,9 -> zero magnitude: 6
    assert O.zero_codes(codes) == 6
