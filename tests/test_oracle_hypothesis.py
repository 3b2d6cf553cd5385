"""Properties of the oracle's quantizer over hypothesis-drawn shapes, value
scales, Philox streams and transform masks (derandomized, so every run draws
the same cases):

* COL blocks of X are the transposed ROW blocks of X^T, codes, scales and
  stochastic-rounding bits included (the two block ids coincide);
* with the transform fused, the result equals quantizing the transformed
  tensor, and the tensor amax is the transformed tensor's;
* dequantizing an RNE quantization lands every element within half a grid
  step (times the block's decoded scale) of its input, or at the saturated
  6 * d for elements that the block scale clips (the E4M3 rounding of the
  scale can put an element just above 6 d).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle as O

SETTINGS = dict(max_examples=60, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow])


def _input(rows, cols, seed, log_scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * 10.0 ** log_scale).astype(np.float32)


def _unpack(c):
    return np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[0], -1)


@settings(**SETTINGS)
@given(r32=st.integers(1, 6), c32=st.integers(1, 6), seed=st.integers(0, 2**20),
       log_scale=st.integers(-30, 30), sr=st.booleans(), pseed=st.integers(0, 2**40))
def test_col_is_transposed_row(r32, c32, seed, log_scale, sr, pseed):
    rows, cols = 32 * r32, 32 * c32
    x = _input(rows, cols, seed, log_scale)
    rnd = O.SR if sr else O.RNE
    qc = O.quantize(x, "col", rounding=rnd, seed=pseed, offset=7)
    qr = O.quantize(np.ascontiguousarray(x.T), "row", rounding=rnd, seed=pseed, offset=7)
    assert np.array_equal(_unpack(qc["codes"]), _unpack(qr["codes"]).T)
    assert np.array_equal(qc["scales"], qr["scales"].T)
    assert qc["amax"] == qr["amax"] and qc["g"] == qr["g"]


@settings(**SETTINGS)
@given(r16=st.integers(1, 8), c32=st.integers(1, 6), seed=st.integers(0, 2**20),
       mask=st.integers(0, 0xFFFF), block=st.sampled_from(["row", "col"]),
       pseed=st.integers(0, 2**40))
def test_fused_transform_equals_transform_then_quantize(r16, c32, seed, mask, block, pseed):
    rows, cols = 16 * r16, 32 * c32
    x = _input(rows, cols, seed, 0)
    fused = O.quantize(x, block, rounding=O.SR, seed=pseed, rht_mask=mask)
    y = O.rht16(x, block, mask)
    two = O.quantize(y, block, rounding=O.SR, seed=pseed)
    for k in ("codes", "scales"):
        assert np.array_equal(fused[k], two[k])
    assert fused["amax"] == np.abs(y).max()


@settings(**SETTINGS)
@given(r16=st.integers(1, 8), c32=st.integers(1, 6), seed=st.integers(0, 2**20),
       log_scale=st.integers(-20, 20))
def test_rne_error_within_half_a_step(r16, c32, seed, log_scale):
    rows, cols = 16 * r16, 32 * c32
    x = _input(rows, cols, seed, log_scale)
    q = O.quantize(x, "row")
    xh = O.dequantize(q["codes"], q["scales"], q["g"], "row").astype(np.float64)
    d = np.repeat(np.array([[O.e4m3_decode(int(e)) for e in row] for row in q["scales"]]),
                  16, axis=1) * float(q["g"])
    y = np.abs(x.astype(np.float64)) / np.where(d > 0, d, np.inf)  # position on the E2M1 grid
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(xh - x)
    # half a step of the grid at y (times d), relative slack for the fp32 products
    bound = (step / 2) * d * (1 + 2.0 ** -20) + 1e-45
    clipped = y > 6
    ok = (err <= bound) | (clipped & (np.abs(np.abs(xh) - 6 * d) <= 6 * d * 2.0 ** -20))
    assert ok.all(), (x[~ok][:4], xh[~ok][:4])
    assert set(np.unique(np.round(np.abs(xh[d > 0]) / d[d > 0], 6))) <= set(grid)
