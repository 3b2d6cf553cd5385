"""GPU parity: fp32 -> fp16 stochastic rounding of an SSM-state cache, bit for
bit against the oracle (Super report summary 4.3: FP16 with Philox<5>
stochastic rounding), called through the C ABI."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from _gpu import assert_same, device

pytestmark = pytest.mark.gpu


def _values(n, seed):
    """Magnitudes over 10^-9 .. 10^5 (fp16 subnormals, normals and
    saturation), plus exact fp16 values, the range edges, NaN, +-inf, +-0."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, 5, n)).astype(np.float32)
    k = min(n, 64)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65520.0, -70000.0,
                        2.0 ** -14, -(2.0 ** -24), 2.0 ** -25, 1.0 + 2.0 ** -11, 2.0 ** -149,
                        3.0, -1.5, 2.0 ** -14 - 2.0 ** -30], dtype=np.float32)
    idx = rng.choice(n, size=min(k, len(special)), replace=False)
    x[idx] = special[:len(idx)]
    return x


def _check(x, seed, offset=0, rounds=5):
    dev = device()
    t = torch.from_numpy(x).to(dev)
    y = nv.sr_fp16(t, nv.Philox(seed, offset, rounds))
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.sr_fp16(x, seed, offset, rounds)
    assert_same(got, want, "fp16 bits")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4097, 65539, 1 << 20])
def test_sr_fp16_ragged(n):
    _check(_values(n, n), seed=99 + n, offset=n)


@pytest.mark.parametrize("rounds", [1, 5, 10, 16])
def test_sr_fp16_streams(rounds):
    _check(_values(20000, 3), seed=2**63 + 17, offset=2**40 + 5, rounds=rounds)


def test_sr_fp16_empty():
    dev = device()
    y = nv.sr_fp16(torch.empty(0, dtype=torch.float32, device=dev), nv.Philox(1))
    assert y.numel() == 0


def test_full_ssm_state():
    """A decode batch's SSM states, 64 x 128 x 64 x 128 fp32 (2^26 elements):
    every element against the oracle."""
    dev = device()
    shape = (64, 128, 64, 128)
    rng = np.random.default_rng(2026)
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-6, 2, shape)).astype(np.float32)
    t = torch.from_numpy(x).to(dev)
    y = nv.sr_fp16(t, nv.Philox(5))
    got = y.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    want = O.sr_fp16(x, 5)
    assert_same(got, want, "fp16 bits")
