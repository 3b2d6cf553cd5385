"""GPU parity: NT GEMMs with few rows of A (decode-like shapes, M <= 64), which
run on the split-K kernel, and the post-training-quantization decode path
(Super report summary section 4.2: MSE-calibrated weight scales, activations
quantized at run time with max-based scales, W4A4 GEMM), against the
oracle's fp64 reference.  Metric and bar as in the other GEMM tests:
max |C - R| / D <= 1e-3 on the fp32 result; bf16 output is the RNE rounding
of the fp32 result; the exact special case is bit-exact."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from nvfp4_block_scaled_07_amd import synth
from _gpu import device, device_input, make_input, to_np

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _check(qa, qb, M, N, K, c):
    R, D = O.gemm_full("N", "T", M, N, K, to_np(qa), to_np(qb))
    err = O.gemm_rel_err(c.float().cpu().numpy(), R, D)
    assert err <= TOL, f"NT {M}x{N}x{K}: max |C-R|/D = {err:.3e}"


def _bf16_is_rne(c_bf16, c_fp32):
    assert torch.equal(c_bf16.view(torch.int16), c_fp32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("M", [1, 2, 7, 16, 31, 32, 33, 48, 63, 64])
@pytest.mark.parametrize("b_block", ["row", "2d"])
def test_small_m_nt(M, b_block):
    """Ragged M on both row-tile variants (<= 32 and <= 64 rows), ragged N
    (a partial 32-column tile) and K = 640: ten 64-k groups over eight waves,
    so the waves' shares are uneven and two of them hold one group."""
    N, K = 272, 640
    dev = device()
    a = make_input("normal", (M, K), 40 + M)
    b = (make_input("normal", (N, K), 41 + M) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_1d(device_input(a, "bf16", dev)[0], "row")
    tb = device_input(b, "bf16", dev)[0]
    qb = nv.quantize_2d(tb) if b_block == "2d" else nv.quantize_1d(tb, "row")
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    _check(qa, qb, M, N, K, c)
    _bf16_is_rne(nv.gemm("N", "T", qa, qb, out_dtype=torch.bfloat16), c)


@pytest.mark.parametrize("K", [64, 128, 64 * 7, 4096])
def test_small_m_k_splits(K):
    """K from one group (seven idle waves) to 64 groups."""
    M, N = 24, 96
    dev = device()
    a = make_input("laplace_zeros", (M, K), 7)
    b = (make_input("normal", (N, K), 8) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_1d(device_input(a, "bf16", dev)[0], "row")
    qb = nv.quantize_2d(device_input(b, "bf16", dev)[0])
    _check(qa, qb, M, N, K, nv.gemm("N", "T", qa, qb, out_dtype=torch.float32))


@pytest.mark.parametrize("M", [65, 100, 128, 200, 300, 512])
@pytest.mark.parametrize("b_block", ["row", "2d"])
def test_small_m_row_blocks(M, b_block):
    """Beyond 64 rows (with few 256 x 256 tiles) the small-M kernel takes row
    blocks of 64: ragged last blocks, both weight block kinds, bf16 output
    the RNE of the fp32 one."""
    N, K = 160, 384
    dev = device()
    a = make_input("normal", (M, K), 70 + M)
    b = (make_input("normal", (N, K), 71 + M) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_1d(device_input(a, "bf16", dev)[0], "row")
    tb = device_input(b, "bf16", dev)[0]
    qb = nv.quantize_2d(tb) if b_block == "2d" else nv.quantize_1d(tb, "row")
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    _check(qa, qb, M, N, K, c)
    _bf16_is_rne(nv.gemm("N", "T", qa, qb, out_dtype=torch.bfloat16), c)
    c0 = torch.ones_like(c)
    nv.gemm("N", "T", qa, qb, out=c0, accumulate=True)
    assert torch.equal(c0.view(torch.int32), (torch.ones_like(c) + c).view(torch.int32))


def test_small_m_row_blocks_2d_activations():
    M, N, K = 208, 96, 256
    dev = device()
    a = make_input("normal", (M, K), 9)
    b = (make_input("normal", (N, K), 10) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_2d(device_input(a, "fp32", dev)[0])
    qb = nv.quantize_1d(device_input(b, "fp32", dev)[0], "row")
    _check(qa, qb, M, N, K, nv.gemm("N", "T", qa, qb, out_dtype=torch.float32))


def test_small_m_2d_activation_operand():
    """A 16x16-block A operand (rows % 16 == 0) on the small-M path."""
    M, N, K = 48, 160, 256
    dev = device()
    a = make_input("normal", (M, K), 3)
    b = (make_input("normal", (N, K), 4) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_2d(device_input(a, "fp32", dev)[0])
    qb = nv.quantize_1d(device_input(b, "fp32", dev)[0], "row")
    _check(qa, qb, M, N, K, nv.gemm("N", "T", qa, qb, out_dtype=torch.float32))


def test_small_m_exact_special_case():
    """Grid-valued operands with a 6 * 448 in every block: unit scales, every
    partial sum exact in fp32 in any order, so C equals the fp64 product."""
    dev = device()
    rng = np.random.default_rng(77)
    M, N, K = 20, 96, 1024
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)

    def draw(r, cc):
        v = grid[rng.integers(0, 8, (r, cc))] * np.where(rng.random((r, cc)) < .5, -1, 1)
        v = v.astype(np.float32)
        v[:, ::16] = 6.0
        return v * np.float32(448)

    a, b = draw(M, K), draw(N, K)
    qa = nv.quantize_1d(torch.from_numpy(a).to(dev), "row")
    qb = nv.quantize_1d(torch.from_numpy(b).to(dev), "row")
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(c.astype(np.float64), a.astype(np.float64) @ b.astype(np.float64).T)


def test_small_m_deterministic_and_matches_tiled_within_bound():
    """Repeated calls give the same bits; rows computed by the small-M kernel
    agree with the same rows of a 1024-row product (tiled kernel) to the bar."""
    M, N, K = 1024, 512, 2048
    dev = device()
    a = make_input("normal", (M, K), 12)
    b = (make_input("normal", (N, K), 13) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_1d(device_input(a, "bf16", dev)[0], "row")
    qb = nv.quantize_2d(device_input(b, "bf16", dev)[0])
    full = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    sub = nv.QTensor(qa.codes[:40], qa.scales[:40], qa.global_dec, qa.amax, 40, K, "row")
    c1 = nv.gemm("N", "T", sub, qb, out_dtype=torch.float32)
    for _ in range(3):
        assert torch.equal(c1, nv.gemm("N", "T", sub, qb, out_dtype=torch.float32))
    R, D = O.gemm_full("N", "T", 40, N, K, to_np(sub), to_np(qb))
    assert O.gemm_rel_err(c1.cpu().numpy(), R, D) <= TOL
    assert O.gemm_rel_err(full[:40].cpu().numpy(), R, D) <= TOL


def test_ptq_decode_small_exact_path():
    """The whole PTQ decode path at a small size: weight quantized with MSE
    scales (checked block for block against the oracle), activations with
    dynamic max-based ROW scales (bit-exact), then the GEMM (to the bar)."""
    M, N, K = 9, 192, 512
    dev = device()
    w = synth.normal((N, K), 0.02, 5)
    x = synth.normal((M, K), 1.0, 6)
    tw, wo = device_input(w, "bf16", dev)
    tx, xo = device_input(x, "bf16", dev)
    qw = nv.quantize_mse(tw)
    qx = nv.quantize_1d(tx, "row")
    gw, gx = to_np(qw), to_np(qx)
    rw, rx = O.quantize_mse(wo), O.quantize(xo, "row")
    for k in ("codes", "scales"):
        assert np.array_equal(gw[k], rw[k]), k
        assert np.array_equal(gx[k], rx[k]), k
    _check(qx, qw, M, N, K, nv.gemm("N", "T", qx, qw, out_dtype=torch.float32))


@pytest.mark.parametrize("M", [1, 32, 64])
def test_full_ptq_decode_super_sampled(M):
    """Super-width decode: W [6144 x 6144] N(0, 0.02) with MSE scales, a batch
    of M tokens quantized at run time; every output of two rows and two
    columns plus 4096 random outputs against the oracle."""
    dev = device()
    N = K = 6144
    w = synth.normal((N, K), 0.02, 2)
    x = synth.normal((M, K), 1.0, 100 + M)
    qw = nv.quantize_mse(device_input(w, "bf16", dev)[0])
    qx = nv.quantize_1d(device_input(x, "bf16", dev)[0], "row")
    c = nv.gemm("N", "T", qx, qw, out_dtype=torch.bfloat16)
    c32 = nv.gemm("N", "T", qx, qw, out_dtype=torch.float32)
    _bf16_is_rne(c, c32)
    rng = np.random.default_rng(M)
    ii = np.concatenate([np.zeros(N, int), np.full(N, M - 1), np.arange(M), np.arange(M),
                         rng.integers(0, M, 4096)])
    jj = np.concatenate([np.arange(N), np.arange(N), np.zeros(M, int), np.full(M, N - 1),
                         rng.integers(0, N, 4096)])
    R, D = O.gemm_entries("N", "T", M, N, K, to_np(qx), to_np(qw), ii, jj)
    err = O.gemm_rel_err(c32[ii, jj].cpu().numpy(), R, D)
    assert err <= TOL, f"sampled max |C-R|/D = {err:.3e}"
