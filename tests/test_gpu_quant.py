"""GPU parity: quantizers, Hadamard transform and dequantizer, bit-exact
against the CPU oracle (codes, scale bytes, amax, decode scale), called
through the C ABI.

Small cases span several workgroups and ragged tails with every combination
of block axis, rounding, transform and input type; full-size cases use the
workloads' own shapes and distributions.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from nvfp4_block_scaled_07_amd import synth
from _gpu import assert_same, device, device_input, make_input, to_np

pytestmark = pytest.mark.gpu

SHAPES = [(16, 32), (48, 96), (1000, 64), (64, 2080), (272, 160)]


def _check_1d(x, dtype, axis, rounding, mask, seed=0, offset=0, rounds=5, amax=None):
    dev = device()
    t, xo = device_input(x, dtype, dev)
    rng = nv.Philox(seed, offset, rounds) if rounding == "sr" else None
    a_t = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=dev)
    q = nv.quantize_1d(t, axis, rounding, rng, mask, amax=a_t)
    got = to_np(q)
    ref = O.quantize(xo, axis, rounding=O.SR if rounding == "sr" else O.RNE, seed=seed,
                     offset=offset, rounds=rounds, rht_mask=mask, amax=amax)
    assert_same(got["amax"][0], ref["amax"], "amax")
    assert_same(np.float32(got["g"]), ref["g"], "global decode scale")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")
    return q, ref


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_1d_small(shape, axis, rounding, rht, dtype):
    if axis == "col" and shape[0] % 16:
        # COL blocks need rows % 16 == 0: the call is rejected before launch.
        t, _ = device_input(make_input("normal", shape, seed=1), dtype, device())
        with pytest.raises(nv.NVFP4Error) as e:
            nv.quantize_1d(t, axis, rounding, nv.Philox(1) if rounding == "sr" else None,
                           0xA5C3 if rht else -1)
        assert e.value.status == nv.NVFP4_ERR_SHAPE
        return
    x = make_input("normal", shape, seed=shape[0] * 7 + shape[1])
    _check_1d(x, dtype, axis, rounding, 0xA5C3 if rht else -1, seed=123, offset=9)


@pytest.mark.parametrize("kind", ["laplace_zeros", "wide", "tiny", "zeros"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quantize_1d_distributions(kind, axis, rounding):
    x = make_input(kind, (64, 256), seed=5)
    _check_1d(x, "bf16", axis, rounding, 0x1234 if axis == "col" else -1, seed=77)
    _check_1d(x, "fp32", axis, rounding, -1, seed=77)


@pytest.mark.parametrize("rows", [1, 5, 64, 66, 130])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_1d_row_launch_paths(rows, rounding, dtype):
    """ROW quantization of tensors up to 64 Ki elements runs in one workgroup
    (tensor amax and encode in one launch), larger ones in the multi-
    workgroup kernels: rows of 1024 columns on both sides of the boundary
    (64 rows = 65536 elements) match the oracle bit for bit, computed amax
    and supplied amax alike."""
    x = make_input("normal", (rows, 1024), seed=500 + rows)
    _check_1d(x, dtype, "row", rounding, -1, seed=rows)
    _check_1d(x, dtype, "row", rounding, -1, seed=rows, amax=3.25)


def test_quantize_1d_philox_rounds_and_offsets():
    x = make_input("normal", (32, 128), seed=3)
    for rounds in (1, 5, 10, 16):
        _check_1d(x, "bf16", "row", "sr", -1, seed=2**40 + 3, offset=2**33 + 1, rounds=rounds)
    _check_1d(x, "bf16", "col", "sr", 0xFFFF, seed=1, offset=0, rounds=10)


def test_quantize_1d_amax_input():
    x = make_input("normal", (64, 128), seed=4)
    # a supplied amax larger than the data: smaller codes, still bit-exact
    _check_1d(x, "bf16", "row", "rne", -1, amax=50.0)
    _check_1d(x, "fp32", "col", "sr", 0x00FF, amax=12.5)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mask", [0x0000, 0xA5C3])
def test_quantize_1d_rht_tail_block(dtype, mask):
    """Zeros except the last 8 elements (the second half of the last block):
    the transform of that block, [0 | v], has max |H8 v|/4; a pass that paired
    the last chunk with a copy of itself would see [v | v] and twice that."""
    x = np.zeros((16, 64), dtype=np.float32)
    x[15, 56:] = np.array([3.0, -1.0, 2.5, 0.25, -7.0, 1.5, 0.5, -2.0], dtype=np.float32)
    _check_1d(x, dtype, "row", "rne", mask)


# Mid-size tensors (several amax trips per workgroup and a ragged last trip).
@pytest.mark.parametrize("rounding,rht", [("rne", False), ("sr", False), ("rne", True),
                                          ("sr", True)])
def test_quantize_1d_row_large(rounding, rht):
    x = make_input("laplace_zeros", (4096, 4160), seed=41)
    _check_1d(x, "bf16", "row", rounding, 0x9C31 if rht else -1, seed=9, offset=4)


def test_quantize_1d_row_large_amax_input():
    x = make_input("normal", (4096, 4096), seed=42)
    _check_1d(x, "bf16", "row", "sr", -1, seed=3, amax=40.0)


@pytest.mark.parametrize("amax", [None, 0.5])
def test_quantize_2d_large(amax):
    dev = device()
    x = make_input("normal", (4096, 4160), seed=43) * np.float32(0.02)
    t, xo = device_input(x, "bf16", dev)
    a_t = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=dev)
    q = nv.quantize_2d(t, amax=a_t)
    got = to_np(q)
    ref = O.quantize(xo, "2d", amax=amax)
    assert_same(got["amax"], np.atleast_1d(np.float32(ref["amax"])), "amax")
    assert_same(q.global_dec.cpu().numpy(), np.atleast_1d(np.float32(ref["g"])), "g")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


def test_quantize_1d_empty():
    dev = device()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    q = nv.quantize_1d(x, "row")
    assert q.codes.numel() == 0


@pytest.mark.parametrize("batch,rows,cols", [(1, 16, 32), (1, 48, 96), (3, 32, 160),
                                             (5, 272, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_2d_small(batch, rows, cols, dtype):
    dev = device()
    x = make_input("normal", (batch, rows, cols), seed=batch + rows)
    x *= np.float32(10.0) ** np.arange(batch, dtype=np.float32)[:, None, None]
    t, xo = device_input(x, dtype, dev)
    q = nv.quantize_2d(t)
    got = to_np(q)
    ref = O.quantize(xo, "2d")
    assert_same(got["amax"], ref["amax"], "amax")
    assert_same(q.global_dec.cpu().numpy(), ref["g"], "g")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rht16_standalone(axis, dtype):
    dev = device()
    x = make_input("normal", (48, 96), seed=8)
    t, xo = device_input(x, dtype, dev)
    y = nv.rht16(t, axis, 0x5A5A)
    assert_same(y.cpu().numpy(), O.rht16(xo, axis, 0x5A5A), "rht16")


@pytest.mark.parametrize("axis", ["row", "col", "2d"])
def test_dequantize(axis):
    dev = device()
    x = make_input("normal", (64, 96), seed=9)
    t, xo = device_input(x, "bf16", dev)
    q = nv.quantize_2d(t) if axis == "2d" else nv.quantize_1d(t, axis, "sr", nv.Philox(4))
    got = nv.dequantize(q, index=None).cpu().numpy()
    r = to_np(q)
    want = O.dequantize(r["codes"], r["scales"], r["g"] if axis != "2d" else r["g"], axis)
    assert_same(got.view(np.uint32), want.view(np.uint32), "dequantized bits")


def test_tiny_config():
    """X fp32 [256x512] ~N(0,1), seed 0, 1x16 RNE, dequantize."""
    dev = device()
    x = synth.normal((256, 512), 1.0, 0)
    q, ref = _check_1d(x, "fp32", "row", "rne", -1)
    got = nv.dequantize(q).cpu().numpy()
    want = O.dequantize(ref["codes"], ref["scales"], ref["g"], "row")
    assert_same(got.view(np.uint32), want.view(np.uint32), "dequantized bits")


# ---- both quantizations of a gradient from one read -------------------------------------------------
def _check_dual(x, dtype, mask, seeds=(11, 12), offsets=(3, 0), rounds=(5, 5), amax=None):
    dev = device()
    t, xo = device_input(x, dtype, dev)
    rr = nv.Philox(seeds[0], offsets[0], rounds[0])
    rc = nv.Philox(seeds[1], offsets[1], rounds[1])
    a_t = None if amax is None else torch.tensor(amax, dtype=torch.float32, device=dev)
    qr, qc, z = nv.quantize_dual(t, rr, rc, mask, amax=a_t)
    ref_r = O.quantize(xo, "row", rounding=O.SR, seed=seeds[0], offset=offsets[0],
                       rounds=rounds[0], amax=None if amax is None else amax[0])
    ref_c = O.quantize(xo, "col", rounding=O.SR, seed=seeds[1], offset=offsets[1],
                       rounds=rounds[1], rht_mask=mask, amax=None if amax is None else amax[1])
    for got, ref, name in ((to_np(qr), ref_r, "row"), (to_np(qc), ref_c, "col")):
        assert_same(got["amax"][0], ref["amax"], name + " amax")
        assert_same(np.float32(got["g"]), ref["g"], name + " g")
        assert_same(got["scales"], ref["scales"], name + " scales")
        assert_same(got["codes"], ref["codes"], name + " codes")
    zeros = z.cpu().numpy()
    assert zeros[0] == O.zero_codes(ref_r["codes"]) and zeros[1] == O.zero_codes(ref_c["codes"])
    return qr, qc, zeros


@pytest.mark.parametrize("shape", [(16, 32), (48, 96), (272, 160), (64, 2080), (1008, 64)])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_dual_small(shape, rht, dtype):
    """Several workgroups and a ragged last one (units not a multiple of 256)."""
    x = make_input("laplace_zeros", shape, seed=shape[0] + 3 * shape[1])
    _check_dual(x, dtype, 0x6C2B if rht else -1)


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny", "zeros"])
def test_quantize_dual_distributions(kind):
    x = make_input(kind, (64, 256), seed=17)
    _check_dual(x, "bf16", 0x0F0F, seeds=(2**40 + 1, 7), offsets=(2**33, 5), rounds=(10, 1))


def test_quantize_dual_amax_input():
    x = make_input("normal", (96, 128), seed=6)
    _check_dual(x, "bf16", 0x1111, amax=[9.5, 3.25])
    _check_dual(x, "fp32", -1, amax=[0.5, 40.0])


def test_quantize_dual_empty():
    dev = device()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    qr, qc, z = nv.quantize_dual(x, nv.Philox(1), nv.Philox(2), 0x5)
    assert qr.codes.numel() == 0 and qc.codes.numel() == 0


# ---- full-size workloads -------------------------------------------------------------------------
def test_full_fprop_super_inputs():
    w = synth.WORKLOADS["fprop_super"]
    dev = device()
    x = synth.normal((w["M"], w["K"]), w["x_std"], w["x_seed"])
    _check_1d(x, "bf16", "row", "rne", -1)
    wt = synth.normal((w["N"], w["K"]), w["w_std"], w["w_seed"])
    t, xo = device_input(wt, "bf16", dev)
    q = nv.quantize_2d(t)
    got = to_np(q)
    ref = O.quantize(xo, "2d")
    assert_same(got["scales"], ref["scales"], "W scales")
    assert_same(got["codes"], ref["codes"], "W codes")
    assert_same(np.float32(got["g"]), ref["g"], "W g")


def test_full_wgrad_super_inputs():
    w = synth.WORKLOADS["wgrad_super"]
    shape = (w["tokens"], w["out"])
    dy = synth.laplace(shape, w["dy_b"], w["dy_seed"], w["zero_frac"], w["zero_seed"])
    mask = synth.rht_mask(w["mask_seed"])
    q, ref = _check_1d(dy, "bf16", "col", "sr", mask, seed=w["philox_seed"])
    zero_codes = (np.stack([ref["codes"] & 7, (ref["codes"] >> 4) & 7]) == 0).mean()
    print(f"dY zero-code fraction {zero_codes:.4f}")
    x = synth.normal((w["tokens"], w["inp"]), 1.0, w["x_seed"])
    _check_1d(x, "bf16", "col", "rne", mask)


def test_full_ultra_dgrad_input():
    w = synth.WORKLOADS["ultra"]
    dy = synth.laplace((w["M"], w["N"]), w["dy_b"], w["dy_seed"])
    _check_1d(dy, "bf16", "row", "sr", -1, seed=w["philox_seed"])


def test_full_grouped_super_weights_sampled():
    """W [512 x 2688 x 1024] 2D-quantized in one call; per-slice amax and g
    for all 512 experts, codes and scales for a sample of slices."""
    w = synth.WORKLOADS["grouped_super"]
    dev = device()
    shape = (w["experts"], w["hidden"], w["latent"])
    x = synth.normal(shape, w["w_std"], w["w_seed"])
    t, xo = device_input(x, "bf16", dev)
    del x
    q = nv.quantize_2d(t)
    torch.cuda.synchronize()
    ref_amax = O.amax(xo, "2d")
    assert_same(q.amax.cpu().numpy(), ref_amax, "per-expert amax")
    g = q.global_dec.cpu().numpy()
    for e in [0, 1, 255, 511]:
        ref = O.quantize(xo[e], "2d")
        assert_same(q.codes[e].cpu().numpy(), ref["codes"], f"codes of expert {e}")
        assert_same(q.scales[e].cpu().numpy(), ref["scales"], f"scales of expert {e}")
        assert g[e] == ref["g"]


def test_full_wgrad_super_dy_dual():
    """dY of the wgrad Super workload [8192 x 6144] (Laplace, 7% exact zeros):
    the single-read quantizer against the oracle's ROW (dgrad) and COL+RHT
    (wgrad) quantizations, and equal to the two separate device calls."""
    w = synth.WORKLOADS["wgrad_super"]
    dev = device()
    dy = synth.laplace((w["tokens"], w["out"]), w["dy_b"], w["dy_seed"], w["zero_frac"],
                       w["zero_seed"])
    mask = synth.rht_mask(w["mask_seed"])
    qr, qc, zeros = _check_dual(dy, "bf16", mask, seeds=(w["philox_seed"] + 100, w["philox_seed"]),
                                offsets=(0, 0))
    t, _ = device_input(dy, "bf16", dev)
    sr = nv.quantize_1d(t, "row", "sr", nv.Philox(w["philox_seed"] + 100))
    sc = nv.quantize_1d(t, "col", "sr", nv.Philox(w["philox_seed"]), mask)
    for a, b, name in ((qr, sr, "row"), (qc, sc, "col")):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales), name
    n = dy.size
    print(f"dY zero-code fraction: ROW {zeros[0] / n:.4f}, COL+RHT {zeros[1] / n:.4f}")


# ---- PTQ weights: MSE-calibrated block scales ---------------------------------------------------
@pytest.mark.parametrize("shape", [(16, 32), (48, 96), (1000, 64), (64, 2080)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_mse_small(shape, dtype):
    dev = device()
    x = make_input("normal", shape, seed=shape[0] + shape[1]) * np.float32(0.02)
    x[0, :16] = 0.0                                    # a zero block
    x[min(1, shape[0] - 1), 16:32] = [6.0] * 15 + [7.2]  # a block the MSE choice moves
    t, xo = device_input(x, dtype, dev)
    q = nv.quantize_mse(t)
    got = to_np(q)
    ref = O.quantize_mse(xo)
    assert_same(got["amax"][0], ref["amax"], "amax")
    assert_same(np.float32(got["g"]), ref["g"], "g")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


@pytest.mark.parametrize("kind", ["wide", "tiny", "zeros", "laplace_zeros"])
def test_quantize_mse_distributions(kind):
    dev = device()
    x = make_input(kind, (64, 256), seed=7)
    t, xo = device_input(x, "bf16", dev)
    q = nv.quantize_mse(t, amax=None)
    got = to_np(q)
    ref = O.quantize_mse(xo)
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


def test_quantize_mse_amax_input():
    dev = device()
    x = make_input("normal", (64, 128), seed=8)
    t, xo = device_input(x, "bf16", dev)
    q = nv.quantize_mse(t, amax=torch.tensor([9.0], device=dev))
    got = to_np(q)
    ref = O.quantize_mse(xo, amax=9.0)
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


def test_full_ptq_weight():
    """A Super-width weight [6144 x 6144] N(0, 0.02): every block against the
    oracle."""
    dev = device()
    w = synth.normal((6144, 6144), 0.02, 2)
    t, xo = device_input(w, "bf16", dev)
    q = nv.quantize_mse(t)
    got = to_np(q)
    ref = O.quantize_mse(xo)
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")
    moved = (got["scales"] != O.quantize(xo, "row")["scales"]).mean()
    print(f"blocks whose scale the MSE choice moved: {moved:.3f}")
