"""GPU parity: NVFP4 GEMMs (NT fprop, NN dgrad, TN wgrad) through the C ABI,
against the oracle's fp64 reference over the same quantized operands.

Metric: max over outputs of |C - R| / D with R = gA gB sum a b (fp64) and
D = gA gB sum |a b|; the bar is 1e-3, applied to the GEMM's fp32 result.  A
bf16 output is checked to be exactly the round-to-nearest-even of that fp32
result: the format's own rounding (up to 2^-9 |C|) is not an error of the
GEMM and can exceed 1e-3 D where |R| is close to D.  An exact special case
(grid-valued operands, unit scales) is bit-exact.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from nvfp4_block_scaled_07_amd import synth
from _gpu import assert_same, device, device_input, make_input, to_np

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _operands(layout, M, N, K, seed, dtype="bf16", a_kind="normal", sr=False, mask=-1):
    """Quantize logical A [M x K] and B^T [N x K] in the storage the layout
    uses; return device QTensors."""
    dev = device()
    a = make_input(a_kind, (M, K), seed)
    b = (make_input("normal", (N, K), seed + 1) * np.float32(0.02)).astype(np.float32)
    rng = nv.Philox(seed + 2) if sr else None
    rnd = "sr" if sr else "rne"
    if layout == "NT":
        qa = nv.quantize_1d(device_input(a, dtype, dev)[0], "row", rnd, rng)
        qb = nv.quantize_2d(device_input(b, dtype, dev)[0])
    elif layout == "NN":
        qa = nv.quantize_1d(device_input(a, dtype, dev)[0], "row", rnd, rng)
        qb = nv.quantize_2d(device_input(np.ascontiguousarray(b.T), dtype, dev)[0])
    else:  # TN: both stored [K x MN], COL blocks, shared transform mask
        qa = nv.quantize_1d(device_input(np.ascontiguousarray(a.T), dtype, dev)[0], "col", rnd,
                            rng, mask)
        qb = nv.quantize_1d(device_input(np.ascontiguousarray(b.T), dtype, dev)[0], "col", "rne",
                            None, mask)
    return qa, qb


def check_bf16_is_rne_of_fp32(c_bf16, c_fp32):
    """The bf16 output equals torch's RNE cast of the same GEMM's fp32 output."""
    want = c_fp32.to(torch.bfloat16)
    assert torch.equal(c_bf16.view(torch.int16), want.view(torch.int16)), \
        "bf16 output is not the RNE rounding of the fp32 result"


def _full_check(layout, qa, qb, M, N, K, out_dtype):
    c = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32)
    if out_dtype == torch.bfloat16:
        check_bf16_is_rne_of_fp32(nv.gemm(layout[0], layout[1], qa, qb, out_dtype=out_dtype), c)
    A, B = to_np(qa), to_np(qb)
    R, D = O.gemm_full(layout[0], layout[1], M, N, K, A, B)
    got = c.cpu().numpy()
    err = O.gemm_rel_err(got, R, D)
    assert err <= TOL, f"{layout} {M}x{N}x{K}: max |C-R|/D = {err:.3e}"
    return err


@pytest.mark.parametrize("layout,M,N,K", [
    ("NT", 256, 256, 256), ("NN", 256, 256, 256), ("TN", 256, 256, 256),
    ("NT", 300, 272, 320), ("NT", 17, 48, 64), ("NT", 513, 784, 128),
    ("NN", 200, 96, 192), ("NN", 520, 288, 256),
    ("TN", 96, 160, 192), ("TN", 288, 544, 128),
])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_small(layout, M, N, K, out):
    qa, qb = _operands(layout, M, N, K, seed=M + N + K, sr=(layout != "NT"),
                       mask=0x3C5A if layout == "TN" else -1)
    _full_check(layout, qa, qb, M, N, K, out)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_tiny_config(layout):
    """M=N=K=256, A 1x16 ~N(0,1) seed 100, B 16x16 ~N(0,1) seed 101, fp32 out
    (for TN both operands use COL blocks)."""
    dev = device()
    a = synth.normal((256, 256), 1.0, 100)
    b = synth.normal((256, 256), 1.0, 101)
    if layout == "NT":
        qa = nv.quantize_1d(torch.from_numpy(a).to(dev), "row")
        qb = nv.quantize_2d(torch.from_numpy(b).to(dev))
    elif layout == "NN":
        qa = nv.quantize_1d(torch.from_numpy(a).to(dev), "row")
        qb = nv.quantize_2d(torch.from_numpy(np.ascontiguousarray(b.T)).to(dev))
    else:
        qa = nv.quantize_1d(torch.from_numpy(np.ascontiguousarray(a.T)).to(dev), "col")
        qb = nv.quantize_1d(torch.from_numpy(np.ascontiguousarray(b.T)).to(dev), "col")
    _full_check(layout, qa, qb, 256, 256, 256, torch.float32)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_exact_special_case(layout):
    """Operands on the E2M1 grid times 448 with a 6*448 in every block: all
    scales 448, g = 1, every product a multiple of 1/4 * 448^2 and the fp32
    sum exact, so C equals the fp64 reference bit for bit."""
    dev = device()
    rng = np.random.default_rng(31)
    M, N, K = 256, 256, 512
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)

    def draw(r, c):
        v = grid[rng.integers(0, 8, (r, c))] * np.where(rng.random((r, c)) < .5, -1, 1)
        return v.astype(np.float32)

    a = draw(M, K); b = draw(N, K)
    a[:, ::16] = 6.0; b[:, ::16] = 6.0
    if layout == "TN":
        a[::16, :] = 6.0; b[::16, :] = 6.0
    a *= 448; b *= 448
    if layout == "NT":
        qa = nv.quantize_1d(torch.from_numpy(a).to(dev), "row")
        qb = nv.quantize_1d(torch.from_numpy(b).to(dev), "row")
    elif layout == "NN":
        qa = nv.quantize_1d(torch.from_numpy(a).to(dev), "row")
        qb = nv.quantize_1d(torch.from_numpy(np.ascontiguousarray(b.T)).to(dev), "col")
    else:
        qa = nv.quantize_1d(torch.from_numpy(np.ascontiguousarray(a.T)).to(dev), "col")
        qb = nv.quantize_1d(torch.from_numpy(np.ascontiguousarray(b.T)).to(dev), "col")
    c = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32).cpu().numpy()
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.array_equal(c.astype(np.float64), exact)


def _pick(n, k, rng):
    """k distinct indices of range(n) including the first and the last (all of
    them when n <= k), sorted."""
    if n <= k:
        return np.arange(n, dtype=np.int64)
    mid = rng.choice(np.arange(1, n - 1), k - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid]).astype(np.int64))


def _sampled_check(layout, qa, qb, M, N, K, c, n_rows=64, n_cols=64, n_random=4096, seed=0):
    """Full rows (n_rows, the first and last included), full columns (n_cols,
    likewise) and n_random random outputs against the oracle."""
    rng = np.random.default_rng(seed)
    rows = _pick(M, n_rows, rng)
    cols = _pick(N, n_cols, rng)
    ii = [np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, n_random)]
    jj = [np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, n_random)]
    ii = np.concatenate(ii); jj = np.concatenate(jj)
    A, B = to_np(qa), to_np(qb)
    R, D = O.gemm_entries(layout[0], layout[1], M, N, K, A, B, ii, jj)
    got = c[torch.from_numpy(ii).to(c.device), torch.from_numpy(jj).to(c.device)]
    got = got.float().cpu().numpy()
    err = O.gemm_rel_err(got, R, D)
    assert err <= TOL, f"{layout} {M}x{N}x{K}: sampled max |C-R|/D = {err:.3e}"
    return err


def test_full_fprop_super():
    w = synth.WORKLOADS["fprop_super"]
    dev = device()
    M, N, K = w["M"], w["N"], w["K"]
    x = synth.to_bf16(synth.normal((M, K), w["x_std"], w["x_seed"])).to(dev)
    wt = synth.to_bf16(synth.normal((N, K), w["w_std"], w["w_seed"])).to(dev)
    qa = nv.quantize_1d(x, "row")
    qb = nv.quantize_2d(wt)
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    check_bf16_is_rne_of_fp32(nv.gemm("N", "T", qa, qb, out_dtype=torch.bfloat16), c)
    _sampled_check("NT", qa, qb, M, N, K, c)


def test_full_wgrad_super():
    w = synth.WORKLOADS["wgrad_super"]
    dev = device()
    T, Mo, Ni = w["tokens"], w["out"], w["inp"]
    mask = synth.rht_mask(w["mask_seed"])
    dy = synth.to_bf16(synth.laplace((T, Mo), w["dy_b"], w["dy_seed"], w["zero_frac"],
                                     w["zero_seed"])).to(dev)
    x = synth.to_bf16(synth.normal((T, Ni), 1.0, w["x_seed"])).to(dev)
    qa = nv.quantize_1d(dy, "col", "sr", nv.Philox(w["philox_seed"]), mask)
    qb = nv.quantize_1d(x, "col", "rne", None, mask)
    c = nv.gemm("T", "N", qa, qb, out_dtype=torch.float32)
    _sampled_check("TN", qa, qb, Mo, Ni, T, c)


def test_full_ultra_dgrad():
    w = synth.WORKLOADS["ultra"]
    dev = device()
    M, N, K = w["M"], w["N"], w["K"]
    dy = synth.to_bf16(synth.laplace((M, K), w["dy_b"], w["dy_seed"])).to(dev)
    wt = synth.to_bf16(synth.normal((K, N), w["w_std"], w["w_seed"])).to(dev)
    qa = nv.quantize_1d(dy, "row", "sr", nv.Philox(w["philox_seed"]))
    qb = nv.quantize_2d(wt)  # W stored [out = K, in = N]; dX = dY W
    c = nv.gemm("N", "N", qa, qb, out_dtype=torch.float32)
    check_bf16_is_rne_of_fp32(nv.gemm("N", "N", qa, qb, out_dtype=torch.bfloat16), c)
    _sampled_check("NN", qa, qb, M, N, K, c)


def test_full_ultra_fprop():
    """Ultra-width fprop: X bf16 [8192 x 8192] N(0,1) 1x16 RNE, W [8192 x
    8192] N(0, 0.015) 16x16, Y = X W^T (NT); bf16 out, the RNE of the fp32
    result, which is sampled against the oracle."""
    w = synth.WORKLOADS["ultra"]
    dev = device()
    M, N, K = w["M"], w["N"], w["K"]
    x = synth.to_bf16(synth.normal((M, K), 1.0, w["x_seed"])).to(dev)
    wt = synth.to_bf16(synth.normal((N, K), w["w_std"], w["w_seed"])).to(dev)
    qa = nv.quantize_1d(x, "row")
    qb = nv.quantize_2d(wt)
    del x, wt
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    check_bf16_is_rne_of_fp32(nv.gemm("N", "T", qa, qb, out_dtype=torch.bfloat16), c)
    _sampled_check("NT", qa, qb, M, N, K, c, seed=1)


def test_gemm_kmajor_operand_past_4gib():
    """A K-major A with 2^20 + 256 rows of K = 8192 (4 GiB of codes): each
    tile's buffer range covers its own rows, so tiles far into the operand,
    and the last one, read their codes (a range running to the operand's end
    would wrap 32 bits and read zeros).  A's codes and scales are drawn
    directly; rows are checked against the oracle on those rows alone (row i
    of an NT product only depends on row i of A)."""
    dev = device()
    M, N, K = (1 << 20) + 256, 64, 8192
    g = torch.Generator(device=dev).manual_seed(41)
    codes = torch.randint(0, 256, (M, K // 2), generator=g, device=dev, dtype=torch.uint8)
    scales = torch.randint(0x30, 0x48, (M, K // 16), generator=g, device=dev,
                           dtype=torch.uint8)
    one = torch.ones(1, device=dev)
    qa = nv.QTensor(codes, scales, one, one, M, K, "row")
    qb = nv.quantize_2d(synth.normal_device((N, K), 0.02, 42, dev))
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    rows = np.array([0, 1, 255, 256, 4097, (1 << 19) + 3, 1 << 20, M - 2, M - 1], dtype=np.int64)
    ridx = torch.from_numpy(rows).to(dev)
    A = dict(codes=codes[ridx].cpu().numpy(), scales=scales[ridx].cpu().numpy(), block="row",
             g=1.0)
    ii = np.repeat(np.arange(len(rows), dtype=np.int64), N)
    jj = np.tile(np.arange(N, dtype=np.int64), len(rows))
    R, D = O.gemm_entries("N", "T", len(rows), N, K, A, to_np(qb), ii, jj)
    got = c[ridx].cpu().numpy().reshape(-1)
    err = O.gemm_rel_err(got, R, D)
    assert err <= TOL, f"max |C-R|/D = {err:.3e}"


SENTINEL = 0x7FC0DEAD  # a NaN pattern no kernel writes


def _guarded(shape, dtype, dev, pad=1024):
    """A tensor of `shape` inside a larger buffer whose other bytes hold a
    sentinel pattern: (view, buffer, pad in elements)."""
    n = int(np.prod(shape))
    esz = torch.empty(0, dtype=dtype).element_size()
    words = (n * esz + 3) // 4 + 2 * pad
    buf = torch.full((words,), SENTINEL, dtype=torch.int32, device=dev)
    view = buf[pad:].view(torch.uint8)[:n * esz].view(dtype).view(shape)
    return view, buf, pad, (n * esz + 3) // 4


def _intact(buf, pad, used):
    b = buf.cpu().numpy()
    return bool(np.all(b[:pad] == SENTINEL) and np.all(b[pad + used:] == SENTINEL))


@pytest.mark.parametrize("layout,M,N,K", [("NT", 300, 272, 320), ("NN", 200, 96, 192),
                                          ("TN", 288, 544, 128), ("NT", 40, 96, 512),
                                          ("NT", 4096, 4096, 128)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_output_canaries(layout, M, N, K, out):
    """The GEMMs write nothing outside C: sentinel words before and after the
    output (partial tiles, small-M kernel, full tiles) are untouched."""
    dev = device()
    qa, qb = _operands(layout, M, N, K, seed=M + N, sr=layout != "NT",
                       mask=0x3C5A if layout == "TN" else -1)
    c, buf, pad, used = _guarded((M, N), out, dev)
    nv.gemm(layout[0], layout[1], qa, qb, out=c)
    torch.cuda.synchronize()
    assert _intact(buf, pad, used)
    want = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=out)
    assert torch.equal(c.view(torch.int16 if out == torch.bfloat16 else torch.int32),
                       want.view(torch.int16 if out == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_large_tiles_full(layout):
    """4096 x 4096 fills exactly one round of 256 x 256 tiles on 256 CUs, so
    the launch takes the 256-row tile; every output is checked."""
    M, N, K = 4096, 4096, 128
    qa, qb = _operands(layout, M, N, K, seed=17, sr=layout != "NT",
                       mask=0x0F0F if layout == "TN" else -1)
    _full_check(layout, qa, qb, M, N, K, torch.bfloat16)


@pytest.mark.parametrize("layout", ["NT", "NN"])
def test_gemm_tile_shape_does_not_change_bits(layout):
    """C for A's first 768 rows (128-row tiles on 256 CUs) and first 3072
    rows (192-row tiles) equals those rows of the 4096 x 4096 product
    (256-row tiles) bit for bit: each output is the same sum in the same
    order whatever the tile shape."""
    M, N, K = 4096, 4096, 256
    qa, qb = _operands(layout, M, N, K, seed=23, sr=layout != "NT")
    full = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32)
    for rows in (768, 3072):
        sub = nv.QTensor(qa.codes[:rows], qa.scales[:rows], qa.global_dec, qa.amax, rows, K,
                         "row")
        part = nv.gemm(layout[0], layout[1], sub, qb, out_dtype=torch.float32)
        assert torch.equal(part, full[:rows]), rows


def test_full_ultra_wgrad():
    """dW = dY^T X at the Ultra width (8192 tokens, 8192 x 8192), COL blocks
    with the transform on both operands and SR on dY (256-row tiles)."""
    w = synth.WORKLOADS["ultra"]
    dev = device()
    T, Mo, Ni = w["K"], w["M"], w["N"]
    mask = synth.rht_mask(6)
    dy = synth.to_bf16(synth.laplace((T, Mo), w["dy_b"], w["dy_seed"])).to(dev)
    x = synth.to_bf16(synth.normal((T, Ni), 1.0, w["x_seed"])).to(dev)
    qa = nv.quantize_1d(dy, "col", "sr", nv.Philox(w["philox_seed"]), mask)
    qb = nv.quantize_1d(x, "col", "rne", None, mask)
    c = nv.gemm("T", "N", qa, qb, out_dtype=torch.float32)
    _sampled_check("TN", qa, qb, Mo, Ni, T, c)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_deterministic_long_k(layout):
    """Repeated runs with many pipeline stages give identical bits (a race
    between the LDS stage buffers would show up as run-to-run differences),
    and bf16 output stays the RNE rounding of the fp32 result."""
    M, N, K = 1024, 768, 8192
    qa, qb = _operands(layout, M, N, K, seed=5, sr=layout != "NT",
                       mask=0x1111 if layout == "TN" else -1)
    c1 = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32)
    for _ in range(4):
        c2 = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32)
        assert torch.equal(c1, c2)
        check_bf16_is_rne_of_fp32(nv.gemm(layout[0], layout[1], qa, qb,
                                          out_dtype=torch.bfloat16), c1)


@pytest.mark.parametrize("layout,M,N,K", [("TN", 288, 544, 256), ("NN", 200, 96, 192),
                                          ("NT", 300, 272, 320), ("NT", 40, 96, 512)])
def test_gemm_accumulate_into_fp32(layout, M, N, K):
    """NVFP4_FP32_ACCUMULATE: C = RN32(C + P) with P the product the plain
    fp32 call writes, bit for bit (tiled kernels with partial tiles, and the
    small-M kernel); P itself meets the oracle bar."""
    dev = device()
    qa, qb = _operands(layout, M, N, K, seed=M + 2 * N + K, sr=layout != "NT",
                       mask=0x2D4B if layout == "TN" else -1)
    p = nv.gemm(layout[0], layout[1], qa, qb, out_dtype=torch.float32)
    c0 = torch.from_numpy(make_input("normal", (M, N), 77)).to(dev)
    c0[0, :8] = 0.0
    c = c0.clone()
    nv.gemm(layout[0], layout[1], qa, qb, out=c, accumulate=True)
    assert torch.equal(c.view(torch.int32), (c0 + p).view(torch.int32))
    nv.gemm(layout[0], layout[1], qa, qb, out=c, accumulate=True)
    assert torch.equal(c.view(torch.int32), ((c0 + p) + p).view(torch.int32))
    A, B = to_np(qa), to_np(qb)
    R, D = O.gemm_full(layout[0], layout[1], M, N, K, A, B)
    assert O.gemm_rel_err(p.cpu().numpy(), R, D) <= TOL


@pytest.mark.parametrize("M,N,K", [(40, 256, 1 << 17), (300, 256, 1 << 16)])
def test_gemm_long_k(M, N, K):
    """Long contractions (small-M and tiled kernels): 2^16 and 2^17 k, far
    past one tile's buffer range, sampled against the oracle."""
    dev = device()
    a = make_input("normal", (M, K), 61)
    b = (make_input("normal", (N, K), 62) * np.float32(0.02)).astype(np.float32)
    qa = nv.quantize_1d(device_input(a, "bf16", dev)[0], "row")
    qb = nv.quantize_2d(device_input(b, "bf16", dev)[0])
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    _sampled_check("NT", qa, qb, M, N, K, c, n_random=512)


@pytest.mark.parametrize("M", [1, 33, 130])
def test_gemm_widest_n(M):
    """N = 2^21 - 32, the widest output the ABI accepts (31-bit store offsets
    within a tile, 65535 small-M workgroups), sampled against the oracle
    including the last columns."""
    dev = device()
    N, K = (1 << 21) - 32, 64
    a = make_input("normal", (M, K), 63)
    qa = nv.quantize_1d(device_input(a, "fp32", dev)[0], "row")
    qb = nv.quantize_1d(synth.normal_device((N, K), 0.02, 64, dev, dtype=torch.float32), "row")
    c = nv.gemm("N", "T", qa, qb, out_dtype=torch.bfloat16)
    c32 = nv.gemm("N", "T", qa, qb, out_dtype=torch.float32)
    check_bf16_is_rne_of_fp32(c, c32)
    rng = np.random.default_rng(M)
    ii = np.concatenate([rng.integers(0, M, 2048), np.full(64, M - 1)])
    jj = np.concatenate([rng.integers(0, N, 2048), np.arange(N - 64, N)])
    R, D = O.gemm_entries("N", "T", M, N, K, to_np(qa), to_np(qb), ii, jj)
    err = O.gemm_rel_err(c32[ii, jj].cpu().numpy(), R, D)
    assert err <= TOL, f"sampled max |C-R|/D = {err:.3e}"
