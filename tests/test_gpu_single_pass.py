"""GPU parity of the single-pass quantizers and of the per-call scratch slots
that replace a cleared amax output.

* Single pass (bf16 ROW without transform, RNE or stochastic rounding; one
  bf16 16x16-blocked matrix): bit-exact against the oracle on both sides of
  the register capacity (the largest tensor the grid's registers hold, and
  one row group more, whose last round is streamed: read for the maximum
  before the grid barrier and again after it), at the Ultra size [8192^2]
  (a quarter of it streamed) and at the wgrad-Super dY size with stochastic
  rounding; equal to the two-pass path; exact when the grid barrier's wait is
  forced to give up (every late workgroup takes the tensor maximum by
  itself) and when two streams run single-pass calls at the same time.
* Batched single pass (bf16 16x16 blocks of a batch of matrices, one amax
  each: groups of workgroups that each hold one matrix, several matrices per
  group in turn): bit-exact against the oracle for batches that give each
  group one, two and three matrices (the board alternates between rounds),
  with slices scaled apart so that a maximum taken from the wrong slice
  shows; equal to the two-pass path, also for matrices larger than the
  grid's registers (one group, streamed rounds); exact when the group
  barrier's wait is forced to give up.
* COL single pass (bf16 16x1 blocks with RNE, with and without the
  transform; the maximum taken after the transform): equal to
  the two-pass path for tensors smaller and larger than the grid's registers
  (the Super and Ultra sizes stream 4 and 8 of their 12 and 16 rounds) and
  ragged against the grid; bit-exact against the oracle; exact when the
  barrier's wait gives up (the late workgroups transform the whole tensor
  for the maximum themselves).
* Slots: hundreds of calls in a row, more than the slots, with tensor maxima
  going up and down (a slot left dirty would hand a stale, larger maximum to
  a later call), and repeated dual quantizations whose zero-code counts must
  not accumulate across calls.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from nvfp4_block_scaled_07_amd import synth
from _gpu import assert_same, device, make_input, to_np

pytestmark = pytest.mark.gpu

THREADS, ROW_HOLD, ROW_HOLD_SR, UNITS_HOLD = 512, 48, 42, 3  # held per thread


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _bf16(x, dev):
    t = synth.to_bf16(x)
    return t.to(dev), synth.bf16_bits(t)


def _check(q, ref):
    got = to_np(q)
    assert_same(got["amax"][0], ref["amax"], "amax")
    assert_same(np.float32(got["g"]), ref["g"], "g")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


def _same(a, b):
    for f in ("codes", "scales", "global_dec", "amax"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("extra_rows", [0, 16])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_row_single_pass_size_limit(extra_rows, rounding):
    """Rows of 4096: the largest ROW tensor held in registers, and 16 rows
    more (a partial last round, streamed), both against the oracle."""
    dev = device()
    hold = ROW_HOLD if rounding == "rne" else ROW_HOLD_SR
    rows = _cus() * THREADS * hold * 8 // 4096 + extra_rows
    x = make_input("normal", (rows, 4096), seed=600 + extra_rows)
    t, xo = _bf16(x, dev)
    if rounding == "rne":
        _check(nv.quantize_1d(t, "row"), O.quantize(xo, "row"))
    else:
        _check(nv.quantize_1d(t, "row", "sr", nv.Philox(31)),
               O.quantize(xo, "row", rounding=O.SR, seed=31))


@pytest.mark.parametrize("extra_rows", [0, 16])
def test_2d_single_pass_size_limit(extra_rows):
    dev = device()
    rows = 16 * _cus() * THREADS * UNITS_HOLD // (4096 // 8) + extra_rows
    x = make_input("normal", (rows, 4096), seed=610 + extra_rows) * np.float32(0.02)
    t, xo = _bf16(x, dev)
    _check(nv.quantize_2d(t), O.quantize(xo, "2d"))


@pytest.mark.parametrize("kind", ["row", "row_sr", "2d"])
def test_single_pass_ultra_size(kind):
    """[8192 x 8192] bf16 (134 MB, a quarter of it streamed), against the
    oracle: the Ultra-width X (ROW), dY (ROW, stochastic rounding) and W."""
    dev = device()
    scale = np.float32(0.015) if kind == "2d" else np.float32(1.0)
    x = make_input("normal", (8192, 8192), seed=615) * scale
    t, xo = _bf16(x, dev)
    del x
    if kind == "row":
        _check(nv.quantize_1d(t, "row"), O.quantize(xo, "row"))
    elif kind == "row_sr":
        _check(nv.quantize_1d(t, "row", "sr", nv.Philox(14)),
               O.quantize(xo, "row", rounding=O.SR, seed=14))
    else:
        _check(nv.quantize_2d(t), O.quantize(xo, "2d"))


def test_single_pass_sr_wgrad_dy():
    """The wgrad-Super dY [8192 x 6144] (Laplace, 7% zeros), ROW with
    stochastic rounding, single pass with streamed rounds, against the
    oracle and the two-pass path."""
    dev = device()
    x = make_input("laplace_zeros", (8192, 6144), seed=3)
    t, xo = _bf16(x, dev)
    one = nv.quantize_1d(t, "row", "sr", nv.Philox(7))
    prev = nv.nvfp4_set_single_pass_wait(-1)
    try:
        two = nv.quantize_1d(t, "row", "sr", nv.Philox(7))
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _same(one, two)
    _check(one, O.quantize(xo, "row", rounding=O.SR, seed=7))


@pytest.mark.parametrize("shape", [(66, 1024), (2000, 6144), (4096, 4160), (1024, 32)])
def test_single_pass_equals_two_pass(shape):
    """The same bits with the single-pass kernels turned off (tensors of
    several sizes, ragged against the grid)."""
    dev = device()
    x = make_input("laplace_zeros", shape, seed=shape[0])
    t, xo = _bf16(x, dev)
    w = t[: shape[0] // 16 * 16]
    one_r, one_w = nv.quantize_1d(t, "row"), nv.quantize_2d(w)
    one_s = nv.quantize_1d(t, "row", "sr", nv.Philox(shape[1]))
    prev = nv.nvfp4_set_single_pass_wait(-1)
    try:
        two_r, two_w = nv.quantize_1d(t, "row"), nv.quantize_2d(w)
        two_s = nv.quantize_1d(t, "row", "sr", nv.Philox(shape[1]))
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _same(one_r, two_r)
    _same(one_w, two_w)
    _same(one_s, two_s)
    _check(one_r, O.quantize(xo, "row"))


def _batch_input(batch, rows, cols, seed, dev):
    """Normal slices scaled 4^(i % 7): neighbouring slices' maxima differ."""
    x = make_input("normal", (batch, rows, cols), seed=seed)
    x *= np.float32(4.0) ** (np.arange(batch, dtype=np.float32) % 7)[:, None, None]
    return _bf16(x, dev)


def _check_batch(q, xo):
    got, ref = to_np(q), O.quantize(xo, "2d")
    assert_same(got["amax"], ref["amax"], "amax")
    assert_same(got["g"], ref["g"], "g")
    assert_same(got["scales"], ref["scales"], "scales")
    assert_same(got["codes"], ref["codes"], "codes")


@pytest.mark.parametrize("batch,rows,cols", [(3, 48, 96), (300, 16, 32), (37, 2688, 1024),
                                             (5, 1024, 4096), (64, 272, 160)])
def test_batch_2d_single_pass(batch, rows, cols):
    """Matrices per group (one workgroup holds 1536 units of 16 x 8):
    [16 x 32] x 300 -> 256 groups, two rounds for 44 of them; [2688 x 1024]
    x 37 (the Super experts' shape) -> 18 groups of 14 workgroups, three
    rounds for one group; [1024 x 4096] x 5 -> 5 groups; ragged column
    counts (96, 160) -> pairs and rows as in the single-matrix kernel."""
    dev = device()
    t, xo = _batch_input(batch, rows, cols, batch + rows, dev)
    _check_batch(nv.quantize_2d(t), xo)


@pytest.mark.parametrize("batch,rows,cols", [(300, 16, 32), (20, 2688, 1024), (2, 8192, 8192)])
def test_batch_2d_single_pass_equals_two_pass(batch, rows, cols):
    """The same bits with the single-pass kernels turned off; [8192^2] x 2 is
    larger than the grid's registers (one group, the last round streamed)."""
    dev = device()
    t, _ = _batch_input(batch, rows, cols, 7 * batch, dev)
    one = nv.quantize_2d(t)
    prev = nv.nvfp4_set_single_pass_wait(-1)
    try:
        two = nv.quantize_2d(t)
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _same(one, two)
    want = t.float().abs().amax(dim=(1, 2))
    assert torch.equal(one.amax, want), "amax"


def test_batch_2d_single_pass_gives_up():
    """With no wait at the group barriers every late workgroup reads its
    matrix for the maximum: the results are still exact."""
    dev = device()
    t, xo = _batch_input(24, 2688, 1024, 640, dev)
    prev = nv.nvfp4_set_single_pass_wait(0)
    try:
        q = nv.quantize_2d(t)
        torch.cuda.synchronize()
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _check_batch(q, xo)


@pytest.mark.parametrize("shape", [(16, 32), (2000, 6144), (8192, 6144), (8192, 8192), (4096, 4160)])
def test_col_single_pass_equals_two_pass(shape):
    """COL with and without the transform: the same bits with the single-pass
    kernels turned off (RNE; the SR cases take the two-pass path either way
    and check that the setting leaves them alone)."""
    dev = device()
    x = make_input("laplace_zeros", shape, seed=shape[1] + 3)
    rows = shape[0] // 16 * 16
    t, _ = _bf16(x[:rows], dev)
    mask = synth.rht_mask(6)
    cases = [("rne", None, -1), ("rne", None, mask), ("sr", 21, -1), ("sr", 22, mask)]

    def run():
        return [nv.quantize_1d(t, "col", r, nv.Philox(sd) if sd else None, m) for r, sd, m in cases]

    one = run()
    prev = nv.nvfp4_set_single_pass_wait(-1)
    try:
        two = run()
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    for a, b in zip(one, two):
        _same(a, b)


def test_col_single_pass_oracle():
    """COL + RHT16 RNE in one pass, bit-exact against the oracle, on a
    tensor whose last round is streamed ([8192 x 4160]: 8 held rounds and a
    partial ninth on 256 CUs)."""
    dev = device()
    x = make_input("normal", (8192, 4160), seed=650)
    t, xo = _bf16(x, dev)
    mask = synth.rht_mask(6)
    q = nv.quantize_1d(t, "col", "rne", None, mask)
    _check(q, O.quantize(xo, "col", rht_mask=mask))


def test_col_single_pass_gives_up():
    """With no wait at the grid barrier the late workgroups take the
    transform's maximum from the whole tensor: still exact."""
    dev = device()
    x = make_input("normal", (2000, 6144), seed=660)
    t, xo = _bf16(x[:1984], dev)
    mask = synth.rht_mask(6)
    prev = nv.nvfp4_set_single_pass_wait(0)
    try:
        qr = nv.quantize_1d(t, "col", "rne", None, mask)
        qp = nv.quantize_1d(t, "col")
        torch.cuda.synchronize()
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _check(qr, O.quantize(xo, "col", rht_mask=mask))
    _check(qp, O.quantize(xo, "col"))


def test_single_pass_barrier_gives_up():
    """With no wait at the grid barrier, workgroups that find it incomplete
    read the whole tensor for the maximum: the results are still exact."""
    dev = device()
    x = make_input("normal", (2000, 6144), seed=620)
    t, xo = _bf16(x, dev)
    w = t[:1984]
    prev = nv.nvfp4_set_single_pass_wait(0)
    try:
        qr, qw = nv.quantize_1d(t, "row"), nv.quantize_2d(w)
        torch.cuda.synchronize()
    finally:
        nv.nvfp4_set_single_pass_wait(prev)
    _check(qr, O.quantize(xo, "row"))
    _check(qw, O.quantize(xo[:1984], "2d"))


def test_single_pass_on_two_streams():
    """Single-pass calls issued on two streams at once (each may find CUs
    held by the other's workgroups) give the single-stream results."""
    dev = device()
    xs = [_bf16(make_input("normal", (2048, 6144), seed=630 + i) * np.float32(1 + i), dev)[0]
          for i in range(2)]
    ref = [nv.quantize_1d(x, "row") for x in xs] + [nv.quantize_2d(x) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    out = []
    for rep in range(4):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                out.append((i, nv.quantize_1d(xs[i], "row", stream=s),
                            nv.quantize_2d(xs[i], stream=s)))
    torch.cuda.synchronize()
    for i, qr, qw in out:
        _same(qr, ref[i])
        _same(qw, ref[2 + i])


def test_slots_reused_and_cleared():
    """600 end-to-end calls (more than the slots), single-pass and two-pass,
    ROW, 2D and COL, with the tensor maximum scaled by powers of two up and
    down between calls: every call's amax is its own tensor's (exact: a
    power-of-two scale scales the maximum exactly)."""
    dev = device()
    base = [make_input("normal", (66, 1024), seed=640),           # ROW single pass (bf16)
            make_input("normal", (256, 1024), seed=641)]          # two-pass (fp32)
    amax0 = [float(O.amax(synth.bf16_bits(synth.to_bf16(base[0])), "row")),
             float(O.amax(base[1], "row"))]
    t_bf = synth.to_bf16(base[0]).to(dev)
    t_32 = torch.from_numpy(base[1]).to(dev)
    for i in range(600):
        k = (i * 7) % 11 - 5                   # scale 2^k, k in -5 .. 5
        f = float(2.0 ** k)
        kind = i % 4
        if kind == 0:
            q, want = nv.quantize_1d(t_bf * f, "row"), amax0[0] * f
        elif kind == 1:
            q, want = nv.quantize_1d(t_32 * f, "row"), amax0[1] * f
        elif kind == 2:
            q, want = nv.quantize_2d(t_bf[:64] * f), None
        else:
            q, want = nv.quantize_1d(t_32 * f, "col"), amax0[1] * f
        got = float(q.amax.item())
        if want is not None:
            assert got == np.float32(want), (i, got, want)
        else:
            want2d = float(O.amax(synth.bf16_bits(synth.to_bf16(base[0][:64])), "row")) * f
            assert got == np.float32(want2d), (i, got, want2d)


def test_dual_zero_counts_do_not_accumulate():
    """The dual quantizer's zero-code counts go through the call's slot: the
    same input gives the same counts call after call, equal to the oracle's
    count of its codes."""
    dev = device()
    x = make_input("laplace_zeros", (512, 1024), seed=650)
    t, xo = _bf16(x, dev)
    mask = 0x5A3C
    counts = []
    for rep in range(5):
        qr, qc, z = nv.quantize_dual(t, nv.Philox(11), nv.Philox(12), mask)
        counts.append(z.cpu().tolist())
    assert all(c == counts[0] for c in counts)
    rr = O.quantize(xo, "row", rounding=O.SR, seed=11)
    rc = O.quantize(xo, "col", rounding=O.SR, seed=12, rht_mask=mask)
    assert counts[0] == [O.zero_codes(rr["codes"]), O.zero_codes(rc["codes"])]
