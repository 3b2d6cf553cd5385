"""GPU parity: grouped NVFP4 GEMM for routed experts, against the oracle's
fp64 reference applied group by group (ragged and empty groups included),
and against the dense GEMM on each group.  As for the dense GEMM, the 1e-3
metric applies to the fp32 result and a bf16 output must be its RNE
rounding bit for bit."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from nvfp4_block_scaled_07_amd import synth
from _gpu import device, to_np

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _grouped_case(counts, N, K, seed, b_block="2d", out=torch.bfloat16):
    dev = device()
    counts = np.asarray(counts, dtype=np.int64)
    G = len(counts)
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    T = int(offsets[-1])
    a = synth.normal((T, K), 1.0, seed)
    w = synth.normal((G, N, K), 0.02, seed + 1)
    w *= (1 + np.arange(G) % 5).astype(np.float32)[:, None, None]  # distinct g per group
    qa = nv.quantize_1d(synth.to_bf16(a).to(dev), "row")
    if b_block == "2d":
        qb = nv.quantize_2d(synth.to_bf16(w).to(dev))
    else:  # ROW-blocked expert weights, one 1D quantization per expert
        qs = [nv.quantize_1d(synth.to_bf16(w[e]).to(dev), "row") for e in range(G)]
        qb = nv.QTensor(torch.stack([q.codes for q in qs]), torch.stack([q.scales for q in qs]),
                        torch.cat([q.global_dec for q in qs]), torch.cat([q.amax for q in qs]),
                        N, K, "row")
    off_d = torch.from_numpy(offsets).to(dev)
    c = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.float32)
    if out == torch.bfloat16:
        cb = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.bfloat16)
        assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))
    return qa, qb, offsets, c


def _check_group(qa, qb, offsets, c, e, N, K, rows=None, A=None):
    A = to_np(qa) if A is None else A
    Bc = qb.codes[e].cpu().numpy()
    Bs = qb.scales[e].cpu().numpy()
    gB = float(qb.global_dec[e].item())
    r0, r1 = int(offsets[e]), int(offsets[e + 1])
    if r1 == r0:
        return 0.0
    Ae = dict(codes=A["codes"][r0:r1], scales=A["scales"][r0:r1], block="row", g=A["g"])
    Be = dict(codes=Bc, scales=Bs, block=qb.block, g=gB)
    if rows is None:
        R, D = O.gemm_full("N", "T", r1 - r0, N, K, Ae, Be)
        got = c[r0:r1].float().cpu().numpy()
    else:
        rr = np.array([r for r in rows if r < r1 - r0], dtype=np.int64)
        ii = np.repeat(rr, N)
        jj = np.tile(np.arange(N), len(rr))
        R, D = O.gemm_entries("N", "T", r1 - r0, N, K, Ae, Be, ii, jj)
        got = c[r0 + ii, jj].float().cpu().numpy()
    err = O.gemm_rel_err(got, R, D)
    assert err <= TOL, f"group {e}: {err:.3e}"
    return err


@pytest.mark.parametrize("b_block", ["2d", "row"])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_grouped_small_ragged(b_block, out):
    counts = [0, 5, 300, 1, 256, 0, 77, 513]
    N, K = 96, 128
    qa, qb, off, c = _grouped_case(counts, N, K, seed=3, b_block=b_block, out=out)
    for e in range(len(counts)):
        _check_group(qa, qb, off, c, e, N, K)


def test_grouped_matches_dense_per_group():
    """Groups of more than 512 rows give exactly the dense GEMM's bits (the
    same sum in the same order); a dense NT call with fewer rows (and few
    tiles) takes the split-K small-M kernel, which rounds differently, so
    those groups are held to the oracle bar instead."""
    counts = [40, 0, 600, 7, 90]
    N, K = 272, 192
    qa, qb, off, c = _grouped_case(counts, N, K, seed=9, out=torch.float32)
    for e, n in enumerate(counts):
        if n == 0:
            continue
        if n <= 512:
            _check_group(qa, qb, off, c, e, N, K)
            continue
        r0 = int(off[e])
        sub = nv.QTensor(qa.codes[r0:r0 + n], qa.scales[r0:r0 + n], qa.global_dec, qa.amax, n, K,
                         "row")
        be = nv.QTensor(qb.codes[e], qb.scales[e], qb.global_dec[e:e + 1], qb.amax[e:e + 1], N, K,
                        "2d")
        d = nv.gemm("N", "T", sub, be, out_dtype=torch.float32)
        assert torch.equal(d, c[r0:r0 + n])


@pytest.mark.parametrize("counts,K", [([40, 0, 600, 7, 100], 192),  # few rows per group: 128-row tiles
                                      ([600, 1100, 0, 700], 256)])  # many: 256-row tiles
def test_grouped_tile_shapes_match_dense(counts, K):
    """Both grouped tile shapes give each group of more than 512 rows exactly
    the dense GEMM's bits (smaller dense NT calls take the small-M kernel)."""
    N = 272
    qa, qb, off, c = _grouped_case(counts, N, K, seed=11, out=torch.float32)
    for e, n in enumerate(counts):
        if n == 0:
            continue
        _check_group(qa, qb, off, c, e, N, K)
        if n <= 512:
            continue
        r0 = int(off[e])
        sub = nv.QTensor(qa.codes[r0:r0 + n], qa.scales[r0:r0 + n], qa.global_dec, qa.amax, n, K,
                         "row")
        be = nv.QTensor(qb.codes[e], qb.scales[e], qb.global_dec[e:e + 1], qb.amax[e:e + 1], N, K,
                        "2d")
        d = nv.gemm("N", "T", sub, be, out_dtype=torch.float32)
        assert torch.equal(d, c[r0:r0 + n])


def test_grouped_all_rows_in_one_group_and_many_groups():
    qa, qb, off, c = _grouped_case([700], 64, 64, seed=1)
    _check_group(qa, qb, off, c, 0, 64, 64)
    counts = np.random.default_rng(2).integers(0, 40, 300)
    qa, qb, off, c = _grouped_case(counts, 32, 64, seed=2)
    for e in range(0, 300, 37):
        _check_group(qa, qb, off, c, e, 32, 64)


def test_full_grouped_super_sampled():
    """8192 tokens x top-22 of 512 experts (Zipf 1.1 routing), latent 1024 ->
    expert hidden 2688; checks full rows of the first, last and a middle row of
    several experts, including the largest and smallest."""
    w = synth.WORKLOADS["grouped_super"]
    dev = device()
    counts, tok, offsets = synth.zipf_routing(w["tokens"], w["experts"], w["topk"], w["zipf_s"],
                                              w["route_seed"])
    x = synth.to_bf16(synth.normal((w["tokens"], w["latent"]), 1.0, w["x_seed"])).to(dev)
    a = x[torch.from_numpy(tok).to(dev)]  # rows gathered by expert
    W = synth.to_bf16(synth.normal((w["experts"], w["hidden"], w["latent"]), w["w_std"],
                                   w["w_seed"])).to(dev)
    qa = nv.quantize_1d(a, "row")
    qb = nv.quantize_2d(W)
    off_d = torch.from_numpy(offsets).to(dev)
    c = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.float32)
    cb = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.bfloat16)
    assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))
    torch.cuda.synchronize()
    A = to_np(qa)
    for e in _spread_experts(counts, 16):
        n = int(counts[e])
        _check_group(qa, qb, offsets, c, e, w["hidden"], w["latent"], rows=[0, n // 2, n - 1],
                     A=A)


def _spread_experts(counts, k):
    """k experts spread over the range of row counts: the largest, the
    smallest non-empty one, and k - 2 between them by rank, plus experts 0
    and the last."""
    order = [int(e) for e in np.argsort(counts, kind="stable") if counts[e] > 0]
    picks = {order[-1], order[0], 0, len(counts) - 1}
    for t in np.linspace(0, len(order) - 1, k).astype(int):
        picks.add(order[t])
    return sorted(e for e in picks if counts[e] > 0)


def test_full_grouped_ultra_sampled():
    """Ultra's routed experts: 8192 tokens x top-22 of 512 experts (Zipf 1.1
    routing, seed 16), latent 2048 -> expert hidden 5120, W_e N(0, 0.015);
    full rows (first, middle, last) of at least 16 experts against the
    oracle, and bf16 output equal to the RNE of the fp32 result."""
    w = synth.WORKLOADS["ultra"]
    dev = device()
    E, L, H = 512, w["glat"], w["ghidden"]
    counts, tok, offsets = synth.zipf_routing(8192, E, 22, 1.1, w["groute_seed"])
    x = synth.to_bf16(synth.normal((8192, L), 1.0, w["gx_seed"])).to(dev)
    a = x[torch.from_numpy(tok).to(dev)]
    W = synth.normal_device((E, H, L), w["w_std"], w["gw_seed"], dev)
    qa = nv.quantize_1d(a, "row")
    qb = nv.quantize_2d(W)
    del W, a
    torch.cuda.empty_cache()
    off_d = torch.from_numpy(offsets).to(dev)
    c = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.float32)
    cb = nv.grouped_gemm(qa, qb, off_d, out_dtype=torch.bfloat16)
    assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))
    del cb
    torch.cuda.synchronize()
    picks = _spread_experts(counts, 16)
    assert len(picks) >= 16
    A = to_np(qa)
    for e in picks:
        n = int(counts[e])
        _check_group(qa, qb, offsets, c, e, H, L, rows=[0, n // 2, n - 1], A=A)


# ---- routed-expert backward: grouped dgrad (NN) and grouped wgrad (TN) -------------------------
def _offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off


def _stack_col(ws, dev):
    """COL-blocked slices [G, K, N]: one 1D quantization per slice."""
    qs = [nv.quantize_1d(synth.to_bf16(w).to(dev), "col") for w in ws]
    K, N = ws[0].shape
    return nv.QTensor(torch.stack([q.codes for q in qs]), torch.stack([q.scales for q in qs]),
                      torch.cat([q.global_dec for q in qs]), torch.cat([q.amax for q in qs]),
                      K, N, "col")


@pytest.mark.parametrize("b_block", ["2d", "col"])
def test_grouped_dgrad_nn_small_ragged(b_block):
    """dX_e = dY_e W_e, W_e stored [K x N]; dY ROW with stochastic rounding."""
    dev = device()
    counts = [0, 5, 300, 1, 256, 0, 77, 513]
    G, N, K = len(counts), 96, 192
    off = _offsets(counts)
    T = int(off[-1])
    dy = synth.laplace((T, K), 1e-3, 61)
    w = synth.normal((G, K, N), 0.02, 62) * (1 + np.arange(G) % 3).astype(np.float32)[:, None, None]
    qa = nv.quantize_1d(synth.to_bf16(dy).to(dev), "row", "sr", nv.Philox(63))
    qb = nv.quantize_2d(synth.to_bf16(w).to(dev)) if b_block == "2d" else _stack_col(list(w), dev)
    off_d = torch.from_numpy(off).to(dev)
    c = nv.grouped_gemm_nn(qa, qb, off_d, out_dtype=torch.float32)
    cb = nv.grouped_gemm_nn(qa, qb, off_d, out_dtype=torch.bfloat16)
    assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))
    A = to_np(qa)
    for e in range(G):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        Ae = dict(codes=A["codes"][r0:r1], scales=A["scales"][r0:r1], block="row", g=A["g"])
        Be = dict(codes=qb.codes[e].cpu().numpy(), scales=qb.scales[e].cpu().numpy(),
                  block=b_block, g=float(qb.global_dec[e].item()))
        R, D = O.gemm_full("N", "N", r1 - r0, N, K, Ae, Be)
        err = O.gemm_rel_err(c[r0:r1].cpu().numpy(), R, D)
        assert err <= TOL, f"group {e}: {err:.3e}"


def _wgrad_case(counts, M, N, seed, dev, mask=0x3C5A):
    """Per-group token segments padded with zero rows to multiples of 16."""
    counts = np.asarray(counts, dtype=np.int64)
    padded = (counts + 15) // 16 * 16
    off = _offsets(padded)
    total = int(off[-1])
    dy = np.zeros((total, M), dtype=np.float32)
    x = np.zeros((total, N), dtype=np.float32)
    rng = np.random.default_rng(seed)
    for e, c in enumerate(counts):
        k0 = int(off[e])
        dy[k0:k0 + c] = rng.laplace(0.0, 1e-3, (c, M)).astype(np.float32)
        x[k0:k0 + c] = rng.standard_normal((c, N)).astype(np.float32)
    qa = nv.quantize_1d(synth.to_bf16(dy).to(dev), "col", "sr", nv.Philox(seed), mask)
    qb = nv.quantize_1d(synth.to_bf16(x).to(dev), "col", "rne", None, mask)
    return qa, qb, off


def _check_wgrad_group(qa, qb, off, c, e, M, N, rows=None, AB=None):
    k0, k1 = int(off[e]), int(off[e + 1])
    got = c[e].cpu().numpy()
    if k1 == k0:
        assert not got.any(), f"empty group {e} must give zeros"
        return
    A, B = (to_np(qa), to_np(qb)) if AB is None else AB
    Ae = dict(codes=A["codes"][k0:k1], scales=A["scales"][k0 // 16:k1 // 16], block="col", g=A["g"])
    Be = dict(codes=B["codes"][k0:k1], scales=B["scales"][k0 // 16:k1 // 16], block="col", g=B["g"])
    if rows is None:
        R, D = O.gemm_full("T", "N", M, N, k1 - k0, Ae, Be)
        err = O.gemm_rel_err(got, R, D)
    else:
        ii = np.repeat(np.asarray(rows, dtype=np.int64), N)
        jj = np.tile(np.arange(N, dtype=np.int64), len(rows))
        R, D = O.gemm_entries("T", "N", M, N, k1 - k0, Ae, Be, ii, jj)
        err = O.gemm_rel_err(got[ii, jj], R, D)
    assert err <= TOL, f"group {e}: {err:.3e}"


def test_grouped_wgrad_tn_small_ragged():
    """dW_e = dY_e^T X_e over each group's own tokens: empty groups, one-block
    groups, and token counts that leave a partial last stage of 64."""
    dev = device()
    counts = [0, 5, 40, 1, 130, 0, 77, 64, 200, 16]
    M, N = 96, 288
    qa, qb, off = _wgrad_case(counts, M, N, 71, dev)
    c = nv.grouped_gemm_tn(qa, qb, torch.from_numpy(off).to(dev), len(counts))
    for e in range(len(counts)):
        _check_wgrad_group(qa, qb, off, c, e, M, N)


def test_grouped_fprop_accumulate_into_fp32():
    """The grouped fprop's NVFP4_FP32_ACCUMULATE output: C = RN32(C + P), bit
    for bit against the plain fp32 call (partial 128- and 256-row tiles)."""
    counts = [40, 0, 300, 7]
    N, K = 272, 192
    qa, qb, off, p = _grouped_case(counts, N, K, seed=13, out=torch.float32)
    dev = p.device
    c0 = torch.randn(p.shape, generator=torch.Generator(device=dev).manual_seed(3), device=dev)
    c = c0.clone()
    nv.nvfp4_grouped_gemm(len(counts), torch.from_numpy(off).to(dev), int(sum(counts)), N, K,
                          qa.operand(), qb.operand(), c, nv.NVFP4_FP32_ACCUMULATE)
    assert torch.equal(c.view(torch.int32), (c0 + p).view(torch.int32))


def test_grouped_wgrad_tn_accumulate():
    """Accumulating into fp32 main-grad buffers: C[e] = RN32(C[e] + P_e), bit
    for bit against the plain call's P_e, twice in a row; a group with no
    tokens adds +0."""
    dev = device()
    counts = [0, 5, 40, 130, 0, 77]
    M, N = 96, 288
    qa, qb, off = _wgrad_case(counts, M, N, 72, dev)
    offs = torch.from_numpy(off).to(dev)
    p = nv.grouped_gemm_tn(qa, qb, offs, len(counts))
    c0 = torch.randn((len(counts), M, N), generator=torch.Generator(device=dev).manual_seed(5),
                     device=dev)
    c = c0.clone()
    nv.grouped_gemm_tn(qa, qb, offs, len(counts), out=c, accumulate=True)
    assert torch.equal(c.view(torch.int32), (c0 + p).view(torch.int32))
    nv.grouped_gemm_tn(qa, qb, offs, len(counts), out=c, accumulate=True)
    assert torch.equal(c.view(torch.int32), ((c0 + p) + p).view(torch.int32))
    assert torch.equal(p[0], torch.zeros_like(p[0]))


def test_grouped_wgrad_tn_matches_dense_per_group():
    """Each group's result equals the dense TN GEMM on that group's rows when
    the group's token count is a multiple of 64 (bit for bit: same sums in
    the same order)."""
    dev = device()
    counts = [128, 0, 64, 320]
    M, N = 256, 512
    qa, qb, off = _wgrad_case(counts, M, N, 72, dev)
    c = nv.grouped_gemm_tn(qa, qb, torch.from_numpy(off).to(dev), len(counts))
    for e in range(len(counts)):
        k0, k1 = int(off[e]), int(off[e + 1])
        if k1 == k0:
            assert not c[e].any()
            continue
        sa = nv.QTensor(qa.codes[k0:k1], qa.scales[k0 // 16:k1 // 16], qa.global_dec, qa.amax,
                        k1 - k0, M, "col")
        sb = nv.QTensor(qb.codes[k0:k1], qb.scales[k0 // 16:k1 // 16], qb.global_dec, qb.amax,
                        k1 - k0, N, "col")
        d = nv.gemm("T", "N", sa, sb, out_dtype=torch.float32)
        assert torch.equal(d.view(torch.int32), c[e].view(torch.int32)), f"group {e}"


def test_full_grouped_super_backward_sampled():
    """Routed-expert backward at the Super shapes (512 experts, 8192 tokens
    top-22, Zipf 1.1 routing; hidden 2688, latent 1024): grouped dgrad
    dX = dY W (bf16 out) and grouped wgrad dW_e = dY_e^T X_e (fp32 out),
    sampled rows of at least 16 experts spread over the row counts."""
    dev = device()
    counts, tok, _ = synth.zipf_routing(8192, 512, 22, 1.1, 9)
    H, L = 2688, 1024
    # dgrad: dY gathered [T x H] ROW SR, W_e stored [H x L] 2D (the fprop's W_e^T layout)
    off = _offsets(counts)
    T = int(off[-1])
    dy = synth.laplace_device((T, H), 1e-3, 81, dev)
    w = synth.normal_device((512, H, L), 0.02, 82, dev)
    qa = nv.quantize_1d(dy, "row", "sr", nv.Philox(83))
    qw = nv.quantize_2d(w)
    del w
    off_d = torch.from_numpy(off).to(dev)
    dx = nv.grouped_gemm_nn(qa, qw, off_d, out_dtype=torch.float32)
    A = to_np(qa)
    picks = _spread_experts(counts, 16)
    assert len(picks) >= 16
    for e in picks:
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = np.unique(np.linspace(0, r1 - r0 - 1, 6).astype(np.int64))
        Ae = dict(codes=A["codes"][r0:r1], scales=A["scales"][r0:r1], block="row", g=A["g"])
        Be = dict(codes=qw.codes[e].cpu().numpy(), scales=qw.scales[e].cpu().numpy(),
                  block="2d", g=float(qw.global_dec[e].item()))
        ii = np.repeat(rows, L)
        jj = np.tile(np.arange(L, dtype=np.int64), len(rows))
        R, D = O.gemm_entries("N", "N", r1 - r0, L, H, Ae, Be, ii, jj)
        err = O.gemm_rel_err(dx[r0 + ii, jj].cpu().numpy(), R, D)
        assert err <= TOL, f"dgrad expert {e}: {err:.3e}"
    del dx, qa, qw, dy
    torch.cuda.empty_cache()
    # wgrad: per-expert token segments padded to 16; dY and X COL with the transform
    padded = (counts + 15) // 16 * 16
    koff = _offsets(padded)
    KT = int(koff[-1])
    rows_idx = np.concatenate([np.arange(int(koff[e]), int(koff[e]) + int(counts[e]))
                               for e in range(512)])
    dyp = torch.zeros((KT, H), dtype=torch.bfloat16, device=dev)
    xp = torch.zeros((KT, L), dtype=torch.bfloat16, device=dev)
    ridx = torch.from_numpy(rows_idx).to(dev)
    dyp[ridx] = synth.laplace_device((T, H), 1e-3, 84, dev)
    xp[ridx] = synth.normal_device((T, L), 1.0, 85, dev)
    mask = synth.rht_mask(6)
    qa = nv.quantize_1d(dyp, "col", "sr", nv.Philox(86), mask)
    qb = nv.quantize_1d(xp, "col", "rne", None, mask)
    del dyp, xp
    dw = nv.grouped_gemm_tn(qa, qb, torch.from_numpy(koff).to(dev), 512)
    AB = (to_np(qa), to_np(qb))
    for e in picks:
        _check_wgrad_group(qa, qb, koff, dw, e, H, L, rows=[0, 1000, 2687], AB=AB)
