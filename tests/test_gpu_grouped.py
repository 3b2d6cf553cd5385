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


def _check_group(qa, qb, offsets, c, e, N, K, rows=None):
    A = to_np(qa)
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
    counts = [40, 0, 260, 7]
    N, K = 272, 192
    qa, qb, off, c = _grouped_case(counts, N, K, seed=9, out=torch.float32)
    for e, n in enumerate(counts):
        if n == 0:
            continue
        r0 = int(off[e])
        sub = nv.QTensor(qa.codes[r0:r0 + n], qa.scales[r0:r0 + n], qa.global_dec, qa.amax, n, K,
                         "row")
        be = nv.QTensor(qb.codes[e], qb.scales[e], qb.global_dec[e:e + 1], qb.amax[e:e + 1], N, K,
                        "2d")
        d = nv.gemm("N", "T", sub, be, out_dtype=torch.float32)
        assert torch.equal(d, c[r0:r0 + n])


@pytest.mark.parametrize("counts,K", [([40, 0, 260, 7], 192),   # few rows per group: 128-row tiles
                                      ([600, 1100, 0, 700], 256)])  # many: 256-row tiles
def test_grouped_tile_shapes_match_dense(counts, K):
    """Both grouped tile shapes give each group exactly the dense GEMM's bits."""
    N = 272
    qa, qb, off, c = _grouped_case(counts, N, K, seed=11, out=torch.float32)
    for e, n in enumerate(counts):
        if n == 0:
            continue
        _check_group(qa, qb, off, c, e, N, K)
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
    big, small = int(np.argmax(counts)), int(np.argmin(counts))
    for e in sorted({0, 1, big, small, 257, 511}):
        n = int(counts[e])
        _check_group(qa, qb, offsets, c, e, w["hidden"], w["latent"], rows=[0, n // 2, n - 1])
