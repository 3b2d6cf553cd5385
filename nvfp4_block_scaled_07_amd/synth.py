"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers (numpy ``default_rng``), converts fp32 samples to bf16 bit patterns
(``torch`` round-to-nearest-even cast) and builds the expert routing.  Both
the GPU path and the CPU oracle consume what it produces.

Workload shapes follow the pages: hidden size 6144 and 88 layers for Super,
8192 for Ultra; 512 routed experts with 22 active, latent 1024 / expert
hidden 2688 (Super) and latent 2048 / expert hidden 5120 (Ultra); 8192-token
sequences ("Nemotron 3 Super" summary, gkm0120.cn/p/20617, pretraining-recipe
table; "Nemotron 3 Ultra" summary, gkm0120.cn/p/65339, recipe table).
"""
import numpy as np
import torch


def normal(shape, std, seed):
    """fp32 samples of N(0, std^2), drawn in float64 then rounded to fp32."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


def laplace(shape, b, seed, zero_frac=0.0, zero_seed=None):
    """fp32 Laplace(0, b) samples; optionally a Bernoulli(zero_frac) mask of
    exact zeros drawn from its own seed."""
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, b, size=shape).astype(np.float32)
    if zero_frac > 0.0:
        zrng = np.random.default_rng(zero_seed)
        x[zrng.random(size=shape) < zero_frac] = 0.0
    return x


def to_bf16(x):
    """fp32 numpy -> torch bf16 tensor (RNE), CPU."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t):
    """bf16 torch tensor -> numpy uint16 bit patterns (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rht_mask(seed):
    """A 16-bit random sign mask for the Hadamard transform."""
    return int(np.random.default_rng(seed).integers(0, 65536))


def zipf_routing(tokens, experts, topk, s, seed):
    """Route every token to ``topk`` distinct experts with Zipf(s) popularity.

    Each token takes the top-``topk`` of log(r^-s) + Gumbel noise over the
    expert ranks r = 1..experts (a draw without replacement in proportion to
    r^-s); ranks map to expert ids through a seeded permutation.  Returns
    (counts [experts] int64, token_ids sorted by expert: [tokens*topk] int64,
    offsets [experts+1] int64).
    """
    rng = np.random.default_rng(seed)
    logw = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    perm = rng.permutation(experts)
    chosen = np.empty((tokens, topk), dtype=np.int64)
    chunk = 1024
    for t0 in range(0, tokens, chunk):
        t1 = min(tokens, t0 + chunk)
        g = rng.gumbel(size=(t1 - t0, experts)) + logw[None, :]
        top = np.argpartition(-g, topk - 1, axis=1)[:, :topk]
        chosen[t0:t1] = perm[top]
    flat_e = chosen.reshape(-1)
    flat_t = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.argsort(flat_e, kind="stable")
    counts = np.bincount(flat_e, minlength=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, flat_t[order], offsets


def max_vio(counts, topk):
    """Peak expert load over the balanced mean; at most experts/topk when no
    expert receives a token twice ("Nemotron 3 Ultra" report, section 2.7)."""
    counts = np.asarray(counts, dtype=np.float64)
    return float(counts.max() / counts.mean())


# Workload definitions: shapes, seeds and value distributions of each workload.
WORKLOADS = {
    "tiny": dict(x=(256, 512), a=(256, 256), b=(256, 256)),
    "fprop_super": dict(M=8192, N=6144, K=6144, x_std=1.0, w_std=0.02,
                        x_seed=1, w_seed=2),
    "wgrad_super": dict(tokens=8192, out=6144, inp=6144, dy_b=1e-3,
                        dy_seed=3, zero_frac=0.07, zero_seed=4, x_seed=5,
                        mask_seed=6, philox_seed=7),
    "grouped_super": dict(tokens=8192, latent=1024, hidden=2688, experts=512,
                          topk=22, zipf_s=1.1, x_seed=8, route_seed=9,
                          w_seed=10, w_std=0.02),
    "ultra": dict(M=8192, N=8192, K=8192, x_seed=11, w_seed=12, w_std=0.015,
                  dy_seed=13, dy_b=1e-3, philox_seed=14, glat=2048,
                  ghidden=5120, gx_seed=15, groute_seed=16, gw_seed=17),
}


def normal_device(shape, std, seed, device, dtype=torch.bfloat16):
    """N(0, std^2) drawn by torch's generator on the device (used for large
    benchmark inputs, where host generation would dominate set-up time)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def laplace_from_uniform(r, b):
    """Laplace(0, b) by inverse CDF from uniform draws r in [0, 1) (float64),
    as float32.  |r - 1/2| is kept below 1/2: r = 0 (one draw in 2^24 for
    float32 draws, so several times in any large tensor) would give
    log1p(-1) = -inf, and one infinite element makes a whole tensor's amax,
    scales and codes meaningless."""
    u = r - 0.5
    a = u.abs().clamp_(max=0.5 - 2.0 ** -40)
    return (-b * torch.sign(u) * torch.log1p(-2.0 * a)).to(torch.float32)


def laplace_device(shape, b, seed, device, zero_frac=0.0, dtype=torch.bfloat16):
    """Laplace(0, b) on the device (inverse CDF of a uniform), optionally with
    a Bernoulli(zero_frac) mask of exact zeros."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = laplace_from_uniform(torch.rand(shape, generator=g, device=device, dtype=torch.float64), b)
    if zero_frac > 0.0:
        z = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < zero_frac
        x = x.masked_fill(z, 0.0)
    return x.to(dtype)
