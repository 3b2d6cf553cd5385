#!/usr/bin/env python3
"""Benchmark of the NVFP4 linear-layer hot path on one MI355X.

One step = the fprop of one Super-width linear layer from bf16 inputs:
  quantize X bf16 [8192 x 6144] with 1x16 blocks (RNE),
  quantize W bf16 [6144 x 6144] with 16x16 blocks,
  Y = X W^T with the NVFP4 GEMM (NT), bf16 out.
Inputs are resident in HBM before timing starts; four input sets rotate so
that the 256 MB Infinity Cache cannot serve a step's inputs from the step
before.  The timed steps hold no mark between calls (ms_per_step and value
come from them alone).  The same number of steps then runs again with one
HIP event recorded before every library call, on the stream the library
launches on (torch's current stream); a call's time runs to the next event,
which gives the per-kernel averages used for the roofline fractions (each
holds one event boundary, a few us).  encode_only entries time the encode
pass alone (amax supplied), launches back to back with no mark between
them.

`--rows` adds further rows of the hot path (wgrad with RHT + stochastic
rounding, routed-expert grouped GEMM, Ultra-width fprop/dgrad, the SSM-state
fp16 rounding, the post-training-quantized decode path), each timed the same
way (the decode path from HIP graph replays) and reported under "rows".
Without --rows the Ultra-width fprop/dgrad row is reported.  "context" holds
hipBLASLt's plain bf16/fp16 GEMM rate at the fprop shape (not a target).

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s + quantize GB/s at 1 MI355X, % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
COPY_BYTES = 256 * 1024 * 1024  # calibration copy: reads and writes this many bytes
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
# On a freshly idle MI355X the fprop GEMM's launches run 470 -> 600 us and
# settle at ~458 us only after about 30 of them (~15 ms of MFMA work; hipBLASLt's
# GEMMs show the same ramp), so at least this many untimed steps (settle steps
# plus warm-up steps) run before the timed ones.  The JSON line reports the
# settle steps beside the requested warm-up.
SETTLE_STEPS = 40


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fprop_super_hbm_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_block_scaled_07_amd", "csrc", "gemm.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def q1d_bytes(rows, cols, in_bytes=2):
    return rows * cols * (in_bytes + 0.5 + 1.0 / 16)


def q2d_bytes(rows, cols, in_bytes=2):
    return rows * cols * (in_bytes + 0.5 + 1.0 / 256)


class Timer:
    """Per-label HIP-event durations within a timed region.  One event is
    recorded before each call and a call's duration runs to the next mark
    (the next call's, or the region's closing event), so every call boundary
    holds one event.  A pair of timing events around each call cost about
    10 us of idle GPU per boundary on MI355X (5% of an fprop step); one costs
    about half that.  pairs=True brackets each call instead, for calls with
    other work between them."""

    def __init__(self, torch, pairs=False):
        self.torch = torch
        self.pairs = pairs
        self.enabled = True
        self.pending = []
        self.total = {}
        self.count = {}

    def run(self, label, fn):
        if not self.enabled:
            fn()
            return
        t = self.torch
        e0 = t.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1 = None
        if self.pairs:
            e1 = t.cuda.Event(enable_timing=True)
            e1.record()
        self.pending.append((label, e0, e1))

    def collect(self, end=None):
        """end: the event recorded after the last call (chained mode)."""
        for k, (label, e0, e1) in enumerate(self.pending):
            if e1 is None:
                e1 = self.pending[k + 1][1] if k + 1 < len(self.pending) else end
            self.total[label] = self.total.get(label, 0.0) + e0.elapsed_time(e1)
            self.count[label] = self.count.get(label, 0) + 1
        self.pending = []

    def avg_ms(self, label):
        return self.total[label] / self.count[label]


def fprop_setup(nv, synth, torch, dev, M, N, K, sets, seed0=1):
    xs = [synth.normal_device((M, K), 1.0, seed0 + 2 * i, dev) for i in range(sets)]
    ws = [synth.normal_device((N, K), 0.02, seed0 + 2 * i + 1, dev) for i in range(sets)]
    qx = nv.quantize_1d(xs[0], "row")
    qw = nv.quantize_2d(ws[0])
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    return xs, ws, qx, qw, y


def fprop_step(nv, timer, xs, ws, qx, qw, y, M, N, K, i):
    x, w = xs[i % len(xs)], ws[i % len(ws)]
    timer.run("quantize_1d", lambda: nv.nvfp4_quantize_1d(
        x, nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, qx.amax, False, qx.codes, qx.scales,
        qx.global_dec))
    timer.run("quantize_2d", lambda: nv.nvfp4_quantize_2d(
        w, qw.amax, False, qw.codes, qw.scales, qw.global_dec))
    timer.run("gemm_nt", lambda: nv.nvfp4_gemm("N", "T", M, N, K, qx.operand(), qw.operand(), y,
                                                nv.NVFP4_BF16))


def timed(torch, timer, step, steps, warmup, settle=0):
    """Settle and warm up, then time exactly `steps` steps between two events
    with no mark inside (each mark between calls idles the GPU for a few us);
    then run `steps` more with the timer's per-call marks, which only
    attribute time to the calls (their durations each hold one mark).
    settle: steps run before the warm-up, untimed and unmarked, so that the
    timed steps start at the device's steady clock (see SETTLE_STEPS)."""
    timer.enabled = False
    for i in range(settle):
        step(i)
    timer.enabled = True
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    timer.enabled = False
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(warmup + i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.enabled = True
    timer.pending = []
    for i in range(steps):
        step(warmup + steps + i)
    end = torch.cuda.Event(enable_timing=True)
    end.record()
    torch.cuda.synchronize()
    timer.collect(end)
    return start.elapsed_time(stop) / steps, wall


def kernel_entry(ms, work, kind):
    if kind == "bytes":
        gbs = work / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": int(work)}
    tf = work / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 4), "flops": int(work)}


def back_to_back(torch, call, reps=20):
    """Average ms of call(i) over reps launches in a row, between two events
    (no mark between the calls).  The callers rotate over their input sets so
    that the input comes from HBM, not the Infinity Cache."""
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def encode_only(nv, torch, qx, xs, reps=20):
    """ROW quantize with the amax supplied (the encode pass only)."""
    return back_to_back(torch, lambda i: nv.nvfp4_quantize_1d(
        xs[i % len(xs)], nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, qx.amax, True, qx.codes,
        qx.scales, qx.global_dec), reps)


def gemm_traffic():
    """HBM bytes per NT launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None when that summary is missing or was taken on another version of
    the GEMM source (its sha256 is recorded in the summary)."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    h = re.search(r"source sha256 gemm.hip: ([0-9a-f]{64})", text)
    t = re.search(r"gemm_nt traffic_bytes_per_launch: (\d+)", text)
    if not h or not t or h.group(1) != src:
        return None
    return int(t.group(1))


# ---- CPU baseline: the oracle on a bounded sample of the same step ---------------------------
def cpu_baseline(torch, synth, xs, ws, M, N, K, q_rows=2048, g_rows=128, g1_rows=8):
    """The oracle on fixed slices of the fprop step (about 15 s of host work):
    ROW quantization of q_rows rows of X and 16x16 quantization of q_rows
    rows of W (one core each, amax given: those blocks only see their own
    rows), and the fp64 GEMM reference of g_rows full rows of Y (g_rows x N
    outputs over all of K, OpenMP over all host cores).  Each part is timed
    and scaled to the full step by its share of rows.  The GEMM reference is
    also timed on one core over g1_rows rows, reported beside it."""
    import numpy as np

    import oracle as O
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    xb = synth.bf16_bits(xs[0][:q_rows].cpu())
    wb_all = synth.bf16_bits(ws[0].cpu())
    amax_x = float(xs[0].float().abs().max())
    amax_w = float(ws[0].float().abs().max())

    t0 = time.perf_counter()
    qa = O.quantize(xb, "row", amax=amax_x)
    t_qx = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.quantize(wb_all[:q_rows], "2d", amax=amax_w)
    t_qw = time.perf_counter() - t0
    qw_full = O.quantize(wb_all, "2d", amax=amax_w)  # the GEMM's B (not timed)
    A = dict(codes=qa["codes"], scales=qa["scales"], block="row", g=qa["g"])
    B = dict(codes=qw_full["codes"], scales=qw_full["scales"], block="2d", g=qw_full["g"])

    def gemm_rows(rows):
        ii = np.repeat(np.arange(rows), N)
        jj = np.tile(np.arange(N), rows)
        t0 = time.perf_counter()
        O.gemm_entries("N", "T", q_rows, N, K, A, B, ii, jj)
        return time.perf_counter() - t0

    used = O.set_threads(threads)
    t_g = gemm_rows(g_rows)
    O.set_threads(1)
    t_g1 = gemm_rows(g1_rows)
    O.set_threads(used)
    est = t_qx * (M / q_rows) + t_qw * (N / q_rows) + t_g * (M / g_rows)
    flops = 2.0 * M * N * K
    return {
        "value": round(flops / est / 1e12, 6), "unit": "TFLOP/s", "cores": used,
        "kind": "oracle",
        "sample": (f"oracle ROW quantize of {q_rows} of {M} rows of X and 16x16 quantize of "
                   f"{q_rows} of {N} rows of W (1 core each), fp64 GEMM reference of {g_rows} "
                   f"full rows of Y ({g_rows} x {N} outputs, K = {K}; {used} OpenMP "
                   f"threads); each part scaled to the full step by rows"),
        "est_step_s": round(est, 2),
        "sample_seconds": round(t_qx + t_qw + t_g + t_g1, 2),
        "parts_s": {"quantize_x": round(t_qx, 3), "quantize_w": round(t_qw, 3),
                    "gemm_rows": round(t_g, 3)},
        "gemm_1core": {"rows": g1_rows, "s": round(t_g1, 3),
                       "est_full_gemm_s": round(t_g1 * (M / g1_rows), 1),
                       "speedup_all_cores": round((t_g1 / g1_rows) / (t_g / g_rows), 2)},
    }


def hipblaslt_context(torch, dev, M, N, K, reps=20):
    """Context only: torch.matmul (hipBLASLt) bf16 and fp16 at the same shape
    (plain GEMMs, no decode), TFLOP/s."""
    out = {}
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        a = torch.randn((M, K), device=dev, dtype=dt)
        b = torch.randn((N, K), device=dev, dtype=dt)
        c = torch.empty((M, N), device=dev, dtype=dt)
        for _ in range(3):
            torch.matmul(a, b.t(), out=c)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b.t(), out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"hipblaslt_{name}_tflops"] = round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    return out


# ---- further rows ------------------------------------------------------------------------------
def row_wgrad(nv, synth, torch, dev, steps, warmup):
    T, Mo, Ni = 8192, 6144, 6144
    mask = synth.rht_mask(6)
    dys = [synth.laplace_device((T, Mo), 1e-3, 30 + i, dev, zero_frac=0.07) for i in range(3)]
    xs = [synth.normal_device((T, Ni), 1.0, 40 + i, dev) for i in range(3)]
    qdy = nv.quantize_1d(dys[0], "col", "sr", nv.Philox(7), mask)
    qx = nv.quantize_1d(xs[0], "col", "rne", None, mask)
    dw = torch.empty((Mo, Ni), dtype=torch.float32, device=dev)
    timer = Timer(torch)
    rng = nv.Philox(7)

    def step(i):
        dy, x = dys[i % 3], xs[i % 3]
        rng.offset = i
        timer.run("quantize_col_rht_sr", lambda: nv.nvfp4_quantize_1d(
            dy, nv.NVFP4_BLOCK_COL, nv.NVFP4_SR, rng, mask, qdy.amax, False, qdy.codes,
            qdy.scales, qdy.global_dec))
        timer.run("quantize_col_rht", lambda: nv.nvfp4_quantize_1d(
            x, nv.NVFP4_BLOCK_COL, nv.NVFP4_RNE, None, mask, qx.amax, False, qx.codes, qx.scales,
            qx.global_dec))
        timer.run("gemm_tn", lambda: nv.nvfp4_gemm("T", "N", Mo, Ni, T, qdy.operand(),
                                                    qx.operand(), dw, nv.NVFP4_FP32))

    ms, _ = timed(torch, timer, step, steps, warmup)
    # The encode pass alone (amax supplied), launches back to back.
    enc_sr = back_to_back(torch, lambda i: nv.nvfp4_quantize_1d(
        dys[i % 3], nv.NVFP4_BLOCK_COL, nv.NVFP4_SR, rng, mask, qdy.amax, True, qdy.codes,
        qdy.scales, qdy.global_dec))
    enc_rne = back_to_back(torch, lambda i: nv.nvfp4_quantize_1d(
        xs[i % 3], nv.NVFP4_BLOCK_COL, nv.NVFP4_RNE, None, mask, qx.amax, True, qx.codes,
        qx.scales, qx.global_dec))
    e_sr = kernel_entry(timer.avg_ms("quantize_col_rht_sr"), q1d_bytes(T, Mo), "bytes")
    e_sr["encode_only"] = kernel_entry(enc_sr, q1d_bytes(T, Mo), "bytes")
    e_rne = kernel_entry(timer.avg_ms("quantize_col_rht"), q1d_bytes(T, Ni), "bytes")
    e_rne["encode_only"] = kernel_entry(enc_rne, q1d_bytes(T, Ni), "bytes")
    return {"workload": "wgrad_super: dY, X bf16 [8192x6144] COL+RHT16 (SR on dY) -> dW fp32 TN",
            "ms_per_step": round(ms, 4),
            "quantize_col_rht_sr": e_sr,
            "quantize_col_rht": e_rne,
            "gemm_tn": kernel_entry(timer.avg_ms("gemm_tn"), 2.0 * Mo * Ni * T, "flops")}


def row_dy_dual(nv, synth, torch, dev, steps, warmup):
    """dY of the Super layer quantized for both backward GEMMs from one read
    (ROW+SR for dgrad, COL+RHT+SR for wgrad, zero-code counts), against the
    two separate calls that produce the same bits."""
    T, Mo = 8192, 6144
    mask = synth.rht_mask(6)
    dys = [synth.laplace_device((T, Mo), 1e-3, 30 + i, dev, zero_frac=0.07) for i in range(3)]
    qr, qc, z = nv.quantize_dual(dys[0], nv.Philox(107), nv.Philox(7), mask)
    g = torch.empty(2, dtype=torch.float32, device=dev)
    a = torch.empty(2, dtype=torch.float32, device=dev)
    rr, rc = nv.Philox(107), nv.Philox(7)
    timer = Timer(torch)

    def dual(i):
        rr.offset = rc.offset = i
        dy = dys[i % 3]
        timer.run("quantize_dual", lambda: nv.nvfp4_quantize_dual(
            dy, rr, rc, mask, a, False, qr.codes, qr.scales, g[0:1], qc.codes, qc.scales, g[1:2],
            z))

    def separate(i):
        rr.offset = rc.offset = i
        dy = dys[i % 3]
        timer.run("separate_row_sr", lambda: nv.nvfp4_quantize_1d(
            dy, nv.NVFP4_BLOCK_ROW, nv.NVFP4_SR, rr, -1, a[0:1], False, qr.codes, qr.scales,
            g[0:1]))
        timer.run("separate_col_rht_sr", lambda: nv.nvfp4_quantize_1d(
            dy, nv.NVFP4_BLOCK_COL, nv.NVFP4_SR, rc, mask, a[1:2], False, qc.codes, qc.scales,
            g[1:2]))

    ms, _ = timed(torch, timer, dual, steps, warmup)
    ms_sep, _ = timed(torch, timer, separate, steps, warmup)
    dual(0)
    torch.cuda.synchronize()
    zeros = z.cpu().tolist()
    both = T * Mo * (2 + 2 * (0.5 + 1.0 / 16))  # one read, two sets of codes and scales
    return {"workload": "dy_dual_super: dY bf16 [8192x6144] Laplace(1e-3), 7% zeros -> ROW+SR "
                        "(dgrad) and COL+RHT16+SR (wgrad) from one read",
            "ms_per_step": round(ms, 4), "ms_separate_calls": round(ms_sep, 4),
            "quantize_dual": kernel_entry(timer.avg_ms("quantize_dual"), both, "bytes"),
            "separate_row_sr": kernel_entry(timer.avg_ms("separate_row_sr"), q1d_bytes(T, Mo),
                                            "bytes"),
            "separate_col_rht_sr": kernel_entry(timer.avg_ms("separate_col_rht_sr"),
                                                q1d_bytes(T, Mo), "bytes"),
            "zero_code_fraction": {"row": round(zeros[0] / (T * Mo), 4),
                                   "col_rht": round(zeros[1] / (T * Mo), 4)}}


def row_grouped(nv, synth, torch, dev, steps, warmup, latent=1024, hidden=2688, route_seed=9,
                name="grouped_super"):
    """Routed-expert fprop: token-major X [8192 x latent] dispatched to 22 of
    512 experts and quantized in the same pass (row-index gather, ROW RNE),
    the experts' weights 16x16, then the grouped GEMM.  The gather done
    apart (torch index_select, then the plain quantizer) is timed beside it
    for comparison."""
    counts, tok, offsets = synth.zipf_routing(8192, 512, 22, 1.1, route_seed)
    x = synth.normal_device((8192, latent), 1.0, 8, dev)
    idx = torch.from_numpy(tok).to(dev)
    a = x[idx].contiguous()
    w = synth.normal_device((512, hidden, latent), 0.02, 10, dev)
    qa = nv.quantize_1d(x, "row", row_index=idx)
    qw = nv.quantize_2d(w)
    off = torch.from_numpy(offsets).to(dev)
    total = int(offsets[-1])
    y = torch.empty((total, hidden), dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)

    def step(i):
        timer.run("quantize_1d_gather", lambda: nv.nvfp4_quantize_1d(
            x, nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, qa.amax, False, qa.codes, qa.scales,
            qa.global_dec, row_index=idx))
        timer.run("quantize_2d_experts", lambda: nv.nvfp4_quantize_2d(
            w, qw.amax, False, qw.codes, qw.scales, qw.global_dec))
        timer.run("grouped_gemm", lambda: nv.nvfp4_grouped_gemm(
            512, off, total, hidden, latent, qa.operand(), qw.operand(), y, nv.NVFP4_BF16))

    ms, _ = timed(torch, timer, step, steps, warmup)
    ref = Timer(torch)
    qb = nv.quantize_1d(a, "row")

    def apart(i):
        ref.run("gather_index_select", lambda: torch.index_select(x, 0, idx, out=a))
        ref.run("quantize_1d", lambda: nv.nvfp4_quantize_1d(
            a, nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, qb.amax, False, qb.codes, qb.scales,
            qb.global_dec))

    timed(torch, ref, apart, steps, warmup)
    return {"workload": f"{name}: 8192 tokens top-22 of 512 experts (Zipf 1.1), "
                        f"{latent} -> {hidden}",
            "ms_per_step": round(ms, 4), "max_vio": round(synth.max_vio(counts, 22), 3),
            "rows_per_expert_min_max": [int(counts.min()), int(counts.max())],
            "quantize_1d_gather": kernel_entry(timer.avg_ms("quantize_1d_gather"),
                                               q1d_bytes(total, latent), "bytes"),
            "gather_then_quantize_ms": {
                "index_select": round(ref.avg_ms("gather_index_select"), 5),
                "quantize_1d": round(ref.avg_ms("quantize_1d"), 5)},
            "quantize_2d_experts": kernel_entry(timer.avg_ms("quantize_2d_experts"),
                                                q2d_bytes(512 * hidden, latent), "bytes"),
            "grouped_gemm": kernel_entry(timer.avg_ms("grouped_gemm"),
                                         2.0 * total * hidden * latent, "flops")}


def row_grouped_bwd(nv, synth, torch, dev, steps, warmup, latent=1024, hidden=2688,
                    route_seed=9, name="grouped_bwd_super"):
    """Routed-expert backward of the experts' up projection.  dY arrives in
    expert order ([rows x hidden], unpadded) and is quantized once for both
    GEMMs (ROW+SR for dgrad, COL+RHT+SR for wgrad) with each expert's rows
    padded to 16 by the row-index gather; X is gathered from the token-major
    latent activations and quantized COL+RHT in the same pass.  Then grouped
    dgrad dX = dY W_e (W_e the fprop's 2D codes, stored [hidden x latent])
    and grouped wgrad dW_e = dY_e^T X_e over each expert's own tokens
    (fp32)."""
    import numpy as np
    counts, tok, offsets = synth.zipf_routing(8192, 512, 22, 1.1, route_seed)
    padded = (counts + 15) // 16 * 16
    koff = np.zeros(513, dtype=np.int64)
    koff[1:] = np.cumsum(padded)
    KT = int(koff[-1])
    T = int(offsets[-1])
    idx_dy = np.full(KT, -1, dtype=np.int64)   # padded row -> row of the unpadded dY
    idx_x = np.full(KT, -1, dtype=np.int64)    # padded row -> token
    for e in range(512):
        n = int(counts[e])
        idx_dy[koff[e]:koff[e] + n] = np.arange(offsets[e], offsets[e] + n)
        idx_x[koff[e]:koff[e] + n] = tok[offsets[e]:offsets[e] + n]
    idx_dy = torch.from_numpy(idx_dy).to(dev)
    idx_x = torch.from_numpy(idx_x).to(dev)
    mask = synth.rht_mask(6)
    dy = synth.laplace_device((T, hidden), 1e-3, 91, dev, zero_frac=0.07)
    x = synth.normal_device((8192, latent), 1.0, 92, dev)
    w = synth.normal_device((512, hidden, latent), 0.02, 93, dev)
    qw = nv.quantize_2d(w)
    del w
    qr, qc, z = nv.quantize_dual(dy, nv.Philox(94), nv.Philox(95), mask, row_index=idx_dy)
    qx = nv.quantize_1d(x, "col", "rne", None, mask, row_index=idx_x)
    koff_d = torch.from_numpy(koff).to(dev)
    dx = torch.empty((KT, latent), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((512, hidden, latent), dtype=torch.float32, device=dev)
    g = torch.empty(2, dtype=torch.float32, device=dev)
    a = torch.empty(2, dtype=torch.float32, device=dev)
    rr, rc = nv.Philox(94), nv.Philox(95)
    timer = Timer(torch)

    def step(i):
        rr.offset = rc.offset = i
        timer.run("quantize_dual_dy", lambda: nv.nvfp4_quantize_dual(
            dy, rr, rc, mask, a, False, qr.codes, qr.scales, g[0:1], qc.codes, qc.scales, g[1:2],
            z, row_index=idx_dy))
        timer.run("quantize_col_rht_x", lambda: nv.nvfp4_quantize_1d(
            x, nv.NVFP4_BLOCK_COL, nv.NVFP4_RNE, None, mask, qx.amax, False, qx.codes, qx.scales,
            qx.global_dec, row_index=idx_x))
        # dgrad over the padded rows (the pad rows of dY are zero: their dX rows are 0)
        timer.run("grouped_dgrad_nn", lambda: nv.nvfp4_grouped_gemm_nn(
            512, koff_d, KT, latent, hidden, qr.operand(), qw.operand(), dx, nv.NVFP4_BF16))
        timer.run("grouped_wgrad_tn", lambda: nv.nvfp4_grouped_gemm_tn(
            512, koff_d, KT, hidden, latent, qc.operand(), qx.operand(), dw))

    ms, _ = timed(torch, timer, step, steps, warmup)
    flops = 2.0 * KT * hidden * latent
    return {"workload": f"{name}: 8192 tokens top-22 of 512 experts (Zipf 1.1), expert rows "
                        f"padded to 16 by the gather ({KT} rows); dY [{T} x {hidden}] in expert "
                        f"order, X [8192 x {latent}] token-major",
            "ms_per_step": round(ms, 4),
            "quantize_dual_dy": kernel_entry(timer.avg_ms("quantize_dual_dy"),
                                             T * hidden * 2 + KT * hidden * 2 * (0.5 + 1.0 / 16),
                                             "bytes"),
            "quantize_col_rht_x": kernel_entry(timer.avg_ms("quantize_col_rht_x"),
                                               T * latent * 2 + KT * latent * (0.5 + 1.0 / 16),
                                               "bytes"),
            "grouped_dgrad_nn": kernel_entry(timer.avg_ms("grouped_dgrad_nn"), flops, "flops"),
            "grouped_wgrad_tn": kernel_entry(timer.avg_ms("grouped_wgrad_tn"), flops, "flops")}


def row_ssm_sr(nv, synth, torch, dev, steps, warmup):
    """An SSM-state cache written back in fp16 with Philox<5> stochastic
    rounding: a decode batch's states, 64 x 128 x 64 x 128 fp32 (256 MiB),
    three rotating sets so that each call reads from HBM."""
    shape = (64, 128, 64, 128)
    n = 64 * 128 * 64 * 128
    xs = [synth.normal_device(shape, 1.0, 120 + i, dev, dtype=torch.float32) for i in range(3)]
    y = torch.empty(shape, dtype=torch.float16, device=dev)
    rng = nv.Philox(5)
    timer = Timer(torch)

    def step(i):
        rng.offset = i
        x = xs[i % 3]
        timer.run("sr_fp16", lambda: nv.nvfp4_sr_fp16(x, rng, y))

    ms, _ = timed(torch, timer, step, steps, warmup)
    return {"workload": "ssm_sr: SSM states fp32 [64x128x64x128] -> fp16, Philox<5> stochastic "
                        "rounding",
            "ms_per_step": round(ms, 4),
            "sr_fp16": kernel_entry(timer.avg_ms("sr_fp16"), n * 6.0, "bytes")}


def row_ptq_decode(nv, synth, torch, dev, steps, warmup, layers=16, hidden=6144, batches=(1, 32)):
    """Post-training-quantized decode: Super-width weights W_l [6144 x 6144]
    N(0, 0.02) quantized offline with MSE-calibrated block scales, then per
    decode step and layer the activations X_l [M x 6144] quantized with
    dynamic max-based ROW scales and Y_l = X_l W_l^T (W4A4, small-M kernel).
    Sixteen layers (340 MB of weight codes, more than the 256 MB last-level
    cache) so every GEMM streams its weight from HBM.  Each step is replayed
    from a HIP graph (the kernels take microseconds, less than a Python
    launch); every replay is checked bit for bit against the eager result."""
    N = K = hidden
    ws = []
    timer = Timer(torch, pairs=True)
    for l in range(layers):
        w = synth.normal_device((N, K), 0.02, 300 + l, dev)
        qw = nv.quantize_mse(w)
        timer.run("quantize_mse_w", lambda w=w, qw=qw: nv.nvfp4_quantize_mse(
            w, qw.amax, False, qw.codes, qw.scales, qw.global_dec))
        ws.append(qw)
        del w
    torch.cuda.synchronize()
    timer.collect()
    out = {"workload": f"ptq_decode: {layers} layers W [{N}x{K}] MSE-scaled 1x16 NVFP4, "
                       f"X [M x {K}] max-scaled 1x16, Y = X W^T bf16 (NT, small-M kernel)",
           "layers": layers,
           "quantize_mse_w": kernel_entry(timer.avg_ms("quantize_mse_w"), N * K * 2.0 + N * K / 2
                                          + N * K / 16, "bytes")}
    w_bytes = N * K / 2 + N * K / 16
    for M in batches:
        xs = [synth.normal_device((M, K), 1.0, 400 + l, dev) for l in range(layers)]
        qxs = [nv.quantize_1d(x, "row") for x in xs]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(layers)]

        def quant(l):
            q = qxs[l]
            nv.nvfp4_quantize_1d(xs[l], nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, q.amax, False,
                                 q.codes, q.scales, q.global_dec)

        def gemm(l):
            nv.nvfp4_gemm("N", "T", M, N, K, qxs[l].operand(), ws[l].operand(), ys[l],
                          nv.NVFP4_BF16)

        def step():
            for l in range(layers):
                quant(l)
                gemm(l)

        def gemms():
            for l in range(layers):
                gemm(l)

        step()
        torch.cuda.synchronize()
        ref = [y.clone() for y in ys]
        graphs = {}
        for name, fn in (("step", step), ("gemms", gemms)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs[name] = g
        match = True
        res = {}
        for name, g in graphs.items():
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / steps
            for l in range(layers):
                match = match and torch.equal(ys[l].view(torch.int16), ref[l].view(torch.int16))
            for y in ys:
                y.zero_()
            torch.cuda.synchronize()
        gemm_ms = res["gemms"] / layers
        gemm_bytes = w_bytes + M * K / 2 + M * K / 16 + M * N * 2
        out[f"M{M}"] = {
            "ms_per_step": round(res["step"], 4),
            "tokens_per_s": round(M / (res["step"] * 1e-3), 1),
            "gemm": {**kernel_entry(gemm_ms, gemm_bytes, "bytes"),
                     "TFLOP/s": round(2.0 * M * N * K / (gemm_ms * 1e-3) / 1e12, 2)},
            "quantize_x_ms_per_layer": round((res["step"] - res["gemms"]) / layers, 5),
            "graph_replays_match_eager": bool(match),
        }
        del xs, qxs, ys, ref, graphs
    return out


def row_ultra(nv, synth, torch, dev, steps, warmup):
    M = N = K = 8192
    xs = [synth.normal_device((M, K), 1.0, 11 + i, dev) for i in range(2)]
    w = synth.normal_device((N, K), 0.015, 12, dev)
    dys = [synth.laplace_device((M, N), 1e-3, 13 + i, dev) for i in range(2)]
    qx = nv.quantize_1d(xs[0], "row")
    qw = nv.quantize_2d(w)
    qdy = nv.quantize_1d(dys[0], "row", "sr", nv.Philox(14))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)
    rng = nv.Philox(14)

    def step(i):
        x, dy = xs[i % 2], dys[i % 2]
        rng.offset = i
        timer.run("quantize_x", lambda: nv.nvfp4_quantize_1d(
            x, nv.NVFP4_BLOCK_ROW, nv.NVFP4_RNE, None, -1, qx.amax, False, qx.codes, qx.scales,
            qx.global_dec))
        timer.run("quantize_w", lambda: nv.nvfp4_quantize_2d(
            w, qw.amax, False, qw.codes, qw.scales, qw.global_dec))
        timer.run("quantize_dy_sr", lambda: nv.nvfp4_quantize_1d(
            dy, nv.NVFP4_BLOCK_ROW, nv.NVFP4_SR, rng, -1, qdy.amax, False, qdy.codes, qdy.scales,
            qdy.global_dec))
        timer.run("gemm_nt", lambda: nv.nvfp4_gemm("N", "T", M, N, K, qx.operand(), qw.operand(),
                                                    y, nv.NVFP4_BF16))
        timer.run("gemm_nn", lambda: nv.nvfp4_gemm("N", "N", M, K, N, qdy.operand(),
                                                    qw.operand(), dx, nv.NVFP4_BF16))

    ms, _ = timed(torch, timer, step, steps, warmup)
    return {"workload": "ultra: X, dY bf16 [8192x8192], W [8192x8192]; fprop NT + dgrad NN",
            "ms_per_step": round(ms, 4),
            "quantize_x": kernel_entry(timer.avg_ms("quantize_x"), q1d_bytes(M, K), "bytes"),
            "quantize_w": kernel_entry(timer.avg_ms("quantize_w"), q2d_bytes(N, K), "bytes"),
            "quantize_dy_sr": kernel_entry(timer.avg_ms("quantize_dy_sr"), q1d_bytes(M, N),
                                           "bytes"),
            "gemm_nt": kernel_entry(timer.avg_ms("gemm_nt"), 2.0 * M * N * K, "flops"),
            "gemm_nn": kernel_entry(timer.avg_ms("gemm_nn"), 2.0 * M * N * K, "flops")}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Fewer than SETTLE_STEPS warm-up steps are topped up by settle steps.
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--rows", default="", help="comma list of extra rows: wgrad,dy_dual,grouped,grouped_bwd,ultra,grouped_ultra,ssm_sr,ptq_decode,all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the hipBLASLt context GEMMs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (a known-size kernel for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "libnvfp4 runs on one GPU: the hot path has no "
                                   "multi-GPU mode, so only --gpus 1 is measured",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import nvfp4_block_scaled_07_amd as nv
    from nvfp4_block_scaled_07_amd import synth

    nv.load()  # the HIP library must be present; no fallback
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    M, N, K = 8192, 6144, 6144
    log("generating inputs")
    xs, ws, qx, qw, y = fprop_setup(nv, synth, torch, dev, M, N, K, sets=4)
    timer = Timer(torch)
    settle = max(0, SETTLE_STEPS - args.warmup)
    log(f"timing {args.steps} steps after {settle} settle and {args.warmup} warm-up steps")
    ms, wall = timed(torch, timer,
                     lambda i: fprop_step(nv, timer, xs, ws, qx, qw, y, M, N, K, i),
                     args.steps, args.warmup, settle)
    flops = 2.0 * M * N * K
    g = kernel_entry(timer.avg_ms("gemm_nt"), flops, "flops")
    qx_e = kernel_entry(timer.avg_ms("quantize_1d"), q1d_bytes(M, K), "bytes")
    qw_e = kernel_entry(timer.avg_ms("quantize_2d"), q2d_bytes(N, K), "bytes")
    enc_ms = encode_only(nv, torch, qx, xs)
    qx_e["encode_only"] = kernel_entry(enc_ms, q1d_bytes(M, K), "bytes")
    enc_w = back_to_back(torch, lambda i: nv.nvfp4_quantize_2d(
        ws[i % len(ws)], qw.amax, True, qw.codes, qw.scales, qw.global_dec))
    qw_e["encode_only"] = kernel_entry(enc_w, q2d_bytes(N, K), "bytes")
    out = {
        "metric": METRIC,
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 codes -> f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, on-device generator)",
        "config": {"workload": "fprop_super: X bf16 [8192x6144] 1x16 RNE + W bf16 [6144x6144] "
                               "16x16 + Y = X W^T (NT) bf16", "M": M, "N": N, "K": K,
                   "input_sets_rotated": 4},
        "roofline": {"bound": "mfma", "achieved": g["TFLOP/s"], "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": g["frac_mfma"], "traffic": gemm_traffic(),
                     "kernel": "gemm_kernel NT 256x256 (fp16 MFMA 32x32x16)"},
        "kernels": {"gemm_nt": g, "quantize_1d_x": qx_e, "quantize_2d_w": qw_e},
        "wall_s_timed": round(wall, 3),
    }
    extra = [r.strip() for r in args.rows.split(",") if r.strip()]
    if not args.rows:  # the default run also reports the Ultra-width GEMMs
        extra = ["ultra"]
    if "none" in extra:
        extra = []
    if "all" in extra:
        extra = ["wgrad", "dy_dual", "grouped", "grouped_bwd", "ultra", "grouped_ultra", "ssm_sr",
                 "ptq_decode"]
    rows = {}
    del xs, ws
    torch.cuda.empty_cache()
    for r in extra:
        log(f"row {r}")
        if r == "wgrad":
            rows[r] = row_wgrad(nv, synth, torch, dev, max(5, args.steps // 5), 2)
        elif r == "dy_dual":
            rows[r] = row_dy_dual(nv, synth, torch, dev, max(5, args.steps // 5), 2)
        elif r == "grouped":
            rows[r] = row_grouped(nv, synth, torch, dev, max(5, args.steps // 5), 2)
        elif r == "grouped_bwd":
            rows[r] = row_grouped_bwd(nv, synth, torch, dev, max(3, args.steps // 10), 1)
        elif r == "ssm_sr":
            rows[r] = row_ssm_sr(nv, synth, torch, dev, max(10, args.steps // 2), 2)
        elif r == "ptq_decode":
            rows[r] = row_ptq_decode(nv, synth, torch, dev, max(20, args.steps), 3)
        elif r == "grouped_ultra":
            rows[r] = row_grouped(nv, synth, torch, dev, max(3, args.steps // 10), 1, latent=2048,
                                  hidden=5120, route_seed=16, name="grouped_ultra")
        elif r == "ultra":
            rows[r] = row_ultra(nv, synth, torch, dev, max(5, args.steps // 5), 2)
        torch.cuda.empty_cache()
    if rows:
        out["rows"] = rows
    if not args.no_context:
        log("context: hipBLASLt plain GEMMs at the fprop shape")
        out["context"] = hipblaslt_context(torch, dev, M, N, K)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, bounded sample)")
        xs1 = [synth.normal_device((M, K), 1.0, 1, dev)]
        ws1 = [synth.normal_device((N, K), 0.02, 2, dev)]
        out["cpu_baseline"] = cpu_baseline(torch, synth, xs1, ws1, M, N, K)
        del xs1, ws1
    # Leave nothing queued or allocated on the device before the interpreter
    # exits (the exit handlers of the HIP runtime, of libnvfp4's code-object
    # registration and of a profiler's tool then find an idle device).
    del qx, qw, y, timer
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
