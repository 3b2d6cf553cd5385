"""On-device proof that the quantizers round every element and every block
scale exactly as the format definitions say, swept over every fp32 input in
the range that matters, through the public ABI (nvfp4_quantize_1d, fp32
input, ROW blocks).  Elements are E2M1 and block scales E4M3 (Super summary,
pretraining-recipe table); the kernels round both with gfx950's conversion
instructions, so these sweeps are what ties them to the definitions.  Each
result is compared with the oracle's brute-force encoders (nearest value by
distance, ties to the even code, saturation), element by element.

* E2M1, unit-scale blocks: one block holds 2688, so the tensor amax A = 2688
  gives S = 1, k = RN32(1/6), g = 1; every other block holds 6.25, so its
  scale s = RN32(6.25 k) rounds to the E4M3 value 1.0 and r = 1: y = x.  The
  other 15 elements of those blocks sweep every fp32 in [0, 6.25] (both
  signs; above 6 the code saturates).
* E4M3, unit-k blocks: one block holds 448, so A = 448 gives S = 6, k = 1 and
  s = a exactly: block b = [a_b, 0 x 15] has the scale code E4M3(a_b).  a_b
  sweeps every fp32 in [0, 448] (at 448: the saturating end).

Inputs are built on the host (arange over fp32 bit patterns) in chunks, so
memory stays bounded; each chunk prints a progress line.
"""
import sys

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import oracle as O
from _gpu import device

pytestmark = pytest.mark.gpu

COLS = 4096  # 256 blocks per row


def _codes_of(q, rows):
    c = q.codes.cpu().numpy().reshape(rows, COLS // 2)
    return np.stack([c & 0xF, c >> 4], axis=-1).reshape(rows, COLS)


def _progress(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


@pytest.mark.parametrize("sign", [0, 1])
def test_e2m1_rne_every_fp32_in_range(sign):
    dev = device()
    hi_bits = int(np.float32(6.25).view(np.uint32))
    total = hi_bits + 1                          # bit patterns 0 .. 6.25
    per_chunk = 15 * (1 << 23)                   # values per launch (divisible by 15)
    done = 0
    while done < total:
        n = min(per_chunk, total - done)
        bits = np.arange(done, done + n, dtype=np.uint32) | np.uint32(sign << 31)
        vals = bits.view(np.float32)
        nb = (n + 14) // 15                      # sweep blocks
        rows = (nb + 1 + 255) // 256             # + the 2688 block, whole rows
        x = np.zeros((rows * 256, 16), dtype=np.float32)
        x[0, 0] = 2688.0
        x[1:, 0] = 6.25                          # every other block: max 6.25
        body = np.zeros(nb * 15, dtype=np.float32)
        body[:n] = vals
        x[1:nb + 1, 1:] = body.reshape(nb, 15)
        x = x.reshape(rows, COLS)
        q = nv.quantize_1d(torch.from_numpy(x).to(dev), "row")
        torch.cuda.synchronize()
        assert q.global_dec.item() == 1.0
        sc = q.scales.cpu().numpy().reshape(-1)
        assert sc[0] == 0x7E and np.all(sc[1:] == 0x38), "unit-scale set-up"
        got = _codes_of(q, rows).reshape(-1, 16)[1:nb + 1, 1:].reshape(-1)[:n]
        want = O.e2m1_encode_rne_array(vals)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} mismatches, first x = {vals[bad[0]]!r}: "
                               f"got {got[bad[0]]} want {want[bad[0]]}")
        done += n
        _progress(f"e2m1 sign {sign}: {done}/{total} values bit-exact")


def test_e4m3_scale_every_fp32_in_range():
    dev = device()
    hi_bits = int(np.float32(448.0).view(np.uint32))
    total = hi_bits + 1                          # bit patterns 0 .. 448
    per_chunk = 1 << 26                          # blocks per launch
    done = 0
    while done < total:
        n = min(per_chunk, total - done)
        a = np.arange(done, done + n, dtype=np.uint32).view(np.float32)
        rows = (n + 1 + 255) // 256
        x = torch.zeros((rows * 256, 16), dtype=torch.float32, device=dev)
        x[0, 0] = 448.0
        x[1:n + 1, 0] = torch.from_numpy(a).to(dev)
        q = nv.quantize_1d(x.view(rows, COLS), "row")
        torch.cuda.synchronize()
        assert q.global_dec.item() == np.float32(448.0) / np.float32(2688.0)
        got = q.scales.cpu().numpy().reshape(-1)[1:n + 1]
        del x, q
        want = O.e4m3_encode_array(a)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} mismatches, first s = {a[bad[0]]!r}: "
                               f"got {got[bad[0]]:#x} want {want[bad[0]]:#x}")
        done += n
        _progress(f"e4m3: {done}/{total} block maxima bit-exact")
