"""Pins for the oracle's Philox4x32 stream (random bits for stochastic rounding).

The ten-round instance is checked against rocRAND's header-only
philox4x32_10 engine compiled for the host, and against the published
known-answer vectors; the round function is shared by every round count, so
this also pins the five-round default.  Uniformity of the 16-bit slots is a
statistical property.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
from _golden import GOLDEN

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    if not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers not present")
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe], check=True)
    return exe


def test_kat_vectors():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for r in rows:
        v = [int(x, 16) for x in r]
        out = O.philox4x32(v[0:4], v[4:6], 10)
        assert list(out) == v[6:10]


def test_ten_rounds_match_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    ins = rng.integers(0, 2**32, size=(2000, 6), dtype=np.uint64)
    ins[:50, :] = 0
    ins[50:100, :] = 2**32 - 1
    text = "\n".join(" ".join(str(int(v)) for v in row) for row in ins) + "\n"
    res = subprocess.run([rocrand_ref], input=text, capture_output=True, text=True, check=True)
    want = np.array([[int(v) for v in l.split()] for l in res.stdout.strip().splitlines()],
                    dtype=np.uint64)
    got = np.array([O.philox4x32(r[:4], r[4:], 10) for r in ins], dtype=np.uint64)
    assert np.array_equal(got, want)


def test_rounds_are_prefixes():
    # R rounds then one more round with the key bumped R times == R+1 rounds:
    # checked indirectly by distinct outputs for every R and by R=0 identity.
    ctr, key = [1, 2, 3, 4], [5, 6]
    assert list(O.philox4x32(ctr, key, 0)) == ctr
    outs = {tuple(O.philox4x32(ctr, key, r)) for r in range(1, 11)}
    assert len(outs) == 10


def test_sr_slot_layout():
    # Element e of block b uses call e>>3 (counter 2b + (e>>3)), word (e>>1)&3,
    # and the low half for even e.
    seed, offset = 0x1234_5678_9ABC_DEF0, 0x0FED_CBA9_8765_4321
    for b in [0, 1, 77, 2**33 + 5]:
        for j in (0, 1):
            n = 2 * b + j
            ctr = [n & 0xFFFFFFFF, n >> 32, offset & 0xFFFFFFFF, offset >> 32]
            key = [seed & 0xFFFFFFFF, seed >> 32]
            out = O.philox4x32(ctr, key, 5)
            for e in range(8 * j, 8 * j + 8):
                w = int(out[(e >> 1) & 3])
                want = (w >> 16) if e & 1 else (w & 0xFFFF)
                assert O.sr_bits(seed, offset, 5, b, e) == want


def test_sr_slots_uniform():
    # chi-square over 256 bins of the top byte of 16-bit slots (5 rounds).
    vals = np.array([O.sr_bits(7, 0, 5, b, e) for b in range(4096) for e in range(16)])
    hist = np.bincount(vals >> 8, minlength=256)
    exp = vals.size / 256
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; 6 sd margin.
    assert chi2 < 255 + 6 * 22.6
    # and the low byte
    hist = np.bincount(vals & 0xFF, minlength=256)
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    assert chi2 < 255 + 6 * 22.6
