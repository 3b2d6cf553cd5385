"""Readers for the hand-written fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def e2m1_values():
    return {int(c, 16): float(v) for c, v in _lines("e2m1_values.txt")}


def e2m1_rne_intervals():
    return [(float(a), float(b), int(lc), int(hc), int(code))
            for a, b, lc, hc, code in _lines("e2m1_rne_intervals.txt")]


def e4m3_examples():
    return [(float(v), int(c, 16)) for v, c in _lines("e4m3_examples.txt")]


def keyed(name):
    out = {}
    for parts in _lines(name):
        out[parts[0]] = parts[1:]
    return out


def quant_example(name):
    d = keyed(name)
    return dict(
        input=np.array([float(v) for v in d["input"]], dtype=np.float32),
        codes=np.array([int(v, 16) for v in d["codes"]], dtype=np.uint8),
        scales=np.array([int(v, 16) for v in d["scales"]], dtype=np.uint8),
        amax=float(d["amax"][0]),
        g=float(d["g"][0]),
    )
