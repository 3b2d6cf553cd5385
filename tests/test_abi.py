"""The C-ABI library loads and exports every entry point that include/nvfp4.h
declares, and its host-side argument checks reject bad calls with the
documented status codes before touching a device (runs without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.path.join(ROOT, "nvfp4_block_scaled_07_amd", "libnvfp4.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libnvfp4.so not built")
    from nvfp4_block_scaled_07_amd import _binding
    return _binding.load()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ["nvfp4_abi_version", "nvfp4_status_string", "nvfp4_quantize_1d",
              "nvfp4_quantize_2d", "nvfp4_rht16", "nvfp4_dequantize", "nvfp4_gemm",
              "nvfp4_grouped_gemm"]:
        assert f in fns


def test_binding_constants_match_header():
    """The Python binding's enum values are the header's #defines."""
    from nvfp4_block_scaled_07_amd import _binding
    text = open(HEADER).read()
    defs = dict((k, int(v)) for k, v in re.findall(r"#define\s+(NVFP4_[A-Z0-9_]+)\s+\(?(-?\d+)\)?",
                                                   text))
    names = [n for n in dir(_binding) if n.startswith("NVFP4_") and n != "NVFP4Error"]
    assert len(names) >= 14
    for n in names:
        assert defs[n] == getattr(_binding, n), n


def test_every_declared_symbol_is_exported(lib):
    for f in declared_functions():
        assert hasattr(lib, f), f


def test_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == 1
    for s in range(-7, 1):
        assert lib.nvfp4_status_string(s)
    assert b"NaN" in lib.nvfp4_status_string(-7)
    assert lib.nvfp4_status_string(-99) == b"unknown status"


FAKE = C.c_void_p(0x100000)  # never dereferenced: every call below fails validation


def test_quantize_1d_validation(lib):
    q = lib.nvfp4_quantize_1d
    args = lambda **kw: [kw.get("x", FAKE), kw.get("dt", 0), kw.get("rows", 64), kw.get("cols", 64),
                         kw.get("axis", 0), kw.get("rnd", 0), kw.get("rng", None),
                         kw.get("mask", -1), kw.get("amax", FAKE), 0, kw.get("codes", FAKE),
                         kw.get("scales", FAKE), kw.get("g", FAKE), None]
    assert q(*args(x=None)) == -1
    assert q(*args(cols=48)) == -2          # cols % 32
    assert q(*args(axis=1, rows=40)) == -2  # COL needs rows % 16
    assert q(*args(axis=2)) == -4           # 2D goes through quantize_2d
    assert q(*args(rnd=1)) == -1            # SR without a Philox stream
    assert q(*args(mask=0x10000)) == -5
    assert q(*args(dt=7)) == -5
    assert q(*args(x=C.c_void_p(0x100004))) == -3
    assert q(*args(rows=0)) == 0            # empty: nothing to do


def test_quantize_dual_validation(lib):
    from nvfp4_block_scaled_07_amd._binding import _Philox
    f = lib.nvfp4_quantize_dual
    r = C.byref(_Philox(1, 0, 5, 0))
    bad_rounds = C.byref(_Philox(1, 0, 0, 0))
    P = FAKE

    def call(rows=64, cols=128, rr=r, rc=r, mask=0x1234, zeros=P, x=P):
        return f(x, 0, rows, cols, rr, rc, mask, P, 0, P, P, P, P, P, P, zeros, None)

    assert call(rows=40) == -2                   # rows % 16
    assert call(cols=80) == -2                   # cols % 32
    assert call(rr=None) == -1 and call(rc=None) == -1
    assert call(rc=bad_rounds) == -5
    assert call(mask=0x10000) == -5 and call(mask=-2) == -5
    assert call(zeros=C.c_void_p(0x100004)) == -3   # zero_codes needs 8-byte alignment
    assert call(x=None) == -1
    assert call(rows=0) == 0                     # empty: nothing launched
    assert f(P, 7, 64, 128, r, r, -1, P, 0, P, P, P, P, P, P, None, None) == -5  # dtype


def test_quantize_gather_validation(lib):
    """The gathering quantizers: the plain calls' checks plus src_rows >= 1,
    a row index for a non-empty G (8-byte aligned) and rows * cols / 8 <
    2^32."""
    q, d = lib.nvfp4_quantize_1d_gather, lib.nvfp4_quantize_dual_gather

    def q1(src_rows=10, idx=FAKE, rows=32, cols=64, axis=0):
        return q(FAKE, 0, src_rows, idx, rows, cols, axis, 0, None, -1, FAKE, 0, FAKE, FAKE,
                 FAKE, None)

    assert q1(src_rows=0) == -2
    assert q1(idx=None) == -1
    assert q1(idx=C.c_void_p(0x100004)) == -3
    assert q1(rows=1 << 26, cols=1 << 10) == -2        # rows * cols / 8 = 2^33
    assert q1(cols=48) == -2                           # cols % 32
    assert q1(rows=40, axis=1) == -2                   # COL: rows % 16
    assert q1(rows=0, idx=None) == 0                   # empty G: no-op
    from nvfp4_block_scaled_07_amd._binding import _Philox
    r = _Philox(1, 0, 5, 0)

    def q2(src_rows=10, idx=FAKE, rows=32, cols=64):
        return d(FAKE, 0, src_rows, idx, rows, cols, C.byref(r), C.byref(r), -1, FAKE, 0, FAKE,
                 FAKE, FAKE, FAKE, FAKE, FAKE, None, None)

    assert q2(src_rows=0) == -2
    assert q2(idx=None) == -1
    assert q2(rows=40) == -2                           # rows % 16
    assert q2(rows=0, idx=None) == 0


def test_gemm_validation(lib):
    from nvfp4_block_scaled_07_amd._binding import _Operand
    A = _Operand(0x100000, 0x200000, 0x300000, 64, 128, 0, 0)
    B = _Operand(0x100000, 0x200000, 0x300000, 64, 128, 2, 0)
    g = lib.nvfp4_gemm
    assert g(b"T", b"T", 64, 64, 128, C.byref(A), C.byref(B), FAKE, 0, None) == -5
    assert g(b"X", b"T", 64, 64, 128, C.byref(A), C.byref(B), FAKE, 0, None) == -4
    assert g(b"N", b"T", 64, 64, 128, C.byref(A), C.byref(B), FAKE, 3, None) == -5  # c_dtype
    assert g(b"N", b"T", 64, 64, 96, C.byref(A), C.byref(B), FAKE, 2, None) == -2   # accumulate
    assert g(b"N", b"T", 64, 64, 96, C.byref(A), C.byref(B), FAKE, 0, None) == -2   # K % 64
    assert g(b"N", b"T", 64, 64, 128, C.byref(A), C.byref(B), None, 0, None) == -1
    bad = _Operand(0x100000, 0x200000, 0x300000, 64, 128, 1, 0)  # COL blocks on a K-major A
    assert g(b"N", b"T", 64, 64, 128, C.byref(bad), C.byref(B), FAKE, 0, None) == -4
    wrong = _Operand(0x100000, 0x200000, 0x300000, 65, 128, 0, 0)
    assert g(b"N", b"T", 64, 64, 128, C.byref(wrong), C.byref(B), FAKE, 0, None) == -2
    # N < 2^21: a tile's output rows must span fewer than 2^31 bytes
    wide = _Operand(0x100000, 0x200000, 0x300000, 1 << 21, 128, 2, 0)
    assert g(b"N", b"T", 64, 1 << 21, 128, C.byref(A), C.byref(wide), FAKE, 0, None) == -2
    # 32-bit buffer offsets: K < 2^24 for a K-major operand, rows * cols < 2^32
    # for an MN-major one
    K = 1 << 24
    ak = _Operand(0x100000, 0x200000, 0x300000, 64, K, 0, 0)
    bk = _Operand(0x100000, 0x200000, 0x300000, 64, K, 2, 0)
    assert g(b"N", b"T", 64, 64, K, C.byref(ak), C.byref(bk), FAKE, 0, None) == -2
    bn = _Operand(0x100000, 0x200000, 0x300000, 1 << 16, 1 << 16, 2, 0)  # [K x N], 2^32 elements
    an = _Operand(0x100000, 0x200000, 0x300000, 64, 1 << 16, 0, 0)
    assert g(b"N", b"N", 64, 1 << 16, 1 << 16, C.byref(an), C.byref(bn), FAKE, 0, None) == -2
    bn_ok = _Operand(0x100000, 0x200000, 0x300000, 1 << 16, (1 << 16) - 32, 2, 0)
    an0 = _Operand(0x100000, 0x200000, 0x300000, 0, 1 << 16, 0, 0)
    assert g(b"N", b"N", 0, (1 << 16) - 32, 1 << 16, C.byref(an0), C.byref(bn_ok), FAKE, 0,
             None) == 0  # just under the limit; M == 0 returns before any device call


def test_grouped_validation(lib):
    from nvfp4_block_scaled_07_amd._binding import _Operand
    A = _Operand(0x100000, 0x200000, 0x300000, 100, 128, 0, 0)
    B = _Operand(0x100000, 0x200000, 0x300000, 64, 128, 2, 0)
    f = lib.nvfp4_grouped_gemm
    assert f(4, None, 100, 64, 128, C.byref(A), C.byref(B), FAKE, 0, None) == -1
    assert f(5000, FAKE, 100, 64, 128, C.byref(A), C.byref(B), FAKE, 0, None) == -2
    assert f(4, FAKE, 100, 60, 128, C.byref(A), C.byref(B), FAKE, 0, None) == -2
    wide = _Operand(0x100000, 0x200000, 0x300000, 1 << 21, 128, 2, 0)
    assert f(4, FAKE, 100, 1 << 21, 128, C.byref(A), C.byref(wide), FAKE, 0, None) == -2


def test_grouped_backward_validation(lib):
    from nvfp4_block_scaled_07_amd._binding import _Operand
    nn, tn = lib.nvfp4_grouped_gemm_nn, lib.nvfp4_grouped_gemm_tn
    A = _Operand(0x100000, 0x200000, 0x300000, 100, 128, 0, 0)          # dY [100 x 128] ROW
    W = _Operand(0x100000, 0x200000, 0x300000, 128, 64, 2, 0)           # W_e [K=128 x N=64] 2D
    assert nn(4, None, 100, 64, 128, C.byref(A), C.byref(W), FAKE, 0, None) == -1
    assert nn(4, FAKE, 100, 48, 128, C.byref(A), C.byref(W), FAKE, 0, None) == -2  # N % 32
    assert nn(5000, FAKE, 100, 64, 128, C.byref(A), C.byref(W), FAKE, 0, None) == -2
    rowW = _Operand(0x100000, 0x200000, 0x300000, 128, 64, 0, 0)        # ROW blocks along N: wrong
    assert nn(4, FAKE, 100, 64, 128, C.byref(A), C.byref(rowW), FAKE, 0, None) == -4
    dY = _Operand(0x100000, 0x200000, 0x300000, 160, 96, 1, 0)          # [tokens=160 x M=96] COL
    X = _Operand(0x100000, 0x200000, 0x300000, 160, 64, 1, 0)           # [tokens=160 x N=64] COL
    assert tn(4, None, 160, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == -1
    assert tn(4, FAKE, 160, 80, 64, C.byref(dY), C.byref(X), FAKE, None) == -2   # M % 32
    assert tn(4, FAKE, 150, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == -2   # total_k % 16
    rowX = _Operand(0x100000, 0x200000, 0x300000, 160, 64, 0, 0)        # ROW blocks: not along tokens
    assert tn(4, FAKE, 160, 96, 64, C.byref(dY), C.byref(rowX), FAKE, None) == -4
    assert tn(4, C.c_void_p(0x100004), 160, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == -3
    assert tn(0, FAKE, 160, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == 0     # no groups: no-op
    acc = lib.nvfp4_grouped_gemm_tn_accumulate  # same checks, C read and written
    assert acc(4, None, 160, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == -1
    assert acc(4, FAKE, 160, 80, 64, C.byref(dY), C.byref(X), FAKE, None) == -2
    assert acc(4, FAKE, 160, 96, 64, C.byref(dY), C.byref(rowX), FAKE, None) == -4
    assert acc(0, FAKE, 160, 96, 64, C.byref(dY), C.byref(X), FAKE, None) == 0


def test_sr_fp16_validation(lib):
    from nvfp4_block_scaled_07_amd._binding import _Philox
    f = lib.nvfp4_sr_fp16
    r = C.byref(_Philox(1, 0, 5, 0))
    assert f(FAKE, -1, r, FAKE, None) == -2
    assert f(FAKE, 64, None, FAKE, None) == -1
    assert f(FAKE, 64, C.byref(_Philox(1, 0, 17, 0)), FAKE, None) == -5
    assert f(None, 64, r, FAKE, None) == -1
    assert f(C.c_void_p(0x100008), 64, r, FAKE, None) == -3   # x needs 16-byte alignment
    assert f(FAKE, 0, r, None, None) == 0                     # empty: nothing launched


def test_quantize_mse_validation(lib):
    f = lib.nvfp4_quantize_mse
    assert f(FAKE, 0, 64, 80, FAKE, 0, FAKE, FAKE, FAKE, None) == -2   # cols % 32
    assert f(FAKE, 3, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, None) == -5   # dtype
    assert f(None, 0, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 0, 64, 64, FAKE, 0, C.c_void_p(0x100008), FAKE, FAKE, None) == -3
    assert f(FAKE, 0, 0, 64, None, 0, None, None, None, None) == 0


def test_single_pass_wait_setting(lib):
    """The single-pass tuning knob is host state only: it returns the previous
    setting, and any negative value reads back as -1 (off)."""
    prev = lib.nvfp4_set_single_pass_wait(123)
    assert lib.nvfp4_set_single_pass_wait(-7) == 123
    assert lib.nvfp4_set_single_pass_wait(0) == -1
    assert lib.nvfp4_set_single_pass_wait(prev) == 0


def test_debug_checks_setting(lib):
    """The debug switch is host state only: it returns the previous setting,
    normalized to 0 / 1, and starts off."""
    prev = lib.nvfp4_set_debug_checks(5)
    assert prev == 0
    assert lib.nvfp4_set_debug_checks(0) == 1
    assert lib.nvfp4_set_debug_checks(prev) == 0
