"""CPU oracle for the NVFP4 linear-layer hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or calls it, and the two share no code.

This module is a thin ctypes wrapper over ``oracle/oracle.c`` (plain C, built
by ``oracle/build.py``).  Arrays are numpy; bf16 tensors are passed as their
raw ``uint16`` bit patterns.  See ``oracle.h`` for the definitions and the
page passages they follow.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

ROW, COL, BLOCK_2D = 0, 1, 2
RNE, SR = 0, 1
BLOCK_NAMES = {"row": ROW, "col": COL, "2d": BLOCK_2D}

_lib = None


def lib():
    """Load liboracle.so, building it first when it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        u8, u32, i32, i64, u64 = C.c_uint8, C.c_uint32, C.c_int32, C.c_int64, C.c_uint64
        vp, fp, dp = C.c_void_p, C.POINTER(C.c_float), C.POINTER(C.c_double)
        L.oracle_e2m1_decode.restype = C.c_float
        L.oracle_e2m1_decode.argtypes = [u8]
        L.oracle_e2m1_encode_rne.restype = u8
        L.oracle_e2m1_encode_rne.argtypes = [C.c_float]
        L.oracle_e2m1_encode_sr.restype = u8
        L.oracle_e2m1_encode_sr.argtypes = [C.c_float, u32]
        L.oracle_e4m3_decode.restype = C.c_float
        L.oracle_e4m3_decode.argtypes = [u8]
        L.oracle_e4m3_encode_rne_sat.restype = u8
        L.oracle_e4m3_encode_rne_sat.argtypes = [C.c_float]
        L.oracle_e2m1_encode_rne_n.restype = None
        L.oracle_e2m1_encode_rne_n.argtypes = [vp, i64, vp]
        L.oracle_e4m3_encode_rne_sat_n.restype = None
        L.oracle_e4m3_encode_rne_sat_n.argtypes = [vp, i64, vp]
        L.oracle_philox4x32.restype = None
        L.oracle_philox4x32.argtypes = [vp, vp, u32, vp]
        L.oracle_sr_bits.restype = u32
        L.oracle_sr_bits.argtypes = [u64, u64, u32, u64, C.c_int]
        L.oracle_rht16_vec.restype = None
        L.oracle_rht16_vec.argtypes = [vp, u32]
        L.oracle_global_scales.restype = None
        L.oracle_global_scales.argtypes = [C.c_float, fp, fp, fp]
        L.oracle_quantize_rows.restype = C.c_int
        L.oracle_quantize_rows.argtypes = [vp, C.c_int, i64, i64, i64, C.c_int, C.c_int,
                                           u64, u64, u32, i32, vp, i64, i64, vp, vp, vp, vp]
        L.oracle_amax.restype = C.c_int
        L.oracle_amax.argtypes = [vp, C.c_int, i64, i64, i64, C.c_int, i32, vp]
        L.oracle_rht16.restype = C.c_int
        L.oracle_rht16.argtypes = [vp, C.c_int, i64, i64, C.c_int, u32, vp]
        L.oracle_quantize_mse.restype = C.c_int
        L.oracle_quantize_mse.argtypes = [vp, C.c_int, i64, i64, vp, vp, vp, vp, vp]
        L.oracle_sr_fp16_one.restype = C.c_uint16
        L.oracle_sr_fp16_one.argtypes = [C.c_float, u32]
        L.oracle_sr_fp16.restype = None
        L.oracle_sr_fp16.argtypes = [vp, i64, u64, u64, u32, vp]
        L.oracle_dequantize.restype = C.c_int
        L.oracle_dequantize.argtypes = [vp, vp, C.c_float, i64, i64, C.c_int, vp]
        L.oracle_gemm_entries.restype = C.c_int
        L.oracle_gemm_entries.argtypes = [C.c_char, C.c_char, i64, i64, i64,
                                          vp, vp, C.c_int, C.c_float,
                                          vp, vp, C.c_int, C.c_float,
                                          vp, vp, i64, vp, vp]
        L.oracle_set_threads.restype = C.c_int
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_gemm_full.restype = C.c_int
        L.oracle_gemm_full.argtypes = [C.c_char, C.c_char, i64, i64, i64,
                                       vp, vp, C.c_int, C.c_float,
                                       vp, vp, C.c_int, C.c_float, vp, vp]
        _lib = L
    return _lib


def _ptr(a):
    return C.c_void_p(a.ctypes.data) if a is not None else None


def _block(b):
    return BLOCK_NAMES[b] if isinstance(b, str) else int(b)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} returned {rc}")


# ---- element formats --------------------------------------------------------
def e2m1_decode(code):
    return lib().oracle_e2m1_decode(int(code))


def e2m1_encode_rne(y):
    return lib().oracle_e2m1_encode_rne(float(y))


def e2m1_encode_sr(y, u16):
    return lib().oracle_e2m1_encode_sr(float(y), int(u16))


def e4m3_decode(e):
    return lib().oracle_e4m3_decode(int(e))


def e4m3_encode(s):
    return lib().oracle_e4m3_encode_rne_sat(float(s))


def e2m1_encode_rne_array(y):
    """oracle_e2m1_encode_rne on every element of a float32 array (uint8
    codes: sign bit 8, magnitude index 0..7)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().oracle_e2m1_encode_rne_n(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode_array(s):
    """oracle_e4m3_encode_rne_sat on every element of a float32 array."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_rne_sat_n(_ptr(s), s.size, _ptr(out))
    return out


def philox4x32(ctr, key, rounds):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32(_ptr(c), _ptr(k), int(rounds), _ptr(out))
    return out


def sr_bits(seed, offset, rounds, block, e):
    return lib().oracle_sr_bits(int(seed), int(offset), int(rounds), int(block), int(e))


def rht16_vec(v, mask):
    a = np.array(v, dtype=np.float32).copy()
    assert a.shape == (16,)
    lib().oracle_rht16_vec(_ptr(a), int(mask))
    return a


def global_scales(amax):
    S, k, g = C.c_float(), C.c_float(), C.c_float()
    lib().oracle_global_scales(float(amax), C.byref(S), C.byref(k), C.byref(g))
    return np.float32(S.value), np.float32(k.value), np.float32(g.value)


# ---- tensors -----------------------------------------------------------------
def _as_input(x):
    """Return (contiguous array, is_bf16, batch, rows, cols)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        is_bf16 = 1
    elif x.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("oracle input must be uint16 (bf16 bits) or float32")
    if x.ndim == 2:
        return x, is_bf16, 1, x.shape[0], x.shape[1]
    if x.ndim == 3:
        return x, is_bf16, x.shape[0], x.shape[1], x.shape[2]
    raise ValueError("2-D or 3-D input expected")


def scale_shape(block, rows, cols):
    block = _block(block)
    if block == ROW:
        return (rows, cols // 16)
    if block == COL:
        return (rows // 16, cols)
    return (rows // 16, cols // 16)


def quantize(x, block, rounding=RNE, seed=0, offset=0, rounds=5, rht_mask=-1,
             amax=None, row_begin=None, row_end=None, out=None):
    """Quantize a 2-D tensor or a batch of 2-D slices (see oracle_quantize).

    Returns dict(codes, scales, amax, g).  ``row_begin/row_end`` restrict the
    work to a window of rows (then ``amax`` must be given); ``out`` may pass
    preallocated codes/scales arrays to fill.
    """
    x, is_bf16, batch, rows, cols = _as_input(x)
    block = _block(block)
    lead = x.shape[:-2]
    if out is None:
        codes = np.zeros(lead + (rows, cols // 2), dtype=np.uint8)
        scales = np.zeros(lead + scale_shape(block, rows, cols), dtype=np.uint8)
    else:
        codes, scales = out["codes"], out["scales"]
    amax_out = np.zeros(batch, dtype=np.float32)
    g = np.zeros(batch, dtype=np.float32)
    amax_in = None if amax is None else np.ascontiguousarray(
        np.broadcast_to(np.asarray(amax, dtype=np.float32), (batch,)))
    rb = 0 if row_begin is None else row_begin
    re = rows if row_end is None else row_end
    rc = lib().oracle_quantize_rows(_ptr(x), is_bf16, batch, rows, cols, block, int(rounding),
                                    int(seed), int(offset), int(rounds), int(rht_mask),
                                    _ptr(amax_in), rb, re, _ptr(codes), _ptr(scales),
                                    _ptr(amax_out), _ptr(g))
    _check(rc, "quantize")
    if x.ndim == 2:
        return dict(codes=codes, scales=scales, amax=amax_out[0], g=g[0])
    return dict(codes=codes, scales=scales, amax=amax_out, g=g)


def gather_rows(x, row_index):
    """The tensor a gathering quantizer quantizes: row r is x[row_index[r]],
    or a row of zeros when row_index[r] lies outside [0, len(x)) -- the MoE
    token dispatch, with the padding that rounds each expert's rows up to a
    multiple of 16 (Super report summary, sections 2.1-2.2).  Works on fp32
    arrays and on bf16 bit patterns (uint16; zero bits are +0.0)."""
    x = np.asarray(x)
    idx = np.asarray(row_index, dtype=np.int64)
    out = np.zeros((idx.shape[0],) + x.shape[1:], dtype=x.dtype)
    ok = (idx >= 0) & (idx < x.shape[0])
    out[ok] = x[idx[ok]]
    return out


def quantize_gather(x, row_index, block, **kw):
    """quantize() of gather_rows(x, row_index): the gathered tensor's own
    amax, scales and Philox block ids (by gathered position)."""
    return quantize(gather_rows(x, row_index), block, **kw)


def quantize_mse(x, amax=None):
    """PTQ weight quantization: ROW blocks, RNE, MSE-calibrated block scales
    (see oracle_quantize_mse).  Returns dict(codes, scales, amax, g)."""
    x, is_bf16, batch, rows, cols = _as_input(x)
    assert batch == 1 and x.ndim == 2
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    a_out = np.zeros(1, dtype=np.float32)
    g = np.zeros(1, dtype=np.float32)
    a_in = None if amax is None else np.array([amax], dtype=np.float32)
    _check(lib().oracle_quantize_mse(_ptr(x), is_bf16, rows, cols, _ptr(a_in), _ptr(codes),
                                     _ptr(scales), _ptr(a_out), _ptr(g)), "quantize_mse")
    return dict(codes=codes, scales=scales, amax=a_out[0], g=g[0])


def sr_fp16_one(x, u16):
    """fp16 bits of x rounded stochastically with the 16-bit value u16."""
    return int(lib().oracle_sr_fp16_one(float(np.float32(x)), int(u16)))


def sr_fp16(x, seed, offset=0, rounds=5):
    """fp32 array -> fp16 bit patterns (uint16), stochastic rounding with the
    Philox stream (seed, offset, rounds): the SSM-state cache recipe."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    y = np.zeros(x.shape, dtype=np.uint16)
    lib().oracle_sr_fp16(_ptr(x), x.size, int(seed), int(offset), int(rounds), _ptr(y))
    return y


def zero_codes(codes):
    """Number of codes of magnitude zero (0x0 or 0x8) in packed codes, two per
    byte: the count behind the share of zero-valued gradient elements that the
    Super report summary, section 2.2 (NVFP4 pretraining), watches."""
    c = np.asarray(codes, dtype=np.uint8)
    return int(np.count_nonzero((c & 0x7) == 0) + np.count_nonzero(((c >> 4) & 0x7) == 0))


def amax(x, block=ROW, rht_mask=-1):
    x, is_bf16, batch, rows, cols = _as_input(x)
    out = np.zeros(batch, dtype=np.float32)
    _check(lib().oracle_amax(_ptr(x), is_bf16, batch, rows, cols, _block(block),
                             int(rht_mask), _ptr(out)), "amax")
    return out[0] if x.ndim == 2 else out


def rht16(x, block, mask):
    x, is_bf16, batch, rows, cols = _as_input(x)
    assert batch == 1 and x.ndim == 2
    y = np.zeros((rows, cols), dtype=np.float32)
    _check(lib().oracle_rht16(_ptr(x), is_bf16, rows, cols, _block(block), int(mask), _ptr(y)),
           "rht16")
    return y


def dequantize(codes, scales, g, block):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = np.zeros((rows, cols), dtype=np.float32)
    _check(lib().oracle_dequantize(_ptr(codes), _ptr(scales), float(g), rows, cols,
                                   _block(block), _ptr(y)), "dequantize")
    return y


def _operand(q):
    return (np.ascontiguousarray(q["codes"], dtype=np.uint8),
            np.ascontiguousarray(q["scales"], dtype=np.uint8),
            _block(q["block"]), float(q["g"]))


def gemm_entries(opA, opB, M, N, K, A, B, ii, jj):
    """fp64 reference R and magnitude sum D at the (ii[t], jj[t]) outputs.

    A and B are dicts with codes, scales, block ("row"/"col"/"2d") and g.
    """
    ac, asc, ab, ag = _operand(A)
    bc, bsc, bb, bg = _operand(B)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.shape[0]
    R = np.zeros(n, dtype=np.float64)
    D = np.zeros(n, dtype=np.float64)
    rc = lib().oracle_gemm_entries(opA.encode(), opB.encode(), M, N, K, _ptr(ac), _ptr(asc), ab,
                                   ag, _ptr(bc), _ptr(bsc), bb, bg, _ptr(ii), _ptr(jj), n,
                                   _ptr(R), _ptr(D))
    _check(rc, "gemm_entries")
    return R, D


def set_threads(n):
    """OpenMP threads of the oracle's parallel loops for later calls from this
    thread (n <= 0: unchanged); returns the count in force."""
    return lib().oracle_set_threads(int(n))


def gemm_full(opA, opB, M, N, K, A, B):
    ac, asc, ab, ag = _operand(A)
    bc, bsc, bb, bg = _operand(B)
    R = np.zeros((M, N), dtype=np.float64)
    D = np.zeros((M, N), dtype=np.float64)
    rc = lib().oracle_gemm_full(opA.encode(), opB.encode(), M, N, K, _ptr(ac), _ptr(asc), ab, ag,
                                _ptr(bc), _ptr(bsc), bb, bg, _ptr(R), _ptr(D))
    _check(rc, "gemm_full")
    return R, D


def gemm_rel_err(C, R, D):
    """Componentwise error max |C - R| / D (0/0 counts as 0; x/0 as inf)."""
    C = np.asarray(C, dtype=np.float64)
    diff = np.abs(C - R)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(D > 0, diff / np.where(D > 0, D, 1.0), np.where(diff == 0, 0.0, np.inf))
    return float(e.max()) if e.size else 0.0
