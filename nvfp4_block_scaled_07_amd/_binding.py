"""ctypes binding of libnvfp4 (argument marshalling only).

Tensors are torch CUDA (HIP) tensors; their ``data_ptr()`` values are passed as
device pointers and torch's current stream as the HIP stream.  Every value the
method computes is computed by the library's kernels.
"""
import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

NVFP4_BF16, NVFP4_FP32, NVFP4_FP32_ACCUMULATE = 0, 1, 2
NVFP4_RNE, NVFP4_SR = 0, 1
NVFP4_BLOCK_ROW, NVFP4_BLOCK_COL, NVFP4_BLOCK_2D = 0, 1, 2
NVFP4_OK, NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN = 0, -1, -2, -3
NVFP4_ERR_LAYOUT, NVFP4_ERR_UNSUPPORTED, NVFP4_ERR_DEVICE = -4, -5, -6
NVFP4_ERR_NONFINITE = -7
_BLOCKS = {"row": NVFP4_BLOCK_ROW, "col": NVFP4_BLOCK_COL, "2d": NVFP4_BLOCK_2D}
_BLOCK_NAMES = {v: k for k, v in _BLOCKS.items()}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "libnvfp4.so")


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({nvfp4_status_string(status)})")
        self.status = status


class _Philox(C.Structure):
    _fields_ = [("seed", C.c_uint64), ("offset", C.c_uint64), ("rounds", C.c_uint32),
                ("reserved", C.c_uint32)]


class _Operand(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("global_dec", C.c_void_p),
                ("rows", C.c_int64), ("cols", C.c_int64), ("block", C.c_int32),
                ("reserved", C.c_int32)]


_lib = None


def load():
    """Load libnvfp4.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libnvfp4.so not built ({path}); run __graft_entry__.build()")
    L = C.CDLL(path)
    i32, i64, vp = C.c_int32, C.c_int64, C.c_void_p
    L.nvfp4_abi_version.restype = i32
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_status_string.restype = C.c_char_p
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_quantize_1d.restype = i32
    L.nvfp4_quantize_1d.argtypes = [vp, i32, i64, i64, i32, i32, C.POINTER(_Philox), i32, vp, i32,
                                     vp, vp, vp, vp]
    L.nvfp4_quantize_dual.restype = i32
    L.nvfp4_quantize_dual.argtypes = [vp, i32, i64, i64, C.POINTER(_Philox), C.POINTER(_Philox),
                                       i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.nvfp4_quantize_1d_gather.restype = i32
    L.nvfp4_quantize_1d_gather.argtypes = [vp, i32, i64, vp, i64, i64, i32, i32,
                                           C.POINTER(_Philox), i32, vp, i32, vp, vp, vp, vp]
    L.nvfp4_quantize_dual_gather.restype = i32
    L.nvfp4_quantize_dual_gather.argtypes = [vp, i32, i64, vp, i64, i64, C.POINTER(_Philox),
                                             C.POINTER(_Philox), i32, vp, i32, vp, vp, vp, vp,
                                             vp, vp, vp, vp]
    L.nvfp4_quantize_mse.restype = i32
    L.nvfp4_quantize_mse.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp, vp]
    L.nvfp4_quantize_2d.restype = i32
    L.nvfp4_quantize_2d.argtypes = [vp, i32, i64, i64, i64, vp, i32, vp, vp, vp, vp]
    L.nvfp4_rht16.restype = i32
    L.nvfp4_rht16.argtypes = [vp, i32, i64, i64, i32, C.c_uint32, vp, vp]
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_dequantize.argtypes = [C.POINTER(_Operand), vp, vp]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm.argtypes = [C.c_char, C.c_char, i64, i64, i64, C.POINTER(_Operand),
                             C.POINTER(_Operand), vp, i32, vp]
    L.nvfp4_grouped_gemm.restype = i32
    L.nvfp4_grouped_gemm.argtypes = [i64, vp, i64, i64, i64, C.POINTER(_Operand),
                                     C.POINTER(_Operand), vp, i32, vp]
    L.nvfp4_sr_fp16.restype = i32
    L.nvfp4_sr_fp16.argtypes = [vp, i64, C.POINTER(_Philox), vp, vp]
    L.nvfp4_grouped_gemm_nn.restype = i32
    L.nvfp4_grouped_gemm_nn.argtypes = [i64, vp, i64, i64, i64, C.POINTER(_Operand),
                                        C.POINTER(_Operand), vp, i32, vp]
    L.nvfp4_grouped_gemm_tn.restype = i32
    L.nvfp4_grouped_gemm_tn.argtypes = [i64, vp, i64, i64, i64, C.POINTER(_Operand),
                                        C.POINTER(_Operand), vp, vp]
    L.nvfp4_grouped_gemm_tn_accumulate.restype = i32
    L.nvfp4_grouped_gemm_tn_accumulate.argtypes = [i64, vp, i64, i64, i64, C.POINTER(_Operand),
                                                   C.POINTER(_Operand), vp, vp]
    L.nvfp4_set_single_pass_wait.restype = i32
    L.nvfp4_set_single_pass_wait.argtypes = [i32]
    L.nvfp4_set_debug_checks.restype = i32
    L.nvfp4_set_debug_checks.argtypes = [i32]
    _lib = L
    return L


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return NVFP4_BF16
    if t.dtype == torch.float32:
        return NVFP4_FP32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _check(fn, status):
    if status != 0:
        raise NVFP4Error(fn, status)


@dataclass
class Philox:
    seed: int
    offset: int = 0
    rounds: int = 5


@dataclass
class QTensor:
    """A quantized tensor (one slice, or a batch of 2D-blocked slices)."""
    codes: torch.Tensor        # uint8 [(batch,) rows, cols/2]
    scales: torch.Tensor       # uint8, layout per block kind
    global_dec: torch.Tensor   # float32 [batch] (batch = 1 for 1D)
    amax: torch.Tensor         # float32 [batch]
    rows: int
    cols: int
    block: str                 # "row" | "col" | "2d"

    def operand(self, index=None):
        """The C operand struct for the whole tensor (or slice ``index``)."""
        codes, scales, g = self.codes, self.scales, self.global_dec
        if index is not None:
            codes, scales, g = codes[index], scales[index], g[index:index + 1]
        return _Operand(codes.data_ptr(), scales.data_ptr(), g.data_ptr(), self.rows, self.cols,
                        _BLOCKS[self.block], 0)


# ---- one-to-one mirrors of the C entry points ------------------------------------------
def nvfp4_set_single_pass_wait(wait_us):
    """Grid-barrier wait of the single-pass quantizers in microseconds (< 0:
    single-pass kernels off); returns the previous setting."""
    return load().nvfp4_set_single_pass_wait(int(wait_us))


def nvfp4_set_debug_checks(on):
    """Debug mode: quantizers first check their input for infinities and NaNs
    (NVFP4_ERR_NONFINITE); returns the previous setting."""
    return load().nvfp4_set_debug_checks(1 if on else 0)


def nvfp4_abi_version():
    return load().nvfp4_abi_version()


def nvfp4_status_string(status):
    try:
        return load().nvfp4_status_string(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def nvfp4_quantize_1d(x, axis, rounding, rng, rht_sign_mask, amax, amax_is_input, codes, scales,
                      global_dec, stream=None, row_index=None):
    """row_index (device int64): quantize the rows x[row_index] (indices
    outside [0, len(x)) give zero rows) through nvfp4_quantize_1d_gather."""
    src_rows, cols = x.shape
    ph = None if rng is None else C.byref(_Philox(rng.seed, rng.offset, rng.rounds, 0))
    if row_index is None:
        st = load().nvfp4_quantize_1d(_p(x), _dtype_code(x), src_rows, cols, int(axis),
                                      int(rounding), ph, int(rht_sign_mask), _p(amax),
                                      int(bool(amax_is_input)), _p(codes), _p(scales),
                                      _p(global_dec), _stream(stream))
        _check("nvfp4_quantize_1d", st)
        return
    st = load().nvfp4_quantize_1d_gather(_p(x), _dtype_code(x), src_rows, _p(row_index),
                                         row_index.numel(), cols, int(axis), int(rounding), ph,
                                         int(rht_sign_mask), _p(amax), int(bool(amax_is_input)),
                                         _p(codes), _p(scales), _p(global_dec), _stream(stream))
    _check("nvfp4_quantize_1d_gather", st)


def nvfp4_quantize_dual(x, rng_row, rng_col, rht_sign_mask, amax, amax_is_input, row_codes,
                        row_scales, row_global_dec, col_codes, col_scales, col_global_dec,
                        zero_codes, stream=None, row_index=None):
    src_rows, cols = x.shape
    pr = C.byref(_Philox(rng_row.seed, rng_row.offset, rng_row.rounds, 0))
    pc = C.byref(_Philox(rng_col.seed, rng_col.offset, rng_col.rounds, 0))
    tail = (int(rht_sign_mask), _p(amax), int(bool(amax_is_input)), _p(row_codes),
            _p(row_scales), _p(row_global_dec), _p(col_codes), _p(col_scales),
            _p(col_global_dec), _p(zero_codes), _stream(stream))
    if row_index is None:
        st = load().nvfp4_quantize_dual(_p(x), _dtype_code(x), src_rows, cols, pr, pc, *tail)
        _check("nvfp4_quantize_dual", st)
        return
    st = load().nvfp4_quantize_dual_gather(_p(x), _dtype_code(x), src_rows, _p(row_index),
                                           row_index.numel(), cols, pr, pc, *tail)
    _check("nvfp4_quantize_dual_gather", st)


def nvfp4_quantize_mse(w, amax, amax_is_input, codes, scales, global_dec, stream=None):
    rows, cols = w.shape
    st = load().nvfp4_quantize_mse(_p(w), _dtype_code(w), rows, cols, _p(amax),
                                   int(bool(amax_is_input)), _p(codes), _p(scales),
                                   _p(global_dec), _stream(stream))
    _check("nvfp4_quantize_mse", st)


def nvfp4_quantize_2d(w, amax, amax_is_input, codes, scales, global_dec, stream=None):
    if w.dim() == 2:
        batch, (rows, cols) = 1, w.shape
    else:
        batch, rows, cols = w.shape
    st = load().nvfp4_quantize_2d(_p(w), _dtype_code(w), batch, rows, cols, _p(amax),
                                  int(bool(amax_is_input)), _p(codes), _p(scales), _p(global_dec),
                                  _stream(stream))
    _check("nvfp4_quantize_2d", st)


def nvfp4_rht16(x, axis, sign_mask, y, stream=None):
    rows, cols = x.shape
    st = load().nvfp4_rht16(_p(x), _dtype_code(x), rows, cols, int(axis), int(sign_mask), _p(y),
                            _stream(stream))
    _check("nvfp4_rht16", st)


def nvfp4_dequantize(q_operand, y, stream=None):
    st = load().nvfp4_dequantize(C.byref(q_operand), _p(y), _stream(stream))
    _check("nvfp4_dequantize", st)


def nvfp4_gemm(opA, opB, M, N, K, A_operand, B_operand, C_out, c_dtype, stream=None):
    st = load().nvfp4_gemm(opA.encode(), opB.encode(), M, N, K, C.byref(A_operand),
                           C.byref(B_operand), _p(C_out), int(c_dtype), _stream(stream))
    _check("nvfp4_gemm", st)


def nvfp4_grouped_gemm(groups, row_offsets, total_rows, N, K, A_operand, B_operand, C_out, c_dtype,
                       stream=None):
    st = load().nvfp4_grouped_gemm(groups, _p(row_offsets), total_rows, N, K, C.byref(A_operand),
                                   C.byref(B_operand), _p(C_out), int(c_dtype), _stream(stream))
    _check("nvfp4_grouped_gemm", st)


def nvfp4_grouped_gemm_nn(groups, row_offsets, total_rows, N, K, A_operand, B_operand, C_out,
                          c_dtype, stream=None):
    st = load().nvfp4_grouped_gemm_nn(groups, _p(row_offsets), total_rows, N, K,
                                      C.byref(A_operand), C.byref(B_operand), _p(C_out),
                                      int(c_dtype), _stream(stream))
    _check("nvfp4_grouped_gemm_nn", st)


def nvfp4_grouped_gemm_tn(groups, k_offsets, total_k, M, N, A_operand, B_operand, C_out,
                          stream=None):
    st = load().nvfp4_grouped_gemm_tn(groups, _p(k_offsets), total_k, M, N, C.byref(A_operand),
                                      C.byref(B_operand), _p(C_out), _stream(stream))
    _check("nvfp4_grouped_gemm_tn", st)


def nvfp4_grouped_gemm_tn_accumulate(groups, k_offsets, total_k, M, N, A_operand, B_operand,
                                     C_inout, stream=None):
    st = load().nvfp4_grouped_gemm_tn_accumulate(groups, _p(k_offsets), total_k, M, N,
                                                 C.byref(A_operand), C.byref(B_operand),
                                                 _p(C_inout), _stream(stream))
    _check("nvfp4_grouped_gemm_tn_accumulate", st)


def nvfp4_sr_fp16(x, rng, y, stream=None):
    st = load().nvfp4_sr_fp16(_p(x), x.numel(), C.byref(_Philox(rng.seed, rng.offset, rng.rounds, 0)),
                              _p(y), _stream(stream))
    _check("nvfp4_sr_fp16", st)


# ---- allocating convenience wrappers ------------------------------------------------------
def _scale_shape(block, rows, cols):
    if block == "row":
        return (rows, cols // 16)
    if block == "col":
        return (rows // 16, cols)
    return (rows // 16, cols // 16)


def quantize_1d(x, axis="row", rounding="rne", rng: Optional[Philox] = None, rht_sign_mask=-1,
                amax=None, stream=None, row_index=None):
    """row_index: quantize x[row_index] (out-of-range indices: zero rows)
    without materializing the gathered rows."""
    rows, cols = x.shape
    if row_index is not None:
        rows = row_index.numel()
    dev = x.device
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty(_scale_shape(axis, rows, cols), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    given = amax is not None
    a = (amax.reshape(1).to(torch.float32).clone() if given
         else torch.empty(1, dtype=torch.float32, device=dev))
    rnd = NVFP4_SR if rounding == "sr" else NVFP4_RNE
    nvfp4_quantize_1d(x, _BLOCKS[axis], rnd, rng, rht_sign_mask, a, given, codes, scales, g, stream,
                      row_index)
    return QTensor(codes, scales, g, a, rows, cols, axis)


def quantize_dual(x, rng_row: Philox, rng_col: Philox, rht_sign_mask=-1, amax=None,
                  count_zeros=True, stream=None, row_index=None):
    """ROW (dgrad) and COL (wgrad) quantization of one gradient from one read
    (of x[row_index] when given).  Returns (row QTensor, col QTensor,
    zero-code counts int64[2] or None)."""
    rows, cols = x.shape
    if row_index is not None:
        rows = row_index.numel()
    dev = x.device
    rc = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    rs = torch.empty(_scale_shape("row", rows, cols), dtype=torch.uint8, device=dev)
    cc = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    cs = torch.empty(_scale_shape("col", rows, cols), dtype=torch.uint8, device=dev)
    g = torch.empty(2, dtype=torch.float32, device=dev)
    given = amax is not None
    a = (amax.reshape(2).to(torch.float32).clone() if given
         else torch.empty(2, dtype=torch.float32, device=dev))
    z = torch.empty(2, dtype=torch.int64, device=dev) if count_zeros else None
    nvfp4_quantize_dual(x, rng_row, rng_col, rht_sign_mask, a, given, rc, rs, g[0:1], cc, cs,
                        g[1:2], z, stream, row_index)
    return (QTensor(rc, rs, g[0:1], a[0:1], rows, cols, "row"),
            QTensor(cc, cs, g[1:2], a[1:2], rows, cols, "col"), z)


def quantize_mse(w, amax=None, stream=None):
    """PTQ weight quantization: ROW blocks with MSE-calibrated scales."""
    rows, cols = w.shape
    dev = w.device
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    given = amax is not None
    a = (amax.reshape(1).to(torch.float32).clone() if given
         else torch.empty(1, dtype=torch.float32, device=dev))
    nvfp4_quantize_mse(w, a, given, codes, scales, g, stream)
    return QTensor(codes, scales, g, a, rows, cols, "row")


def quantize_2d(w, amax=None, stream=None):
    dev = w.device
    batched = w.dim() == 3
    batch = w.shape[0] if batched else 1
    rows, cols = w.shape[-2:]
    lead = (batch,) if batched else ()
    codes = torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty(lead + (rows // 16, cols // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(batch, dtype=torch.float32, device=dev)
    given = amax is not None
    a = (amax.reshape(batch).to(torch.float32).clone() if given
         else torch.empty(batch, dtype=torch.float32, device=dev))
    nvfp4_quantize_2d(w, a, given, codes, scales, g, stream)
    return QTensor(codes, scales, g, a, rows, cols, "2d")


def rht16(x, axis="col", sign_mask=0, stream=None):
    y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    nvfp4_rht16(x, _BLOCKS[axis], sign_mask, y, stream)
    return y


def dequantize(q: QTensor, index=None, stream=None):
    y = torch.empty((q.rows, q.cols), dtype=torch.float32, device=q.codes.device)
    nvfp4_dequantize(q.operand(index), y, stream)
    return y


def gemm(opA, opB, A: QTensor, B: QTensor, out_dtype=torch.bfloat16, out=None, stream=None,
         accumulate=False):
    """C = op(A) op(B) * gA * gB with row-major op letters (see nvfp4.h);
    accumulate=True adds the product to the fp32 tensor `out`."""
    M = A.rows if opA == "N" else A.cols
    K = A.cols if opA == "N" else A.rows
    N = B.rows if opB == "T" else B.cols
    if accumulate:
        if out is None or out.dtype != torch.float32:
            raise ValueError("accumulate needs an fp32 `out`")
        cd = NVFP4_FP32_ACCUMULATE
    else:
        if out is None:
            out = torch.empty((M, N), dtype=out_dtype, device=A.codes.device)
        cd = NVFP4_BF16 if out.dtype == torch.bfloat16 else NVFP4_FP32
    nvfp4_gemm(opA, opB, M, N, K, A.operand(), B.operand(), out, cd, stream)
    return out


def grouped_gemm(A: QTensor, B: QTensor, row_offsets, out_dtype=torch.bfloat16, out=None,
                 stream=None):
    """Per group e: C[o_e:o_e+1] = A[o_e:o_e+1] B_e^T (B batched [groups, N, K])."""
    groups = B.codes.shape[0]
    total, K = A.rows, A.cols
    N = B.rows
    if out is None:
        out = torch.empty((total, N), dtype=out_dtype, device=A.codes.device)
    cd = NVFP4_BF16 if out.dtype == torch.bfloat16 else NVFP4_FP32
    nvfp4_grouped_gemm(groups, row_offsets, total, N, K, A.operand(), B.operand(), out, cd, stream)
    return out


def grouped_gemm_nn(A: QTensor, B: QTensor, row_offsets, out_dtype=torch.bfloat16, out=None,
                    stream=None):
    """Per group e: C[o_e:o_e+1] = A[o_e:o_e+1] B_e (B batched [groups, K, N])."""
    groups = B.codes.shape[0]
    total, K = A.rows, A.cols
    N = B.cols
    if out is None:
        out = torch.empty((total, N), dtype=out_dtype, device=A.codes.device)
    cd = NVFP4_BF16 if out.dtype == torch.bfloat16 else NVFP4_FP32
    nvfp4_grouped_gemm_nn(groups, row_offsets, total, N, K, A.operand(), B.operand(), out, cd,
                          stream)
    return out


def grouped_gemm_tn(A: QTensor, B: QTensor, k_offsets, groups, out=None, stream=None,
                    accumulate=False):
    """Per group e: C[e] = A[k_e:k_e+1]^T B[k_e:k_e+1], fp32 [groups, M, N];
    accumulate=True adds it to `out` instead."""
    total, M = A.rows, A.cols
    N = B.cols
    if accumulate:
        if out is None:
            raise ValueError("accumulate needs `out`")
        nvfp4_grouped_gemm_tn_accumulate(groups, k_offsets, total, M, N, A.operand(),
                                         B.operand(), out, stream)
        return out
    if out is None:
        out = torch.empty((groups, M, N), dtype=torch.float32, device=A.codes.device)
    nvfp4_grouped_gemm_tn(groups, k_offsets, total, M, N, A.operand(), B.operand(), out, stream)
    return out


def sr_fp16(x, rng: Philox, stream=None):
    """fp32 tensor -> fp16 tensor of the same shape, stochastic rounding."""
    y = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    nvfp4_sr_fp16(x, rng, y, stream)
    return y
