"""libnvfp4: NVFP4 quantizers and GEMMs for AMD MI355X (gfx950).

The compute path is the HIP library ``libnvfp4.so`` (C ABI in
``include/nvfp4.h``).  This package only marshals torch tensors into that ABI:
``nvfp4_*`` functions mirror the C entry points one to one, and the
convenience wrappers (``quantize_1d``, ``quantize_dual``, ``quantize_mse``, ``quantize_2d``, ``rht16``,
``dequantize``, ``gemm``, ``grouped_gemm``, ``grouped_gemm_nn``,
``grouped_gemm_tn``, ``sr_fp16``) allocate outputs with torch and
call them.  Nothing here computes a value of the method; if the library is
missing, every call raises.
"""
from ._binding import (  # noqa: F401
    NVFP4_BF16, NVFP4_FP32, NVFP4_FP32_ACCUMULATE, NVFP4_RNE, NVFP4_SR,
    NVFP4_BLOCK_ROW, NVFP4_BLOCK_COL, NVFP4_BLOCK_2D, NVFP4_OK, NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN, NVFP4_ERR_LAYOUT,
    NVFP4_ERR_UNSUPPORTED, NVFP4_ERR_DEVICE, NVFP4_ERR_NONFINITE,
    NVFP4Error, Philox, QTensor, library_path, load,
    nvfp4_abi_version, nvfp4_status_string, nvfp4_quantize_1d, nvfp4_quantize_dual,
    nvfp4_quantize_mse, nvfp4_quantize_2d, nvfp4_rht16,
    nvfp4_dequantize, nvfp4_gemm, nvfp4_grouped_gemm, nvfp4_grouped_gemm_nn, nvfp4_grouped_gemm_tn,
    nvfp4_grouped_gemm_tn_accumulate, nvfp4_sr_fp16, nvfp4_set_single_pass_wait, nvfp4_set_debug_checks,
    quantize_1d, quantize_dual, quantize_mse, quantize_2d, rht16, dequantize, gemm, grouped_gemm,
    grouped_gemm_nn, grouped_gemm_tn, sr_fp16,
)
