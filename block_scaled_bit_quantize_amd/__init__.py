"""block_scaled_bit_quantize_amd: NVFP4 / MXFP8 block-scaled quantization and
expert grouped GEMMs for AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/bsq.h`` (``libbsq.so``). Every
step runs in the library's HIP kernels; this module only checks arguments,
allocates outputs and workspaces with PyTorch and passes raw device pointers
and the current stream. There is no CPU fallback: importing works without a
GPU, but calling an operation without the built library or a GPU raises.
"""
from ._lib import BsqError, library_path, load_library
from .ops import (BF16, F32, MXFP8, NVFP4, OUTER_GIVEN, OUTER_ROW, OUTER_TENSOR, RN, SR,
                  dequantize_mxfp8, dequantize_nvfp4, grouped_gemm_mxfp8, grouped_gemm_nvfp4,
                  grouped_gemm_nvfp4_s2f6,
                  padded_segment_layout, quantize_mxfp8, quantize_mxfp8_dual, quantize_nvfp4, quantize_nvfp4_square,
                  requant_transpose_sr,
                  rht_s2f6_combine, rht_s2f6_encode, rng_bits16, mfma_rate_probe, route, route_noalloc, gemm_nvfp4_inreg_scale, swiglu_quantize_nvfp4)

__all__ = [
    "BsqError", "library_path", "load_library",
    "F32", "BF16", "OUTER_TENSOR", "OUTER_ROW", "OUTER_GIVEN", "RN", "SR", "NVFP4", "MXFP8",
    "quantize_nvfp4", "quantize_mxfp8", "quantize_mxfp8_dual", "requant_transpose_sr", "grouped_gemm_nvfp4",
    "grouped_gemm_mxfp8", "route", "route_noalloc", "gemm_nvfp4_inreg_scale", "dequantize_nvfp4", "dequantize_mxfp8", "rng_bits16", "mfma_rate_probe",
    "padded_segment_layout", "quantize_nvfp4_square", "rht_s2f6_encode", "rht_s2f6_combine",
    "swiglu_quantize_nvfp4", "grouped_gemm_nvfp4_s2f6",
]
