"""Loading of libbsq.so and the C signatures of include/bsq.h."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

c_i64 = ctypes.c_int64
c_u64 = ctypes.c_uint64
c_int = ctypes.c_int
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p

# include/bsq.h: BSQ_ROUTE_NOALLOC_MAX_BYTES
ROUTE_NOALLOC_MAX_BYTES = 1 << 20

# name -> (restype, argtypes); mirrors include/bsq.h
SIGNATURES = {
    "bsq_status_string": (ctypes.c_char_p, [c_int]),
    "bsq_version": (c_int, []),
    "bsq_quantize_nvfp4_workspace": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "bsq_quantize_nvfp4": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                   c_size, c_vp]),
    "bsq_swiglu_quantize_nvfp4": (c_int, [c_vp, c_int, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp]),
    "bsq_quantize_nvfp4_square_workspace": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "bsq_quantize_nvfp4_square": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_size, c_vp]),
    "bsq_quantize_mxfp8_workspace": (c_size, [c_i64, c_int, c_i64]),
    "bsq_quantize_mxfp8": (c_int, [c_vp, c_int, c_i64, c_i64, c_int, c_vp, c_i64, c_int, c_u64, c_u64, c_vp, c_vp,
                                   c_vp, c_size, c_vp]),
    "bsq_quantize_mxfp8_dual": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_int, c_u64, c_u64, c_u64, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "bsq_requant_workspace": (c_size, [c_i64, c_i64, c_i64, c_int, c_int]),
    "bsq_requant_transpose_sr": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_i64,
                                         c_int, c_int, c_u64, c_u64, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "bsq_grouped_gemm_nvfp4": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                       c_i64, c_i64, c_vp, c_int, c_vp]),
    "bsq_grouped_gemm_nvfp4_s2f6": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                            c_i64, c_i64, ctypes.c_uint32, c_vp, c_vp, c_vp]),
    "bsq_grouped_gemm_mxfp8": (c_int, [c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp,
                                       c_int, c_vp]),
    "bsq_gemm_nvfp4_inreg_scale": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "bsq_route_workspace": (c_size, [c_i64, c_i64]),
    "bsq_route": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "bsq_route_noalloc": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "bsq_rht_s2f6_encode": (c_int, [c_vp, c_int, c_i64, c_i64, ctypes.c_uint32, c_vp, c_vp, c_vp]),
    "bsq_rht_s2f6_combine": (c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_i64, c_i64, ctypes.c_uint32, c_vp, c_int,
                                     c_vp]),
    "bsq_dequantize_nvfp4": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "bsq_dequantize_mxfp8": (c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "bsq_rng_bits16": (c_int, [c_u64, c_u64, c_u64, c_i64, c_vp, c_vp]),
    "bsq_mfma_rate_probe": (c_int, [c_int, c_int, c_i64, c_i64, c_vp, c_vp]),
}


class BsqError(RuntimeError):
    """A bsq_* call returned a non-zero status, or the library is missing."""


def library_path():
    return os.environ.get("BSQ_LIBRARY", os.path.join(_HERE, "libbsq.so"))


def load_library():
    """Load libbsq.so once and attach the C signatures. Raises BsqError when
    the library has not been built (there is no fallback path)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise BsqError(f"{path} not found: build the HIP library first "
                       "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(status, what):
    if status != 0:
        msg = load_library().bsq_status_string(status).decode()
        raise BsqError(f"{what}: status {status} ({msg})")
