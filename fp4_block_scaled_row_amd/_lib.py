"""ctypes loader for libfp4q.so (the C ABI declared in include/fp4q.h).

Argument marshalling only: every step of quantization runs in the HIP kernels
of the library.  There is no CPU fallback -- if the shared library is missing
or cannot be loaded, every call raises.
"""
import ctypes as C
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# FP4Q_LIB selects another build of the same sources (the sanitizer run of the
# host-side tests loads a host-only AddressSanitizer/UBSan build this way)
LIB_PATH = os.environ.get("FP4Q_LIB") or os.path.join(HERE, "libfp4q.so")

FP4Q_OK, FP4Q_ERR_INVALID_ARG, FP4Q_ERR_UNSUPPORTED, FP4Q_ERR_WORKSPACE, FP4Q_ERR_NONFINITE, FP4Q_ERR_HIP = range(6)
FP4Q_F32, FP4Q_BF16 = 0, 1
FP4Q_MXFP4, FP4Q_NVFP4, FP4Q_IF4 = 0, 1, 2
FP4Q_SCALE_OCP_MAX, FP4Q_SCALE_MANUAL, FP4Q_SCALE_NV_MAX6, FP4Q_SCALE_FOUR_OVER_SIX, FP4Q_SCALE_IF4 = 0, 1, 2, 3, 4
FP4Q_ROUND_RNE, FP4Q_ROUND_STOCHASTIC = 0, 1
FP4Q_ROT_NONE, FP4Q_ROT_FWHT_ROW, FP4Q_ROT_RHT16, FP4Q_ROT_FWHT128 = 0, 1, 2, 3

EXPORTED = [
    "fp4q_workspace_bytes", "fp4q_quantize_mxfp4", "fp4q_quantize_nvfp4", "fp4q_quantize_nvfp4_noalloc",
    "fp4q_silu_mul_fwht_mxfp4", "fp4q_fwht",
    "fp4q_dequantize", "fp4q_mxfp4_gemm", "fp4q_check_counters", "fp4q_status_string", "fp4q_version",
]


class QuantArgs(C.Structure):
    _fields_ = [
        ("rows", C.c_int64), ("cols", C.c_int64), ("in_row_stride", C.c_int64),
        ("in_dtype", C.c_int32), ("block_size", C.c_int32), ("scale_policy", C.c_int32),
        ("manual_exponent", C.c_int32), ("rounding", C.c_int32), ("rotation", C.c_int32),
        ("seed", C.c_uint64),
    ]


class Outputs(C.Structure):
    _fields_ = [
        ("codes", C.c_void_p), ("scales", C.c_void_p), ("global_scale", C.c_void_p),
        ("choice_bits", C.c_void_p), ("rotated", C.c_void_p), ("counters", C.c_void_p),
    ]


class Fp4qError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


_lock = threading.Lock()
_lib = None


def load():
    """Load libfp4q.so (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4q.so is not built (run `python -m fp4_block_scaled_row_amd.build`); "
                               "there is no CPU fallback")
        lib = C.CDLL(LIB_PATH)
        vp, i64, i32, u64 = C.c_void_p, C.c_int64, C.c_int32, C.c_uint64
        lib.fp4q_workspace_bytes.argtypes = [C.POINTER(QuantArgs)]
        lib.fp4q_workspace_bytes.restype = C.c_size_t
        lib.fp4q_quantize_mxfp4.argtypes = [C.POINTER(QuantArgs), vp, C.POINTER(Outputs), vp, C.c_size_t, vp]
        lib.fp4q_quantize_mxfp4.restype = C.c_int
        lib.fp4q_quantize_nvfp4.argtypes = [C.POINTER(QuantArgs), vp, vp, C.POINTER(Outputs), vp, C.c_size_t, vp]
        lib.fp4q_quantize_nvfp4.restype = C.c_int
        lib.fp4q_quantize_nvfp4_noalloc.argtypes = [C.POINTER(QuantArgs), vp, vp, C.POINTER(Outputs), vp]
        lib.fp4q_quantize_nvfp4_noalloc.restype = C.c_int
        lib.fp4q_silu_mul_fwht_mxfp4.argtypes = [C.POINTER(QuantArgs), vp, vp, C.POINTER(Outputs), vp]
        lib.fp4q_silu_mul_fwht_mxfp4.restype = C.c_int
        lib.fp4q_fwht.argtypes = [i64, i64, i64, i32, vp, vp, i32, i32, u64, vp]
        lib.fp4q_fwht.restype = C.c_int
        lib.fp4q_dequantize.argtypes = [i32, i64, i64, i32, vp, vp, vp, i32, vp, vp]
        lib.fp4q_dequantize.restype = C.c_int
        lib.fp4q_mxfp4_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32, vp, vp]
        lib.fp4q_mxfp4_gemm.restype = C.c_int
        lib.fp4q_check_counters.argtypes = [vp]
        lib.fp4q_check_counters.restype = C.c_int
        lib.fp4q_status_string.argtypes = [C.c_int]
        lib.fp4q_status_string.restype = C.c_char_p
        lib.fp4q_version.argtypes = []
        lib.fp4q_version.restype = C.c_char_p
        _lib = lib
        return lib


def status_string(status):
    return load().fp4q_status_string(int(status)).decode()


def check(status, where):
    if status != FP4Q_OK:
        raise Fp4qError(status, where)
