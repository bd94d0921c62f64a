"""ctypes binding of the C oracle (test infrastructure only).

Arrays are numpy; bf16 tensors are passed as their raw uint16 bits.  Every
function mirrors one in ``fp4_oracle.c`` and returns freshly allocated numpy
outputs.
"""
import ctypes as C
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
# FP4Q_ORACLE_LIB selects another build of the same source (the sanitizer
# run of the CPU tests loads an AddressSanitizer/UBSan build this way)
LIB = os.environ.get("FP4Q_ORACLE_LIB") or os.path.join(HERE, "libfp4oracle.so")

F32, BF16 = 0, 1
MX, NV, IF4 = 0, 1, 2
_lock = threading.Lock()
_lib = None


def build(force=True):
    """Compile the oracle with gcc (IEEE semantics: no contraction, no fast-math)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(HERE, "libfp4oracle_san.so")


def build_sanitized(cc="/opt/rocm/llvm/bin/clang"):
    """The same source with AddressSanitizer and UBSan (clang, shared
    sanitizer runtime, so that it can share a process with the sanitized
    host build of the HIP library), for the sanitizer run of the CPU tests."""
    tmp = SAN_LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
           "-fno-omit-frame-pointer", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.environ.get("FP4Q_ORACLE_LIB") and (not os.path.exists(LIB) or
                                                          os.path.getmtime(LIB) < os.path.getmtime(SRC)):
                build()
            lib = C.CDLL(LIB)
            i64, i32, u64, vp, dp = C.c_int64, C.c_int, C.c_uint64, C.c_void_p, C.c_double
            lib.oracle_e2m1_value.argtypes = [i32]; lib.oracle_e2m1_value.restype = dp
            lib.oracle_e8m0_value.argtypes = [i32]; lib.oracle_e8m0_value.restype = dp
            lib.oracle_e4m3_value.argtypes = [i32]; lib.oracle_e4m3_value.restype = dp
            lib.oracle_e4m3_encode.argtypes = [dp]; lib.oracle_e4m3_encode.restype = i32
            lib.oracle_e2m1_round.argtypes = [dp, i32, C.c_uint, C.POINTER(C.c_int)]
            lib.oracle_e2m1_round.restype = i32
            lib.oracle_int4_round.argtypes = [dp, C.POINTER(C.c_int)]; lib.oracle_int4_round.restype = i32
            lib.oracle_mx_exponent.argtypes = [dp]; lib.oracle_mx_exponent.restype = i32
            lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]; lib.oracle_philox4x32_10.restype = None
            lib.oracle_sr_draw.argtypes = [u64, u64]; lib.oracle_sr_draw.restype = C.c_uint
            lib.oracle_rht_sign_negative.argtypes = [u64, i64]; lib.oracle_rht_sign_negative.restype = i32
            lib.oracle_quantize_mx.argtypes = [i64, i64, i64, i32, vp, i32, i32, i32, u64, vp, vp, vp]
            lib.oracle_quantize_mx.restype = i32
            lib.oracle_quantize_nv.argtypes = [i64, i64, i64, i32, vp, i32, i32, u64, vp, vp, vp, vp, vp, vp]
            lib.oracle_quantize_nv.restype = i32
            lib.oracle_fwht.argtypes = [i64, i64, i64, i32, vp, vp, i64, i32, u64]
            lib.oracle_silu_mul.argtypes = [i64, i64, i64, i32, vp, vp, vp]
            lib.oracle_mx_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, i64, i64, vp, vp]
            lib.oracle_mx_gemm.restype = i32
            lib.oracle_silu_mul.restype = i32
            lib.oracle_fwht.restype = i32
            lib.oracle_dequantize.argtypes = [i32, i64, i64, i32, vp, vp, vp, i32, vp]
            lib.oracle_dequantize.restype = i32
            lib.oracle_tensor_amax.argtypes = [i64, i64, i64, i32, vp]
            lib.oracle_tensor_amax.restype = C.c_float
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_input(x):
    """Return (array, dtype code) for an fp32 array or a uint16 array of bf16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits), got %s" % x.dtype)


def e2m1_value(code):
    return load().oracle_e2m1_value(int(code))


def e8m0_value(b):
    return load().oracle_e8m0_value(int(b))


def e4m3_value(b):
    return load().oracle_e4m3_value(int(b))


def e4m3_encode(t):
    return load().oracle_e4m3_encode(float(t))


def e2m1_round(q, rounding=0, u=0):
    sat = C.c_int(0)
    code = load().oracle_e2m1_round(float(q), int(rounding), int(u), C.byref(sat))
    return code, sat.value


def int4_round(q):
    sat = C.c_int(0)
    code = load().oracle_int4_round(float(q), C.byref(sat))
    return code, sat.value


def mx_exponent(amax):
    return load().oracle_mx_exponent(float(amax))


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, np.uint32)
    load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_draw(seed, i):
    return load().oracle_sr_draw(int(seed), int(i))


def rht_sign_negative(seed, j):
    return load().oracle_rht_sign_negative(int(seed), int(j))


def quantize_mx(x, policy=0, manual_exponent=0, rounding=0, seed=0, cols=None):
    """x: [rows, stride] float32 or uint16 (bf16 bits); the first ``cols`` columns are quantized."""
    x, dt = _as_input(x)
    rows, stride = x.shape
    cols = stride if cols is None else cols
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    counters = np.zeros(3, np.uint64)
    rc = load().oracle_quantize_mx(rows, cols, stride, dt, _ptr(x), policy, manual_exponent, rounding,
                                   seed, _ptr(codes), _ptr(scales), _ptr(counters))
    if rc != 0:
        raise ValueError("oracle_quantize_mx rejected the arguments")
    return codes, scales, counters


def quantize_nv(x, policy=2, rounding=0, seed=0, global_amax=None, cols=None):
    """x: [rows, stride] float32 or uint16 (bf16 bits); the first ``cols`` columns are quantized."""
    x, dt = _as_input(x)
    rows, stride = x.shape
    cols = stride if cols is None else cols
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    gs = np.zeros(1, np.float32)
    nblk = rows * (cols // 16)
    choice = np.zeros((nblk + 7) // 8, np.uint8) if policy == 3 else None
    counters = np.zeros(3, np.uint64)
    ga = None if global_amax is None else np.array([global_amax], np.float32)
    rc = load().oracle_quantize_nv(rows, cols, stride, dt, _ptr(x), policy, rounding, seed, _ptr(ga),
                                   _ptr(codes), _ptr(scales), _ptr(gs), _ptr(choice), _ptr(counters))
    if rc != 0:
        raise ValueError("oracle_quantize_nv rejected the arguments")
    return codes, scales, gs[0], choice, counters


def tensor_amax(x):
    """Largest finite |x| (the NVFP4 per-tensor amax)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    return np.float32(load().oracle_tensor_amax(rows, cols, cols, dt, _ptr(x)))


def fwht(x, t=None, random_signs=False, seed=0):
    """Normalised Walsh-Hadamard transform of each t-chunk of each row (fp64 out).
    x: float32, uint16 (bf16 bits) or float64."""
    if np.asarray(x).dtype == np.float64:
        x, dt = np.ascontiguousarray(x), 2
    else:
        x, dt = _as_input(x)
    rows, d = x.shape
    t = d if t is None else t
    y = np.zeros((rows, d), np.float64)
    rc = load().oracle_fwht(rows, d, d, dt, _ptr(x), _ptr(y), t, int(bool(random_signs)), seed)
    if rc != 0:
        raise ValueError("oracle_fwht rejected the arguments")
    return y


def mx_gemm(a_codes, a_scales, b_codes, b_scales, rows=None):
    """C = A B^T over reconstructed MXFP4 values (fp64), with sum |a b| per output.
    A: codes [M, K/2], scales [M, K/32]; B likewise [N, ...].  rows: optional
    (row0, nrows) of A to compute.  Returns (C, absC), both [nrows, N] fp64."""
    ac = np.ascontiguousarray(a_codes, dtype=np.uint8)
    asc = np.ascontiguousarray(a_scales, dtype=np.uint8)
    bc = np.ascontiguousarray(b_codes, dtype=np.uint8)
    bsc = np.ascontiguousarray(b_scales, dtype=np.uint8)
    M, K = ac.shape[0], ac.shape[1] * 2
    N = bc.shape[0]
    if bc.shape[1] * 2 != K or asc.shape != (M, K // 32) or bsc.shape != (N, K // 32):
        raise ValueError("mx_gemm: inconsistent shapes")
    row0, nrows = (0, M) if rows is None else rows
    c = np.zeros((nrows, N), np.float64)
    absc = np.zeros((nrows, N), np.float64)
    rc = load().oracle_mx_gemm(M, N, K, _ptr(ac), _ptr(asc), _ptr(bc), _ptr(bsc), row0, nrows, _ptr(c), _ptr(absc))
    if rc != 0:
        raise ValueError("oracle_mx_gemm rejected the arguments")
    return c, absc


def silu_mul(gate, up):
    """SiLU(gate) * up in fp64 for two same-shape float32 or uint16 (bf16 bits) arrays."""
    gate, dt = _as_input(gate)
    up, dt2 = _as_input(up)
    if gate.shape != up.shape or dt != dt2:
        raise ValueError("silu_mul: gate and up must have the same shape and dtype")
    rows, cols = gate.shape
    out = np.zeros((rows, cols), np.float64)
    rc = load().oracle_silu_mul(rows, cols, cols, dt, _ptr(gate), _ptr(up), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_silu_mul rejected the arguments")
    return out


def dequantize(fmt, codes, scales, global_scale=None, out_dtype=F32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    block = 32 if fmt == MX else 16
    gs = None if global_scale is None else np.array([global_scale], np.float32)
    out = np.zeros((rows, cols), np.float32 if out_dtype == F32 else np.uint16)
    rc = load().oracle_dequantize(fmt, rows, cols, block, _ptr(codes), _ptr(scales), _ptr(gs),
                                  out_dtype, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequantize rejected the arguments")
    return out
