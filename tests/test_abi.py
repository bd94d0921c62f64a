"""Host-side checks of the C ABI (no GPU compute): the library loads, exports
every function include/fp4q.h declares, and refuses bad arguments with the
documented status before anything is enqueued."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from fp4_block_scaled_row_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfp4q.so not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp4q_quantize_mxfp4", "fp4q_quantize_nvfp4", "fp4q_silu_mul_fwht_mxfp4", "fp4q_fwht",
              "fp4q_dequantize", "fp4q_mxfp4_gemm"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = _lib_or_skip()
    for s in range(6):
        assert lib.fp4q_status_string(s)
    assert b"gfx950" in lib.fp4q_version()


def test_check_counters_host():
    lib = _lib_or_skip()
    ok = (C.c_uint64 * 3)(5, 7, 0)
    bad = (C.c_uint64 * 3)(0, 0, 2)
    assert lib.fp4q_check_counters(C.addressof(ok)) == _lib.FP4Q_OK
    assert lib.fp4q_check_counters(C.addressof(bad)) == _lib.FP4Q_ERR_NONFINITE
    assert lib.fp4q_check_counters(None) == _lib.FP4Q_ERR_INVALID_ARG


def test_workspace_bytes():
    lib = _lib_or_skip()
    a = _lib.QuantArgs()
    a.block_size = 16
    assert lib.fp4q_workspace_bytes(a) == 80 * 1024   # the layout include/fp4q.h documents
    a.block_size = 32
    assert lib.fp4q_workspace_bytes(a) == 4096                 # counter slots (optional)
    a.block_size = 8
    assert lib.fp4q_workspace_bytes(a) == 0


def _args(rows=4, cols=64, block=32, policy=_lib.FP4Q_SCALE_OCP_MAX, dtype=_lib.FP4Q_BF16, stride=None,
          rounding=0, rotation=0, manual=0):
    a = _lib.QuantArgs()
    a.rows, a.cols = rows, cols
    a.in_row_stride = cols if stride is None else stride
    a.in_dtype, a.block_size, a.scale_policy = dtype, block, policy
    a.rounding, a.rotation, a.manual_exponent = rounding, rotation, manual
    return a


# Fake (never dereferenced) but suitably aligned device addresses: every call
# below must be rejected by the host-side checks before any HIP call.
FAKE = 0x10000000
OUTS = _lib.Outputs(FAKE, FAKE, FAKE, FAKE, None, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(block=16), _lib.FP4Q_ERR_UNSUPPORTED),                               # MXFP4 with 16-blocks
    (dict(policy=_lib.FP4Q_SCALE_NV_MAX6), _lib.FP4Q_ERR_UNSUPPORTED),          # NV policy on MX
    (dict(cols=48), _lib.FP4Q_ERR_INVALID_ARG),                                # incomplete block
    (dict(stride=32), _lib.FP4Q_ERR_INVALID_ARG),                              # stride < cols
    (dict(rows=-1), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(rounding=3), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(rotation=9), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(policy=_lib.FP4Q_SCALE_MANUAL, manual=128), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, cols=96), _lib.FP4Q_ERR_UNSUPPORTED),  # not a power of two
    (dict(stride=68), _lib.FP4Q_ERR_UNSUPPORTED),                              # unaligned row pitch
    (dict(rotation=_lib.FP4Q_ROT_FWHT128, cols=128), _lib.FP4Q_ERR_UNSUPPORTED),  # per-head rotation is NV only
])
def test_mxfp4_rejects(kwargs, status):
    lib = _lib_or_skip()
    assert lib.fp4q_quantize_mxfp4(_args(**kwargs), FAKE, OUTS, None, 0, None) == status


def test_mxfp4_workspace_checked_when_given():
    lib = _lib_or_skip()
    o = _lib.Outputs(FAKE, FAKE, None, None, None, FAKE)
    assert lib.fp4q_quantize_mxfp4(_args(), FAKE, o, FAKE, 64, None) == _lib.FP4Q_ERR_WORKSPACE      # too small
    assert lib.fp4q_quantize_mxfp4(_args(), FAKE, o, FAKE + 4, 4096, None) == _lib.FP4Q_ERR_WORKSPACE  # misaligned


@pytest.mark.parametrize("kwargs,status", [
    (dict(block=32, policy=_lib.FP4Q_SCALE_NV_MAX6), _lib.FP4Q_ERR_UNSUPPORTED),   # NVFP4 with 32-blocks
    (dict(block=16, policy=_lib.FP4Q_SCALE_OCP_MAX), _lib.FP4Q_ERR_UNSUPPORTED),   # MX policy on NV
    (dict(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6, rotation=_lib.FP4Q_ROT_FWHT_ROW), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6, cols=40), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(block=16, policy=_lib.FP4Q_SCALE_IF4, rounding=_lib.FP4Q_ROUND_STOCHASTIC), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=16, policy=_lib.FP4Q_SCALE_IF4, rotation=_lib.FP4Q_ROT_FWHT_ROW), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=32, policy=_lib.FP4Q_SCALE_IF4), _lib.FP4Q_ERR_UNSUPPORTED),       # IF4 needs 16-blocks
    (dict(block=16, policy=5), _lib.FP4Q_ERR_INVALID_ARG),
    (dict(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6, rotation=_lib.FP4Q_ROT_FWHT128, cols=64), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6, rotation=_lib.FP4Q_ROT_FWHT128, cols=128,
          rounding=_lib.FP4Q_ROUND_STOCHASTIC), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=16, policy=_lib.FP4Q_SCALE_FOUR_OVER_SIX, rotation=_lib.FP4Q_ROT_FWHT128, cols=128),
     _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6, rotation=4), _lib.FP4Q_ERR_INVALID_ARG),
])
def test_nvfp4_rejects(kwargs, status):
    lib = _lib_or_skip()
    assert lib.fp4q_quantize_nvfp4(_args(**kwargs), FAKE, None, OUTS, FAKE, 1 << 20, None) == status


def test_nvfp4_needs_workspace_or_amax():
    lib = _lib_or_skip()
    a = _args(block=16, policy=_lib.FP4Q_SCALE_NV_MAX6)
    assert lib.fp4q_quantize_nvfp4(a, FAKE, None, OUTS, None, 0, None) == _lib.FP4Q_ERR_WORKSPACE
    assert lib.fp4q_quantize_nvfp4(a, FAKE, None, OUTS, FAKE, 16, None) == _lib.FP4Q_ERR_WORKSPACE
    o = _lib.Outputs(FAKE, FAKE, None, None, None, None)
    assert lib.fp4q_quantize_nvfp4(a, FAKE, None, o, FAKE, 1 << 20, None) == _lib.FP4Q_ERR_INVALID_ARG
    # the single-read kernel keeps 64-bit atomic words in the workspace: 8-byte alignment
    assert lib.fp4q_quantize_nvfp4(a, FAKE, None, OUTS, FAKE + 4, 1 << 20, None) == _lib.FP4Q_ERR_WORKSPACE
    a46 = _args(block=16, policy=_lib.FP4Q_SCALE_FOUR_OVER_SIX)
    o = _lib.Outputs(FAKE, FAKE, FAKE, None, None, None)
    assert lib.fp4q_quantize_nvfp4(a46, FAKE, None, o, FAKE, 1 << 20, None) == _lib.FP4Q_ERR_INVALID_ARG


@pytest.mark.parametrize("kwargs,status", [
    (dict(rotation=_lib.FP4Q_ROT_NONE), _lib.FP4Q_ERR_UNSUPPORTED),           # the fused op always rotates
    (dict(rotation=_lib.FP4Q_ROT_RHT16), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, cols=96), _lib.FP4Q_ERR_UNSUPPORTED),  # not a power of two
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, cols=32768), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, block=16), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, policy=_lib.FP4Q_SCALE_NV_MAX6), _lib.FP4Q_ERR_UNSUPPORTED),
    (dict(rotation=_lib.FP4Q_ROT_FWHT_ROW, stride=32), _lib.FP4Q_ERR_INVALID_ARG),
])
def test_silu_mul_fwht_rejects(kwargs, status):
    lib = _lib_or_skip()
    assert lib.fp4q_silu_mul_fwht_mxfp4(_args(**kwargs), FAKE, FAKE, OUTS, None) == status


def test_silu_mul_fwht_needs_up():
    lib = _lib_or_skip()
    a = _args(rotation=_lib.FP4Q_ROT_FWHT_ROW)
    assert lib.fp4q_silu_mul_fwht_mxfp4(a, FAKE, None, OUTS, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_silu_mul_fwht_mxfp4(a, FAKE, FAKE + 8, OUTS, None) == _lib.FP4Q_ERR_UNSUPPORTED


def test_mxfp4_gemm_rejects():
    lib = _lib_or_skip()
    F = FAKE
    assert lib.fp4q_mxfp4_gemm(4, 4, 80, F, F, F, F, 0, F, None) == _lib.FP4Q_ERR_INVALID_ARG   # K % 32
    assert lib.fp4q_mxfp4_gemm(4, 4, 96, F, F, F, F, 0, F, None) == _lib.FP4Q_ERR_UNSUPPORTED   # K % 128
    assert lib.fp4q_mxfp4_gemm(4, 4, (1 << 23) + 128, F, F, F, F, 0, F, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_mxfp4_gemm(-1, 4, 128, F, F, F, F, 0, F, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_mxfp4_gemm(4, 4, 128, F, F, F, F, 7, F, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_mxfp4_gemm(4, 4, 128, None, F, F, F, 0, F, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_mxfp4_gemm(4, 4, 128, F + 8, F, F, F, 0, F, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_mxfp4_gemm(0, 4, 128, None, None, None, None, 0, None, None) == _lib.FP4Q_OK


def test_fwht_and_dequant_reject():
    lib = _lib_or_skip()
    assert lib.fp4q_fwht(4, 64, 64, 1, FAKE, FAKE, 24, 0, 0, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_fwht(4, 64, 64, 1, FAKE, FAKE, 128, 0, 0, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_fwht(4, 64, 32, 1, FAKE, FAKE, 64, 0, 0, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_fwht(4, 64, 64, 5, FAKE, FAKE, 64, 0, 0, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_dequantize(0, 4, 64, 16, FAKE, FAKE, None, 0, FAKE, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_dequantize(1, 4, 64, 16, FAKE, FAKE, None, 0, FAKE, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_dequantize(3, 4, 64, 16, FAKE, FAKE, FAKE, 0, FAKE, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_dequantize(2, 4, 64, 32, FAKE, FAKE, FAKE, 0, FAKE, None) == _lib.FP4Q_ERR_UNSUPPORTED
    assert lib.fp4q_dequantize(2, 4, 64, 16, FAKE, FAKE, None, 0, FAKE, None) == _lib.FP4Q_ERR_INVALID_ARG
    assert lib.fp4q_dequantize(0, 4, 48, 32, FAKE, FAKE, None, 0, FAKE, None) == _lib.FP4Q_ERR_INVALID_ARG


def test_empty_tensors_are_no_ops():
    lib = _lib_or_skip()
    assert lib.fp4q_dequantize(0, 0, 64, 32, None, None, None, 0, None, None) == _lib.FP4Q_OK
    assert lib.fp4q_fwht(0, 64, 64, 1, None, None, 64, 0, 0, None) == _lib.FP4Q_OK
    assert lib.fp4q_quantize_mxfp4(_args(rows=0), None, _lib.Outputs(None, None, None, None, None, None),
                                   None, 0, None) == _lib.FP4Q_OK


def test_tensor_scale_product_equals_quotient():
    """The single-read kernel forms g = RN32(amax / 2688) as RN32(RN64(amax * RN64(1/2688))):
    the two agree for every positive finite bf16 amax and for a seeded sample of fp32 amax
    (the quotient is never within 2^-30 of an fp32 rounding boundary unless exact)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    rng = np.random.default_rng(5)
    more = rng.integers(1, 0x7F800000, size=1 << 20, dtype=np.uint32)
    for b in (bits, more):
        a = b.view(np.float32).astype(np.float64)
        q = (a / 2688.0).astype(np.float32)
        p = (a * (1.0 / 2688.0)).astype(np.float32)
        assert np.array_equal(q.view(np.uint32), p.view(np.uint32))
