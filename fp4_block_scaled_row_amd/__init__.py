"""fp4q -- block-scaled FP4 quantization on MI355X (gfx950).

Thin Python binding over the C ABI of libfp4q.so (include/fp4q.h).  PyTorch
supplies device memory and the current HIP stream; every step of the
quantization runs in the library's HIP kernels.  There is no CPU fallback.

Formats (pages cited by title and section):
  * MXFP4: 32-element blocks, E8M0 scale, OCP max rule ("MXFP4 Quantization:
    Audit the 4.25-Bit Blocks", "Read the shared E8M0 scale").
  * NVFP4: 16-element blocks, E4M3 block scale and fp32 tensor scale
    ("Sub-4-Bit Microscaling", section 2); Four Over Six ("Adaptive
    Block-Scaled Data Types" transcript, cue 10); IF4, FP4 or 7/6-scaled
    INT4 per block flagged in the scale's sign bit (transcript, cues 14, 17).
  * Rotations: full-row FWHT ("Sub-4-Bit Microscaling", section 3) and the
    16-point random Hadamard transform (transcript, cue 8).
  * Fused SwiGLU epilogue: SiLU(gate) * up -> row FWHT -> MXFP4 in one kernel
    ("Sub-4-Bit Microscaling", section 3, the online SiLU_and_Mul rotation).
"""
from collections import namedtuple

import torch

from . import _lib
from ._lib import Fp4qError, load  # noqa: F401

__all__ = [
    "quantize_mxfp4", "quantize_nvfp4", "silu_mul_fwht_mxfp4", "fwht", "dequantize", "mxfp4_gemm",
    "workspace_bytes",
    "check_counters", "version", "MxResult", "NvResult", "Fp4qError",
]

MxResult = namedtuple("MxResult", "codes scales rotated counters")
NvResult = namedtuple("NvResult", "codes scales global_scale choice_bits rotated counters")

_ROUND = {"rne": _lib.FP4Q_ROUND_RNE, "stochastic": _lib.FP4Q_ROUND_STOCHASTIC, "sr": _lib.FP4Q_ROUND_STOCHASTIC}
_ROT = {None: _lib.FP4Q_ROT_NONE, "none": _lib.FP4Q_ROT_NONE, "fwht_row": _lib.FP4Q_ROT_FWHT_ROW,
        "rht16": _lib.FP4Q_ROT_RHT16, "fwht128": _lib.FP4Q_ROT_FWHT128}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _in_dtype(x):
    if x.dtype == torch.float32:
        return _lib.FP4Q_F32
    if x.dtype == torch.bfloat16:
        return _lib.FP4Q_BF16
    raise TypeError("fp4q: input must be float32 or bfloat16, got %s" % x.dtype)


def _check_input(x):
    if not x.is_cuda:
        raise ValueError("fp4q: the input must be a GPU tensor (no CPU path exists)")
    if x.dim() != 2:
        raise ValueError("fp4q: the input must be 2-D [rows, cols]")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("fp4q: rows must be contiguous (stride(1) == 1)")


def _check_buf(t, shape, dtype, what):
    """A buffer handed to the library: a contiguous GPU tensor of this shape
    (None: any shape) and dtype, since the kernels write or read it densely."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("fp4q: %s must be a GPU tensor" % what)
    if t.dtype != dtype:
        raise ValueError("fp4q: %s must be %s, got %s" % (what, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("fp4q: %s must have shape %s, got %s" % (what, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("fp4q: %s must be contiguous" % what)


def _check_mx_out(out, rows, cols):
    _check_buf(out.codes, (rows, cols // 2), torch.uint8, "out.codes")
    _check_buf(out.scales, (rows, cols // 32), torch.uint8, "out.scales")
    if out.rotated is not None:
        _check_buf(out.rotated, (rows, cols), torch.float32, "out.rotated")
    if out.counters is not None:
        _check_buf(out.counters, (3,), torch.int64, "out.counters")


def _args(x, block, policy, manual_exponent, rounding, rotation, seed):
    a = _lib.QuantArgs()
    a.rows, a.cols = int(x.shape[0]), int(x.shape[1])
    a.in_row_stride = int(x.stride(0)) if x.shape[0] > 1 else int(x.shape[1])
    a.in_dtype = _in_dtype(x)
    a.block_size = block
    a.scale_policy = policy
    a.manual_exponent = int(manual_exponent)
    a.rounding = _ROUND[rounding]
    a.rotation = _ROT[rotation]
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return a


def workspace_bytes(block_size):
    a = _lib.QuantArgs()
    a.block_size = block_size
    return int(_lib.load().fp4q_workspace_bytes(a))


# One zero-filled workspace per (format, device, stream), kept for the life of
# the process: calls on one stream are ordered, which is all the library asks
# of calls that share a workspace.
_workspaces = {}


def _default_workspace(dev, block_size=16):
    stream = torch.cuda.current_stream(dev)
    key = (block_size, dev.index if dev.index is not None else torch.cuda.current_device(), stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("fp4q: no workspace exists yet for this stream; pass workspace= or make one "
                               "call on the stream before capturing it")
        ws = torch.zeros(workspace_bytes(block_size), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def quantize_mxfp4(x, *, policy="ocp", manual_exponent=0, rounding="rne", seed=0, rotation=None,
                   return_rotated=False, counters=False, out=None):
    """MXFP4-quantize a 2-D fp32/bf16 GPU tensor along its rows.

    Returns MxResult(codes [rows, cols/2] uint8, scales [rows, cols/32] uint8
    (E8M0), rotated fp32 or None, counters int64[3] or None).  `out` may be a
    previous MxResult of the same shape to reuse its buffers."""
    _check_input(x)
    rows, cols = x.shape
    pol = {"ocp": _lib.FP4Q_SCALE_OCP_MAX, "manual": _lib.FP4Q_SCALE_MANUAL}[policy]
    a = _args(x, 32, pol, manual_exponent, rounding, rotation, seed)
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        rot = torch.empty((rows, cols), dtype=torch.float32, device=dev) if return_rotated else None
        cnt = torch.empty(3, dtype=torch.int64, device=dev) if counters else None
        out = MxResult(codes, scales, rot, cnt)
    _check_mx_out(out, rows, cols)
    o = _lib.Outputs(_ptr(out.codes), _ptr(out.scales), None, None, _ptr(out.rotated), _ptr(out.counters))
    # (a counting call sums its counts through the workspace's counter slots)
    ws = _default_workspace(dev, 32) if out.counters is not None and rows * cols > 0 else None
    ws_bytes = 0 if ws is None else ws.numel()
    _lib.check(_lib.load().fp4q_quantize_mxfp4(a, _ptr(x), o, _ptr(ws), ws_bytes, _stream()), "fp4q_quantize_mxfp4")
    return out


def quantize_nvfp4(x, *, policy="max6", rounding="rne", seed=0, rotation=None, global_amax=None,
                   return_rotated=False, counters=False, out=None, workspace=None):
    """NVFP4-quantize a 2-D fp32/bf16 GPU tensor along its rows.

    policy "max6" (g = amax/2688), "four_over_six" (g = amax/1792, per-block
    max->6 / max->4 choice) or "if4" (g as max6, per-block FP4 / scaled INT4
    choice in bit 7 of the scale byte; round to nearest only).  global_amax: optional 1-element fp32 GPU tensor.
    Returns NvResult(codes, scales (E4M3), global_scale fp32[1], choice_bits
    uint8 or None, rotated or None, counters or None)."""
    _check_input(x)
    rows, cols = x.shape
    pol = {"max6": _lib.FP4Q_SCALE_NV_MAX6, "four_over_six": _lib.FP4Q_SCALE_FOUR_OVER_SIX,
           "if4": _lib.FP4Q_SCALE_IF4}[policy]
    a = _args(x, 16, pol, 0, rounding, rotation, seed)
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty(1, dtype=torch.float32, device=dev)
        nb = rows * (cols // 16)
        choice = torch.empty(((nb + 7) // 8,), dtype=torch.uint8, device=dev) if policy == "four_over_six" else None
        rot = torch.empty((rows, cols), dtype=torch.float32, device=dev) if return_rotated else None
        cnt = torch.empty(3, dtype=torch.int64, device=dev) if counters else None
        out = NvResult(codes, scales, gs, choice, rot, cnt)
    _check_buf(out.codes, (rows, cols // 2), torch.uint8, "out.codes")
    _check_buf(out.scales, (rows, cols // 16), torch.uint8, "out.scales")
    _check_buf(out.global_scale, (1,), torch.float32, "out.global_scale")
    if out.choice_bits is not None:
        _check_buf(out.choice_bits, ((rows * (cols // 16) + 7) // 8,), torch.uint8, "out.choice_bits")
    if out.rotated is not None:
        _check_buf(out.rotated, (rows, cols), torch.float32, "out.rotated")
    if out.counters is not None:
        _check_buf(out.counters, (3,), torch.int64, "out.counters")
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("fp4q: the workspace must be a GPU tensor")
    if workspace is None and global_amax is None:
        workspace = _default_workspace(dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if global_amax is not None and (global_amax.dtype != torch.float32 or not global_amax.is_cuda):
        raise TypeError("fp4q: global_amax must be a float32 GPU tensor")
    o = _lib.Outputs(_ptr(out.codes), _ptr(out.scales), _ptr(out.global_scale), _ptr(out.choice_bits),
                     _ptr(out.rotated), _ptr(out.counters))
    _lib.check(_lib.load().fp4q_quantize_nvfp4(a, _ptr(x), _ptr(global_amax), o, _ptr(workspace), ws_bytes,
                                               _stream()), "fp4q_quantize_nvfp4")
    return out


def silu_mul_fwht_mxfp4(gate, up, *, policy="ocp", manual_exponent=0, rounding="rne", seed=0,
                        return_rotated=False, counters=False, out=None):
    """Fused SwiGLU epilogue: MXFP4 of the row FWHT of SiLU(gate) * up, for two
    same-shape 2-D fp32/bf16 GPU tensors with the same row stride (e.g.
    x[:, :d] and x[:, d:]).  Returns an MxResult like quantize_mxfp4."""
    _check_input(gate)
    _check_input(up)
    if gate.shape != up.shape or gate.dtype != up.dtype or (gate.shape[0] > 1 and gate.stride(0) != up.stride(0)):
        raise ValueError("fp4q: gate and up must have the same shape, dtype and row stride")
    rows, cols = gate.shape
    pol = {"ocp": _lib.FP4Q_SCALE_OCP_MAX, "manual": _lib.FP4Q_SCALE_MANUAL}[policy]
    a = _args(gate, 32, pol, manual_exponent, rounding, "fwht_row", seed)
    dev = gate.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        rot = torch.empty((rows, cols), dtype=torch.float32, device=dev) if return_rotated else None
        cnt = torch.empty(3, dtype=torch.int64, device=dev) if counters else None
        out = MxResult(codes, scales, rot, cnt)
    _check_mx_out(out, rows, cols)
    o = _lib.Outputs(_ptr(out.codes), _ptr(out.scales), None, None, _ptr(out.rotated), _ptr(out.counters))
    _lib.check(_lib.load().fp4q_silu_mul_fwht_mxfp4(a, _ptr(gate), _ptr(up), o, _stream()),
               "fp4q_silu_mul_fwht_mxfp4")
    return out


def fwht(x, transform_size=None, random_signs=False, seed=0, out=None):
    """Normalised Walsh-Hadamard transform of each transform_size-chunk of
    each row of a 2-D fp32/bf16 GPU tensor; fp32 result."""
    _check_input(x)
    rows, d = x.shape
    t = d if transform_size is None else int(transform_size)
    y = torch.empty((rows, d), dtype=torch.float32, device=x.device) if out is None else out
    _check_buf(y, (rows, d), torch.float32, "out")
    stride = int(x.stride(0)) if rows > 1 else d
    _lib.check(_lib.load().fp4q_fwht(rows, d, stride, _in_dtype(x), _ptr(x), _ptr(y), t, int(bool(random_signs)),
                                     int(seed) & 0xFFFFFFFFFFFFFFFF, _stream()), "fp4q_fwht")
    return y


def dequantize(fmt, codes, scales, global_scale=None, out_dtype=torch.float32, out=None):
    """Reconstruct [rows, cols] from packed codes and block scales.  fmt is
    "mxfp4", "nvfp4" or "if4" (the latter two need the fp32 global_scale tensor)."""
    f = {"mxfp4": _lib.FP4Q_MXFP4, "nvfp4": _lib.FP4Q_NVFP4, "if4": _lib.FP4Q_IF4}[fmt]
    rows, half = codes.shape
    cols = half * 2
    block = 32 if f == _lib.FP4Q_MXFP4 else 16
    _check_buf(codes, None, torch.uint8, "codes")
    _check_buf(scales, (rows, cols // block), torch.uint8, "scales")
    if global_scale is not None:
        _check_buf(global_scale, (1,), torch.float32, "global_scale")
    od = {torch.float32: _lib.FP4Q_F32, torch.bfloat16: _lib.FP4Q_BF16}[out_dtype]
    y = torch.empty((rows, cols), dtype=out_dtype, device=codes.device) if out is None else out
    _check_buf(y, (rows, cols), out_dtype, "out")
    _lib.check(_lib.load().fp4q_dequantize(f, rows, cols, block, _ptr(codes),
                                           _ptr(scales), _ptr(global_scale), od, _ptr(y), _stream()),
               "fp4q_dequantize")
    return y


def mxfp4_gemm(a, b, out_dtype=torch.float32, out=None):
    """C = A B^T for two MxResult-like operands (codes [rows, K/2], scales
    [rows, K/32]): A [M, K] and B [N, K] (e.g. activations and a weight
    quantized by quantize_mxfp4).  K must be a multiple of 128."""
    ac, asc = a[0], a[1]
    bc, bsc = b[0], b[1]
    M, K = ac.shape[0], ac.shape[1] * 2
    N = bc.shape[0]
    if bc.shape[1] * 2 != K or asc.shape != (M, K // 32) or bsc.shape != (N, K // 32):
        raise ValueError("fp4q: inconsistent GEMM operand shapes")
    for t in (ac, asc, bc, bsc):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError("fp4q: GEMM operands must be contiguous uint8 GPU tensors")
    od = {torch.float32: _lib.FP4Q_F32, torch.bfloat16: _lib.FP4Q_BF16}[out_dtype]
    c = torch.empty((M, N), dtype=out_dtype, device=ac.device) if out is None else out
    _check_buf(c, (M, N), out_dtype, "out")
    _lib.check(_lib.load().fp4q_mxfp4_gemm(M, N, K, _ptr(ac), _ptr(asc), _ptr(bc), _ptr(bsc), od, _ptr(c),
                                           _stream()), "fp4q_mxfp4_gemm")
    return c


def check_counters(counters):
    """Raise Fp4qError(FP4Q_ERR_NONFINITE) if the (device) counters report non-finite inputs."""
    import ctypes as C
    host = counters.detach().to("cpu").contiguous()
    buf = (C.c_uint64 * 3)(*[int(v) for v in host.tolist()])
    _lib.check(_lib.load().fp4q_check_counters(C.addressof(buf)), "fp4q_check_counters")


def version():
    return _lib.load().fp4q_version().decode()
