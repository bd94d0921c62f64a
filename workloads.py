"""Seeded synthetic input tensors for the quantization workloads.

This module only draws random numbers and casts them; it holds none of the
quantizer's arithmetic.  Both the GPU path's tests/benchmark and the CPU
oracle's tests take their inputs from here.  Every generator uses
``numpy.random.Generator(PCG64(seed))`` in fp64, then casts to fp32 (IEEE
round-to-nearest-even) and, for bf16 workloads, from fp32 to bf16 with
round-to-nearest-even.  bf16 tensors are returned as their raw uint16 bits.

The shapes and value distributions stand in for the activation, weight and
gradient tensors the pages discuss: outlier channels after a SwiGLU-like
gate (Sub-4-Bit Microscaling, section 3), heavy-tailed activations, sparse
large weights, and small Laplace-distributed gradients (Adaptive
Block-Scaled Data Types transcript, cues 8 and 21).
"""
from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(a):
    """Round fp32 -> bf16 (nearest, ties to even) and return the uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    cols: int
    dtype: str          # "f32" or "bf16"
    seed: int
    description: str


WORKLOADS = {
    "mx_f32_1024": Workload("mx_f32_1024", 1024, 1024, "f32", 101,
                            "N(0,1) fp32 1024x1024, 10 random columns x50"),
    "act_bf16_8192": Workload("act_bf16_8192", 8192, 8192, "bf16", 102,
                              "2*Student-t(nu=4) bf16 8192x8192 activations"),
    "swiglu_bf16_16384x8192": Workload("swiglu_bf16_16384x8192", 16384, 8192, "bf16", 103,
                                       "|N(0,1)| bf16 16384x8192, 8 fixed outlier channels x100"),
    "weight_bf16_8192x28672": Workload("weight_bf16_8192x28672", 8192, 28672, "bf16", 104,
                                       "N(0,0.02) bf16 8192x28672, 0.1% of entries x20"),
    "grad_bf16_8192": Workload("grad_bf16_8192", 8192, 8192, "bf16", 105,
                               "Laplace(0,1e-3) bf16 8192x8192 gradients"),
    "gate_up_bf16_16384x8192": Workload("gate_up_bf16_16384x8192", 16384, 16384, "bf16", 106,
                                        "[gate | up] bf16 16384x(2x8192): gate N(0,1.5), up N(0,1) with "
                                        "8 fixed outlier channels x100"),
}

SR_SEED = 0x5EED  # Philox key of the gradient workload


def _draw(name, rows, cols, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "mx_f32_1024":
        x = rng.standard_normal((rows, cols))
        c = rng.choice(cols, 10, replace=False)
        x[:, c] *= 50.0
    elif name == "act_bf16_8192":
        x = 2.0 * rng.standard_t(4, size=(rows, cols))
    elif name == "swiglu_bf16_16384x8192":
        x = np.abs(rng.standard_normal((rows, cols)))
        c = rng.choice(cols, 8, replace=False)
        x[:, c] *= 100.0
    elif name == "weight_bf16_8192x28672":
        x = rng.normal(0.0, 0.02, size=(rows, cols))
        n = rows * cols
        k = int(0.001 * n)
        idx = rng.choice(n, k, replace=False)
        x.reshape(-1)[idx] *= 20.0
    elif name == "grad_bf16_8192":
        x = rng.laplace(0.0, 1e-3, size=(rows, cols))
    elif name == "gate_up_bf16_16384x8192":
        # gate and up halves of a SwiGLU input row (the up-projection output
        # carries a few outlier channels, which SiLU_and_Mul keeps)
        d = cols // 2
        x = np.empty((rows, cols), np.float32)
        x[:, :d] = 1.5 * rng.standard_normal((rows, d))
        x[:, d:] = rng.standard_normal((rows, d))
        c = rng.choice(d, 8, replace=False)
        x[:, d + c] *= 100.0
    else:
        raise KeyError(name)
    return x


def make(name, rows=None, cols=None):
    """Return the workload tensor: float32 array or uint16 bf16 bits.

    ``rows``/``cols`` override the shape (same recipe, same seed) for the
    small parity cases."""
    w = WORKLOADS[name]
    rows = w.rows if rows is None else rows
    cols = w.cols if cols is None else cols
    x = _draw(name, rows, cols, w.seed).astype(np.float32)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def random_tensor(rows, cols, dtype, seed, scale=1.0, dist="normal"):
    """Generic seeded tensor for edge-case and ragged-shape tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "normal":
        x = rng.standard_normal((rows, cols)) * scale
    elif dist == "t":
        x = rng.standard_t(3, size=(rows, cols)) * scale
    elif dist == "uniform":
        x = rng.uniform(-scale, scale, size=(rows, cols))
    else:
        raise KeyError(dist)
    x = x.astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x
