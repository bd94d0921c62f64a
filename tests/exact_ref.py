"""Exact-rational brute-force reference used to pin the C oracle.

Independent of the oracle by construction: it works in Python
``fractions.Fraction`` (no floating point in any decision), decodes the
E2M1 codes through the metrale_circuit "hardware::exec" E2M1 -> E4M3 bit
identity and torch's E4M3 byte decode (a library routine), decodes E4M3 and
E8M0 scales through torch's float8 byte decodes, finds the OCP exponent by
an integer search instead of frexp, and picks every code as the nearest
*reconstruction* over all candidate codes rather than by rounding a
normalised value.  Meant for tiny inputs only.
"""
from fractions import Fraction as Fr

import numpy as np
import torch


def _e4m3_byte_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    return [float(v) for v in b]


_E4M3 = _e4m3_byte_values()


def e4m3_byte_value(b):
    return _E4M3[b]


def e8m0_byte_value(b):
    t = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e8m0fnu).float()
    return float(t[0])


def e2m1_value_via_exec_identity(code):
    """value(code) = E4M3_decode(((c<<4) & 0x80) | (((c<<4) & 0x70) >> 2)) * 2^6."""
    q = (code & 0xF) << 4
    b = (q & 0x80) | ((q & 0x70) >> 2)
    return Fr(e4m3_byte_value(b)) * 64


E2M1 = [e2m1_value_via_exec_identity(c) for c in range(16)]


def _signbit(x):
    return bool(np.signbit(np.float64(x)))


def nearest_code(x, scale):
    """Code whose reconstruction value(c)*scale is nearest to x (exact), among the
    codes carrying x's sign; ties go to the code with an even mantissa bit.
    Returns (code, saturated)."""
    xs = Fr(float(x))
    sgn = 8 if _signbit(x) else 0
    best = None
    for m in range(8):
        c = sgn | m
        d = abs(xs - E2M1[c] * scale)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c)
    sat = abs(xs) > 6 * scale
    return best[1], sat


def stochastic_code(x, scale, u):
    """Round |x|/scale up iff it exceeds lo + (u/65536)(hi - lo) for the
    neighbouring lattice points lo <= |x|/scale < hi."""
    xs = Fr(float(x))
    sgn = 8 if _signbit(x) else 0
    a = abs(xs) / scale
    mags = [E2M1[m] for m in range(8)]
    if a > 6:
        return sgn | 7, True
    if a == 6:
        return sgn | 7, False
    for k in range(7):
        if mags[k] <= a < mags[k + 1]:
            t = mags[k] + Fr(int(u), 65536) * (mags[k + 1] - mags[k])
            return sgn | (k + 1 if a > t else k), False
    raise AssertionError("unreachable")


def ocp_exponent(amax):
    """Largest integer e with 2^e <= amax/4, clamped to [-127, 127]; 0 for amax 0."""
    if amax == 0:
        return 0
    q = Fr(float(amax)) / 4
    e = 0
    while Fr(2) ** e > q:
        e -= 1
    while Fr(2) ** (e + 1) <= q:
        e += 1
    return max(-127, min(127, e))


def e4m3_nearest(t):
    """Nearest finite non-negative E4M3 byte to the exact rational t; ties to the
    even code; t above 448 saturates."""
    if t >= 448:
        return 0x7E
    best = None
    for b in range(0x7F):
        d = abs(t - Fr(e4m3_byte_value(b)))
        if best is None or d < best[0] or (d == best[0] and (b & 1) == 0 and (best[1] & 1) == 1):
            best = (d, b)
    return best[1]


def mx_quantize(x, rounding=0, draws=None):
    """x: 2-D float64 array of exactly representable inputs; rows split into
    32-blocks.  Returns codes (int array, one per element), scale bytes and
    [saturated, underflowed]."""
    rows, cols = x.shape
    codes = np.zeros((rows, cols), np.int64)
    scales = np.zeros((rows, cols // 32), np.int64)
    sat = und = 0
    for r in range(rows):
        for b in range(cols // 32):
            blk = x[r, b * 32:(b + 1) * 32]
            e = ocp_exponent(max(abs(float(v)) for v in blk))
            scales[r, b] = e + 127
            sc = Fr(e8m0_byte_value(e + 127))
            for i, v in enumerate(blk):
                if rounding:
                    c, s = stochastic_code(v, sc, draws[r, b * 32 + i])
                else:
                    c, s = nearest_code(v, sc)
                codes[r, b * 32 + i] = c
                sat += s
                und += (v != 0 and (c & 7) == 0)
    return codes, scales, [sat, und]


def nv_global_scale(amax, divisor):
    if amax == 0:
        return np.float32(1.0)
    g = np.float32(amax) / np.float32(divisor)
    return np.float32(2.0 ** -149) if g == 0 else g


def nv_quantize(x, divisor=2688, mult=6, rounding=0, draws=None):
    """Two-level NVFP4 of a small 2-D float64 array: g = RN32(amax/divisor),
    per 16-block s = nearest E4M3 to bamax/(mult*g), codes nearest to x/(s*g)."""
    rows, cols = x.shape
    g = nv_global_scale(float(np.max(np.abs(x))), divisor)
    gF = Fr(float(g))
    codes = np.zeros((rows, cols), np.int64)
    scales = np.zeros((rows, cols // 16), np.int64)
    sat = und = 0
    for r in range(rows):
        for b in range(cols // 16):
            blk = x[r, b * 16:(b + 1) * 16]
            bam = Fr(max(abs(float(v)) for v in blk))
            sb = e4m3_nearest(bam / (mult * gF))
            scales[r, b] = sb
            sc = Fr(e4m3_byte_value(sb)) * gF
            for i, v in enumerate(blk):
                if sc == 0:
                    c, s = (8 if _signbit(v) else 0), False
                elif rounding:
                    c, s = stochastic_code(v, sc, draws[r, b * 16 + i])
                else:
                    c, s = nearest_code(v, sc)
                codes[r, b * 16 + i] = c
                sat += s
                und += (v != 0 and (c & 7) == 0)
    return codes, scales, g, [sat, und]


def nearest_int4_code(x, step):
    """Scaled INT4 of IF4: the sign-magnitude nibble (x's sign) whose
    reconstruction k*step, 0 <= k <= 7, is nearest to |x|; ties go to the even
    k.  Returns (code, saturated) with saturated = |x| > 7*step."""
    xs = abs(Fr(float(x)))
    best = None
    for k in range(8):
        d = abs(xs - k * step)
        if best is None or d < best[0] or (d == best[0] and k % 2 == 0 and best[1] % 2 == 1):
            best = (d, k)
    return (8 if _signbit(x) else 0) | best[1], xs > 7 * step


def if4_blocks(x):
    """IF4 of a small 2-D float64 array in exact arithmetic: g and the scale
    byte s of NVFP4 max->6, then per 16-block both candidates -- FP4 codes on
    the step s*g and INT4 codes on the step 6*s*g/7 -- with their exact sums
    of squared errors.  Yields (r, b, sb, fp4_codes, int4_codes, sse_fp4,
    sse_int4, int4_sat) and returns nothing else; g via nv_global_scale."""
    rows, cols = x.shape
    g = nv_global_scale(float(np.max(np.abs(x))), 2688)
    gF = Fr(float(g))
    for r in range(rows):
        for b in range(cols // 16):
            blk = x[r, b * 16:(b + 1) * 16]
            sb = e4m3_nearest(Fr(max(abs(float(v)) for v in blk)) / (6 * gF))
            sg = Fr(e4m3_byte_value(sb)) * gF
            if sg == 0:
                zero = [8 if _signbit(v) else 0 for v in blk]
                yield r, b, sb, zero, zero, Fr(0), Fr(0), 0
                continue
            cf = [nearest_code(v, sg)[0] for v in blk]
            ci = [nearest_int4_code(v, sg * 6 / 7) for v in blk]
            ef = sum((Fr(float(v)) - E2M1[c] * sg) ** 2 for v, c in zip(blk, cf))
            ei = sum((Fr(float(v)) - (-1 if c & 8 else 1) * (c & 7) * sg * 6 / 7) ** 2 for v, (c, _) in zip(blk, ci))
            yield r, b, sb, cf, [c for c, _ in ci], ef, ei, sum(int(s) for _, s in ci)


def round_to_f32_exact(v):
    """Nearest fp32 to the exact rational v (ties to even), as a Fraction."""
    if v == 0:
        return Fr(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    q = Fr(2) ** (max(e, -126) - 23)  # quantum: 24 significant bits, subnormals below 2^-126
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * q


def unpack_codes(packed):
    """[rows, cols/2] bytes -> [rows, cols] codes, element 2k in the low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.int64)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def round_to_bf16_exact(v):
    """Nearest bf16 to the exact rational v (ties to even), as a Fraction."""
    if v == 0:
        return Fr(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    q = Fr(2) ** (max(e, -126) - 7)  # quantum: 8 significant bits, subnormals below 2^-126
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * q
