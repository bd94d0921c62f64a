"""The bound that lets the kernels decide Four-Over-Six and IF4 blocks by
cheaper sums ("Adaptive Block-Scaled Data Types" transcript, cues 10, 14 and
17: the candidate with the lower block SSE is kept; the library freezes one
fp32 order for that SSE).

Frozen order, per half block of 8 elements (S_lo, S_hi), then S = S_lo + S_hi:
    dq = fl(fl(value * s) * g)     (INT4: dq = RN32(k * 6 s g / 7))
    d = fl(x - dq), acc = fl(acc + fl(d * d))
FMA sums: h = fl(s g) (INT4: h = RN32(6 s g / 7), value = k), d' = fma(-value,
h, x), acc = fma(d', d', acc), A = A_lo + A_hi.

The kernels decide a block by the FMA sums only when they differ by more than
bound(A_default) + bound(A_alt), bound(A) = 2^-18 A + 2^-19 M^2 + 2^-129 with
M = 6 s g (INT4: 7 h); the derivation gives |S - A| below half of that.  This
checks |S - A| <= bound / 2 on random blocks over a wide range of magnitudes,
with nearest codes and with arbitrary codes.  numpy evaluates the float32
steps one rounding at a time; an FMA is evaluated in float64 and rounded to
float32 (the 48-bit product is exact there, the sum is rounded twice, which
moves the result by far less than the margin tested).
"""
import numpy as np
import pytest

# blocks near the top of the float range overflow (they are left out of the check)
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

f32 = np.float32
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _e4m3_values():
    v = []
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        v.append((m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v)


E4M3 = _e4m3_values()


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _bound(a, m):
    return 2.0 ** -18 * a.astype(np.float64) + 2.0 ** -19 * m.astype(np.float64) ** 2 + 2.0 ** -129


def _blocks(rng, n):
    scale = 2.0 ** rng.integers(-60, 61, (n, 1))
    kind = rng.integers(0, 4, (n, 1))
    t = rng.standard_t(3, (n, 16))
    u = rng.uniform(-1, 1, (n, 16))
    w = np.ldexp(rng.uniform(0.5, 1, (n, 16)) * rng.choice([-1, 1], (n, 16)), rng.integers(-20, 1, (n, 16)))
    x = np.where(kind == 0, t, np.where(kind == 1, u, w)) * scale
    return x.astype(np.float32)


def _scale_value(amax, g, target):
    want = amax / (target * g.astype(np.float64))
    return E4M3[np.argmin(np.abs(E4M3[None, :] - want[:, None]), axis=1)].astype(np.float32)


def _half_sums(terms_frozen, terms_fma):
    s = [np.zeros(terms_frozen.shape[0], np.float32) for _ in range(2)]
    a = [np.zeros(terms_frozen.shape[0], np.float32) for _ in range(2)]
    for h in range(2):
        for i in range(8 * h, 8 * h + 8):
            d = terms_frozen[:, i]
            s[h] = (s[h] + (d * d).astype(np.float32)).astype(np.float32)
            dp = terms_fma[:, i]
            a[h] = _fma32(dp, dp, a[h])
    return (s[0] + s[1]).astype(np.float32), (a[0] + a[1]).astype(np.float32)


def _check(S, A, M):
    ok = np.isfinite(S) & np.isfinite(A) & (np.maximum(S, A) < 2.0 ** 120)
    ratio = np.abs(S[ok].astype(np.float64) - A[ok].astype(np.float64)) / (_bound(A[ok], M[ok]) / 2)
    assert ok.sum() > 0.9 * len(S)
    assert ratio.max() <= 1.0, ratio.max()
    return ratio.max()


def test_fp4_candidate_sums_within_bound():
    rng = np.random.default_rng(5)
    n = 60000
    x = _blocks(rng, n)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    keep = amax > 0
    x, amax = x[keep], amax[keep]
    g = (amax / 1792 * rng.uniform(0.3, 3.0, len(x))).astype(np.float32)
    worst = 0.0
    for target in (6.0, 4.0):
        sd = _scale_value(amax, g, target)
        step = sd.astype(np.float64) * g.astype(np.float64)
        q = np.abs(x.astype(np.float64)) / step[:, None]
        val = np.sign(x) * E2M1[np.argmin(np.abs(q[:, :, None] - E2M1[None, None, :]), axis=2)]
        wild = rng.random(len(x)) < 0.3          # arbitrary codes obey the bound too
        val[wild] = rng.choice(np.concatenate([E2M1, -E2M1]), (wild.sum(), 16))
        val = val.astype(np.float32)
        vs = (val * sd[:, None]).astype(np.float32)
        dq = (vs * g[:, None]).astype(np.float32)
        d = (x - dq).astype(np.float32)
        h = (sd * g).astype(np.float32)
        dp = _fma32(-val, np.broadcast_to(h[:, None], val.shape), x)
        S, A = _half_sums(d, dp)
        worst = max(worst, _check(S, A, (6 * h).astype(np.float32)))
    assert worst > 0.01   # the check is not vacuous


def test_int4_candidate_sums_within_bound():
    rng = np.random.default_rng(6)
    n = 60000
    x = _blocks(rng, n)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    keep = amax > 0
    x, amax = x[keep], amax[keep]
    g = (amax / 2688 * rng.uniform(0.3, 3.0, len(x))).astype(np.float32)
    sd = _scale_value(amax, g, 6.0)
    sg = sd.astype(np.float64) * g.astype(np.float64)
    k = np.minimum(np.rint(np.abs(x.astype(np.float64)) / (6 * sg[:, None] / 7)), 7)
    wild = rng.random(len(x)) < 0.3
    k[wild] = rng.integers(0, 8, (wild.sum(), 16))
    dq = (k * 6.0 * sg[:, None] / 7.0).astype(np.float32)       # one rounding of the exact value
    d = (np.abs(x) - dq).astype(np.float32)
    h7 = (6.0 * sg / 7.0).astype(np.float32)
    dp = _fma32(-k.astype(np.float32), np.broadcast_to(h7[:, None], k.shape), np.abs(x))
    S, A = _half_sums(d, dp)
    worst = _check(S, A, (7 * h7).astype(np.float32))
    assert worst > 0.01
