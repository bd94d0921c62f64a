"""16-blocks on which the frozen fp32 order of the block sum of squared errors
picks a different candidate than exact arithmetic does.

Four Over Six ("Adaptive Block-Scaled Data Types" transcript, cue 10) keeps
the max->4 scaling of a block iff its sum of squared errors is lower; IF4
(cues 14 and 17) keeps scaled INT4 iff its sum is lower.  The pages fix no
precision for these sums, so the library freezes one fp32 evaluation order:

    dq = fl32(fl32(value * s) * g)          (INT4: fl32(k * 6 s g / 7))
    d  = fl32(x - dq),  sq = fl32(d * d)
    S_lo = sequential fl32 sum of sq over elements 0..7, S_hi over 8..15
    SSE  = fl32(S_lo + S_hi)

A block whose two exact sums are closer than that order's rounding error is
decided by the order alone.  This module builds such blocks without the
oracle: candidate codes and scale bytes come from the exact-rational
reference (exact_ref), the frozen order is evaluated here in numpy float32
(one rounding per operation, never fused), and one element of a random block
is walked in fp32 ulps across the point where the two exact sums cross.  It
keeps the values at which the frozen choice and the exact choice differ.

It also evaluates two plausible slips of that order (one sequential 16-term
sum instead of S_lo + S_hi, and a fused d * d + acc), so a test can show
that the blocks tell each of them apart from the frozen order.
"""
from fractions import Fraction as Fr

import numpy as np

import exact_ref as X

FOS, IF4 = "four_over_six", "if4"


def _f32(v):
    return np.float32(v)


def global_scale(kind, amax):
    """g = RN32(amax / (4 * 448)) for Four Over Six, RN32(amax / (6 * 448)) for IF4."""
    return X.nv_global_scale(float(amax), 1792 if kind == FOS else 2688)


def candidates(kind, xs, g):
    """Both candidates of one block of float values xs under tensor scale g.
    Returns (sb_a, codes_a, recon_a, sb_b, codes_b, recon_b, int4) where a is
    the default (max->6 / FP4) and b the alternative (max->4 / INT4); recon
    are exact reconstructions (Fractions); int4 tells how recon_b is formed."""
    gF = Fr(float(g))
    bam = Fr(max(abs(float(v)) for v in xs))
    sa = X.e4m3_nearest(bam / (6 * gF))
    step_a = Fr(X.e4m3_byte_value(sa)) * gF
    ca = [X.nearest_code(v, step_a)[0] for v in xs]
    ra = [X.E2M1[c] * step_a for c in ca]
    if kind == FOS:
        sb = X.e4m3_nearest(bam / (4 * gF))
        step_b = Fr(X.e4m3_byte_value(sb)) * gF
        cb = [X.nearest_code(v, step_b)[0] for v in xs]
        rb = [X.E2M1[c] * step_b for c in cb]
    else:
        sb = sa
        step_b = step_a * 6 / 7
        cb = [X.nearest_int4_code(v, step_b)[0] for v in xs]
        rb = [(-1 if c & 8 else 1) * (c & 7) * step_b for c in cb]
    return sa, ca, ra, sb, cb, rb


def _dq_f32(kind_b, codes, sb, g, order):
    """fp32 reconstructions of one candidate in the frozen order (or a slip)."""
    s = _f32(X.e4m3_byte_value(sb))
    if kind_b == "int4":
        step = Fr(X.e4m3_byte_value(sb)) * Fr(float(g)) * 6 / 7
        return np.array([float(X.round_to_f32_exact((-1 if c & 8 else 1) * (c & 7) * step)) for c in codes],
                        np.float32)
    vals = np.array([float(X.E2M1[c]) for c in codes], np.float32)
    return (vals * s) * g


def sse_f32(x, dq, order="frozen"):
    """Block SSE of rows of x (float32, [n, 16]) against dq ([n, 16] or [16]) in
    the frozen order, or in one of the slips 'seq16' and 'fma'."""
    x = np.asarray(x, np.float32)
    d = x - np.asarray(dq, np.float32)
    if order == "fma":
        out = []
        for row in d:
            lo = hi = Fr(0)
            for i, di in enumerate(row):
                e = Fr(float(di)) ** 2
                if i < 8:
                    lo = X.round_to_f32_exact(lo + e)
                else:
                    hi = X.round_to_f32_exact(hi + e)
            out.append(np.float32(float(lo)) + np.float32(float(hi)))
        return np.array(out, np.float32)
    sq = d * d
    if order == "seq16":
        acc = np.zeros(x.shape[0], np.float32)
        for i in range(16):
            acc = acc + sq[:, i]
        return acc
    lo = np.zeros(x.shape[0], np.float32)
    hi = np.zeros(x.shape[0], np.float32)
    for i in range(8):
        lo = lo + sq[:, i]
    for i in range(8, 16):
        hi = hi + sq[:, i]
    return lo + hi


def choice_f32(kind, x, cand, g, order="frozen"):
    """True where the frozen order (or a slip) keeps the alternative candidate."""
    sa, ca, _, sb, cb, _ = cand
    dqa = _dq_f32("fp4", ca, sa, g, order)
    dqb = _dq_f32("int4" if kind == IF4 else "fp4", cb, sb, g, order)
    ea = sse_f32(x, dqa, order)
    eb = sse_f32(x, dqb, order)
    return eb < ea


def build(kind, n_blocks, seed, amax=7.3, walk=48, per_block=2, max_tries=5000):
    """Return (x, info): x float32 [1 + n, 16], row 0 holding the tensor
    maximum amax (so g is fixed), rows 1.. near-tie blocks; info[r] =
    (frozen_choice, exact_choice, cand) for every row r >= 1, where a choice
    is True for the alternative candidate (max->4 / INT4)."""
    rng = np.random.default_rng(seed)
    amax = _f32(amax)
    g = global_scale(kind, amax)
    rows = [np.array([amax] + [0.0] * 15, np.float32)]
    info = [None]
    tries = 0
    while len(rows) <= n_blocks and tries < max_tries:
        tries += 1
        bam = _f32(amax * rng.uniform(0.05, 0.95))
        if rng.random() < 0.5:
            blk = rng.uniform(-1.0, 1.0, 16) * float(bam)
        else:
            blk = np.clip(rng.normal(0.0, 0.4, 16), -1.0, 1.0) * float(bam)
        blk = blk.astype(np.float32)
        im = int(rng.integers(16))
        blk[im] = bam if rng.random() < 0.5 else -bam
        blk = np.where(np.abs(blk) > bam, np.sign(blk) * bam, blk).astype(np.float32)
        xs = [float(v) for v in blk]
        cand = candidates(kind, xs, g)
        sa, ca, ra, sb, cb, rb = cand
        terms = [(Fr(v) - b) ** 2 - (Fr(v) - a) ** 2 for v, a, b in zip(xs, ra, rb)]
        total = sum(terms)
        order = rng.permutation(16)
        kept = 0
        for k in order:
            k = int(k)
            if k == im or ra[k] == rb[k] or kept >= per_block:
                continue
            c_rest = total - terms[k]
            root = (-c_rest - rb[k] ** 2 + ra[k] ** 2) / (2 * (ra[k] - rb[k]))
            if abs(root) >= Fr(float(bam)) or (root < 0) != (xs[k] < 0) or root == 0:
                continue
            x0 = _f32(float(root))
            vals = [x0]
            lo = hi = x0
            for _ in range(walk):
                lo = np.nextafter(lo, _f32(-np.inf))
                hi = np.nextafter(hi, _f32(np.inf))
                vals += [lo, hi]
            vals = np.array(vals, np.float32)
            xmat = np.tile(blk, (len(vals), 1))
            xmat[:, k] = vals
            frozen = choice_f32(kind, xmat, cand, g)
            # the exact difference SSE_b - SSE_a is linear in the walked element:
            # slope * (v - root), zero at the root (a tie keeps candidate a)
            slope_pos = ra[k] > rb[k]
            for v, fz in zip(vals, frozen):
                vF = Fr(float(v))
                exact = (vF < root) if slope_pos else (vF > root)
                if bool(fz) == exact:
                    continue
                # the walked element must keep its codes under both scalings
                step_a = Fr(X.e4m3_byte_value(sa)) * Fr(float(g))
                if X.nearest_code(float(v), step_a)[0] != ca[k]:
                    continue
                if kind == FOS:
                    ok = X.nearest_code(float(v), Fr(X.e4m3_byte_value(sb)) * Fr(float(g)))[0] == cb[k]
                else:
                    ok = X.nearest_int4_code(float(v), step_a * 6 / 7)[0] == cb[k]
                if not ok or abs(float(v)) >= float(bam):
                    continue
                row = blk.copy()
                row[k] = v
                rows.append(row)
                info.append((bool(fz), exact, cand))
                kept += 1
                break
            if len(rows) > n_blocks:
                break
    return np.stack(rows), info
