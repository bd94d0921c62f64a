"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Codes, scale bytes, global scales, choice bits, counters
and dequantized values must be bit-identical; rotations are checked against
the fp64 oracle transform at relative L2 <= 1e-5, and the oracle quantizer is
applied to the GPU's rotated fp32 values."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_row_amd")

RTOL_ROT = 1e-5
_cache = {}


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(gpu()).view(torch.bfloat16)
    return torch.from_numpy(a).to(gpu())


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def workload(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = workloads.make(name)
    return _cache[name]


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint16)


def assert_same(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %s want %s" % (
        what, bad.size, bad[:5], got.reshape(-1)[bad[:5]], want.reshape(-1)[bad[:5]])


def rel_l2(got, want):
    got = got.astype(np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def choice_bits_rows(choice, r0, r1, blocks_per_row):
    allbits = np.unpackbits(choice, bitorder="little")
    return allbits[r0 * blocks_per_row:r1 * blocks_per_row]


# ------------------------------------------------------------------ full-size workloads
def test_mx_fp32_1024_quant_dequant_counts():
    x = workload("mx_f32_1024")
    r = fq.quantize_mxfp4(to_dev(x), counters=True)
    c, s, cnt = oracle.quantize_mx(x)
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    d32 = fq.dequantize("mxfp4", r.codes, r.scales, out_dtype=torch.float32)
    assert_same(bits(host(d32)), bits(oracle.dequantize(oracle.MX, c, s)), "dequant fp32")
    d16 = fq.dequantize("mxfp4", r.codes, r.scales, out_dtype=torch.bfloat16)
    assert_same(host(d16), oracle.dequantize(oracle.MX, c, s, out_dtype=oracle.BF16), "dequant bf16")


def test_mx_bf16_8192_headline():
    x = workload("act_bf16_8192")
    xd = to_dev(x)
    r = fq.quantize_mxfp4(xd)
    c, s, cnt = oracle.quantize_mx(x)
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.scales), s, "scales")
    r2 = fq.quantize_mxfp4(xd, counters=True)            # counting variant: same codes
    assert_same(host(r2.codes), c, "codes (counting kernel)")
    assert_same(host(r2.counters).astype(np.uint64), cnt, "counters")


def test_nv_bf16_8192_headline_and_dequant():
    x = workload("act_bf16_8192")
    xd = to_dev(x)
    r = fq.quantize_nvfp4(xd, counters=True)
    c, s, g, _, cnt = oracle.quantize_nv(x)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    d16 = fq.dequantize("nvfp4", r.codes, r.scales, r.global_scale, out_dtype=torch.bfloat16)
    assert_same(host(d16), oracle.dequantize(oracle.NV, c, s, g, out_dtype=oracle.BF16), "dequant bf16")
    r2 = fq.quantize_nvfp4(xd)            # no counters: the single-read kernel
    assert host(r2.global_scale)[0] == g
    assert_same(host(r2.scales), s, "scales (single-read kernel)")
    assert_same(host(r2.codes), c, "codes (single-read kernel)")


def test_fwht_mx_swiglu_16384x8192():
    x = workload("swiglu_bf16_16384x8192")
    xd = to_dev(x)
    r = fq.quantize_mxfp4(xd, rotation="fwht_row", return_rotated=True)
    rot = host(r.rotated)
    c, s, _ = oracle.quantize_mx(rot)
    assert_same(host(r.codes), c, "codes of the rotated values")
    assert_same(host(r.scales), s, "scales of the rotated values")
    r2 = fq.quantize_mxfp4(xd, rotation="fwht_row")       # no rotated store: identical codes
    assert_same(host(r2.codes), c, "codes without the rotated hook")
    rows = np.random.default_rng(0).choice(x.shape[0], 64, replace=False)
    ref = oracle.fwht(x[rows])
    assert rel_l2(rot[rows], ref) <= RTOL_ROT


def oracle_nv_all_rows(x, policy, amax, rows_per_chunk=128):
    """The oracle's NVFP4 of every row of x, rows split over host threads
    (the C oracle runs without the GIL); amax is the tensor amax, so every
    chunk uses the tensor's g.  Returns codes, scales, g, choice bytes (or
    None) and the summed counters."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    R, cols = x.shape
    nbr = cols // 16
    assert (rows_per_chunk * nbr) % 8 == 0          # chunk choice bits start on byte boundaries
    chunks = [(r0, min(R, r0 + rows_per_chunk)) for r0 in range(0, R, rows_per_chunk)]
    nthreads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(nthreads) as ex:
        parts = list(ex.map(lambda c: oracle.quantize_nv(x[c[0]:c[1]], policy=policy, global_amax=amax), chunks))
    codes = np.concatenate([p[0] for p in parts])
    scales = np.concatenate([p[1] for p in parts])
    g = parts[0][2]
    assert all(p[2] == g for p in parts)
    choice = None
    if parts[0][3] is not None:
        bitsall = np.concatenate([np.unpackbits(p[3], bitorder="little")[:(c[1] - c[0]) * nbr]
                                  for p, c in zip(parts, chunks)])
        choice = np.packbits(bitsall, bitorder="little")
    cnt = np.sum([p[4] for p in parts], axis=0).astype(np.uint64)
    return codes, scales, g, choice, cnt


# The three tests below share the 8192 x 28672 weight (generated once), every
# row compared.
def test_four_over_six_weight_8192x28672_all_rows():
    x = workload("weight_bf16_8192x28672")
    amax = oracle.tensor_amax(x)
    c, s, g, ch, cnt = oracle_nv_all_rows(x, 3, amax)
    assert g == np.float32(amax) / np.float32(1792)
    xd = to_dev(x)
    for counters in (False, True):   # (without counters: the kernel the bench times)
        r = fq.quantize_nvfp4(xd, policy="four_over_six", counters=counters)
        assert host(r.global_scale)[0] == g
        assert_same(host(r.scales), s, "scales (counters %s)" % counters)
        assert_same(host(r.codes), c, "codes (counters %s)" % counters)
        assert_same(host(r.choice_bits), ch, "choice bits (counters %s)" % counters)
        if counters:
            assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
        del r


def test_if4_weight_8192x28672_all_rows():
    x = workload("weight_bf16_8192x28672")
    amax = oracle.tensor_amax(x)
    c, s, g, _, cnt = oracle_nv_all_rows(x, 4, amax)
    xd = to_dev(x)
    for counters in (False, True):
        _if4_check(fq.quantize_nvfp4(xd, policy="if4", counters=counters), c, s, g, cnt if counters else None)


def test_nv_max6_weight_8192x28672_two_pass_all_rows():
    """max->6, RNE, no counters, amax in the call, over 64 Mi elements: too
    large for the single-read kernel, so the amax pass and the streaming
    paired encode run on the per-workgroup partials in the workspace."""
    x = workload("weight_bf16_8192x28672")
    amax = oracle.tensor_amax(x)
    c, s, g, _, cnt = oracle_nv_all_rows(x, 2, amax)
    r = fq.quantize_nvfp4(to_dev(x))
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    r = fq.quantize_nvfp4(to_dev(x), counters=True)   # the two-pass kernel with counters: same bytes
    assert_same(host(r.codes), c, "codes (counters)")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


def test_rht_sr_grad_8192():
    x = workload("grad_bf16_8192")
    xd = to_dev(x)
    seed = workloads.SR_SEED
    r = fq.quantize_nvfp4(xd, rotation="rht16", rounding="stochastic", seed=seed, return_rotated=True,
                          counters=True)
    rot = host(r.rotated)
    c, s, g, _, cnt = oracle.quantize_nv(rot, rounding=1, seed=seed)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    ref = oracle.fwht(x[:512], t=16, random_signs=True, seed=seed)
    assert rel_l2(rot[:512], ref) <= RTOL_ROT
    r2 = fq.quantize_nvfp4(xd, rotation="rht16", rounding="stochastic", seed=seed)
    assert_same(host(r2.codes), c, "codes without the rotated hook")


# ------------------------------------------------------------------ small and ragged shapes
SHAPES = [(1, 32), (3, 64), (17, 96), (5, 160), (64, 256), (7, 1024), (33, 544)]


def make_input(rows, cols, dtype, seed, dist="t", pad=0):
    full = workloads.random_tensor(rows, cols + pad, dtype, seed, scale=3.0, dist=dist)
    return full


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rounding", ["rne", "stochastic"])
@pytest.mark.parametrize("rotation", [None, "rht16"])
@pytest.mark.parametrize("counters", [True, False])
def test_mx_small(rows, cols, dtype, rounding, rotation, counters):
    # odd row counts read every row from a wider padded tensor (strided input)
    pad = 32 if rows % 2 else 0
    full = make_input(rows, cols, dtype, rows * 1000 + cols, pad=pad)
    xd = to_dev(full)[:, :cols]
    r = fq.quantize_mxfp4(xd, rounding=rounding, seed=77, rotation=rotation, counters=counters,
                          return_rotated=rotation is not None)
    if rotation is None:
        c, s, cnt = oracle.quantize_mx(full, cols=cols, rounding=int(rounding != "rne"), seed=77)
    else:
        rot = host(r.rotated)
        ref = oracle.fwht(np.ascontiguousarray(full[:, :cols]), t=16, random_signs=True, seed=77)
        assert rel_l2(rot, ref) <= RTOL_ROT
        c, s, cnt = oracle.quantize_mx(rot, rounding=int(rounding != "rne"), seed=77)
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.scales), s, "scales")
    if counters:
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("policy", ["max6", "four_over_six"])
@pytest.mark.parametrize("rounding", ["rne", "stochastic"])
@pytest.mark.parametrize("counters", [True, False])
def test_nv_small(rows, cols, dtype, policy, rounding, counters):
    # odd row counts read every row from a wider padded tensor (strided input)
    pad = 16 if rows % 2 else 0
    full = make_input(rows, cols, dtype, rows * 7 + cols, pad=pad)
    xd = to_dev(full)[:, :cols]
    r = fq.quantize_nvfp4(xd, policy=policy, rounding=rounding, seed=123, counters=counters)
    c, s, g, ch, cnt = oracle.quantize_nv(full, cols=cols, policy=3 if policy == "four_over_six" else 2,
                                         rounding=int(rounding != "rne"), seed=123)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    if counters:
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    if ch is not None:
        assert_same(host(r.choice_bits), ch, "choice bits")


@pytest.mark.parametrize("rows,cols", [(4, 64), (9, 4096), (3, 8192), (2, 16384), (5, 32), (6, 2048)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwht_row_mx_small(rows, cols, dtype):
    full = make_input(rows, cols, dtype, cols + rows, dist="normal")
    xd = to_dev(full)
    for rounding in ("rne", "stochastic"):
        r = fq.quantize_mxfp4(xd, rotation="fwht_row", return_rotated=True, counters=True, rounding=rounding,
                              seed=9)
        rot = host(r.rotated)
        assert rel_l2(rot, oracle.fwht(full)) <= RTOL_ROT
        c, s, cnt = oracle.quantize_mx(rot, rounding=int(rounding != "rne"), seed=9)
        assert_same(host(r.codes), c, "codes")
        assert_same(host(r.scales), s, "scales")
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


@pytest.mark.parametrize("t", [2, 4, 8, 16, 32, 64, 256, 1024, 4096, 8192, 16384])
@pytest.mark.parametrize("signs", [False, True])
def test_fwht_standalone(t, signs):
    rows = 3
    d = max(t, 64)
    full = make_input(rows, d, "bf16", t, dist="normal", pad=64)
    xd = to_dev(full)[:, :d]
    y = host(fq.fwht(xd, transform_size=t, random_signs=signs, seed=0xABC))
    ref = oracle.fwht(np.ascontiguousarray(full[:, :d]), t=t, random_signs=signs, seed=0xABC)
    assert rel_l2(y, ref) <= RTOL_ROT


# ------------------------------------------------------------------ edge cases
def test_empty_inputs():
    dev = gpu()
    for dtype in (torch.float32, torch.bfloat16):
        x = torch.empty((0, 64), dtype=dtype, device=dev)
        r = fq.quantize_mxfp4(x, counters=True)
        assert r.codes.numel() == 0 and host(r.counters).tolist() == [0, 0, 0]
        n = fq.quantize_nvfp4(x, counters=True)
        assert host(n.global_scale)[0] == 1.0 and host(n.counters).tolist() == [0, 0, 0]
        n = fq.quantize_nvfp4(x, policy="four_over_six")
        assert host(n.global_scale)[0] == 1.0
        assert fq.fwht(x).numel() == 0
        assert fq.dequantize("mxfp4", torch.empty((0, 32), dtype=torch.uint8, device=dev),
                             torch.empty((0, 2), dtype=torch.uint8, device=dev)).numel() == 0


def _special_tensor(dtype):
    rng = np.random.default_rng(42)
    x = (rng.standard_t(3, (6, 128)) * 2).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    x[1, 41] = -np.inf
    x[2, :32] = 0.0
    x[2, 32:48] = -0.0
    x[3, :] = np.ldexp(rng.uniform(-1, 1, 128), -130).astype(np.float32)   # subnormal block
    x[4, :] *= 1e30
    x[5, 0] = -0.0
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_zero_subnormal_huge(dtype):
    x = _special_tensor(dtype)
    xd = to_dev(x)
    r = fq.quantize_mxfp4(xd, counters=True)
    c, s, cnt = oracle.quantize_mx(x)
    assert_same(host(r.codes), c, "mx codes")
    assert_same(host(r.scales), s, "mx scales")
    assert_same(host(r.counters).astype(np.uint64), cnt, "mx counters")
    for pol, p in (("max6", 2), ("four_over_six", 3)):
        n = fq.quantize_nvfp4(xd, policy=pol, counters=True)
        c, s, g, ch, cnt = oracle.quantize_nv(x, policy=p)
        assert host(n.global_scale)[0] == g
        assert_same(host(n.scales), s, "nv scales")
        assert_same(host(n.codes), c, "nv codes")
        assert_same(host(n.counters).astype(np.uint64), cnt, "nv counters")
        if ch is not None:
            assert_same(host(n.choice_bits), ch, "choice")
    with pytest.raises(fq.Fp4qError):
        fq.check_counters(n.counters)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rotation,rounding", [("rht16", "rne"), ("rht16", "stochastic"), ("fwht128", "rne")])
@pytest.mark.parametrize("kind", ["inf", "nan"])
def test_nv_rotated_nonfinite_amax(dtype, rotation, rounding, kind):
    """The tensor amax of rotated values is the largest finite rotated value.
    'inf': an infinite input and a row of huge finite inputs whose rotated
    sums overflow, next to ordinary rows (the amax pass then rescans with a
    filter per value); 'nan': a NaN input only (the float maxima pass over
    it).  Compared with the oracle on the GPU's rotated values."""
    rng = np.random.default_rng(91)
    x = (rng.standard_t(3, (8, 128)) * 2).astype(np.float32)
    if kind == "inf":
        x[1, 40] = np.inf
        x[2, :] = rng.choice([-1.0, 1.0], 128) * np.float32(3.0e38)
    else:
        x[1, 40] = np.nan
    x[3, :] = np.ldexp(rng.uniform(-1, 1, 128), -130).astype(np.float32)
    x[4, :] *= 1e30
    xin = f32_to_bf16_bits(x) if dtype == "bf16" else x
    r = fq.quantize_nvfp4(to_dev(xin), rotation=rotation, rounding=rounding, seed=0x77, return_rotated=True)
    rot = host(r.rotated)
    if kind == "inf":
        assert np.isinf(rot).any() and np.isfinite(rot).any()
    else:
        assert np.isnan(rot).any() and not np.isinf(rot).any()
    if rounding == "rne":
        c, s, g, _, _ = oracle.quantize_nv(rot, policy=2)
    else:
        c, s, g, _, _ = oracle.quantize_nv(rot, policy=2, rounding=1, seed=0x77)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rotation", ["none", "rht16"])
@pytest.mark.parametrize("counters", [False, True])
def test_nv_stochastic_signed_zeros_and_subnormal_elements(dtype, rotation, counters):
    """Stochastic rounding keeps the sign of every code, zeros and underflows
    included (R-5, R-17): 16-blocks whose maximum is a normal value and whose
    other elements are +-0, subnormals of either sign and tiny normals, so
    that the scaled products of the small ones are zero or subnormal."""
    rng = np.random.default_rng(77)
    rows, cols = 24, 128
    x = np.empty((rows, cols), np.float32)
    kinds = rng.integers(0, 5, (rows, cols))
    x[kinds == 0] = 0.0
    x[kinds == 1] = -0.0
    sub = np.ldexp(rng.uniform(0.5, 1.0, (rows, cols)), rng.integers(-149, -127, (rows, cols)))
    x[kinds == 2] = -sub[kinds == 2]
    x[kinds == 3] = sub[kinds == 3]
    tiny = np.ldexp(rng.uniform(-1, 1, (rows, cols)), -120)
    x[kinds == 4] = tiny[kinds == 4]
    x[:, ::16] = rng.choice([-1, 1], (rows, cols // 16)) * rng.uniform(0.5, 4.0, (rows, cols // 16))
    x = x.astype(np.float32)
    xin = f32_to_bf16_bits(x) if dtype == "bf16" else x
    rot = 1 if rotation == "rht16" else 0
    n = fq.quantize_nvfp4(to_dev(xin), rotation=rotation, rounding="stochastic", seed=0x5EED, counters=counters,
                          return_rotated=True)
    if rot:
        # codes against the oracle's NVFP4 of the GPU's own rotated values (as the other rotation tests)
        xr = host(n.rotated)
        c, s, g, _, cnt = oracle.quantize_nv(xr, rounding=1, seed=0x5EED)
    else:
        c, s, g, _, cnt = oracle.quantize_nv(xin, rounding=1, seed=0x5EED)
    assert host(n.global_scale)[0] == g
    assert_same(host(n.scales), s, "scales")
    assert_same(host(n.codes), c, "codes")
    if counters:
        assert_same(host(n.counters).astype(np.uint64), cnt, "counters")


@pytest.mark.parametrize("scale_exp", [-140, -120, -101, -60, 0, 100, 120])
def test_nv_tiny_and_huge_tensors(scale_exp):
    """Tensors whose global scale is tiny take the all-fp64 path (g < 2^-100)."""
    rng = np.random.default_rng(scale_exp + 500)
    x = np.ldexp(rng.standard_t(4, (8, 64)), scale_exp).astype(np.float32)
    for rounding in (0, 1):
        n = fq.quantize_nvfp4(to_dev(x), rounding=("stochastic" if rounding else "rne"), seed=3, counters=True)
        c, s, g, _, cnt = oracle.quantize_nv(x, rounding=rounding, seed=3)
        assert host(n.global_scale)[0] == g
        assert_same(host(n.scales), s, "scales")
        assert_same(host(n.codes), c, "codes")
        assert_same(host(n.counters).astype(np.uint64), cnt, "counters")
        d = fq.dequantize("nvfp4", n.codes, n.scales, n.global_scale, out_dtype=torch.bfloat16)
        assert_same(host(d), oracle.dequantize(oracle.NV, c, s, g, out_dtype=oracle.BF16), "dequant bf16")
        d = fq.dequantize("nvfp4", n.codes, n.scales, n.global_scale, out_dtype=torch.float32)
        assert_same(bits(host(d)), bits(oracle.dequantize(oracle.NV, c, s, g)), "dequant fp32")


@pytest.mark.parametrize("scale_exp", [None, -140, -101, -60, 0, 100, 120])
def test_four_over_six_streaming_specials_tiny_huge(scale_exp):
    """Four Over Six of contiguous bf16 without counters (the streaming
    kernel): non-finite, zero and subnormal blocks, and tensors whose g is
    below 2^-100 (every block on the exact path) or near the top of the range,
    with ragged tile counts and a caller amax."""
    if scale_exp is None:
        x = _special_tensor("bf16")
    else:
        rng = np.random.default_rng(scale_exp + 700)
        x = f32_to_bf16_bits(np.ldexp(rng.standard_t(4, (24, 96)), scale_exp).astype(np.float32))
    c, s, g, ch, _ = oracle.quantize_nv(x, policy=3)
    xd = to_dev(x)
    r = fq.quantize_nvfp4(xd, policy="four_over_six")
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.choice_bits), ch, "choice bits")
    amax = oracle.tensor_amax(x)
    r = fq.quantize_nvfp4(xd, policy="four_over_six", global_amax=torch.tensor([amax], dtype=torch.float32,
                                                                              device=xd.device))
    assert_same(host(r.codes), c, "codes (caller amax)")
    assert_same(host(r.choice_bits), ch, "choice bits (caller amax)")


def test_nv_exact_ties_and_caller_amax():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    x = np.zeros((2, 64), np.float32)
    x[0, 0] = 2688.0                      # g = 1 exactly
    x[0, 16:32] = [9.0] + [m * 1.5 for m in mids] + [-m * 1.5 for m in mids[:7]]
    x[1] = np.random.default_rng(1).standard_normal(64) * 3
    xd = to_dev(x)
    n = fq.quantize_nvfp4(xd, counters=True)
    c, s, g, _, cnt = oracle.quantize_nv(x)
    assert_same(host(n.codes), c, "codes with exact ties")
    assert_same(host(n.counters).astype(np.uint64), cnt, "counters")
    amax = torch.tensor([1.0], dtype=torch.float32, device=xd.device)   # saturating caller amax
    n = fq.quantize_nvfp4(xd, global_amax=amax, counters=True)
    c, s, g, _, cnt = oracle.quantize_nv(x, global_amax=1.0)
    assert host(n.global_scale)[0] == g
    assert_same(host(n.scales), s, "scales (caller amax)")
    assert_same(host(n.codes), c, "codes (caller amax)")
    assert_same(host(n.counters).astype(np.uint64), cnt, "counters (caller amax)")


@pytest.mark.parametrize("e", [-127, -20, 0, 5, 125, 126, 127])
def test_mx_manual_exponent(e):
    x = make_input(4, 128, "f32", 11)
    for rounding in ("rne", "stochastic"):
        r = fq.quantize_mxfp4(to_dev(x), policy="manual", manual_exponent=e, rounding=rounding, seed=5,
                              counters=True)
        c, s, cnt = oracle.quantize_mx(x, policy=1, manual_exponent=e, rounding=int(rounding != "rne"), seed=5)
        assert_same(host(r.codes), c, "codes")
        assert_same(host(r.scales), s, "scales")
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
        d = fq.dequantize("mxfp4", r.codes, r.scales)
        assert_same(bits(host(d)), bits(oracle.dequantize(oracle.MX, c, s)), "dequant")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequant_all_codes_and_scales(fmt, out_dtype):
    rng = np.random.default_rng(3)
    rows, cols = 16, 512
    block = 32 if fmt == "mxfp4" else 16
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    codes[0, :128] = np.arange(128, dtype=np.uint8) * 2     # every nibble value
    scales = rng.integers(0, 255 if fmt == "mxfp4" else 0x7F, (rows, cols // block), dtype=np.uint8)
    scales[0, :] = np.arange(scales.shape[1]) % (256 if fmt == "mxfp4" else 128)
    scales[1, 0] = 0xFF if fmt == "mxfp4" else 0x7F
    gs = np.float32(0.0123457) if fmt == "nvfp4" else None
    gdev = torch.tensor([gs], dtype=torch.float32, device=gpu()) if gs is not None else None
    d = fq.dequantize(fmt, to_dev(codes), to_dev(scales), gdev, out_dtype=out_dtype)
    od = oracle.F32 if out_dtype == torch.float32 else oracle.BF16
    want = oracle.dequantize(oracle.MX if fmt == "mxfp4" else oracle.NV, codes, scales, gs, out_dtype=od)
    got = host(d)
    if out_dtype == torch.float32:
        got, want = bits(got), bits(want)
    nan_got = np.isnan(bf16_bits_to_f32(got)) if out_dtype == torch.bfloat16 else np.isnan(got.view(np.float32))
    nan_want = np.isnan(bf16_bits_to_f32(want)) if out_dtype == torch.bfloat16 else np.isnan(want.view(np.float32))
    assert_same(nan_got, nan_want, "NaN positions")
    assert_same(np.where(nan_got, 0, got), np.where(nan_want, 0, want), "values")


def test_deterministic_repeat():
    x = to_dev(make_input(64, 512, "bf16", 99))
    a = fq.quantize_nvfp4(x, policy="four_over_six", rounding="stochastic", rotation="rht16", seed=1)
    b = fq.quantize_nvfp4(x, policy="four_over_six", rounding="stochastic", rotation="rht16", seed=1)
    for u, v in zip(a, b):
        if u is not None:
            assert torch.equal(u, v)
    c = fq.quantize_nvfp4(x, policy="four_over_six", rounding="stochastic", rotation="rht16", seed=2)
    assert not torch.equal(a.codes, c.codes)


# ------------------------------------------------------------------ single-read NVFP4 kernel
# Contiguous bf16, max->6, RNE, no rotation, no counters, no caller amax: one
# launch holding the tensor on chip.  Compared with the oracle like every
# other path; the two-pass path is covered by the tests above (counters on).
def _nv_single(x, ws=None):
    xd = to_dev(x)
    r = fq.quantize_nvfp4(xd, workspace=ws)
    c, s, g, _, _ = oracle.quantize_nv(x)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    return r


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 64), (17, 96), (64, 256), (33, 544), (1000, 1024),
                                       (2048, 4096), (4097, 2048), (8192, 8192 - 16)])
def test_nv_single_read_shapes(rows, cols):
    _nv_single(workloads.random_tensor(rows, cols, "bf16", rows + 3 * cols, scale=2.0, dist="t"))


def _nv_caller_amax(x):
    """Contiguous bf16, max->6, RNE, no counters, caller amax: the streaming
    paired encode."""
    xd = to_dev(x)
    amax = oracle.tensor_amax(x)
    amax_dev = torch.tensor([amax], dtype=torch.float32, device=xd.device)
    r = fq.quantize_nvfp4(xd, global_amax=amax_dev)
    c, s, g, _, _ = oracle.quantize_nv(x, global_amax=amax)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales (caller amax)")
    assert_same(host(r.codes), c, "codes (caller amax)")


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 64), (17, 96), (64, 256), (33, 544), (1000, 1024),
                                       (2048, 4096), (4097, 2048)])
def test_nv_caller_amax_shapes(rows, cols):
    _nv_caller_amax(workloads.random_tensor(rows, cols, "bf16", 7 * rows + cols, scale=2.0, dist="t"))


def test_nv_caller_amax_specials_and_tiny():
    _nv_caller_amax(_special_tensor("bf16"))
    rng = np.random.default_rng(31)
    for e in (-133, -101, 100):
        _nv_caller_amax(f32_to_bf16_bits(np.ldexp(rng.standard_t(4, (8, 64)), e).astype(np.float32)))


def test_nv_single_read_full_workgroups():
    """64 Mi elements in a shape other than the headline: every workgroup full."""
    x = workloads.random_tensor(4096, 16384, "bf16", 77, scale=2.0)
    _nv_single(x)


def test_nv_single_read_full_workgroups_nonfinite():
    """Full workgroups with NaN and inf planted in slots held in registers, in
    LDS and re-read from memory, in several workgroups (the block maxima are
    taken on chip; a lane holding a non-finite value takes its finite maximum
    apart).  Slot s of a 256-thread workgroup w with 32 slots per thread is
    flat slot 8192 w + 2048 wave + 64 j + lane (8 elements each)."""
    x = workloads.random_tensor(4096, 16384, "bf16", 78, scale=2.0)
    flat = x.reshape(-1)
    plant = [(5, 2, 3, 7, 0x7FC0), (100, 1, 20, 40, 0x7F80), (700, 3, 29, 63, 0xFF80),
             (1023, 0, 31, 0, 0xFFC1), (400, 0, 16, 1, 0x7F80), (401, 3, 17, 62, 0x7FC0)]
    for wg, wave, j, lane, bits in plant:
        slot = 8192 * wg + 2048 * wave + 64 * j + lane
        flat[slot * 8 + (wg % 8)] = bits
    _nv_single(x)


def test_nv_single_read_specials_and_ties():
    _nv_single(_special_tensor("bf16"))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    x = np.zeros((2, 64), np.float32)
    x[0, 0] = 2688.0                      # g = 1 exactly: exact ties at every decision point
    x[0, 16:32] = [9.0] + [m * 1.5 for m in mids] + [-m * 1.5 for m in mids[:7]]
    x[1] = np.random.default_rng(1).standard_normal(64) * 3
    _nv_single(f32_to_bf16_bits(x))


@pytest.mark.parametrize("scale_exp", [-133, -120, -101, -60, 100, 120])
def test_nv_single_read_tiny_and_huge(scale_exp):
    rng = np.random.default_rng(scale_exp + 900)
    x = np.ldexp(rng.standard_t(4, (8, 64)), scale_exp).astype(np.float32)
    _nv_single(f32_to_bf16_bits(x))


def test_nv_single_read_workspace_reuse_and_fallback():
    """One workspace across calls of different sizes (stale flags must never
    match), then a wait limit of one tick so every workgroup's wait runs out
    and each takes the tensor maximum from its own scan."""
    ws = torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8, device=gpu())
    for shape, seed in (((512, 4096), 1), ((64, 256), 2), ((2048, 8192), 3), ((512, 4096), 4)):
        _nv_single(workloads.random_tensor(shape[0], shape[1], "bf16", seed, scale=2.0), ws)
    ws.view(torch.int64)[2] = 1
    for shape, seed in (((96, 1024), 5), ((1500, 2048), 6)):
        _nv_single(workloads.random_tensor(shape[0], shape[1], "bf16", seed, scale=2.0), ws)
    ws.view(torch.int64)[2] = 0
    _nv_single(workloads.random_tensor(300, 4096, "bf16", 7, scale=2.0), ws)


def test_nv_single_read_graph_replay():
    """The single-read kernel captured in a HIP graph and replayed on new
    data: each replay takes its epoch from the workspace, so flags and result
    words of the previous replay never pass for its own (the tensors differ
    in amax, so a stale tensor scale would show)."""
    dev = gpu()
    rows, cols = 2048, 4096
    xs = [workloads.random_tensor(rows, cols, "bf16", 40 + k, scale=sc, dist="t")
          for k, sc in enumerate((2.0, 50.0, 0.01, 2.0))]
    static_x = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        static_x.copy_(to_dev(xs[0]))
        fq.quantize_nvfp4(static_x)                   # the stream's workspace exists before capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        out = fq.quantize_nvfp4(static_x)
    for k in (1, 2, 0, 3, 1):
        static_x.copy_(to_dev(xs[k]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        c, s, g, _, _ = oracle.quantize_nv(xs[k])
        assert host(out.global_scale)[0] == g, k
        assert_same(host(out.scales), s, "scales (replay of input %d)" % k)
        assert_same(host(out.codes), c, "codes (replay of input %d)" % k)
        with torch.cuda.stream(stream):               # eager work on the same stream and workspace
            e = fq.quantize_nvfp4(static_x)
        stream.synchronize()
        assert_same(host(e.codes), c, "codes (eager call between replays)")


# ------------------------------------------------------------------ exhaustive NVFP4 coverage
def _e4m3_value(c):
    return c * 2.0 ** -9 if c < 8 else (1 + (c & 7) / 8.0) * 2.0 ** ((c >> 3) - 7)


def _exhaustive_nv_tensor(amax_bits):
    """Block 0 holds the tensor max; then, for every E4M3 scale code c, blocks
    whose max makes c the block's scale (near bamax = amax * s_c / 448) and
    whose other 15 elements run through every bf16 magnitude up to that max,
    with alternating signs: every (scale code, bf16 magnitude) pair once."""
    amax = float(bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
    allmag = np.arange(1, 0x7F80, dtype=np.uint16)
    blocks = [np.array([amax_bits] + [0] * 15, np.uint16)]
    for c in range(1, 127):
        b = f32_to_bf16_bits(np.array([amax * _e4m3_value(c) / 448.0], np.float32))[0]
        if b == 0:
            continue
        sel = allmag[allmag <= b]
        sel = np.concatenate([sel, np.zeros((-len(sel)) % 15, np.uint16)]).reshape(-1, 15)
        sel[:, 1::2] |= 0x8000
        blocks.append(np.concatenate([np.full((len(sel), 1), b, np.uint16), sel], axis=1).reshape(-1))
    flat = np.concatenate(blocks)
    cols = 4096
    flat = np.concatenate([flat, np.zeros((-len(flat)) % cols, np.uint16)])
    return flat.reshape(-1, cols)


@pytest.mark.parametrize("amax", [418.0, 168.0, 3.7e-3, 2.0 ** -95, 3.0e38])
def test_nv_exhaustive_scale_codes_and_magnitudes(amax):
    """418: the workload's amax (near-ties from the rounding of g); 168: g
    exact, so exact ties at every decision point; 2^-95: g < 2^-100; 3e38:
    near the top of the range.  Single-read, two-pass and caller-amax paths."""
    a_bits = int(f32_to_bf16_bits(np.array([amax], np.float32))[0])
    x = _exhaustive_nv_tensor(a_bits)
    c, s, g, _, cnt = oracle.quantize_nv(x)
    xd = to_dev(x)
    r = fq.quantize_nvfp4(xd)                                   # single read
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales (single read)")
    assert_same(host(r.codes), c, "codes (single read)")
    r = fq.quantize_nvfp4(xd, counters=True)                    # two passes
    assert_same(host(r.scales), s, "scales (two-pass)")
    assert_same(host(r.codes), c, "codes (two-pass)")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters (two-pass)")
    amax_dev = torch.tensor([float(bf16_bits_to_f32(np.array([a_bits], np.uint16))[0])], dtype=torch.float32,
                            device=xd.device)
    r = fq.quantize_nvfp4(xd, global_amax=amax_dev)             # caller amax, encode pass only
    assert_same(host(r.scales), s, "scales (caller amax)")
    assert_same(host(r.codes), c, "codes (caller amax)")
    c4, s4, g4, ch4, cnt4 = oracle.quantize_nv(x, policy=3)
    for counters in (True, False):      # (without counters: the streaming Four Over Six kernel)
        r = fq.quantize_nvfp4(xd, policy="four_over_six", counters=counters)
        assert host(r.global_scale)[0] == g4
        assert_same(host(r.scales), s4, "scales (four over six, counters %s)" % counters)
        assert_same(host(r.codes), c4, "codes (four over six, counters %s)" % counters)
        assert_same(host(r.choice_bits), ch4, "choice bits (four over six, counters %s)" % counters)
        if counters:
            assert_same(host(r.counters).astype(np.uint64), cnt4, "counters (four over six)")
    seed = 0xC0FFEE
    cs, ss, gs_, _, cnts = oracle.quantize_nv(x, rounding=1, seed=seed)
    r = fq.quantize_nvfp4(xd, rounding="stochastic", seed=seed, counters=True)
    assert host(r.global_scale)[0] == gs_
    assert_same(host(r.scales), ss, "scales (stochastic)")
    assert_same(host(r.codes), cs, "codes (stochastic)")
    assert_same(host(r.counters).astype(np.uint64), cnts, "counters (stochastic)")


_E2M1_LATTICE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("rounding", ["rne", "stochastic"])
@pytest.mark.parametrize("counters", [False, True])
def test_nv_fp32_decision_points(rounding, counters):
    """fp32 elements on, and one ulp either side of, the values where the code
    changes: with round to nearest the midpoints of neighbouring E2M1 values
    (and 6 for the saturation count), with stochastic rounding the thresholds
    lo + u 2^-16 (hi - lo) of each element's own draw u and the lattice points
    themselves, all times the block's s g.  Product-based decisions are within
    rounding error of every one of them and must fall back to exact ones."""
    rng = np.random.default_rng(11)
    rows, cols, seed = 64, 512, 0x5EED
    rmode = 1 if rounding == "stochastic" else 0
    x = np.zeros((rows, cols), np.float32)
    x[:, ::16] = rng.uniform(1.0, 400.0, size=(rows, cols // 16)).astype(np.float32)
    x[0, 0] = 1000.0
    _, s0, g0, _, _ = oracle.quantize_nv(x, rounding=rmode, seed=seed)
    lat = _E2M1_LATTICE
    for r in range(rows):
        for b in range(cols // 16):
            sg = oracle.e4m3_value(int(s0[r, b])) * float(g0)
            for j in range(1, 16):
                col = b * 16 + j
                k = int(rng.integers(0, 6))
                mode = int(rng.integers(0, 3))
                if rmode == 0:
                    t = 6.0 if (k == 5 and mode == 0) else 0.5 * (lat[k] + lat[k + 1])
                elif mode == 0:
                    u = oracle.sr_draw(seed, r * cols + col)
                    t = lat[k] + u * 2.0 ** -16 * (lat[k + 1] - lat[k])
                else:
                    t = lat[k + mode - 1]
                v = np.float32(t * sg)              # t * s * g is exact in fp64
                d = int(rng.integers(-1, 2))
                if d:
                    v = np.nextafter(v, np.float32(np.inf if d > 0 else 0.0))
                if v >= x[r, b * 16]:               # keep the block max (and so s)
                    v = np.float32(0.25 * sg)
                x[r, col] = -v if rng.integers(0, 2) else v
    c, s, g, _, cnt = oracle.quantize_nv(x, rounding=rmode, seed=seed)
    assert g == g0 and (s == s0).all()
    r = fq.quantize_nvfp4(to_dev(x), rounding=rounding, seed=seed, counters=counters)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    if counters:
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


@pytest.mark.parametrize("kind", ["four_over_six", "if4"])
def test_near_tie_sse_choices(kind):
    """Blocks on which the frozen fp32 order of the block SSE and exact
    arithmetic pick different candidates (tests/near_tie.py, fp32 inputs; the
    oracle is pinned to the frozen order on the same blocks): the kernels'
    per-lane half sums must reproduce that order, with counters on and off."""
    import near_tie as N
    x, _ = N.build(kind, 200, seed=7 if kind == N.FOS else 8)
    x = np.ascontiguousarray(np.concatenate([x, np.zeros((x.shape[0], 48), np.float32)], axis=1))  # 4 blocks a row
    policy = 3 if kind == N.FOS else 4
    c, s, g, ch, cnt = oracle.quantize_nv(x, policy=policy)
    xd = to_dev(x)
    for counters in (False, True):
        r = fq.quantize_nvfp4(xd, policy=kind, counters=counters)
        assert host(r.global_scale)[0] == g
        assert_same(host(r.scales), s, "scales")
        assert_same(host(r.codes), c, "codes")
        if ch is not None:
            assert_same(host(r.choice_bits), ch, "choice bits")
        if counters:
            assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


# ------------------------------------------------------------------ IF4
def _if4_check(r, c, s, g, cnt=None):
    assert host(r.global_scale)[0] == g
    assert r.choice_bits is None
    assert_same(host(r.scales), s, "scales (bit 7: INT4)")
    assert_same(host(r.codes), c, "codes")
    if cnt is not None:
        assert_same(host(r.counters).astype(np.uint64), cnt, "counters")


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rotation", [None, "rht16"])
def test_if4_small(rows, cols, dtype, rotation):
    pad = 16 if rows % 2 else 0
    full = make_input(rows, cols, dtype, rows * 11 + cols, pad=pad)
    xd = to_dev(full)[:, :cols]
    for counters in (False, True):
        r = fq.quantize_nvfp4(xd, policy="if4", rotation=rotation, seed=321, counters=counters,
                              return_rotated=rotation is not None)
        if rotation is None:
            c, s, g, _, cnt = oracle.quantize_nv(full, cols=cols, policy=4)
        else:
            rot = host(r.rotated)
            assert rel_l2(rot, oracle.fwht(np.ascontiguousarray(full[:, :cols]), t=16, random_signs=True,
                                           seed=321)) <= RTOL_ROT
            c, s, g, _, cnt = oracle.quantize_nv(rot, policy=4)
        _if4_check(r, c, s, g, cnt if counters else None)


def test_if4_grid_blocks_and_decision_points():
    """g = 7/1024 (tensor amax 18.375) and block maxima 42 S / 1024 give block
    scales S exactly, so the INT4 grid k * 6 S / 1024, its half-integer
    decision points and FP4's grid are exact fp32 numbers.  Blocks mix INT4
    grid points with elements on, and one ulp either side of, the INT4
    decision points (exact ties go to the even integer) and the saturation
    threshold, so that both candidates, the bracket fallbacks and the choice
    are exercised."""
    rng = np.random.default_rng(17)
    S = [0.5, 1.0, 1.25, 2.0, 3.5, 10.0, 104.0, 448.0]
    rows, nb = 64, 32
    x = np.zeros((rows, nb * 16), np.float32)
    for r in range(rows):
        for b in range(nb):
            sv = S[(r + b) % len(S)]
            step = 6.0 * sv / 1024.0
            blk = np.zeros(16)
            blk[0] = 7 * step                           # block max: s = S exactly
            n_grid = int(rng.integers(6, 15))
            for j in range(1, 16):
                if j <= n_grid:
                    t = float(rng.integers(0, 8))
                else:
                    t = float(rng.integers(0, 7)) + 0.5 if rng.integers(0, 4) else 7.0
                v = np.float32(t * step)
                d = int(rng.integers(-1, 2))
                if d:
                    v = np.nextafter(v, np.float32(np.inf if d > 0 else 0.0))
                blk[j] = min(float(v), 7 * step)
            blk *= np.where(rng.integers(0, 2, 16) == 1, -1.0, 1.0)
            blk[0] = 7 * step
            x[r, b * 16:(b + 1) * 16] = blk
    x[0, 0] = 18.375
    c, s, g, _, cnt = oracle.quantize_nv(x, policy=4)
    assert g == np.float32(7 / 1024)
    n_int4 = int(np.count_nonzero(s & 0x80))
    assert n_int4 > rows * nb // 4 and n_int4 < rows * nb    # both candidates are kept somewhere
    xd = to_dev(x)
    for counters in (False, True):
        r = fq.quantize_nvfp4(xd, policy="if4", counters=counters)
        _if4_check(r, c, s, g, cnt if counters else None)
    amax = torch.tensor([18.375], dtype=torch.float32, device=xd.device)
    _if4_check(fq.quantize_nvfp4(xd, policy="if4", global_amax=amax), c, s, g)


@pytest.mark.parametrize("amax", [418.0, 168.0, 2.0 ** -95])
def test_if4_exhaustive_scale_codes_and_magnitudes(amax):
    a_bits = int(f32_to_bf16_bits(np.array([amax], np.float32))[0])
    x = _exhaustive_nv_tensor(a_bits)
    c, s, g, _, cnt = oracle.quantize_nv(x, policy=4)
    if amax > 1.0:   # (at 2^-95 every squared error underflows in fp32: the SSEs tie and FP4 is kept)
        assert np.count_nonzero(s & 0x80) > 0
    xd = to_dev(x)
    _if4_check(fq.quantize_nvfp4(xd, policy="if4", counters=True), c, s, g, cnt)
    _if4_check(fq.quantize_nvfp4(xd, policy="if4"), c, s, g)          # the streaming IF4 kernel


def test_if4_specials_and_empty():
    for dtype in ("f32", "bf16"):
        x = _special_tensor(dtype)
        c, s, g, _, cnt = oracle.quantize_nv(x, policy=4)
        _if4_check(fq.quantize_nvfp4(to_dev(x), policy="if4", counters=True), c, s, g, cnt)
        _if4_check(fq.quantize_nvfp4(to_dev(x), policy="if4"), c, s, g)
    rng = np.random.default_rng(77)
    for e in (-140, -101, 100):           # g below 2^-100 (every block exact) and near the top
        x = f32_to_bf16_bits(np.ldexp(rng.standard_t(4, (24, 96)), e).astype(np.float32))
        c, s, g, _, _ = oracle.quantize_nv(x, policy=4)
        _if4_check(fq.quantize_nvfp4(to_dev(x), policy="if4"), c, s, g)
    e = fq.quantize_nvfp4(torch.empty((0, 64), dtype=torch.bfloat16, device=gpu()), policy="if4")
    assert host(e.global_scale)[0] == 1.0
    with pytest.raises(fq.Fp4qError):
        fq.quantize_nvfp4(to_dev(np.zeros((2, 32), np.float32)), policy="if4", rounding="stochastic")


def test_if4_rht_grad_8192():
    """IF4 on the Hadamard-rotated gradient workload, where INT4 is expected to win often."""
    x = workload("grad_bf16_8192")
    r = fq.quantize_nvfp4(to_dev(x), policy="if4", rotation="rht16", seed=workloads.SR_SEED, return_rotated=True,
                          counters=True)
    rot = host(r.rotated)
    c, s, g, _, cnt = oracle.quantize_nv(rot, policy=4)
    _if4_check(r, c, s, g, cnt)
    assert np.count_nonzero(s & 0x80) > s.size // 4


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequant_if4_all_codes_and_scales(out_dtype):
    rng = np.random.default_rng(5)
    rows, cols = 16, 512
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    codes[0, :128] = np.arange(128, dtype=np.uint8) * 2
    scales = rng.integers(0, 256, (rows, cols // 16), dtype=np.uint8)
    scales[0, :] = np.arange(32) * 8 + 1                     # both flag values over the code range
    scales[1, 0], scales[1, 1] = 0x7F, 0xFF
    od = oracle.F32 if out_dtype == torch.float32 else oracle.BF16
    for gs in (np.float32(0.0123457), np.float32(7 / 1024), np.float32(2.0 ** -149), np.float32(1e30)):
        gdev = torch.tensor([gs], dtype=torch.float32, device=gpu())
        got = host(fq.dequantize("if4", to_dev(codes), to_dev(scales), gdev, out_dtype=out_dtype))
        want = oracle.dequantize(oracle.IF4, codes, scales, gs, out_dtype=od)
        if out_dtype == torch.float32:
            got, want = bits(got), bits(want)
            isnan = lambda a: np.isnan(a.view(np.float32))
        else:
            isnan = lambda a: np.isnan(bf16_bits_to_f32(a))
        assert_same(isnan(got), isnan(want), "NaN positions")
        assert_same(np.where(isnan(got), 0, got), np.where(isnan(want), 0, want), "values g=%r" % gs)


def test_if4_round_trip_8192():
    x = workload("act_bf16_8192")
    xd = to_dev(x)
    r = fq.quantize_nvfp4(xd, policy="if4")
    codes, scales, g = host(r.codes), host(r.scales), host(r.global_scale)[0]
    rows = slice(0, 256)
    c, s, g_ref, _, _ = oracle.quantize_nv(x[rows], policy=4, global_amax=oracle.tensor_amax(x))
    assert g == g_ref
    assert_same(codes[rows], c, "codes")
    assert_same(scales[rows], s, "scales")
    d = host(fq.dequantize("if4", r.codes, r.scales, r.global_scale, out_dtype=torch.bfloat16))
    want = oracle.dequantize(oracle.IF4, codes[rows], scales[rows], g, out_dtype=oracle.BF16)
    assert_same(d[rows], want, "bf16 reconstruction")


# ------------------------------------------------------------------ fused SwiGLU epilogue
@pytest.mark.parametrize("rows,d", [(3, 32), (5, 64), (17, 512), (4, 4096), (6, 8192), (2, 16384)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rounding", ["rne", "stochastic"])
def test_silu_mul_fwht_small(rows, d, dtype, rounding):
    x = make_input(rows, 2 * d, dtype, rows * 13 + d)            # [gate | up] per row
    xd = to_dev(x)
    r = fq.silu_mul_fwht_mxfp4(xd[:, :d], xd[:, d:], rounding=rounding, seed=55, return_rotated=True,
                               counters=True)
    rot = host(r.rotated)
    ref = oracle.fwht(oracle.silu_mul(np.ascontiguousarray(x[:, :d]), np.ascontiguousarray(x[:, d:])))
    assert rel_l2(rot, ref) <= RTOL_ROT
    c, s, cnt = oracle.quantize_mx(rot, rounding=int(rounding != "rne"), seed=55)
    assert_same(host(r.codes), c, "codes of the rotated activation")
    assert_same(host(r.scales), s, "scales of the rotated activation")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    r2 = fq.silu_mul_fwht_mxfp4(xd[:, :d], xd[:, d:], rounding=rounding, seed=55)
    assert_same(host(r2.codes), c, "codes without the rotated hook")


def test_silu_mul_fwht_16384x8192():
    x = workload("gate_up_bf16_16384x8192")
    d = x.shape[1] // 2
    xd = to_dev(x)
    r = fq.silu_mul_fwht_mxfp4(xd[:, :d], xd[:, d:], return_rotated=True, counters=True)
    rot = host(r.rotated)
    c, s, cnt = oracle.quantize_mx(rot)
    assert_same(host(r.codes), c, "codes of the rotated activation")
    assert_same(host(r.scales), s, "scales of the rotated activation")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    rows = np.random.default_rng(1).choice(x.shape[0], 32, replace=False)
    ref = oracle.fwht(oracle.silu_mul(np.ascontiguousarray(x[rows, :d]), np.ascontiguousarray(x[rows, d:])))
    assert rel_l2(rot[rows], ref) <= RTOL_ROT
    r2 = fq.silu_mul_fwht_mxfp4(xd[:, :d], xd[:, d:])
    assert_same(host(r2.codes), c, "codes without the rotated hook")


# ------------------------------------------------------------------ per-head FWHT-128 + NVFP4
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 256), (17, 384), (64, 1024), (5, 4096)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("policy", ["max6", "if4"])
def test_fwht128_nv_small(rows, cols, dtype, policy):
    pad = 16 if rows % 2 else 0
    full = make_input(rows, cols, dtype, rows * 17 + cols, pad=pad)
    xd = to_dev(full)[:, :cols]
    ref = oracle.fwht(np.ascontiguousarray(full[:, :cols]), t=128)
    for counters in (False, True):
        r = fq.quantize_nvfp4(xd, policy=policy, rotation="fwht128", counters=counters, return_rotated=True)
        rot = host(r.rotated)
        assert rel_l2(rot, ref) <= RTOL_ROT
        c, s, g, _, cnt = oracle.quantize_nv(rot, policy=2 if policy == "max6" else 4)
        assert host(r.global_scale)[0] == g
        assert_same(host(r.scales), s, "scales")
        assert_same(host(r.codes), c, "codes")
        if counters:
            assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    r2 = fq.quantize_nvfp4(xd, policy=policy, rotation="fwht128")
    assert_same(host(r2.codes), c, "codes without the rotated hook")


def test_fwht128_nv_act_8192_heads():
    """The 8192x8192 activation read as 8192 tokens x 64 heads of 128."""
    x = workload("act_bf16_8192")
    r = fq.quantize_nvfp4(to_dev(x), rotation="fwht128", return_rotated=True, counters=True)
    rot = host(r.rotated)
    c, s, g, _, cnt = oracle.quantize_nv(rot)
    assert host(r.global_scale)[0] == g
    assert_same(host(r.scales), s, "scales")
    assert_same(host(r.codes), c, "codes")
    assert_same(host(r.counters).astype(np.uint64), cnt, "counters")
    rows = np.random.default_rng(2).choice(x.shape[0], 64, replace=False)
    assert rel_l2(rot[rows], oracle.fwht(x[rows], t=128)) <= RTOL_ROT


# ------------------------------------------------------------------ MXFP4 GEMM
def _gemm_check(c_gpu, c_ref, absc, K, extra_rel=0.0):
    """fp32 accumulation of exact products in any order is within K 2^-24 sum|a b|
    of the exact sum (bf16 output adds half an ulp of the result)."""
    c_gpu = c_gpu.astype(np.float64)
    tol = K * 2.0 ** -24 * absc + extra_rel * np.abs(c_ref)
    bad = np.abs(c_gpu - c_ref) > tol
    assert not bad.any(), "%d of %d outside the bound; worst at %s" % (
        bad.sum(), bad.size, np.unravel_index(np.argmax(np.abs(c_gpu - c_ref) - tol), bad.shape))
    rel = np.abs(c_gpu - c_ref) / np.maximum(absc, 1e-300)
    return float(rel.max())


# K covers 1 to 9 pipeline stages of 128 (the load ring runs three stages ahead);
# 256x256 tiles wholly inside C (N a multiple of 8) take the staged epilogue
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (33, 17, 128), (130, 257, 256), (300, 520, 384), (64, 64, 512),
                                   (257, 129, 640), (256, 128, 1024), (40, 300, 1152), (97, 300, 4096), (5, 7, 0),
                                   (512, 264, 256), (256, 256, 384), (256, 260, 128)])
def test_mxfp4_gemm_small(M, N, K):
    a = make_input(M, K, "bf16", M * 7 + K) if K else np.zeros((M, 0), np.uint16)
    b = make_input(N, K, "f32", N * 11 + K) if K else np.zeros((N, 0), np.float32)
    if K == 0:
        qa = (torch.zeros((M, 0), dtype=torch.uint8, device=gpu()), torch.zeros((M, 0), dtype=torch.uint8, device=gpu()))
        qb = (torch.zeros((N, 0), dtype=torch.uint8, device=gpu()), torch.zeros((N, 0), dtype=torch.uint8, device=gpu()))
        assert not host(fq.mxfp4_gemm(qa, qb)).any()
        return
    qa = fq.quantize_mxfp4(to_dev(a))
    qb = fq.quantize_mxfp4(to_dev(b))
    ref, absc = oracle.mx_gemm(host(qa.codes), host(qa.scales), host(qb.codes), host(qb.scales))
    _gemm_check(host(fq.mxfp4_gemm(qa, qb)), ref, absc, K)
    c16 = bf16_bits_to_f32(host(fq.mxfp4_gemm(qa, qb, out_dtype=torch.bfloat16)))
    _gemm_check(c16, ref, absc, K, extra_rel=2.0 ** -8)


def test_mxfp4_gemm_unaligned_out():
    """C at a 4-byte but not 16-byte aligned address: whole tiles take the
    element-wise epilogue, with the same bits as an aligned C."""
    M, N, K = 512, 264, 256
    qa = fq.quantize_mxfp4(to_dev(make_input(M, K, "bf16", 5)))
    qb = fq.quantize_mxfp4(to_dev(make_input(N, K, "bf16", 6)))
    for dt, off in ((torch.float32, 1), (torch.bfloat16, 2)):
        want = host(fq.mxfp4_gemm(qa, qb, out_dtype=dt).view(torch.int32 if dt == torch.float32 else torch.int16))
        buf = torch.zeros(M * N + 8, dtype=dt, device=gpu())
        c = buf[off:off + M * N].view(M, N)
        assert c.data_ptr() % 16 != 0 and c.data_ptr() % 4 == 0
        fq.mxfp4_gemm(qa, qb, out_dtype=dt, out=c)
        got = host(c.view(torch.int32 if dt == torch.float32 else torch.int16))
        assert np.array_equal(got, want), dt
        assert not host(buf[:off]).any() and not host(buf[off + M * N:]).any()   # nothing outside C


def test_binding_rejects_bad_buffers():
    """Buffers the kernels would write or read densely are checked in the
    binding: wrong shape, dtype, device or layout raises before any launch."""
    dev = gpu()
    x = to_dev(make_input(4, 64, "bf16", 9))
    q = fq.quantize_mxfp4(x)
    with pytest.raises(ValueError):
        fq.mxfp4_gemm(q, q, out=torch.empty((4, 5), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        fq.mxfp4_gemm(q, q, out=torch.empty((4, 4), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        fq.mxfp4_gemm(q, q, out=torch.empty((4, 8), dtype=torch.float32, device=dev)[:, ::2])
    with pytest.raises(ValueError):
        fq.quantize_mxfp4(x, out=fq.MxResult(q.codes[:2], q.scales, None, None))
    with pytest.raises(ValueError):
        fq.dequantize("mxfp4", q.codes.cpu(), q.scales)
    with pytest.raises(ValueError):
        fq.dequantize("mxfp4", q.codes, q.scales, out=torch.empty((4, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        fq.fwht(x, out=torch.empty((4, 64), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        fq.quantize_nvfp4(x, workspace=torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8))


def test_mxfp4_gemm_nan_scale_and_exact_case():
    M, N, K = 64, 64, 256
    ac = np.full((M, K // 2), 0x22, np.uint8)                   # all 1.0
    asc = np.full((M, K // 32), 127, np.uint8)
    rng = np.random.default_rng(61)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bsc = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    asc[3, 5] = 255                                             # NaN scale: row 3 is NaN
    ref, _ = oracle.mx_gemm(ac, asc, bc, bsc)
    c = host(fq.mxfp4_gemm((to_dev(ac), to_dev(asc)), (to_dev(bc), to_dev(bsc))))
    assert np.isnan(c[3]).all() and not np.isnan(np.delete(c, 3, axis=0)).any()
    # row sums of B: every partial sum is a short dyadic number, exact in fp32
    ok = np.delete(np.arange(M), 3)
    assert np.array_equal(c[ok].astype(np.float64), ref[ok])


@pytest.mark.parametrize("M,N", [(256, 256), (300, 520)])
def test_mxfp4_gemm_exact_k8192(M, N):
    """K = 8192 with every A and B scale byte 126 or 127 (exponents -1 and
    0, varying per block): each product is a multiple of 2^-4 of magnitude at
    most 36, so every partial sum is a multiple of 2^-4 below 36 * 8192 < 2^19,
    i.e. fewer than 2^23 units: every summation order is exact in fp32.  The fp32 result equals the exact sum
    and the bf16 result is its round-to-nearest-even."""
    K = 8192
    rng = np.random.default_rng(M + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = rng.integers(126, 128, (M, K // 32), dtype=np.uint8)
    bsc = rng.integers(126, 128, (N, K // 32), dtype=np.uint8)
    ref, absc = oracle.mx_gemm(ac, asc, bc, bsc)
    assert np.abs(ref).max() < 2.0 ** 19                       # (2^23 units of 2^-4)
    qa, qb = (to_dev(ac), to_dev(asc)), (to_dev(bc), to_dev(bsc))
    c32 = host(fq.mxfp4_gemm(qa, qb)).astype(np.float64)
    assert np.array_equal(c32, ref)
    c16 = host(fq.mxfp4_gemm(qa, qb, out_dtype=torch.bfloat16))
    assert_same(c16, f32_to_bf16_bits(ref.astype(np.float32)), "bf16 output")


def test_mxfp4_gemm_8192_sampled_rows():
    a = workload("act_bf16_8192")
    w = np.ascontiguousarray(workloads.make("weight_bf16_8192x28672", rows=8192, cols=8192))
    qa = fq.quantize_mxfp4(to_dev(a))
    qb = fq.quantize_mxfp4(to_dev(w))
    c = host(fq.mxfp4_gemm(qa, qb))
    ac, asc, bc, bsc = host(qa.codes), host(qa.scales), host(qb.codes), host(qb.scales)
    for r0 in (0, 4093, 8192 - 3):
        ref, absc = oracle.mx_gemm(ac, asc, bc, bsc, rows=(r0, 3))
        _gemm_check(c[r0:r0 + 3], ref, absc, 8192)


def test_mx_counters_without_workspace_through_the_abi():
    """A counting MXFP4 call with no workspace adds each workgroup's counts
    straight into the counters (the binding always passes its workspace, so
    this path is driven through the C ABI)."""
    from fp4_block_scaled_row_amd import _lib
    lib = _lib.load()
    x = workload("mx_f32_1024")
    xd = to_dev(x)
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=xd.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=xd.device)
    cnt = torch.full((3,), 12345, dtype=torch.int64, device=xd.device)
    a = _lib.QuantArgs()
    a.rows, a.cols, a.in_row_stride = rows, cols, cols
    a.in_dtype, a.block_size, a.scale_policy = _lib.FP4Q_F32, 32, _lib.FP4Q_SCALE_OCP_MAX
    o = _lib.Outputs(codes.data_ptr(), scales.data_ptr(), None, None, None, cnt.data_ptr())
    for _ in range(2):                       # counters start from zero on every call
        st = lib.fp4q_quantize_mxfp4(a, xd.data_ptr(), o, None, 0, torch.cuda.current_stream().cuda_stream)
        assert st == _lib.FP4Q_OK
        c, s, ref = oracle.quantize_mx(x)
        assert_same(host(codes), c, "codes")
        assert_same(host(cnt).astype(np.uint64), ref, "counters")
