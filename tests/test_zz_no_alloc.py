"""fp4q_quantize_nvfp4_noalloc (the NVFP4 entry point that allocates nothing,
its workspace a scratch array the library holds on the device) against
fp4q_quantize_nvfp4 with a caller workspace, through the C ABI: bit-identical
codes, scales, tensor scale, choice bits and counters on two calls in a row,
the second with a smaller input, on the single-read path and on the two-pass
path (whose per-workgroup partials live in the scratch)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp4_block_scaled_row_amd import _lib

pytestmark = pytest.mark.gpu


def _quantize(entry, x, policy, counters, ws=None):
    lib = _lib.load()
    rows, cols = x.shape
    dev = x.device
    a = _lib.QuantArgs()
    a.rows, a.cols, a.in_row_stride = rows, cols, cols
    a.in_dtype, a.block_size, a.scale_policy = _lib.FP4Q_BF16, 16, policy
    a.rounding, a.rotation, a.manual_exponent, a.seed = _lib.FP4Q_ROUND_RNE, _lib.FP4Q_ROT_NONE, 0, 0
    codes = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device=dev)
    scales = torch.full((rows, cols // 16), 0xCD, dtype=torch.uint8, device=dev)
    gs = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    nb = rows * (cols // 16)
    choice = torch.zeros(((nb + 7) // 8,), dtype=torch.uint8, device=dev) \
        if policy == _lib.FP4Q_SCALE_FOUR_OVER_SIX else None
    cnt = torch.full((3,), 7, dtype=torch.int64, device=dev) if counters else None
    p = lambda t: None if t is None else t.data_ptr()
    o = _lib.Outputs(p(codes), p(scales), p(gs), p(choice), None, p(cnt))
    stream = torch.cuda.current_stream().cuda_stream
    if entry == "noalloc":
        st = lib.fp4q_quantize_nvfp4_noalloc(a, x.data_ptr(), None, o, stream)
    else:
        st = lib.fp4q_quantize_nvfp4(a, x.data_ptr(), None, o, ws.data_ptr(), ws.numel(), stream)
    assert st == _lib.FP4Q_OK, _lib.status_string(st)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy() for t in (codes, scales, gs, choice, cnt)]


@pytest.mark.parametrize("policy,counters", [(_lib.FP4Q_SCALE_NV_MAX6, False),          # single read
                                             (_lib.FP4Q_SCALE_FOUR_OVER_SIX, True)])    # two passes
def test_noalloc_matches_workspace_entry_point(policy, counters):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    ws = torch.zeros(80 * 1024, dtype=torch.uint8, device=dev)
    for k, (rows, cols) in enumerate(((2048, 4096), (300, 1024))):   # the second call smaller
        xb = workloads.random_tensor(rows, cols, "bf16", 900 + k, scale=2.0 if k == 0 else 40.0, dist="t")
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        want = _quantize("ws", x, policy, counters, ws)
        got = _quantize("noalloc", x, policy, counters)
        for name, g, w in zip(("codes", "scales", "global scale", "choice bits", "counters"), got, want):
            if w is None:
                assert g is None
            else:
                assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), (name, rows, cols)
        c, s, gsc, ch, cnt = oracle.quantize_nv(xb, policy=policy)
        assert np.array_equal(got[0], c) and np.array_equal(got[1], s) and got[2][0] == gsc
        if ch is not None:
            assert np.array_equal(got[3], ch)
        if counters:
            assert np.array_equal(got[4].astype(np.uint64), cnt)
