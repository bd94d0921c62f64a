"""Benchmark: quantize GB/s and fraction of HBM peak, 8192x8192 bf16 -> NVFP4
(headline) and MXFP4, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]

    python bench.py --profile-kernels   # a few launches of each kernel, for rocprofv3

A step is one NVFP4 quantization of the 8192x8192 bf16 activation tensor
(2 * Student-t(4), seed 102): tensor amax computed in the call, E2M1 codes,
E4M3 block scales and the fp32 tensor scale (one launch of the single-read
kernel).  Inputs are resident in HBM before timing; the step cycles over 4
replicas of the input (4 x 128 MiB) so every step reads an input the Infinity
Cache no longer holds.  value = algorithmic bytes (read the input once, write
every output once) x K / wall time of the K steps.  Before the W warmup steps
the headline step runs back to back, untimed, for MS milliseconds (default
50): the GPU clock idles low and needs ~30 ms of load to reach its sustained
level, which a few warmup steps do not give.

The same line carries the MXFP4 quantization of the same tensor and the
NVFP4 dequantization back to bf16 as sub-objects, the roofline of the
dominant kernel (HIP events on the launch stream), and the CPU oracle timed on
a bounded sample of the workload.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
ROWS, COLS = 8192, 8192
N = ROWS * COLS
BYTES_IN = N * 2
NV_BYTES = BYTES_IN + N // 2 + N // 16 + 4          # 171,966,468
MX_BYTES = BYTES_IN + N // 2 + N // 32              # 169,869,312
DQ_BYTES = N // 2 + N // 16 + 4 + BYTES_IN          # dequant NVFP4 -> bf16
REPLICAS = 4
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_sha():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp4_block_scaled_row_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, launch_units=1):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None when
    the kernels changed since the counters were taken."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or t.get("source_sha") != kernel_source_sha():
        return None
    return int(k["hbm_bytes_per_launch"]) * launch_units


def cpu_baseline(x_np, rows=4096, min_seconds=10.0, max_reps=4):
    """The oracle, untuned and single-threaded, on the first `rows` rows of the
    workload, repeated until about `min_seconds` of CPU work."""
    import oracle
    sample = x_np[:rows]
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t = time.perf_counter()
        oracle.quantize_nv(sample)
        dt += time.perf_counter() - t
        reps += 1
    elems = rows * COLS * reps
    gbps = elems * (NV_BYTES / N) / dt / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "NVFP4 quantize (tensor amax, scales, codes) of rows 0..%d (%d elements) of the 8192x8192 "
                      "workload, %d pass(es), single-threaded C oracle, %.1f s" % (rows - 1, rows * COLS, reps, dt),
            "elements_per_s": round(elems / dt, 1)}


def profile_kernels(dev, reps=5):
    """A few launches of every kernel on the five workloads' full sizes, plus a
    plain 128 MiB device copy (the reference for HBM byte counters).  Prints
    one text line per kernel with its average event time."""
    import numpy as np
    import torch

    import fp4_block_scaled_row_amd as fq
    import workloads

    def dev_tensor(name):
        x = workloads.make(name)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    def settle(fn, seconds=0.04):
        # back-to-back launches until the GPU clock is at its sustained level
        # (it drops while the host prepares the next workload)
        t = time.perf_counter()
        while time.perf_counter() - t < seconds:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()

    def run(label, fn, nbytes):
        settle(fn)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print("%-58s %9.2f us  %8.1f GB/s" % (label, us, nbytes / us / 1e3), flush=True)

    src = torch.empty(BYTES_IN, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    run("copy 128 MiB (reference for byte counters)", lambda: dst.copy_(src), 2 * BYTES_IN)
    del src, dst

    x = dev_tensor("act_bf16_8192")
    ws = torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8, device=dev)
    o = fq.quantize_nvfp4(x, workspace=ws)
    run("C2 NVFP4 bf16 8192x8192, amax in call", lambda: fq.quantize_nvfp4(x, out=o, workspace=ws), NV_BYTES)
    amax = torch.max(torch.abs(x.float())).reshape(1)
    run("C2 NVFP4 bf16 8192x8192, amax given (encode pass)",
        lambda: fq.quantize_nvfp4(x, out=o, global_amax=amax), NV_BYTES)
    ox = fq.quantize_mxfp4(x)
    run("H2 MXFP4 bf16 8192x8192", lambda: fq.quantize_mxfp4(x, out=ox), MX_BYTES)
    y = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev)
    run("C2 dequantize NVFP4 -> bf16 8192x8192",
        lambda: fq.dequantize("nvfp4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=y), DQ_BYTES)
    o6 = fq.quantize_nvfp4(x, rotation="fwht128", workspace=ws)
    run("FWHT-128 per head + NVFP4 bf16 8192x8192 (64 heads of 128)",
        lambda: fq.quantize_nvfp4(x, rotation="fwht128", out=o6, workspace=ws), NV_BYTES)
    del o6
    o5 = fq.quantize_nvfp4(x, rotation="rht16", rounding="stochastic", seed=workloads.SR_SEED, workspace=ws)
    run("C5 RHT16 + stochastic NVFP4 bf16 8192x8192",
        lambda: fq.quantize_nvfp4(x, rotation="rht16", rounding="stochastic", seed=workloads.SR_SEED, out=o5,
                                  workspace=ws), NV_BYTES)
    del x, o, ox, y, o5

    x3 = dev_tensor("swiglu_bf16_16384x8192")
    o3 = fq.quantize_mxfp4(x3, rotation="fwht_row")
    n3 = x3.numel()
    run("C3 FWHT-8192 + MXFP4 bf16 16384x8192",
        lambda: fq.quantize_mxfp4(x3, rotation="fwht_row", out=o3), n3 * 2 + n3 // 2 + n3 // 32)
    del x3, o3

    x4 = dev_tensor("weight_bf16_8192x28672")
    o4 = fq.quantize_nvfp4(x4, policy="four_over_six", workspace=ws)
    n4 = x4.numel()
    run("C4 Four-Over-Six NVFP4 bf16 8192x28672",
        lambda: fq.quantize_nvfp4(x4, policy="four_over_six", out=o4, workspace=ws),
        n4 * 2 + n4 // 2 + n4 // 16 + 4 + n4 // 128)
    del o4
    oi = fq.quantize_nvfp4(x4, policy="if4", workspace=ws)
    run("IF4 bf16 8192x28672 (weights of C4)",
        lambda: fq.quantize_nvfp4(x4, policy="if4", out=oi, workspace=ws), n4 * 2 + n4 // 2 + n4 // 16 + 4)
    del x4
    yi = torch.empty((oi.codes.shape[0], oi.codes.shape[1] * 2), dtype=torch.bfloat16, device=dev)
    run("IF4 dequantize -> bf16 8192x28672",
        lambda: fq.dequantize("if4", oi.codes, oi.scales, oi.global_scale, out_dtype=torch.bfloat16, out=yi),
        n4 * 2 + n4 // 2 + n4 // 16 + 4)
    del oi, yi

    xg = dev_tensor("gate_up_bf16_16384x8192")
    d = xg.shape[1] // 2
    gate, up = xg[:, :d], xg[:, d:]
    og = fq.silu_mul_fwht_mxfp4(gate, up)
    ng = gate.numel()
    run("SiLU_and_Mul + FWHT-8192 + MXFP4 bf16 16384x(2x8192), fused",
        lambda: fq.silu_mul_fwht_mxfp4(gate, up, out=og), 2 * ng * 2 + ng // 2 + ng // 32)
    hb = torch.empty_like(gate)

    def unfused():
        torch.mul(torch.nn.functional.silu(gate), up, out=hb)
        fq.quantize_mxfp4(hb, rotation="fwht_row", out=og)
    run("  unfused reference: torch SiLU*up to bf16, then FWHT-8192 + MXFP4", unfused,
        2 * ng * 2 + ng // 2 + ng // 32)
    del xg, gate, up, og, hb

    # MXFP4 GEMM: C = A W^T, A the 8192x8192 activation, W 8192x8192 of the weight recipe
    xa = dev_tensor("act_bf16_8192")
    wn = workloads.make("weight_bf16_8192x28672", rows=8192, cols=8192)
    xw = torch.from_numpy(wn.view(np.int16)).to(dev).view(torch.bfloat16)
    qa, qw = fq.quantize_mxfp4(xa), fq.quantize_mxfp4(xw)
    cg = torch.empty((8192, 8192), dtype=torch.float32, device=dev)
    flops = 2.0 * 8192 ** 3

    def run_flops(label, fn):
        settle(fn)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print("%-58s %9.2f us  %8.1f TFLOP/s" % (label, us, flops / us / 1e6), flush=True)

    run_flops("MXFP4 GEMM 8192x8192x8192 -> fp32", lambda: fq.mxfp4_gemm(qa, qw, out=cg))
    cb = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    run_flops("MXFP4 GEMM 8192x8192x8192 -> bf16", lambda: fq.mxfp4_gemm(qa, qw, out_dtype=torch.bfloat16, out=cb))
    wt = xw.t().contiguous()
    run_flops("  reference: torch bf16 matmul 8192x8192x8192", lambda: torch.matmul(xa, wt, out=cb))
    del xa, xw, qa, qw, cg, cb, wt

    x1 = dev_tensor("mx_f32_1024")
    o1 = fq.quantize_mxfp4(x1, counters=True)
    y1 = torch.empty_like(x1)
    n1 = x1.numel()
    run("C1 MXFP4 fp32 1024x1024 (with counters)", lambda: fq.quantize_mxfp4(x1, counters=True, out=o1),
        n1 * 4 + n1 // 2 + n1 // 32)
    run("C1 dequantize MXFP4 -> fp32 1024x1024",
        lambda: fq.dequantize("mxfp4", o1.codes, o1.scales, out_dtype=torch.float32, out=y1), n1 // 2 + n1 // 32 + n1 * 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed back-to-back headline steps before the warmup steps, so that the GPU clock "
                         "reaches its sustained level (it idles low and ramps within ~30 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="launch each kernel of the five workloads and of IF4 a few times (for rocprofv3) and print "
                         "event timings as text; no JSON line")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding); "
              "--gpus %d is not supported" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_block_scaled_row_amd as fq
    import workloads

    dev = torch.device("cuda:0")
    if a.profile_kernels:
        profile_kernels(dev)
        return
    x_np = workloads.make("act_bf16_8192")
    x0 = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(REPLICAS - 1)]
    nv_out = [fq.quantize_nvfp4(x) for x in xs]          # allocates outputs once per replica
    ws = torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8, device=dev)
    mx_out = [fq.quantize_mxfp4(x) for x in xs]
    dq_out = [torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev) for _ in range(REPLICAS)]
    amax_dev = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(REPLICAS)]
    torch.cuda.synchronize()

    def nv_step(i):
        k = i % REPLICAS
        fq.quantize_nvfp4(xs[k], out=nv_out[k], workspace=ws)

    def timed(fn, steps, warmup):
        """(wall seconds per step, HIP-event seconds per step) of `steps` steps
        after `warmup` untimed ones; the events bracket the timed steps on the
        launch stream (torch's current stream, which the library launches on)."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record(st)
        for i in range(steps):
            fn(i)
        e1.record(st)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps, e0.elapsed_time(e1) / 1e3 / steps

    def event_avg(fn, steps, pre=None):
        """Average per-call GPU duration from HIP events on the launch stream
        (torch's current stream, which is the stream the library launches on);
        `pre` runs untimed before each timed call."""
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            if pre is not None:
                pre(i)
            ev[i][0].record(st)
            fn(i)
            ev[i][1].record(st)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps / 1e3

    def settle(fn, ms):
        n, t = 0, time.perf_counter()
        while (time.perf_counter() - t) * 1e3 < ms:
            for _ in range(50):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return n

    # ---- headline: NVFP4 quantize, K steps (one launch of nv_resident_kernel each)
    settle_steps = settle(nv_step, a.settle_ms)
    # roofline of the dominant kernel: the single-read NVFP4 kernel, the only
    # launch of a step, so the events over the timed steps give its average
    # launch duration (back-to-back launches: the gaps between them included)
    sec, call_sec = timed(nv_step, a.steps, a.warmup)
    value = NV_BYTES / sec / 1e9
    call_gbps = NV_BYTES / call_sec / 1e9

    # ---- the two-pass NVFP4 encode (used when the caller hands in the
    # tensor amax, and for shapes the single-read kernel does not take)
    for k in range(REPLICAS):
        amax_dev[k].copy_(torch.max(torch.abs(xs[k].float())).reshape(1))
    torch.cuda.synchronize()

    def encode_only(i):
        k = i % REPLICAS
        fq.quantize_nvfp4(xs[k], out=nv_out[k], global_amax=amax_dev[k])

    for i in range(a.warmup):
        encode_only(i)
    enc_sec = event_avg(encode_only, a.steps, pre=nv_step)

    # ---- MXFP4 of the same tensor
    def mx_step(i):
        k = i % REPLICAS
        fq.quantize_mxfp4(xs[k], out=mx_out[k])
    mx_sec, mx_ev = timed(mx_step, a.steps, a.warmup)

    # ---- NVFP4 dequantize back to bf16
    def dq_step(i):
        k = i % REPLICAS
        o = nv_out[k]
        fq.dequantize("nvfp4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=dq_out[k])
    dq_sec = timed(dq_step, a.steps, a.warmup)[0]

    # ---- IF4 of the same tensor (amax pass + encode pass) and its dequantize
    if4_out = [fq.quantize_nvfp4(x, policy="if4", workspace=ws) for x in xs]

    def if4_step(i):
        k = i % REPLICAS
        fq.quantize_nvfp4(xs[k], policy="if4", out=if4_out[k], workspace=ws)
    if4_sec = timed(if4_step, a.steps, a.warmup)[0]

    def if4_dq_step(i):
        k = i % REPLICAS
        o = if4_out[k]
        fq.dequantize("if4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=dq_out[k])
    if4_dq_sec = timed(if4_dq_step, a.steps, a.warmup)[0]
    if4_int4_frac = float((if4_out[0].scales >= 0x80).float().mean())

    line = {
        "metric": "quantize GB/s and % HBM peak, 8192² bf16→NVFP4/MXFP4, 1×MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle_ms": a.settle_ms,
        "settle_steps": settle_steps,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (2*Student-t(4), seed 102, bf16)",
        "config": {"workload": "NVFP4 two-level quantize of bf16 8192x8192 (tensor amax computed in-call), "
                               "E4M3 16-blocks + fp32 tensor scale, RNE",
                   "rows": ROWS, "cols": COLS, "algorithmic_bytes_per_step": NV_BYTES,
                   "elements_per_s": round(N / sec, 1), "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "input_replicas": REPLICAS},
        "roofline": {"bound": "hbm", "kernel": "nv_resident_kernel",
                     "achieved": round(call_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / HBM_PEAK_GBPS, 4),
                     "avg_launch_us": round(call_sec * 1e6, 3),
                     "bytes_per_launch": NV_BYTES,
                     "traffic": traffic_for("nv_resident_kernel")},
        "nvfp4_encode_given_amax": {"kernel": "nv_fast_kernel", "event_us": round(enc_sec * 1e6, 3),
                                    "value": round(NV_BYTES / enc_sec / 1e9, 2), "unit": "GB/s",
                                    "traffic": traffic_for("nv_fast_kernel")},
        "mxfp4": {"value": round(MX_BYTES / mx_sec / 1e9, 2), "unit": "GB/s",
                  "frac_of_hbm_peak": round(MX_BYTES / mx_sec / 1e9 / HBM_PEAK_GBPS, 4),
                  "ms_per_step": round(mx_sec * 1e3, 5), "event_us": round(mx_ev * 1e6, 3),
                  "bytes_per_step": MX_BYTES, "kernel": "mx_quant_kernel",
                  "traffic": traffic_for("mx_quant_kernel")},
        "dequant_nvfp4_to_bf16": {"value": round(DQ_BYTES / dq_sec / 1e9, 2), "unit": "GB/s",
                                  "ms_per_step": round(dq_sec * 1e3, 5), "bytes_per_step": DQ_BYTES,
                                  "kernel": "dequant_kernel", "traffic": traffic_for("dequant_kernel")},
        "if4": {"value": round(NV_BYTES / if4_sec / 1e9, 2), "unit": "GB/s",
                "frac_of_hbm_peak": round(NV_BYTES / if4_sec / 1e9 / HBM_PEAK_GBPS, 4),
                "ms_per_step": round(if4_sec * 1e3, 5), "bytes_per_step": NV_BYTES,
                "kernels": "nv_amax_kernel + nv_quant_kernel (IF4 policy)", "int4_block_fraction": round(if4_int4_frac, 4),
                "dequant_to_bf16": {"value": round(NV_BYTES / if4_dq_sec / 1e9, 2), "unit": "GB/s",
                                    "ms_per_step": round(if4_dq_sec * 1e3, 5)}},
        "kernel_source_sha": kernel_source_sha(),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
