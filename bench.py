"""Benchmark: quantize GB/s and fraction of HBM peak, 8192x8192 bf16 -> NVFP4
(headline) and MXFP4, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one NVFP4 quantization of the 8192x8192 bf16 activation tensor
(2 * Student-t(4), seed 102): the in-call tensor-amax pass, then the encode
pass writing E2M1 codes, E4M3 block scales and the fp32 tensor scale.  Inputs
are resident in HBM before timing; the step cycles over 4 replicas of the
input (4 x 128 MiB) so every step reads an input the Infinity Cache no longer
holds.  value = algorithmic bytes (read the input once, write every output
once) x K / wall time of the K steps.

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


def cpu_baseline(x_np):
    """The oracle, untuned, on the first 512 rows (4 Mi elements) of the workload."""
    import numpy as np  # noqa: F401
    import oracle
    rows = 512
    sample = x_np[:rows]
    t = time.perf_counter()
    oracle.quantize_nv(sample)
    dt = time.perf_counter() - t
    elems = rows * COLS
    gbps = elems * (NV_BYTES / N) / dt / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "NVFP4 quantize of rows 0..511 (4,194,304 elements) of the 8192x8192 workload, "
                      "single-threaded C oracle, %.2f s" % dt,
            "elements_per_s": round(elems / dt, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps

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

    # ---- headline: NVFP4 quantize (amax pass + encode pass), K steps
    sec = timed(nv_step, a.steps, a.warmup)
    value = NV_BYTES / sec / 1e9

    # ---- roofline of the dominant kernel: the encode pass (nv_quant_kernel)
    # launched alone with the tensor amax handed in, after an untimed amax
    # pass on the same replica so its input is where the real step finds it.
    for k in range(REPLICAS):
        amax_dev[k].copy_(torch.max(torch.abs(xs[k].float())).reshape(1))
    torch.cuda.synchronize()

    def encode_only(i):
        k = i % REPLICAS
        fq.quantize_nvfp4(xs[k], out=nv_out[k], global_amax=amax_dev[k])

    for i in range(a.warmup):
        encode_only(i)
    enc_sec = event_avg(encode_only, a.steps, pre=nv_step)
    call_sec = event_avg(nv_step, a.steps)
    enc_gbps = NV_BYTES / enc_sec / 1e9

    # ---- MXFP4 of the same tensor
    def mx_step(i):
        k = i % REPLICAS
        fq.quantize_mxfp4(xs[k], out=mx_out[k])
    mx_sec = timed(mx_step, a.steps, a.warmup)
    mx_ev = event_avg(mx_step, a.steps)

    # ---- NVFP4 dequantize back to bf16
    def dq_step(i):
        k = i % REPLICAS
        o = nv_out[k]
        fq.dequantize("nvfp4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=dq_out[k])
    dq_sec = timed(dq_step, a.steps, a.warmup)

    line = {
        "metric": "quantize GB/s and % HBM peak, 8192² bf16→NVFP4/MXFP4, 1×MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
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
        "roofline": {"bound": "hbm", "kernel": "nv_quant_kernel (encode pass)",
                     "achieved": round(enc_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
                     "avg_launch_us": round(enc_sec * 1e6, 3),
                     "bytes_per_launch": NV_BYTES,
                     "traffic": traffic_for("nv_quant_kernel")},
        "nvfp4_call_event_us": round(call_sec * 1e6, 3),
        "mxfp4": {"value": round(MX_BYTES / mx_sec / 1e9, 2), "unit": "GB/s",
                  "frac_of_hbm_peak": round(MX_BYTES / mx_sec / 1e9 / HBM_PEAK_GBPS, 4),
                  "ms_per_step": round(mx_sec * 1e3, 5), "event_us": round(mx_ev * 1e6, 3),
                  "bytes_per_step": MX_BYTES, "kernel": "mx_quant_kernel",
                  "traffic": traffic_for("mx_quant_kernel")},
        "dequant_nvfp4_to_bf16": {"value": round(DQ_BYTES / dq_sec / 1e9, 2), "unit": "GB/s",
                                  "ms_per_step": round(dq_sec * 1e3, 5), "bytes_per_step": DQ_BYTES},
        "kernel_source_sha": kernel_source_sha(),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
