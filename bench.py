"""Benchmark: quantize GB/s and fraction of HBM peak, 8192x8192 bf16 -> NVFP4
(headline) and MXFP4, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                    [--no-cpu-baseline] [--no-report]

    python bench.py --profile-kernels   # a few launches of each kernel, for rocprofv3

A step is one NVFP4 quantization of the 8192x8192 bf16 activation tensor
(2 * Student-t(4), seed 102): tensor amax computed in the call, E2M1 codes,
E4M3 block scales and the fp32 tensor scale (one launch of the single-read
kernel).  Inputs are resident in HBM before timing; the step cycles over 4
replicas of the input (4 x 128 MiB) so every step reads an input the 256 MB
Infinity Cache no longer holds.  value = algorithmic bytes (read the input
once, write every output once) x K / wall time of the K steps.  Before the W
warmup steps the headline step runs back to back, untimed, for MS
milliseconds (default 50): the GPU clock idles low and needs ~30 ms of load
to reach its sustained level, which a few warmup steps do not give.

The same JSON line carries:
  * roofline: the headline kernel's algorithmic bytes over its average launch
    time (HIP events on the launch stream over the K timed steps), and the
    median / p10 / p90 of per-launch event times;
  * report: every other workload timed the same way, cold (input replicas
    cycled past 256 MB): MXFP4 of the same tensor, the NVFP4 dequantize, the
    encode pass with a caller amax, the 1024x1024 fp32 MXFP4 quantize and
    dequantize, FWHT-8192 + MXFP4 of 16384x8192, Four Over Six of the
    8192x28672 weight, RHT16 + stochastic-rounding NVFP4 of the gradient,
    IF4 (and its dequantize) of both tensors, the per-head FWHT-128, the
    fused SwiGLU epilogue; each with GB/s, elements/s, fraction of 8 TB/s and
    the median / p10 / p90 per call, and an `alu` object: the VALU issue
    quad-cycles per call (committed rocprofv3 SQ counters) over the call
    time, against one quad-cycle per SIMD every 4 clocks at 2.4 GHz;
  * quality: NVFP4 and MXFP4 mean squared error on the headline tensor and
    their ratio, beside the pages' "~2.4x lower for NVFP4";
  * gemm: the MXFP4 GEMM 8192^3 with the bf16 and, where torch runs it, the
    fp8 matmul of the library routine, beside the pages' "FP4 ~2x FP8";
  * cpu_baseline: the CPU oracle on the host's cores (all threads it can use,
    and one), with the core count and CPU model.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense fp4 matrix peak
VALU_PEAK_TSLOTS = 256 * 4 * 2.4e9 / 4 * 64 / 1e12   # 39.32: VALU issue of 256 CUs x 4 SIMDs
ROWS, COLS = 8192, 8192
N = ROWS * COLS
BYTES_IN = N * 2
NV_BYTES = BYTES_IN + N // 2 + N // 16 + 4          # 171,966,468
MX_BYTES = BYTES_IN + N // 2 + N // 32              # 169,869,312
DQ_BYTES = N // 2 + N // 16 + 4 + BYTES_IN          # dequant NVFP4 -> bf16
REPLICAS = 4
COLD_BYTES = 320 << 20          # inputs cycled per timed workload: past the 256 MB Infinity Cache
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
PROFILE_VALU = os.path.join(ROOT, "profiles", "valu.json")


def kernel_source_sha():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp4_block_scaled_row_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _profile(path):
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("source_sha") == kernel_source_sha() else None


def traffic_for(kernel, launch_units=1):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None when
    the kernels changed since the counters were taken."""
    t = _profile(PROFILE_TRAFFIC)
    k = t.get("kernels", {}).get(kernel) if t else None
    if not k:
        return None
    return int(k["hbm_bytes_per_launch"]) * launch_units


def traffic_for_workload(workload):
    """HBM bytes per call of a workload's kernels (the sum over them) from the
    committed rocprofv3 PMC summary, or None when stale or absent."""
    t = _profile(PROFILE_TRAFFIC)
    w = t.get("workloads", {}).get(workload) if t else None
    return int(w["hbm_bytes_per_call"]) if w else None


def profiled(workload):
    """The counter-based fields of a report row: measured HBM bytes per call
    and the VALU issue roofline (summary() turns `valu` into `alu`)."""
    return {"traffic": traffic_for_workload(workload), "valu": valu_for(workload)}


def valu_for(workload):
    """VALU issue quad-cycles per call of a workload's kernels, from the
    committed rocprofv3 SQ counters (ACTIVE_INST_VALU - ACTIVE_INST_VALU2: a
    dual-issued pair counts once, a half-rate conversion twice), or None when
    the kernels changed since the counters were taken."""
    t = _profile(PROFILE_VALU)
    w = t.get("workloads", {}).get(workload) if t else None
    return int(w["valu_issue_quad_cycles_per_call"]) if w else None


def alu_roofline(quad_cycles, seconds):
    """VALU issue roofline: one quad-cycle (a 64-lane wave instruction at full
    rate) per SIMD every 4 clocks, 256 CUs x 4 SIMDs at 2.4 GHz, in 64-lane
    slots per second."""
    if quad_cycles is None:
        return None
    achieved = quad_cycles * 64 / seconds / 1e12
    return {"bound": "alu", "achieved": round(achieved, 2), "peak": round(VALU_PEAK_TSLOTS, 2),
            "unit": "T lane-slots/s", "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
            "valu_issue_quad_cycles_per_call": quad_cycles}


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return model, os.cpu_count() or 1, usable


def cpu_baseline(x_np, min_cpu_seconds=10.0):
    """The oracle as it stands (plain C, one call per row chunk) on the
    headline workload: all the threads the host gives this process, over the
    whole tensor (tensor amax of the row chunks, then their encoding with that
    amax), repeated until about min_cpu_seconds of CPU work; and one thread on
    its first 2048 rows.  ctypes releases the GIL, so the row chunks run in
    parallel."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    model, nproc, usable = cpu_info()
    threads = max(1, min(16, usable))      # at most 16 threads: one GPU's share of a multi-GPU host's cores
    chunk = 256
    starts = list(range(0, ROWS, chunk))

    def full_pass(ex):
        amax = max(ex.map(lambda r0: oracle.tensor_amax(x_np[r0:r0 + chunk]), starts))
        list(ex.map(lambda r0: oracle.quantize_nv(x_np[r0:r0 + chunk], global_amax=amax), starts))

    with ThreadPoolExecutor(threads) as ex:
        reps, dt, cpu = 0, 0.0, 0.0
        while reps == 0 or (cpu < min_cpu_seconds and reps < 8):
            t, c = time.perf_counter(), time.process_time()
            full_pass(ex)
            dt += time.perf_counter() - t
            cpu += time.process_time() - c
            reps += 1
    gbps = N * reps * (NV_BYTES / N) / dt / 1e9
    rows1 = 2048
    t = time.perf_counter()
    oracle.quantize_nv(x_np[:rows1])
    dt1 = time.perf_counter() - t
    gbps1 = rows1 * COLS * (NV_BYTES / N) / dt1 / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "NVFP4 quantize (tensor amax, scales, codes) of the whole 8192x8192 workload, %d pass(es), "
                      "row chunks of %d over %d threads, %.2f s wall, %.1f s CPU" % (reps, chunk, threads, dt, cpu),
            "elements_per_s": round(N * reps / dt, 1),
            "nproc": nproc, "cpu_model": model,
            "single_thread": {"value": round(gbps1, 4), "unit": "GB/s", "cores": 1,
                              "elements_per_s": round(rows1 * COLS / dt1, 1),
                              "sample": "rows 0..%d (%d elements), one call, %.2f s" % (rows1 - 1, rows1 * COLS, dt1)}}


class Timer:
    """HIP-event timing on the launch stream (torch's current stream, which the
    library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def settle(self, fn, ms):
        torch = self.torch
        n, t = 0, time.perf_counter()
        while (time.perf_counter() - t) * 1e3 < ms:
            for _ in range(8):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return n

    def per_call(self, fn, steps, warmup):
        """Event duration of each of `steps` calls (seconds), after `warmup`."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(st)
            fn(warmup + i)
            ev[i][1].record(st)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)

    def wall(self, fn, steps, warmup):
        """(wall seconds per step, event seconds per step) of `steps` back-to-back calls."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record(st)
        for i in range(steps):
            fn(warmup + i)
        e1.record(st)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps, e0.elapsed_time(e1) / 1e3 / steps


def pct(sorted_s, q):
    i = min(len(sorted_s) - 1, max(0, int(round(q * (len(sorted_s) - 1)))))
    return sorted_s[i]


def summary(timing, nbytes, nelems, kernels, **extra):
    """GB/s, elements/s and fraction of HBM peak at the mean call time of
    back-to-back calls (events at both ends), with the median / p10 / p90 of
    calls timed one by one (events around each call, which adds the dispatch
    of each launch: ~1-2 us above the back-to-back mean)."""
    mean, times = timing
    d = {"value": round(nbytes / mean / 1e9, 2), "unit": "GB/s",
         "elements_per_s": round(nelems / mean, 1),
         "frac_of_hbm_peak": round(nbytes / mean / 1e9 / HBM_PEAK_GBPS, 4),
         "us_mean": round(mean * 1e6, 3),
         "us_median": round(pct(times, 0.5) * 1e6, 3), "us_p10": round(pct(times, 0.1) * 1e6, 3),
         "us_p90": round(pct(times, 0.9) * 1e6, 3),
         "bytes_per_call": int(nbytes), "kernels": kernels}
    valu = extra.pop("valu", None)
    if valu is not None:
        d["alu"] = alu_roofline(valu, mean)
    if extra.get("traffic") is not None:
        d["traffic_over_algorithmic"] = round(extra["traffic"] / nbytes, 3)
    d.update(extra)
    return d


def n_replicas(nbytes_in, lo=2):
    return max(lo, -(-COLD_BYTES // nbytes_in))


def report(dev, timer, steps, warmup, ws, xs_act, nv_out):
    """Every other workload, timed cold.  Returns the `report` object."""
    import numpy as np
    import torch

    import fp4_block_scaled_row_amd as fq
    import workloads

    rep = {}

    def replicas(x_np, k):
        x0 = torch.from_numpy(x_np.view(np.int16) if x_np.dtype == np.uint16 else x_np).to(dev)
        if x_np.dtype == np.uint16:
            x0 = x0.view(torch.bfloat16)
        return [x0] + [x0.clone() for _ in range(k - 1)]

    def graph_rate(fn, k, nbytes, replays=20):
        """The same calls (k of them, one per replica) captured in a HIP graph and
        replayed back to back: the GPU's time per call without the host's
        dispatch of each launch, which bounds calls on tensors this small."""
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for i in range(k):
                fn(i)           # (the binding keeps a workspace per stream: made here, outside capture)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(k):
                fn(i)
        timer.settle(lambda i: g.replay(), 20)
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(replays):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        per_call = e0.elapsed_time(e1) / 1e3 / (replays * k)
        return {"us_per_call": round(per_call * 1e6, 3), "value": round(nbytes / per_call / 1e9, 2), "unit": "GB/s",
                "calls_per_graph": k, "replays": replays}

    def timed(fn, n_calls=None):
        n = n_calls or steps
        timer.settle(fn, 30)     # (the clock drops while the host prepares each workload)
        mean = timer.wall(fn, n, warmup)[1]
        return mean, timer.per_call(fn, n, 2)

    # ---- H2: MXFP4 of the headline tensor
    mx_out = [fq.quantize_mxfp4(x) for x in xs_act]
    t = timed(lambda i: fq.quantize_mxfp4(xs_act[i % REPLICAS], out=mx_out[i % REPLICAS]))
    rep["H2_mxfp4_bf16_8192"] = summary(t, MX_BYTES, N, "mx_quant_kernel", **profiled("H2_mxfp4_bf16_8192"))

    # ---- NVFP4 dequantize -> bf16, and the encode pass with a caller amax
    dq_out = [torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev) for _ in range(REPLICAS)]

    def dq(i):
        o = nv_out[i % REPLICAS]
        fq.dequantize("nvfp4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=dq_out[i % REPLICAS])
    rep["C2_dequant_nvfp4_to_bf16"] = summary(timed(dq), DQ_BYTES, N, "dequant_kernel",
                                              **profiled("C2_dequant_nvfp4_to_bf16"))
    amax_dev = [torch.max(torch.abs(x.float())).reshape(1) for x in xs_act]
    t = timed(lambda i: fq.quantize_nvfp4(xs_act[i % REPLICAS], out=nv_out[i % REPLICAS],
                                          global_amax=amax_dev[i % REPLICAS]))
    rep["C2_nvfp4_encode_given_amax"] = summary(t, NV_BYTES, N, "nv_fast_kernel",
                                                **profiled("C2_nvfp4_encode_given_amax"))

    # ---- IF4 of the headline tensor and its dequantize
    if4_out = [fq.quantize_nvfp4(x, policy="if4", workspace=ws) for x in xs_act]
    t = timed(lambda i: fq.quantize_nvfp4(xs_act[i % REPLICAS], policy="if4", out=if4_out[i % REPLICAS], workspace=ws))
    frac = float((if4_out[0].scales >= 0x80).float().mean())
    rep["IF4_bf16_8192"] = summary(t, NV_BYTES, N, "nv_amax_kernel + nv_quant_kernel (IF4)",
                                   int4_block_fraction=round(frac, 4), **profiled("IF4_bf16_8192"))

    def if4dq(i):
        o = if4_out[i % REPLICAS]
        fq.dequantize("if4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=dq_out[i % REPLICAS])
    rep["IF4_dequant_to_bf16_8192"] = summary(timed(if4dq), NV_BYTES, N, "dequant_kernel (IF4)")
    del if4_out, dq_out

    # ---- per-head FWHT-128 + NVFP4 of the headline tensor (64 heads of 128)
    h_out = [fq.quantize_nvfp4(x, rotation="fwht128", workspace=ws) for x in xs_act]
    t = timed(lambda i: fq.quantize_nvfp4(xs_act[i % REPLICAS], rotation="fwht128", out=h_out[i % REPLICAS],
                                          workspace=ws))
    rep["F4_fwht128_nvfp4_bf16_8192"] = summary(t, NV_BYTES, N, "nv_amax_kernel + nv_quant_kernel (FWHT-128)",
                                                **profiled("F4_fwht128_nvfp4_bf16_8192"))
    del h_out, amax_dev
    torch.cuda.empty_cache()

    # ---- C1: MXFP4 quantize (counters) and dequantize of fp32 1024x1024
    x1 = workloads.make("mx_f32_1024")
    n1 = x1.size
    b1 = n1 * 4 + n1 // 2 + n1 // 32
    k1 = n_replicas(x1.nbytes)
    xs1 = replicas(x1, k1)
    o1 = [fq.quantize_mxfp4(x, counters=True) for x in xs1]
    q1 = lambda i: fq.quantize_mxfp4(xs1[i % k1], counters=True, out=o1[i % k1])
    rep["C1_mxfp4_f32_1024_counters"] = summary(timed(q1), b1, n1, "mx_quant_kernel + count_reduce_kernel",
                                                replicas=k1, **profiled("C1_mxfp4_f32_1024_counters"),
                                                graph_replay=graph_rate(q1, k1, b1))
    y1 = [torch.empty_like(x) for x in xs1]
    d1 = lambda i: fq.dequantize("mxfp4", o1[i % k1].codes, o1[i % k1].scales, out_dtype=torch.float32,
                                 out=y1[i % k1])
    rep["C1_dequant_mxfp4_to_f32_1024"] = summary(timed(d1), b1, n1, "dequant_kernel", replicas=k1,
                                                  graph_replay=graph_rate(d1, k1, b1))
    del xs1, o1, y1

    # ---- C5: RHT16 + stochastic-rounding NVFP4 of the gradient
    x5 = workloads.make("grad_bf16_8192")
    xs5 = replicas(x5, REPLICAS)
    del x5
    seed = workloads.SR_SEED
    o5 = [fq.quantize_nvfp4(x, rotation="rht16", rounding="stochastic", seed=seed, workspace=ws) for x in xs5]
    t = timed(lambda i: fq.quantize_nvfp4(xs5[i % REPLICAS], rotation="rht16", rounding="stochastic", seed=seed,
                                          out=o5[i % REPLICAS], workspace=ws))
    rep["C5_rht16_sr_nvfp4_bf16_8192"] = summary(t, NV_BYTES, N, "nv_amax_kernel + nv_quant_kernel (RHT16, SR)",
                                                 **profiled("C5_rht16_sr_nvfp4_bf16_8192"))
    del xs5, o5
    torch.cuda.empty_cache()

    # ---- C3: full-row FWHT-8192 + MXFP4 of 16384x8192
    x3 = workloads.make("swiglu_bf16_16384x8192")
    n3 = x3.size
    xs3 = replicas(x3, 2)
    del x3
    o3 = [fq.quantize_mxfp4(x, rotation="fwht_row") for x in xs3]
    t = timed(lambda i: fq.quantize_mxfp4(xs3[i % 2], rotation="fwht_row", out=o3[i % 2]), max(20, steps // 2))
    rep["C3_fwht8192_mxfp4_bf16_16384x8192"] = summary(t, n3 * 2 + n3 // 2 + n3 // 32, n3, "fwht8192_kernel (+MXFP4)",
                                                       **profiled("C3_fwht8192_mxfp4_bf16_16384x8192"))
    del xs3, o3
    torch.cuda.empty_cache()

    # ---- fused SwiGLU epilogue: SiLU(gate) * up -> FWHT-8192 -> MXFP4, 16384 x (2 x 8192)
    xg = workloads.make("gate_up_bf16_16384x8192")
    xgd = replicas(xg, 2)
    del xg
    d = COLS
    og = [fq.silu_mul_fwht_mxfp4(x[:, :d], x[:, d:]) for x in xgd]
    ng = xgd[0].numel() // 2
    t = timed(lambda i: fq.silu_mul_fwht_mxfp4(xgd[i % 2][:, :d], xgd[i % 2][:, d:], out=og[i % 2]),
              max(20, steps // 2))
    rep["F2_silu_mul_fwht8192_mxfp4_bf16_16384x8192"] = summary(t, 2 * ng * 2 + ng // 2 + ng // 32, ng,
                                                                "fwht8192_kernel (SwiGLU + MXFP4)",
                                                                **profiled("F2_silu_mul_fwht8192_mxfp4_bf16_16384x8192"))
    del xgd, og
    torch.cuda.empty_cache()

    # ---- C4: Four Over Six of the 8192x28672 weight (and IF4 of it)
    x4 = workloads.make("weight_bf16_8192x28672")
    n4 = x4.size
    xs4 = replicas(x4, 2)
    del x4
    o4 = [fq.quantize_nvfp4(x, policy="four_over_six", workspace=ws) for x in xs4]
    t = timed(lambda i: fq.quantize_nvfp4(xs4[i % 2], policy="four_over_six", out=o4[i % 2], workspace=ws),
              max(20, steps // 2))
    rep["C4_four_over_six_bf16_8192x28672"] = summary(t, n4 * 2 + n4 // 2 + n4 // 16 + 4 + n4 // 128, n4,
                                                      "nv_amax_kernel + nv_quant_kernel (Four Over Six)",
                                                      max4_block_fraction=round(float(np.unpackbits(
                                                          o4[0].choice_bits.cpu().numpy()).mean()), 4),
                                                      **profiled("C4_four_over_six_bf16_8192x28672"))
    del o4
    oi = [fq.quantize_nvfp4(x, policy="if4", workspace=ws) for x in xs4]
    t = timed(lambda i: fq.quantize_nvfp4(xs4[i % 2], policy="if4", out=oi[i % 2], workspace=ws), max(20, steps // 2))
    rep["IF4_bf16_8192x28672"] = summary(t, n4 * 2 + n4 // 2 + n4 // 16 + 4, n4,
                                         "nv_amax_kernel + nv_quant_kernel (IF4)",
                                         **profiled("IF4_bf16_8192x28672"))
    yi = [torch.empty_like(xs4[0]) for _ in range(2)]

    def if4dq4(i):
        o = oi[i % 2]
        fq.dequantize("if4", o.codes, o.scales, o.global_scale, out_dtype=torch.bfloat16, out=yi[i % 2])
    rep["IF4_dequant_to_bf16_8192x28672"] = summary(timed(if4dq4, max(20, steps // 2)),
                                                    n4 // 2 + n4 // 16 + 4 + n4 * 2, n4, "dequant_kernel (IF4)",
                                                    **profiled("IF4_dequant_to_bf16_8192x28672"))
    del xs4, oi, yi
    torch.cuda.empty_cache()
    return rep


def quality(xs_act, nv_out):
    """NVFP4 vs MXFP4 mean squared error on the headline tensor (GPU
    dequantize, fp64 sums): the pages quote ~2.4x lower block MSE for NVFP4."""
    import torch

    import fp4_block_scaled_row_amd as fq
    x = xs_act[0]
    o = nv_out[0]
    fq.quantize_nvfp4(x, out=o)
    m = fq.quantize_mxfp4(x)
    xf = x.float()
    ynv = fq.dequantize("nvfp4", o.codes, o.scales, o.global_scale, out_dtype=torch.float32)
    ymx = fq.dequantize("mxfp4", m.codes, m.scales, out_dtype=torch.float32)
    mse_nv = float(((ynv - xf).double() ** 2).mean())
    mse_mx = float(((ymx - xf).double() ** 2).mean())
    return {"mse_nvfp4": mse_nv, "mse_mxfp4": mse_mx, "mxfp4_over_nvfp4": round(mse_mx / mse_nv, 3),
            "pages": "~2.4x lower block MSE for NVFP4 than MXFP4 (Sub-4-Bit Microscaling, section 2; NVIDIA "
                     "Blackwell context, no workload stated)",
            "workload": "2*Student-t(4) bf16 8192x8192, dequantized to fp32"}


def gemm_context(dev, timer, reps=10):
    """MXFP4 GEMM 8192^3 (this library) beside the library matmul in bf16 and,
    where torch runs it, fp8 (e4m3, per-tensor scales)."""
    import numpy as np
    import torch

    import fp4_block_scaled_row_amd as fq
    import workloads
    M = Nn = K = 8192
    flops = 2.0 * M * Nn * K
    xa_np = workloads.make("act_bf16_8192")
    xa = torch.from_numpy(xa_np.view(np.int16)).to(dev).view(torch.bfloat16)
    wn = workloads.make("weight_bf16_8192x28672", rows=8192, cols=8192)
    xw = torch.from_numpy(wn.view(np.int16)).to(dev).view(torch.bfloat16)
    qa, qw = fq.quantize_mxfp4(xa), fq.quantize_mxfp4(xw)
    cb = torch.empty((M, Nn), dtype=torch.bfloat16, device=dev)
    out = {}

    def rate(fn):
        timer.settle(lambda i: fn(), 30)
        t = timer.per_call(lambda i: fn(), reps, 2)
        med = pct(t, 0.5)
        return {"tflops": round(flops / med / 1e12, 1), "us_median": round(med * 1e6, 2)}

    out["mxfp4_gemm_bf16_out"] = rate(lambda: fq.mxfp4_gemm(qa, qw, out_dtype=torch.bfloat16, out=cb))
    out["mxfp4_gemm_bf16_out"]["frac_of_fp4_peak"] = round(out["mxfp4_gemm_bf16_out"]["tflops"] / FP4_PEAK_TFLOPS, 4)
    wt = xw.t().contiguous()
    out["torch_bf16_matmul"] = rate(lambda: torch.matmul(xa, wt, out=cb))
    try:
        f8 = torch.float8_e4m3fn
        sa = (torch.max(torch.abs(xa.float())) / 448.0).reshape(()).float()
        sw = (torch.max(torch.abs(xw.float())) / 448.0).reshape(()).float()
        a8 = (xa.float() / sa).to(f8)
        w8 = (xw.float() / sw).to(f8)
        b8 = w8.t()     # column-major [K, N]
        out["torch_fp8_scaled_mm"] = rate(lambda: torch._scaled_mm(a8, b8, scale_a=sa, scale_b=sw,
                                                                    out_dtype=torch.bfloat16))
        out["fp4_over_fp8"] = round(out["mxfp4_gemm_bf16_out"]["tflops"] / out["torch_fp8_scaled_mm"]["tflops"], 3)
    except Exception as e:          # the library routine may not run fp8 on this machine
        out["torch_fp8_scaled_mm"] = {"error": "%s: %s" % (type(e).__name__, str(e)[:160])}
    out["pages"] = "FP4 matmul ~2x FP8 and ~4x FP16/BF16 with both operands in FP4 (on B200 and MI355X; podcast)"
    out["shape"] = "8192x8192x8192, bf16 output"
    return out


def profile_kernels(dev, reps=5):
    """A few launches of every kernel on the five workloads' full sizes, inputs
    cycled over replicas as in the bench, plus a plain 128 MiB device copy (the
    reference for HBM byte counters).  Prints one text line per kernel with its
    average event time."""
    import numpy as np
    import torch

    import fp4_block_scaled_row_amd as fq
    import workloads

    def dev_replicas(name, k):
        x = workloads.make(name)
        if x.dtype == np.uint16:
            x0 = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            x0 = torch.from_numpy(x).to(dev)
        return [x0] + [x0.clone() for _ in range(k - 1)]

    timer = Timer(torch)

    def run(label, fn, nbytes, k):
        timer.settle(lambda i: fn(i % k), 40)
        t = timer.wall(lambda i: fn(i % k), reps, 1)[1]
        print("%-58s %9.2f us  %8.1f GB/s" % (label, t * 1e6, nbytes / t / 1e9), flush=True)

    src = torch.empty(BYTES_IN, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    run("copy 128 MiB (reference for byte counters)", lambda k: dst.copy_(src), 2 * BYTES_IN, 1)
    del src, dst

    xs = dev_replicas("act_bf16_8192", REPLICAS)
    ws = torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8, device=dev)
    o = [fq.quantize_nvfp4(x, workspace=ws) for x in xs]
    run("C2 NVFP4 bf16 8192x8192, amax in call", lambda k: fq.quantize_nvfp4(xs[k], out=o[k], workspace=ws),
        NV_BYTES, REPLICAS)
    amax = [torch.max(torch.abs(x.float())).reshape(1) for x in xs]
    run("C2 NVFP4 bf16 8192x8192, amax given (encode pass)",
        lambda k: fq.quantize_nvfp4(xs[k], out=o[k], global_amax=amax[k]), NV_BYTES, REPLICAS)
    ox = [fq.quantize_mxfp4(x) for x in xs]
    run("H2 MXFP4 bf16 8192x8192", lambda k: fq.quantize_mxfp4(xs[k], out=ox[k]), MX_BYTES, REPLICAS)
    y = [torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev) for _ in range(REPLICAS)]
    run("C2 dequantize NVFP4 -> bf16 8192x8192",
        lambda k: fq.dequantize("nvfp4", o[k].codes, o[k].scales, o[k].global_scale, out_dtype=torch.bfloat16,
                                out=y[k]), DQ_BYTES, REPLICAS)
    o6 = [fq.quantize_nvfp4(x, rotation="fwht128", workspace=ws) for x in xs]
    run("FWHT-128 per head + NVFP4 bf16 8192x8192 (64 heads of 128)",
        lambda k: fq.quantize_nvfp4(xs[k], rotation="fwht128", out=o6[k], workspace=ws), NV_BYTES, REPLICAS)
    oi = [fq.quantize_nvfp4(x, policy="if4", workspace=ws) for x in xs]
    run("IF4 bf16 8192x8192", lambda k: fq.quantize_nvfp4(xs[k], policy="if4", out=oi[k], workspace=ws),
        NV_BYTES, REPLICAS)
    del xs, o, ox, y, o6, oi, amax
    torch.cuda.empty_cache()

    x5 = dev_replicas("grad_bf16_8192", REPLICAS)
    sd = workloads.SR_SEED
    o5 = [fq.quantize_nvfp4(x, rotation="rht16", rounding="stochastic", seed=sd, workspace=ws) for x in x5]
    run("C5 RHT16 + stochastic NVFP4 bf16 8192x8192",
        lambda k: fq.quantize_nvfp4(x5[k], rotation="rht16", rounding="stochastic", seed=sd, out=o5[k], workspace=ws),
        NV_BYTES, REPLICAS)
    del x5, o5
    torch.cuda.empty_cache()

    x3 = dev_replicas("swiglu_bf16_16384x8192", 2)
    o3 = [fq.quantize_mxfp4(x, rotation="fwht_row") for x in x3]
    n3 = x3[0].numel()
    run("C3 FWHT-8192 + MXFP4 bf16 16384x8192",
        lambda k: fq.quantize_mxfp4(x3[k], rotation="fwht_row", out=o3[k]), n3 * 2 + n3 // 2 + n3 // 32, 2)
    del x3, o3
    torch.cuda.empty_cache()

    x4 = dev_replicas("weight_bf16_8192x28672", 2)
    n4 = x4[0].numel()
    o4 = [fq.quantize_nvfp4(x, policy="four_over_six", workspace=ws) for x in x4]
    run("C4 Four-Over-Six NVFP4 bf16 8192x28672",
        lambda k: fq.quantize_nvfp4(x4[k], policy="four_over_six", out=o4[k], workspace=ws),
        n4 * 2 + n4 // 2 + n4 // 16 + 4 + n4 // 128, 2)
    del o4
    oi = [fq.quantize_nvfp4(x, policy="if4", workspace=ws) for x in x4]
    run("IF4 bf16 8192x28672 (weights of C4)",
        lambda k: fq.quantize_nvfp4(x4[k], policy="if4", out=oi[k], workspace=ws), n4 * 2 + n4 // 2 + n4 // 16 + 4, 2)
    del x4
    yi = [torch.empty((oi[0].codes.shape[0], oi[0].codes.shape[1] * 2), dtype=torch.bfloat16, device=dev)
          for _ in range(2)]
    run("IF4 dequantize -> bf16 8192x28672",
        lambda k: fq.dequantize("if4", oi[k].codes, oi[k].scales, oi[k].global_scale, out_dtype=torch.bfloat16,
                                out=yi[k]), n4 * 2 + n4 // 2 + n4 // 16 + 4, 2)
    del oi, yi
    torch.cuda.empty_cache()

    xg = dev_replicas("gate_up_bf16_16384x8192", 2)
    d = xg[0].shape[1] // 2
    og = [fq.silu_mul_fwht_mxfp4(x[:, :d], x[:, d:]) for x in xg]
    ng = xg[0].numel() // 2
    run("SiLU_and_Mul + FWHT-8192 + MXFP4 bf16 16384x(2x8192), fused",
        lambda k: fq.silu_mul_fwht_mxfp4(xg[k][:, :d], xg[k][:, d:], out=og[k]), 2 * ng * 2 + ng // 2 + ng // 32, 2)
    hb = torch.empty((xg[0].shape[0], d), dtype=torch.bfloat16, device=dev)

    def unfused(k):
        torch.mul(torch.nn.functional.silu(xg[k][:, :d]), xg[k][:, d:], out=hb)
        fq.quantize_mxfp4(hb, rotation="fwht_row", out=og[k])
    run("  unfused reference: torch SiLU*up to bf16, then FWHT-8192 + MXFP4", unfused,
        2 * ng * 2 + ng // 2 + ng // 32, 2)
    del xg, og, hb
    torch.cuda.empty_cache()

    x1 = dev_replicas("mx_f32_1024", n_replicas(1024 * 1024 * 4))
    k1 = len(x1)
    o1 = [fq.quantize_mxfp4(x, counters=True) for x in x1]
    y1 = [torch.empty_like(x) for x in x1]
    n1 = x1[0].numel()
    run("C1 MXFP4 fp32 1024x1024 (with counters)", lambda k: fq.quantize_mxfp4(x1[k], counters=True, out=o1[k]),
        n1 * 4 + n1 // 2 + n1 // 32, k1)
    run("C1 dequantize MXFP4 -> fp32 1024x1024",
        lambda k: fq.dequantize("mxfp4", o1[k].codes, o1[k].scales, out_dtype=torch.float32, out=y1[k]),
        n1 // 2 + n1 // 32 + n1 * 4, k1)
    del x1, o1, y1
    torch.cuda.empty_cache()

    g = gemm_context(dev, timer, reps=reps)
    print("MXFP4 GEMM 8192^3 -> bf16 %s; torch bf16 %s; torch fp8 %s" % (
        g["mxfp4_gemm_bf16_out"], g["torch_bf16_matmul"], g["torch_fp8_scaled_mm"]), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed back-to-back headline steps before the warmup steps, so that the GPU clock "
                         "reaches its sustained level (it idles low and ramps within ~30 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-report", action="store_true",
                    help="time the headline only (no report workloads, quality or GEMM context)")
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
    timer = Timer(torch)
    x_np = workloads.make("act_bf16_8192")
    x0 = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(REPLICAS - 1)]
    ws = torch.zeros(fq.workspace_bytes(16), dtype=torch.uint8, device=dev)
    nv_out = [fq.quantize_nvfp4(x, workspace=ws) for x in xs]          # outputs allocated once per replica
    torch.cuda.synchronize()

    def nv_step(i):
        k = i % REPLICAS
        fq.quantize_nvfp4(xs[k], out=nv_out[k], workspace=ws)

    # ---- headline: NVFP4 quantize, K steps (one launch of nv_resident_kernel each)
    settle_steps = timer.settle(nv_step, a.settle_ms)
    # roofline of the dominant kernel: the single-read NVFP4 kernel, the only
    # launch of a step, so the events over the timed steps give its average
    # launch duration (back-to-back launches: the gaps between them included)
    sec, call_sec = timer.wall(nv_step, a.steps, a.warmup)
    value = NV_BYTES / sec / 1e9
    call_gbps = NV_BYTES / call_sec / 1e9
    per_launch = timer.per_call(nv_step, a.steps, 2)

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
        "dtype": "f32",     # the arithmetic: bf16 inputs are widened to fp32 (the tensor scale in fp64)
        "data": "synthetic (2*Student-t(4), seed 102, bf16)",
        "config": {"workload": "NVFP4 two-level quantize of bf16 8192x8192 (tensor amax computed in-call), "
                               "E4M3 16-blocks + fp32 tensor scale, RNE",
                   "rows": ROWS, "cols": COLS, "algorithmic_bytes_per_step": NV_BYTES,
                   "elements_per_s": round(N / sec, 1), "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "input_replicas": REPLICAS, "input_dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "nv_resident_kernel",
                     "achieved": round(call_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / HBM_PEAK_GBPS, 4),
                     "avg_launch_us": round(call_sec * 1e6, 3),
                     "launch_us_median": round(pct(per_launch, 0.5) * 1e6, 3),
                     "launch_us_p10": round(pct(per_launch, 0.1) * 1e6, 3),
                     "launch_us_p90": round(pct(per_launch, 0.9) * 1e6, 3),
                     "bytes_per_launch": NV_BYTES,
                     "traffic": traffic_for("nv_resident_kernel"),
                     "alu": alu_roofline(valu_for("headline_nvfp4_bf16_8192"), call_sec)},
        "kernel_source_sha": kernel_source_sha(),
    }
    if not a.no_report:
        line["report"] = report(dev, timer, a.steps, a.warmup, ws, xs, nv_out)
        line["quality"] = quality(xs, nv_out)
        del xs, nv_out
        torch.cuda.empty_cache()
        line["gemm"] = gemm_context(dev, timer)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
