#!/usr/bin/env python3
"""Benchmark of the ConvLinear4bit forward pass on one MI355X.

One step = the whole hot path on one batch: rotate + quantize the activations
(convrot_rotate_quant_act) and the W4A4 GEMM with the fused dequant epilogue
(convrot_w4a4_gemm), i.e. the two kernels convrot_w4a4_linear enqueues, launched through
the C ABI.  The weights are rotated and quantized once, before timing (offline path).
Activations rotate through more than twice the 256 MB Infinity Cache, so they come from HBM.

Prints ONE JSON line.  `value` is the full-layer throughput 2 M N K' / step time over the
timed steps.  The `roofline` object is for the dominant kernel (the GEMM, int8 matrix
cores); the rotate+quantize kernel's HBM roofline is reported alongside.  Each kernel's
launch duration comes from HIP events on the launch stream around batches of back-to-back
launches of that kernel, after a time-based ramp of launches that brings the clocks to their
sustained level; this runs before the warm-up and timed steps.  The CPU oracle is timed over
whole passes of the same layer (`cpu_baseline`).

`--codes int8` measures the W8A8 variant the same way (convrot_rotate_quant_act_i8 and
convrot_w8a8_gemm, the kernels convrot_w8a8_linear enqueues) and prints its own line;
`--codes mxfp4` the MXFP4 variant (convrot_rotate_quant_act_mxfp4 and convrot_mxfp4_gemm),
its GEMM against the FP4 matrix peak (10.1 PFLOP/s).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear TOPS + rotate-quant GB/s (% of roofline) at M=4608,K=3072,g=256"
METRIC_W8A8 = "W8A8 linear TOPS + rotate-quant GB/s (% of roofline) at M=4608,K=3072,g=256"
METRIC_MXFP4 = "MXFP4 linear TOPS + rotate-quant GB/s (% of roofline) at M=4608,K=3072,g=256"
FP4_PEAK_TOPS = 10100.0         # MI355X dense FP4 matrix throughput (10.1 PFLOP/s)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 matrix throughput (5.0 POP/s)
MALL_BYTES = 256 << 20          # Infinity Cache; rotate inputs through > 2x this


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="attn_proj")
    p.add_argument("--codes", choices=("int4", "int8", "mxfp4"), default="int4",
                   help="int4: the W4A4 layer (default); int8: the W8A8 variant; mxfp4: the "
                        "floating-point 4-bit variant")
    p.add_argument("--ramp-seconds", type=float, default=0.2,
                   help="back-to-back launches of each kernel before its timed batches")
    p.add_argument("--batches", type=int, default=5)
    p.add_argument("--batch-launches", type=int, default=200,
                   help="launches per timed batch of each kernel")
    p.add_argument("--fused", action="store_true",
                   help="int4 only: one step is a single launch of the fused kernel "
                        "(convrot_w4a4_linear_fused) instead of the two kernels")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = all)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="time the oracle over whole passes until this many seconds")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain device copy of known size (for HBM counter scaling)")
    return p.parse_args()


class Hip:
    """hipEvent* through ctypes on an explicit stream."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        self.lib.hipEventRecord(e, stream)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value


def gpu_bench(args, wl):
    import numpy as np
    import torch

    import workloads as wkmod
    import rotation_w4a4_quantized_convrot_amd as cr

    lib = cr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, K, N, g = wl.M, wl.K, wl.N, wl.g
    Kp = wl.Kp
    tdt = torch.bfloat16 if wl.x_dtype == "bf16" else torch.float32
    x_np = wkmod.activations(wl)
    x0 = torch.from_numpy(x_np).to(tdt).to(dev)
    x_bytes = x0.numel() * x0.element_size()
    n_x = max(2, -(-2 * MALL_BYTES // x_bytes) + 1)
    xs_list = [x0] + [x0.clone() for _ in range(n_x - 1)]
    w = torch.from_numpy(wkmod.weights(wl)).to(tdt).to(dev)
    b = wkmod.bias(wl)
    bias = None if b is None else torch.from_numpy(b).to(torch.bfloat16).to(dev)
    i8, mx = args.codes == "int8", args.codes == "mxfp4"
    qbytes = Kp if i8 else Kp // 2              # code bytes per row
    sbytes = cr.mx_scale_stride(Kp) if mx else 4  # scale bytes per row
    quant_w = (cr.convrot_quant_weight_i8 if i8 else
               cr.convrot_quant_weight_mxfp4 if mx else cr.convrot_quant_weight)
    wq, ws = quant_w(w, g)
    # With few activation rows the GEMM streams the weights: rotate them through copies too,
    # so that they come from HBM rather than from the Infinity Cache.
    w_bytes = wq.numel() * wq.element_size()
    n_w = max(1, -(-2 * MALL_BYTES // w_bytes) + 1) if M <= 512 else 1
    wq_list = [wq] + [wq.clone() for _ in range(n_w - 1)]
    n_y = 4
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(n_y)]
    xq = torch.empty((M, qbytes), dtype=torch.uint8, device=dev)
    xsc = (torch.empty((M, sbytes), dtype=torch.uint8, device=dev) if mx else
           torch.empty((M,), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev).cuda_stream
    dt_code = cr.CONVROT_BF16 if wl.x_dtype == "bf16" else cr.CONVROT_F32
    x_ptrs = [t.data_ptr() for t in xs_list]
    y_ptrs = [t.data_ptr() for t in ys]
    b_ptr = None if bias is None else bias.data_ptr()
    rq, gemm = lib.convrot_rotate_quant_act, lib.convrot_w4a4_gemm
    if i8:
        rq, gemm = lib.convrot_rotate_quant_act_i8, lib.convrot_w8a8_gemm
    if mx:  # the same arguments, block scales in place of row scales
        rq, gemm = lib.convrot_rotate_quant_act_mxfp4, lib.convrot_mxfp4_gemm
    xq_p, xs_p, ws_p = xq.data_ptr(), xsc.data_ptr(), ws.data_ptr()
    wq_ptrs = [t.data_ptr() for t in wq_list]

    def step(i):
        st = rq(x_ptrs[i % n_x], dt_code, M, K, K, g, xq_p, xs_p, None, stream)
        st |= gemm(xq_p, xs_p, wq_ptrs[i % n_w], ws_p, b_ptr, M, N, Kp, y_ptrs[i % n_y], None,
                   stream)
        return st

    if args.fused:
        # one launch per step: the workspace holds the codes and scales; status stays zero
        # unless the kernel's grid barrier times out (checked after the run)
        work = torch.empty((cr.convrot_w4a4_workspace_bytes(M, K, g),), dtype=torch.uint8,
                           device=dev)
        status = torch.zeros((1,), dtype=torch.int32, device=dev)
        work_p, status_p, nbytes = work.data_ptr(), status.data_ptr(), work.numel()
        fused = lib.convrot_w4a4_linear_fused

        def step(i):  # noqa: F811
            return fused(x_ptrs[i % n_x], dt_code, M, K, g, wq_ptrs[i % n_w], ws_p, N, b_ptr,
                         y_ptrs[i % n_y], work_p, nbytes, status_p, stream)
        rq = gemm = None

    hip = Hip()
    e0, e1 = hip.event(), hip.event()

    # Launch duration of each kernel: the kernel alone, launched back to back on the launch
    # stream (the activations still rotate through the HBM-sized buffer set), first for
    # --ramp-seconds of wall time so that the clocks reach the level they hold under
    # sustained load (a GPU coming out of idle runs the first milliseconds slower), then
    # --batches batches of --batch-launches launches with events around each batch.  This
    # does not depend on --steps, and it runs before the steps, which then start warm.
    def batches(fn):
        t_end = time.perf_counter() + args.ramp_seconds
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(50):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        out = []
        for bi in range(args.batches):
            hip.record(e0, stream)
            for j in range(args.batch_launches):
                fn(i + bi * args.batch_launches + j)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            out.append(hip.ms(e0, e1) / args.batch_launches)
        return np.array(out), i

    if args.fused:  # the whole step is one kernel: time it as both
        gemm_ms, gemm_ramp = batches(step)
        rq_ms, rq_ramp = gemm_ms, 0
    else:
        rq_ms, rq_ramp = batches(
            lambda i: rq(x_ptrs[i % n_x], dt_code, M, K, K, g, xq_p, xs_p, None, stream))
        gemm_ms, gemm_ramp = batches(lambda i: gemm(xq_p, xs_p, wq_ptrs[i % n_w], ws_p, b_ptr, M,
                                                    N, Kp, y_ptrs[i % n_y], None, stream))

    for i in range(args.warmup):
        assert step(i) == 0
    torch.cuda.synchronize()

    K_steps = args.steps
    # Timed region: K whole steps back to back, bracketed by a synchronisation on each side
    # (events only at the two ends: an event between kernels costs several microseconds).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, stream)
    for i in range(K_steps):
        step(i)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms_events = hip.ms(e0, e1) / K_steps
    if args.fused:
        assert int(status.item()) == 0, "the fused kernel's grid barrier timed out"
    for x in (e0, e1):
        hip.lib.hipEventDestroy(x)

    copy = None
    if args.copy_calibration:
        # a plain elementwise kernel that reads 256 MiB and writes 256 MiB, for scaling the
        # HBM byte counters (see rotation_w4a4_quantized_convrot_amd/profiling.py)
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        copy = {"bytes_each_way": src.numel() * 4, "launches": 3}

    ms_step = (t1 - t0) * 1e3 / K_steps
    ops = 2.0 * M * N * Kp
    rq_bytes = M * K * x0.element_size() + M * qbytes + M * sbytes
    rq_us = float(np.mean(rq_ms) * 1e3)
    gemm_us = float(np.mean(gemm_ms) * 1e3)
    rq_gbps = rq_bytes / (rq_us * 1e-6) / 1e9
    gemm_tops = ops / (gemm_us * 1e-6) / 1e12
    # GEMM algorithmic bytes: code operands once, scales, bias, bf16 output
    gemm_bytes = ((M + N) * (qbytes + sbytes) + (2 * N if bias is not None else 0)
                  + 2 * M * N)
    return {
        "ms_per_step": ms_step, "ms_per_step_events": step_ms_events,
        "value": ops / (ms_step * 1e-3) / 1e12,
        "rq_us": rq_us, "rq_us_median": float(np.median(rq_ms) * 1e3), "rq_bytes": rq_bytes,
        "rq_gbps": rq_gbps, "gemm_us": gemm_us, "gemm_us_median": float(np.median(gemm_ms) * 1e3),
        "gemm_tops": gemm_tops, "gemm_ops": ops, "gemm_bytes": gemm_bytes,
        "x_buffers": n_x, "x_buffer_bytes": x_bytes * n_x, "w_buffers": n_w,
        "copy_calibration": copy,
        "kernel_timing": {"ramp_seconds": args.ramp_seconds, "ramp_launches_rq": rq_ramp,
                          "ramp_launches_gemm": gemm_ramp, "batches": args.batches,
                          "launches_per_batch": args.batch_launches},
    }


def cpu_baseline(args, wl):
    """The oracle, as it stands, timed on the host: whole passes of the same layer (all rows,
    rotate + quantize, integer GEMM, dequantization) until about --cpu-seconds have passed."""
    import threadpoolctl

    import workloads as wkmod
    from oracle import convrot_oracle as O

    x = wkmod.activations(wl)
    w = wkmod.weights(wl)
    b = wkmod.bias(wl)
    i8, mx = args.codes == "int8", args.codes == "mxfp4"
    quant = (O.rotate_quantize_int8 if i8 else O.rotate_quantize_mxfp4 if mx else
             O.rotate_quantize)
    refw = quant(w, wl.g)                                                   # offline, untimed
    rows = args.cpu_rows or wl.M
    xs = x[:rows]
    passes, t0 = 0, time.perf_counter()
    while True:
        r = quant(xs, wl.g)
        if mx:
            O.mxfp4_linear_from_codes(r["codes"], r["scales"], refw["codes"], refw["scales"], b)
        else:
            lin = O.w8a8_linear_from_codes if i8 else O.w4a4_linear_from_codes
            lin(r["codes"], r["scale"], refw["codes"], refw["scale"], b)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds or passes >= 100:
            break
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    blas = sorted({p.get("internal_api", "?") for p in threadpoolctl.threadpool_info()})
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ops = 2.0 * rows * wl.N * wl.Kp * passes
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "blas": ",".join(blas),
            "sample": f"{passes} passes of the layer on {rows} of {wl.M} rows, all {wl.N} "
                      f"outputs (rotate+quantize, int GEMM, dequant; {dt:.1f} s)",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent: the path would shard by rows, with no communication).", file=sys.stderr)
        sys.exit(2)
    import workloads as wkmod
    wl = wkmod.WORKLOADS[args.workload]
    if wl.N is None:
        raise SystemExit("the benchmark needs a workload with a weight (N)")
    r = gpu_bench(args, wl)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, wl)
    from rotation_w4a4_quantized_convrot_amd import profiling
    i8, mx = args.codes == "int8", args.codes == "mxfp4"
    if args.fused and (i8 or mx):
        raise SystemExit("--fused is the int4 layer only")
    # which GEMM kernel the library picks for this shape (see w4a4_gemm.hip)
    rows16 = i8 or (wl.Kp // 2) % 16 == 0
    if mx:
        gemm_kernel, big = "mxfp4_gemm", True
    elif rows16 and wl.M <= (256 if i8 else 512):
        gemm_kernel, big = "skinny_gemm", False
    elif i8 or (rows16 and wl.M * wl.N >= (1 << 21) and wl.M >= 128):
        gemm_kernel, big = ("w8a8_gemm" if i8 else "w4a4_gemm"), True
    else:
        gemm_kernel, big = "w4a4_gemm_kernel", False
    rq_kernel = "rht_quant_i8" if i8 else "rht_quant_mx4" if mx else "rht_quant_i4"
    if args.fused:
        gemm_kernel, rq_kernel, big = "fused_linear", "fused_linear", False
    mfma_peak = FP4_PEAK_TOPS if mx else INT8_PEAK_TOPS
    traffic_file = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    # the recorded counters are for the attention-projection workload's launches
    profiled = wl.name == "attn_proj"
    tg = profiling.read_traffic(traffic_file, gemm_kernel) if big and profiled else None
    tq = profiling.read_traffic(traffic_file, rq_kernel) if profiled else None
    # The GEMM's binding roof: matrix cores, unless its bytes take longer at the HBM peak
    # than its operations at the matrix peak of its code type (few activation rows).
    if r["gemm_bytes"] / (HBM_PEAK_GBPS * 1e9) > r["gemm_ops"] / (mfma_peak * 1e12):
        roof = {"bound": "hbm", "achieved": r["gemm_bytes"] / (r["gemm_us"] * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": r["gemm_tops"], "peak": mfma_peak,
                "unit": "TFLOP/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"],
                 "traffic": None if tg is None else tg["fetch_bytes"] + tg["write_bytes"],
                 "kernel": gemm_kernel, "launch_us": r["gemm_us"],
                 "launch_us_median": r["gemm_us_median"],
                 "algorithmic_ops_per_launch": r["gemm_ops"],
                 "algorithmic_bytes_per_launch": r["gemm_bytes"]})
    roof_rq = {"bound": "hbm", "achieved": r["rq_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": r["rq_gbps"] / HBM_PEAK_GBPS,
               "traffic": None if tq is None else tq["fetch_bytes"] + tq["write_bytes"],
               "kernel": rq_kernel, "launch_us": r["rq_us"],
               "launch_us_median": r["rq_us_median"],
               "algorithmic_bytes_per_launch": r["rq_bytes"]}
    out = {
        "metric": METRIC_W8A8 if i8 else METRIC_MXFP4 if mx else METRIC, "value": r["value"], "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4" if mx else "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "g": wl.g, "Kp": wl.Kp,
                   "path": "fused single launch" if args.fused else "rotate+quantize, GEMM",
                   "x_dtype": wl.x_dtype, "bias": wl.bias_std is not None,
                   "x_buffers": r["x_buffers"], "w_buffers": r["w_buffers"]},
        "rotate_quant_GBps": r["rq_gbps"], "rotate_quant_us": r["rq_us"],
        "gemm_TOPS": r["gemm_tops"], "gemm_us": r["gemm_us"],
        "roofline": roof, "roofline_rotate_quant": roof_rq, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
