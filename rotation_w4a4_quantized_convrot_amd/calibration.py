"""Matrix-core rates and shader clock of the GPU, measured with libconvrot_calib.so.

``python -m rotation_w4a4_quantized_convrot_amd.calibration [--out FILE]`` runs the
MFMA-only kernels (one instruction in four independent chains per wave, nothing else in
flight), one workgroup per compute unit, each launch about 0.15 s long:
v_mfma_i32_32x32x32_i8 (the int4 and int8 GEMMs) at one, two and four waves per SIMD, and the
E2M1 forms of v_mfma_scale_f32_32x32x64_f8f6f4 (the MXFP4 GEMM) and
v_mfma_scale_f32_16x16x128_f8f6f4 at two, and the int8 instruction again at two with operands
that change every instruction (random full-range int8, and random 16 q as the int4 GEMM feeds
it).  For each it reports:
  * the rate in POP/s (two ops per multiply-accumulate) and its fraction of MI355X's
    published dense peak for that type (int8 5.0 POP/s, fp4 10.1 PFLOP/s);
  * the shader clock while the loop ran: for every workgroup, shader clock cycles
    (s_memtime) over the 100 MHz real-time counter (s_memrealtime) between the same two
    points; median, minimum and maximum over the workgroups.
The published peak assumes 2.4 GHz; at a lower sustained clock the reachable rate scales
with it, which is what the clock column is for.  Needs a GPU; loads only the calibration
library (the oracle and the layer's library are not involved).

``--gemm-tiles`` instead times the layer library's W4A4 GEMM (convrot_w4a4_gemm, the 256 x 256
tiled kernel) at K' = 3072 and output shapes of 64 to 256 tiles, one tile per compute unit,
with codes drawn uniformly from [-7, 7] (the range the quantizer produces): how the time of
one tile, and the chip's aggregate rate, change with the number of compute units at work.

``--reference-gemms`` times, at the attention-projection shape (4608 x 3072 x 3072), the
vendor library's GEMMs next to the layer library's W4A4 GEMM: the int8 GEMM behind
torch._int_mm (int32 output) with operands 16 q (q uniform in [-8, 7], the values the W4A4
GEMM feeds its matrix instruction), full-range int8 and zeros, and the bf16 GEMM x @ w^T.
They are a reference for what the chip sustains on this shape, not part of the layer.

``--reference-copies`` times plain device copies (torch's copy kernel): one moving the bytes
of the attention-projection rotate+quantize (28.3 MB read + 7.1 MB written, here as 17.7 MB
each way), and larger ones, as the practical ceiling of a streaming kernel of that size.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CALIB_PATH = os.path.join(PKG, "libconvrot_calib.so")
PEAK_INT8_POPS = 5.0e15
PEAK_CLOCK_HZ = 2.4e9
# instruction kind -> (name, published dense peak of its type in ops/s)
KINDS = {0: ("i8_32x32x32", 5.0e15), 1: ("fp4_32x32x64_scaled", 10.1e15),
         2: ("fp4_16x16x128_scaled", 10.1e15), 3: ("i8_32x32x32_random_int8", 5.0e15),
         4: ("i8_32x32x32_random_16q", 5.0e15)}
REALTIME_HZ = 100e6


def load() -> ctypes.CDLL:
    if not os.path.exists(CALIB_PATH):
        raise RuntimeError(f"{CALIB_PATH} is not built (python -m "
                           "rotation_w4a4_quantized_convrot_amd.build)")
    lib = ctypes.CDLL(CALIB_PATH)
    lib.convrot_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.convrot_calib_mfma.restype = ctypes.c_int
    lib.convrot_calib_ops_per_inst.argtypes = [ctypes.c_int]
    lib.convrot_calib_ops_per_inst.restype = ctypes.c_int64
    lib.convrot_calib_chains.restype = ctypes.c_int
    return lib


def run(lib, grid: int, block: int, iters: int, kind: int = 0) -> dict:
    """One timed launch; returns its POP/s and the per-workgroup clocks in Hz."""
    import torch
    sink = torch.empty(grid * block, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    rc = lib.convrot_calib_mfma(kind, grid, block, iters, ctypes.c_void_p(sink.data_ptr()),
                                ctypes.c_void_p(clocks.data_ptr()),
                                ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"convrot_calib_mfma failed: hipError {rc}")
    b.record(stream)
    b.synchronize()
    sec = a.elapsed_time(b) / 1e3
    ops = lib.convrot_calib_ops_per_inst(kind) * lib.convrot_calib_chains() * iters * grid * (block // 64)
    c = clocks.view(grid, 4).cpu().tolist()
    hz = [(t1 - t0) / ((r1 - r0) / REALTIME_HZ) for t0, t1, r0, r1 in c if r1 > r0]
    return {"sec": sec, "pops": ops / sec, "sclk_hz": hz}


def measure(target_sec: float = 0.15) -> list:
    import torch
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for kind, waves in ((0, 1), (0, 2), (0, 4), (1, 2), (2, 2), (3, 2), (4, 2)):
        name, peak = KINDS[kind]
        block = 256 * waves
        run(lib, cus, block, 1000, kind)                        # warm-up
        probe = run(lib, cus, block, 20000, kind)
        iters = max(1000, int(20000 * target_sec / probe["sec"]))
        r = run(lib, cus, block, iters, kind)
        hz = r["sclk_hz"]
        out.append({"inst": name, "waves_per_simd": waves, "grid": cus, "block": block,
                    "iters": iters, "ms": r["sec"] * 1e3, "pops": r["pops"],
                    "frac": r["pops"] / peak,
                    "sclk_ghz_median": statistics.median(hz) / 1e9,
                    "sclk_ghz_min": min(hz) / 1e9, "sclk_ghz_max": max(hz) / 1e9})
    return out


# (M, N) at K' = 3072: 64, 144, 216, 224, 255 and 256 tiles of 256 x 256 (attention
# projection, 4608 x 3072, is the 216)
GEMM_TILE_SHAPES = ((2048, 2048), (3072, 3072), (4608, 3072), (4096, 3584), (4352, 3840),
                    (4096, 4096))


def _median_launch_us(fn, launches: int, batches: int, ramp_sec: float) -> float:
    """Median over `batches` of the mean time of `launches` back-to-back calls of `fn`, timed
    with events on the current stream after `ramp_sec` of untimed calls."""
    import time
    import torch
    t0 = time.time()
    while time.time() - t0 < ramp_sec:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    per = []
    for _ in range(batches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(launches):
            fn()
        b.record()
        b.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / launches)
    return statistics.median(per)


def _packed_codes(rows: int, cols: int, gen, lo: int = -7, hi: int = 7):
    """Packed int4 codes (two per byte, column 2j in the low nibble), uniform in [lo, hi]."""
    import torch
    q = torch.randint(lo, hi + 1, (rows, cols), generator=gen, dtype=torch.int16) & 0xF
    return (q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8)


def reference_gemms(M: int = 4608, N: int = 3072, K: int = 3072, launches: int = 200,
                    batches: int = 5, ramp_sec: float = 0.3, seed: int = 0) -> list:
    """Median per-launch time of the vendor int8 and bf16 GEMMs and of convrot_w4a4_gemm at
    one shape, with the rate in POP/s (2 M N K per launch)."""
    import torch
    import rotation_w4a4_quantized_convrot_amd as cr
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(seed)
    out = []

    def add(name, fn):
        us = _median_launch_us(fn, launches, batches, ramp_sec)
        out.append({"gemm": name, "M": M, "N": N, "K": K, "us": us,
                    "pops": 2.0 * M * N * K / (us * 1e-6) / 1e15})

    for data, lo, hi, mul in (("16q", -8, 7, 16), ("int8_full", -128, 127, 1), ("zeros", 0, 0, 1)):
        a = (torch.randint(lo, hi + 1, (M, K), generator=gen, dtype=torch.int32) * mul).to(torch.int8)
        w = (torch.randint(lo, hi + 1, (N, K), generator=gen, dtype=torch.int32) * mul).to(torch.int8)
        a, w = a.to(dev), w.to(dev)
        add(f"vendor_int8_int32out_{data}", lambda a=a, w=w: torch._int_mm(a, w.t()))
    x = torch.randn(M, K, generator=gen).to(torch.bfloat16).to(dev)
    w = torch.randn(N, K, generator=gen).to(torch.bfloat16).to(dev)
    add("vendor_bf16", lambda: x @ w.t())
    xq, wq = _packed_codes(M, K, gen).to(dev), _packed_codes(N, K, gen).to(dev)
    xs = (torch.rand(M, generator=gen) * 1e-2 + 1e-3).to(dev)
    ws = (torch.rand(N, generator=gen) * 1e-2 + 1e-3).to(dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    add("convrot_w4a4_bf16out_codes_-7_7", lambda: cr.convrot_w4a4_gemm(xq, xs, wq, ws, None, y))
    return out


# bytes each way: half the attention projection's rotate+quantize traffic (35,407,872 B),
# 256 MiB and 1 GiB
COPY_SIZES = (17_703_936, 1 << 28, 1 << 30)


def reference_copies(launches: int = 200, batches: int = 5, ramp_sec: float = 0.3) -> list:
    """Median per-launch time of a device-to-device copy of each size in COPY_SIZES (fewer
    launches per batch for the large ones), with the rate over the bytes read plus written.
    Copies smaller than 256 MiB cycle through buffer pairs of at least 600 MB each way, so
    that, as for the benchmark's rotating inputs, the data comes from HBM and not from the
    256 MB Infinity Cache."""
    import torch
    dev = torch.device("cuda:0")
    out = []
    for n in COPY_SIZES:
        pairs = 1 if n >= (1 << 28) else -(-600_000_000 // n)
        src = [torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(pairs)]
        dst = [torch.empty_like(t) for t in src]
        turn = [0]

        def copy():
            i = turn[0] % pairs
            turn[0] += 1
            dst[i].copy_(src[i])

        k = max(5, launches * COPY_SIZES[0] // n)
        us = _median_launch_us(copy, k, batches, ramp_sec)
        out.append({"copy_bytes_each_way": n, "buffer_pairs": pairs, "launches": k, "us": us,
                    "tb_s": 2.0 * n / (us * 1e-6) / 1e12, "frac_of_8tb_s": 2.0 * n / (us * 1e-6) / 8e12})
        del src, dst
    return out


def gemm_tiles(kp: int = 3072, launches: int = 200, batches: int = 5, ramp_sec: float = 0.3,
               seed: int = 0) -> list:
    """Median per-launch time of convrot_w4a4_gemm at GEMM_TILE_SHAPES (back-to-back launches
    after a ramp), with the aggregate rate in POP/s."""
    import torch
    import rotation_w4a4_quantized_convrot_amd as cr
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(seed)
    out = []
    for M, N in GEMM_TILE_SHAPES:
        xq, wq = _packed_codes(M, kp, gen).to(dev), _packed_codes(N, kp, gen).to(dev)
        xs = (torch.rand(M, generator=gen) * 1e-2 + 1e-3).to(dev)
        ws = (torch.rand(N, generator=gen) * 1e-2 + 1e-3).to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        us = _median_launch_us(lambda: cr.convrot_w4a4_gemm(xq, xs, wq, ws, None, y),
                               launches, batches, ramp_sec)
        tiles = -(-M // 256) * -(-N // 256)
        out.append({"M": M, "N": N, "Kp": kp, "tiles": tiles, "us": us,
                    "pops": 2.0 * M * N * kp / (us * 1e-6) / 1e15})
    return out


def main(argv=None) -> int:
    p = argparse.ArgumentParser()
    p.add_argument("--out", default=None, help="write the summary here as well")
    p.add_argument("--command", default=None, help="the command line to record in the summary")
    p.add_argument("--gemm-tiles", action="store_true",
                   help="time the W4A4 GEMM at 64 to 256 tiles instead (layer library)")
    p.add_argument("--reference-gemms", action="store_true",
                   help="time the vendor int8 and bf16 GEMMs and the W4A4 GEMM at 4608 x 3072 x 3072")
    p.add_argument("--reference-copies", action="store_true",
                   help="time plain device copies of the rotate+quantize bytes and larger")
    a = p.parse_args(argv)
    if a.command is None:
        a.command = "python -m rotation_w4a4_quantized_convrot_amd.calibration" + (
            " --gemm-tiles" if a.gemm_tiles else "") + (
            " --reference-gemms" if a.reference_gemms else "") + (
            " --reference-copies" if a.reference_copies else "")
    import torch
    name = torch.cuda.get_device_properties(0).name
    if a.reference_copies:
        rows = reference_copies()
        lines = ["# device-to-device copies (torch's copy kernel): median per-launch time of 5 "
                 "batches of back-to-back launches; tb_s = (bytes read + bytes written) / time",
                 f"# command (repository root): {a.command}",
                 f"device={name}; cus={torch.cuda.get_device_properties(0).multi_processor_count}"]
    elif a.reference_gemms:
        rows = reference_gemms()
        lines = ["# GEMMs at 4608 x 3072 x 3072 (attention projection): the vendor library's int8 "
                 "(torch._int_mm, int32 output) and bf16 (x @ w^T) GEMMs and convrot_w4a4_gemm "
                 "(int4 codes, bf16 output with the dequantization epilogue); median per-launch "
                 "time of 5 batches of 200 back-to-back launches; pops = 2 M N K / time",
                 f"# command (repository root): {a.command}",
                 f"device={name}; cus={torch.cuda.get_device_properties(0).multi_processor_count}"]
    elif a.gemm_tiles:
        rows = gemm_tiles()
        lines = ["# W4A4 GEMM (256 x 256 tiles, one per CU) at K' = 3072, codes uniform in "
                 "[-7, 7]: median per-launch time of 5 batches of 200 back-to-back launches",
                 f"# command (repository root): {a.command}",
                 f"device={name}; cus={torch.cuda.get_device_properties(0).multi_processor_count}"]
    else:
        rows = measure()
        lines = ["# MFMA-only rates (4 independent chains per wave, one workgroup per CU) and "
                 "the shader clock under them",
                 "# sclk = s_memtime cycles / s_memrealtime (100 MHz) per workgroup; frac = "
                 "rate / published dense peak of the type at 2.4 GHz (int8 5.0e15, fp4 10.1e15)",
                 f"# command (repository root): {a.command}",
                 f"device={name}; cus={rows[0]['grid']}"]
    for r in rows:
        lines.append("; ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                               for k, v in r.items()))
    text = "\n".join(lines) + "\n"
    print(text, end="")
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
