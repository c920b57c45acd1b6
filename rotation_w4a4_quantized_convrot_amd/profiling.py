"""Summaries of rocprofv3 CSV output for the two kernels of the layer.

Two uses:
  * ``python -m rotation_w4a4_quantized_convrot_amd.profiling stats <kernel_stats.csv>``
    prints the per-kernel duration table of a ``--kernel-trace --stats`` run, and
    ``... trace <kernel_trace.csv> --last N`` the average over each kernel's last N
    dispatches, and ``... batches <kernel_trace.csv> --last N`` the average over the last N
    dispatches of each kernel's longest back-to-back run (bench.py's timed batches).
  * ``python -m rotation_w4a4_quantized_convrot_amd.profiling traffic --fetch <dir>
    --write <dir> --out <file> --command <text>`` turns two ``--pmc FETCH_SIZE`` /
    ``--pmc WRITE_SIZE`` runs of ``bench.py --copy-calibration`` into HBM bytes per launch.
    Each counter is scaled by what it reads for a plain elementwise copy of known size
    (256 MiB read, 256 MiB written) run in the same process.  The summary records the
    SHA-256 of each kernel's source files, so a reader (bench.py) can tell whether the
    kernel has changed since the counters were taken.
  * ``python -m rotation_w4a4_quantized_convrot_amd.profiling counters --pmc <dir> ...
    --stats <kernel_stats.csv> --out <file>`` summarises ``--pmc`` runs of bench.py and of
    the MFMA-only calibration kernel (calibration.py): per-dispatch counter values of the
    GEMM, the rotate+quantize kernel and the calibration kernel, and what follows from them
    (matrix-core busy fraction relative to the MFMA-only kernel, MFMA instructions against
    the count the tile shape implies, VALU / SALU / LDS instructions per element).

Nothing here touches the GPU; it only reads files.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys
from typing import Dict, List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_BYTES = 256 << 20          # bench.py --copy-calibration: bytes read and written

# The files a kernel's device code comes from (the kernel source and the headers holding its
# body), hashed together.
GEMM_SRC = ("w4a4_gemm.hip", "gemm_device.h", "convrot_internal.h")
RQ_SRC = ("rht_quant.hip", "rht_quant_device.h", "convrot_internal.h")

# kernel key -> (substring of the demangled name, source files under csrc/)
KERNELS = {
    "w4a4_gemm": ("quant_gemm_kernel<false, 4, false>", GEMM_SRC),
    "w8a8_gemm": ("quant_gemm_kernel<false, 8, false>", GEMM_SRC),
    "rht_quant_i4": ("rht_quant_kernel<256, unsigned short, 16, 4", RQ_SRC),
    "rht_quant_i8": ("rht_quant_kernel<256, unsigned short, 16, 8", RQ_SRC),
    "rht_quant_mx4": ("rht_quant_kernel<256, unsigned short, 16, 1", RQ_SRC),
    "mxfp4_gemm": ("quant_gemm_kernel<false, 1, false>", GEMM_SRC),
}
# calibration.py's int8 MFMA loop with fixed operands (kind 0)
CALIB_KERNEL = "mfma_loop<0>("


def source_sha256(src) -> str:
    """SHA-256 of one source file under csrc/, or of several concatenated in order."""
    h = hashlib.sha256()
    for name in ((src,) if isinstance(src, str) else src):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(path: str) -> List[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counter_file(d: str) -> str:
    for name in sorted(os.listdir(d)):
        if name.endswith("counter_collection.csv"):
            return os.path.join(d, name)
    raise FileNotFoundError(f"no *counter_collection.csv under {d}")


def per_launch(rows: List[dict], needle: str) -> Optional[float]:
    """Median counter value (KiB) over the dispatches of the kernel whose name contains
    `needle`, the first dispatch (cold caches) left out when there are several."""
    vals = [float(r["Counter_Value"]) for r in rows if needle in r["Kernel_Name"]]
    if len(vals) > 1:
        vals = vals[1:]
    return statistics.median(vals) if vals else None


def calibration_kib(rows: List[dict]) -> float:
    """Counter value (KiB) of the calibration copy: the elementwise kernel with the largest
    grid (torch's multiply-by-one over 64 Mi floats)."""
    cand = [r for r in rows if "elementwise" in r["Kernel_Name"]]
    if not cand:
        raise ValueError("calibration kernel not found (run bench.py with --copy-calibration)")
    g = max(int(r["Grid_Size"]) for r in cand)
    return statistics.median(float(r["Counter_Value"]) for r in cand if int(r["Grid_Size"]) == g)


def traffic(fetch_dir, write_dir) -> Dict[str, dict]:
    """Per-launch HBM bytes of each known kernel.  fetch_dir / write_dir may be lists of
    paired runs (say one per code width); each pair is calibrated by its own copy kernel."""
    if not isinstance(fetch_dir, str):
        out = {}
        for f, w in zip(fetch_dir, write_dir):
            out.update(traffic(f, w))
        return out
    fr, wr = _rows(_counter_file(fetch_dir)), _rows(_counter_file(write_dir))
    f_cal, w_cal = calibration_kib(fr), calibration_kib(wr)
    f_scale = CALIBRATION_BYTES / (f_cal * 1024.0)
    w_scale = CALIBRATION_BYTES / (w_cal * 1024.0)
    out = {}
    for key, (needle, src) in KERNELS.items():
        fk, wk = per_launch(fr, needle), per_launch(wr, needle)
        if fk is None or wk is None:
            continue
        out[key] = {
            "fetch_kib": fk, "write_kib": wk, "fetch_scale": f_scale, "write_scale": w_scale,
            "fetch_bytes": fk * 1024.0 * f_scale, "write_bytes": wk * 1024.0 * w_scale,
            "source_sha256": source_sha256(src),
        }
    return out


def write_traffic(out_path: str, table: Dict[str, dict], command: str) -> None:
    lines = ["# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
             "# each scaled by its reading for a 256 MiB elementwise copy in the same run.",
             f"# command: {command}"]
    for key, d in table.items():
        fields = "; ".join(f"{k}={v}" for k, v in d.items())
        lines.append(f"kernel={key}; {fields}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str, key: str) -> Optional[dict]:
    """The recorded traffic of `key`, or None when absent or when the kernel's source has
    changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if not line.startswith(f"kernel={key};"):
                continue
            d = {}
            for part in line.strip().split("; "):
                k, _, v = part.partition("=")
                d[k] = v
            src = KERNELS[key][1]
            if d.get("source_sha256") != source_sha256(src):
                return None
            return {"fetch_bytes": float(d["fetch_bytes"]), "write_bytes": float(d["write_bytes"])}
    return None


def counter_medians(dirs: List[str], needle: str) -> Dict[str, float]:
    """Median per-dispatch value of every counter in the ``--pmc`` runs under `dirs`, over the
    dispatches of the kernel whose name contains `needle` (the first dispatch of each run,
    with cold caches, left out when there are several)."""
    out: Dict[str, float] = {}
    for d in dirs:
        per: Dict[str, List[float]] = {}
        for r in _rows(_counter_file(d)):
            if needle in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for name, vals in per.items():
            out[name] = statistics.median(vals[1:] if len(vals) > 1 else vals)
    return out


def counters_of_largest(dirs: List[str], needle: str, by: str) -> Dict[str, float]:
    """Every counter of the one dispatch (per run) of the kernel whose name contains `needle`
    with the largest value of counter `by` (calibration.py's timed launch of its last
    configuration is the longest one)."""
    out: Dict[str, float] = {}
    for d in dirs:
        per: Dict[str, Dict[str, float]] = {}
        for r in _rows(_counter_file(d)):
            if needle in r["Kernel_Name"]:
                per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        if per:
            out.update(max(per.values(), key=lambda c: c.get(by, 0.0)))
    return out


def read_calibration(path: str, inst: str = "i8_32x32x32") -> Dict[int, dict]:
    """calibration.py's summary for one instruction: waves per SIMD -> {pops, sclk_ghz_median,
    ...}."""
    out = {}
    with open(path) as f:
        for line in f:
            if not line.startswith(f"inst={inst};"):
                continue
            d = {}
            for part in line.strip().split("; ")[1:]:
                k, _, v = part.partition("=")
                d[k] = float(v)
            out[int(d["waves_per_simd"])] = d
    return out


def counter_summary(pmc_dirs: List[str], calib_dirs: List[str], stats_csv: str,
                    calib_txt: str, M: int, N: int, Kp: int, cus: int) -> List[str]:
    """Text lines: raw counter values per kernel and what follows from them."""
    gemm = counter_medians(pmc_dirs, KERNELS["w4a4_gemm"][0])
    rq = counter_medians(pmc_dirs, KERNELS["rht_quant_i4"][0])
    cal = counters_of_largest(calib_dirs, CALIB_KERNEL, "SQ_INSTS_MFMA")
    peak = read_calibration(calib_txt)[2]          # two waves per SIMD, as the GEMM runs
    dur = {}
    for r in kernel_stats(stats_csv):
        for key in ("w4a4_gemm", "rht_quant_i4"):
            if KERNELS[key][0] in r["name"]:
                dur[key] = r["avg_us"]
    lines = []
    for label, d in (("w4a4_gemm", gemm), ("rht_quant_i4", rq), ("mfma_only", cal)):
        lines.append(f"raw kernel={label}; " + "; ".join(f"{k}={v:.6g}" for k, v in sorted(d.items())))
    lines.append(f"calibration (2 waves per SIMD): MFMA-only {peak['pops'] / 1e15:.4g} POP/s at "
                 f"sclk {peak['sclk_ghz_median']:.4g} GHz (median over workgroups)")
    if "SQ_INSTS_MFMA" in gemm:
        expect = (-(-M // 32)) * (-(-N // 32)) * (Kp // 32)
        lines.append(f"derived w4a4_gemm mfma_insts={gemm['SQ_INSTS_MFMA']:.7g} expected={expect} "
                     "(one v_mfma_i32_32x32x32_i8 per 32x32 output block per 32 codes of K')")
    for label, d in (("w4a4_gemm", gemm), ("mfma_only", cal)):
        if d.get("SQ_INSTS_MFMA"):
            lines.append(f"derived {label} mfma_busy_cycles_per_mfma="
                         f"{d['SQ_VALU_MFMA_BUSY_CYCLES'] / d['SQ_INSTS_MFMA']:.4g}")
    lines.append("note: SQ_VALU_MFMA_BUSY_CYCLES adds the same fixed amount per instruction in both "
                 "kernels, so it counts instructions, not time; the matrix cores' busy fraction is "
                 "the achieved rate over the MFMA-only rate at the same occupancy")
    if "w4a4_gemm" in dur:
        pops = 2.0 * M * N * Kp / (dur["w4a4_gemm"] * 1e-6)
        lines.append(f"derived w4a4_gemm kernel_us={dur['w4a4_gemm']:.4g} pops={pops / 1e15:.4g} "
                     f"mfma_busy_fraction={pops / peak['pops']:.4f} (of the MFMA-only rate) "
                     f"frac_of_published={pops / 5.0e15:.4f}")
    elems = M * Kp
    for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
              "SQ_INSTS_VMEM_WR", "SQ_INSTS_BRANCH"):
        if c in rq:
            lines.append(f"derived rht_quant_i4 {c}_per_element={rq[c] * 64 / elems:.4g} "
                         f"(wave instructions x 64 lanes / (M x K' = {elems}))")
    if "rht_quant_i4" in dur and rq.get("SQ_INSTS_VALU"):
        # 16-lane SIMDs: a wave64 VALU instruction holds its SIMD four cycles, so a CU issues at
        # most one per cycle
        cyc = cus * dur["rht_quant_i4"] * 1e-6 * peak["sclk_ghz_median"] * 1e9
        lines.append(f"derived rht_quant_i4 kernel_us={dur['rht_quant_i4']:.4g} "
                     f"valu_issue_fraction={rq['SQ_INSTS_VALU'] / cyc:.4f} (VALU instructions over "
                     "CU cycles at the calibrated clock; one wave64 VALU instruction per CU per "
                     "cycle at most)")
    return lines


def kernel_stats(path: str) -> List[dict]:
    out = []
    for r in _rows(path):
        out.append({"name": r["Name"], "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def trace_tail(path: str, last: int) -> List[dict]:
    """Average duration of the last `last` dispatches of each kernel in a kernel-trace CSV
    (bench.py ends with batches of back-to-back launches of each kernel)."""
    per = {}
    for r in _rows(path):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = []
    for name, v in per.items():
        v.sort()
        tail = [d for _, d in v[-last:]]
        out.append({"name": name, "n": len(tail), "avg_us": statistics.mean(tail),
                    "median_us": statistics.median(tail)})
    return out


def trace_batches(path: str, last: int) -> List[dict]:
    """Average duration of the last `last` dispatches of each kernel's longest run of
    consecutive dispatches (no other kernel in between): bench.py's back-to-back batches of
    that kernel alone, wherever they sit in the trace."""
    rows = []
    for r in _rows(path):
        rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    best: Dict[str, List[float]] = {}
    cur_name, cur = None, []
    for _, name, dur in rows + [(0, None, 0.0)]:
        if name != cur_name:
            if cur_name is not None and len(cur) > len(best.get(cur_name, [])):
                best[cur_name] = cur
            cur_name, cur = name, []
        cur.append(dur)
    out = []
    for name, v in best.items():
        tail = v[-last:]
        out.append({"name": name, "n": len(tail), "run": len(v), "avg_us": statistics.mean(tail),
                    "median_us": statistics.median(tail)})
    return out


def main(argv=None) -> int:
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    tt = sub.add_parser("trace")
    tt.add_argument("csv")
    tt.add_argument("--last", type=int, required=True)
    tb = sub.add_parser("batches")
    tb.add_argument("csv")
    tb.add_argument("--last", type=int, required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True, nargs="+")
    t.add_argument("--write", required=True, nargs="+")
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="")
    c = sub.add_parser("counters")
    c.add_argument("--pmc", required=True, nargs="+", help="--pmc runs of bench.py")
    c.add_argument("--calib", required=True, nargs="+", help="--pmc runs of calibration.py")
    c.add_argument("--stats", required=True, help="kernel_stats.csv of the bench command")
    c.add_argument("--calibration", required=True, help="calibration.py's summary file")
    c.add_argument("--M", type=int, default=4608)
    c.add_argument("--N", type=int, default=3072)
    c.add_argument("--Kp", type=int, default=3072)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--out", required=True)
    c.add_argument("--command", default="")
    a = p.parse_args(argv)
    if a.cmd == "counters":
        lines = ["# Hardware counters per dispatch (rocprofv3 --pmc, median over dispatches), "
                 f"W4A4 layer M={a.M} N={a.N} K'={a.Kp}, and the MFMA-only calibration kernel",
                 f"# command: {a.command}"]
        lines += counter_summary(a.pmc, a.calib, a.stats, a.calibration, a.M, a.N, a.Kp, a.cus)
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return 0
    if a.cmd == "stats":
        for r in kernel_stats(a.csv):
            print(f"{r['calls']:6d} calls  avg {r['avg_us']:9.2f} us  min {r['min_us']:9.2f}  "
                  f"max {r['max_us']:9.2f}  {r['pct']:6.2f}%  {r['name'][:110]}")
        return 0
    if a.cmd == "trace":
        for r in trace_tail(a.csv, a.last):
            print(f"{r['n']:6d} last launches  avg {r['avg_us']:9.2f} us  median "
                  f"{r['median_us']:9.2f} us  {r['name'][:110]}")
        return 0
    if a.cmd == "batches":
        for r in trace_batches(a.csv, a.last):
            print(f"{r['n']:6d} of {r['run']:6d} back-to-back  avg {r['avg_us']:9.2f} us  median "
                  f"{r['median_us']:9.2f} us  {r['name'][:110]}")
        return 0
    table = traffic(a.fetch, a.write)
    write_traffic(a.out, table, a.command)
    for k, d in table.items():
        print(f"{k}: fetch {d['fetch_bytes'] / 1e6:.2f} MB, write {d['write_bytes'] / 1e6:.2f} MB "
              f"(scales {d['fetch_scale']:.3f}, {d['write_scale']:.3f})")
    return 0


if __name__ == "__main__":
    sys.exit(main())
