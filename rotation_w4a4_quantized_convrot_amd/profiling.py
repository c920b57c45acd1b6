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
    SHA-256 of each kernel's source file, so a reader (bench.py) can tell whether the
    kernel has changed since the counters were taken.

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

# kernel key -> (substring of the demangled name, source file under csrc/)
KERNELS = {
    "w4a4_gemm": ("quant_gemm_kernel<false, 4>", "w4a4_gemm.hip"),
    "w8a8_gemm": ("quant_gemm_kernel<false, 8>", "w4a4_gemm.hip"),
    "rht_quant_i4": ("rht_quant_kernel<256, unsigned short, 16, 4", "rht_quant.hip"),
    "rht_quant_i8": ("rht_quant_kernel<256, unsigned short, 16, 8", "rht_quant.hip"),
    "rht_quant_mx4": ("rht_quant_kernel<256, unsigned short, 16, 1", "rht_quant.hip"),
    "mxfp4_gemm": ("quant_gemm_kernel<false, 1>", "w4a4_gemm.hip"),
}


def source_sha256(src: str) -> str:
    with open(os.path.join(PKG, "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    a = p.parse_args(argv)
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
