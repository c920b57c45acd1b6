"""Host-side checks of the rocprofv3 summary helpers (no GPU, synthetic CSV files)."""
import csv
import os

import pytest

from rotation_w4a4_quantized_convrot_amd import profiling as P

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
          "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "bench_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, val) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                        "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": val})


GEMM = "void convrot::(anonymous namespace)::big::quant_gemm_kernel<false, 4>(...)"
CAL = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<...>>"


def test_traffic_scaling_and_staleness(tmp_path):
    # the calibration copy reads half of its 256 MiB according to the counter: scale 2
    _write(tmp_path / "f", "FETCH_SIZE", [(GEMM, 55296, 999.0), (GEMM, 55296, 100.0),
                                          (GEMM, 55296, 100.0), (CAL, 262144, 131072.0),
                                          (CAL, 1024, 5.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(GEMM, 55296, 50.0), (GEMM, 55296, 50.0),
                                          (CAL, 262144, 262144.0)])
    t = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    g = t["w4a4_gemm"]
    assert g["fetch_scale"] == pytest.approx(2.0) and g["write_scale"] == pytest.approx(1.0)
    assert g["fetch_bytes"] == pytest.approx(100.0 * 1024 * 2)    # first (cold) dispatch left out
    assert g["write_bytes"] == pytest.approx(50.0 * 1024)
    out = tmp_path / "traffic.txt"
    P.write_traffic(str(out), t, "cmd")
    r = P.read_traffic(str(out), "w4a4_gemm")
    assert r == {"fetch_bytes": pytest.approx(204800.0), "write_bytes": pytest.approx(51200.0)}
    # a different source hash means the kernel changed since: no traffic figure
    text = out.read_text().replace(g["source_sha256"], "0" * 64)
    out.write_text(text)
    assert P.read_traffic(str(out), "w4a4_gemm") is None
    assert P.read_traffic(str(tmp_path / "missing.txt"), "w4a4_gemm") is None


def test_calibration_required(tmp_path):
    _write(tmp_path / "f", "FETCH_SIZE", [(GEMM, 55296, 1.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(GEMM, 55296, 1.0)])
    with pytest.raises(ValueError):
        P.traffic(str(tmp_path / "f"), str(tmp_path / "w"))


def test_trace_batches_picks_longest_back_to_back_run(tmp_path):
    p = tmp_path / "bench_kernel_trace.csv"
    rows, t = [], 0
    def add(name, dur_ns):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur_ns})
        t += dur_ns + 100
    for _ in range(3):                       # interleaved steps
        add("A", 5000)
        add("B", 9000)
    for _ in range(10):                      # A alone: 10 back to back
        add("A", 2000)
    for _ in range(4):
        add("B", 7000)
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    got = {r["name"]: r for r in P.trace_batches(str(p), 5)}
    assert got["A"]["run"] == 10 and got["A"]["n"] == 5 and got["A"]["avg_us"] == 2.0
    assert got["B"]["run"] == 4 and got["B"]["avg_us"] == 7.0
