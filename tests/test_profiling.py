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


GEMM = "void convrot::(anonymous namespace)::big::quant_gemm_kernel<false, 4, false>(...)"
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


def _write_multi(d, stem, rows):
    """rows: (dispatch id, kernel name, {counter: value})."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"{stem}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, counters in rows:
            for c, v in counters.items():
                w.writerow({"Correlation_Id": disp, "Dispatch_Id": disp, "Kernel_Name": name,
                            "Grid_Size": 1, "Counter_Name": c, "Counter_Value": v})


RQ = "void convrot::(anonymous namespace)::rht_quant_kernel<256, unsigned short, 16, 4, 16>(...)"


def test_counter_summary_derivations(tmp_path):
    M, N, Kp = 256, 128, 512
    mfma = (M // 32) * (N // 32) * (Kp // 32)         # 512 instructions
    gemm = {"SQ_INSTS_MFMA": mfma, "SQ_VALU_MFMA_BUSY_CYCLES": 32 * mfma, "GRBM_GUI_ACTIVE": 10}
    _write_multi(tmp_path / "pmc", "bench", [
        (1, GEMM, {k: 7 * v for k, v in gemm.items()}),   # cold first dispatch: left out
        (2, GEMM, gemm), (3, GEMM, gemm),
        (4, RQ, {"SQ_INSTS_VALU": 2 * M * Kp // 64, "SQ_INSTS_SALU": M * Kp // 64}),
        (5, RQ, {"SQ_INSTS_VALU": 2 * M * Kp // 64, "SQ_INSTS_SALU": M * Kp // 64})])
    # calibration: three launches of the int8 loop with fixed operands, the counters of the
    # largest one taken, and a larger launch of another kind (scaled FP4), which is not
    loop = "void (anonymous namespace)::mfma_loop<{}>(int, int*, unsigned long*)"
    _write_multi(tmp_path / "cal", "calib", [
        (1, loop.format(0), {"SQ_INSTS_MFMA": 10, "SQ_VALU_MFMA_BUSY_CYCLES": 999}),
        (2, loop.format(0), {"SQ_INSTS_MFMA": 1000, "SQ_VALU_MFMA_BUSY_CYCLES": 32000}),
        (3, loop.format(0), {"SQ_INSTS_MFMA": 100, "SQ_VALU_MFMA_BUSY_CYCLES": 1}),
        (4, loop.format(1), {"SQ_INSTS_MFMA": 5000, "SQ_VALU_MFMA_BUSY_CYCLES": 7})])
    stats = tmp_path / "bench_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        # 2 M N K' ops in 1 us: 33.55 TOPS; the GEMM at a quarter of a 134.2 TOPS MFMA-only rate
        w.writerow({"Name": GEMM, "Calls": 2, "TotalDurationNs": 2000, "AverageNs": 1000,
                    "Percentage": 50, "MinNs": 1000, "MaxNs": 1000, "StdDev": 0})
        # 256 CUs x 2 us x 2 GHz = 1024000 CU cycles
        w.writerow({"Name": RQ, "Calls": 2, "TotalDurationNs": 4000, "AverageNs": 2000,
                    "Percentage": 50, "MinNs": 2000, "MaxNs": 2000, "StdDev": 0})
    cal_txt = tmp_path / "mfma_peak_sclk.txt"
    ops = 2 * M * N * Kp / 1e-6
    cal_txt.write_text("# header\ndevice=x; cus=256\n"
                       "inst=i8_32x32x32; waves_per_simd=1; pops=1e15; sclk_ghz_median=1.5\n"
                       f"inst=i8_32x32x32; waves_per_simd=2; pops={4 * ops}; sclk_ghz_median=2.0\n"
                       "inst=fp4_32x32x64_scaled; waves_per_simd=2; pops=1e12; sclk_ghz_median=1.0\n")
    lines = P.counter_summary([str(tmp_path / "pmc")], [str(tmp_path / "cal")], str(stats),
                              str(cal_txt), M, N, Kp, 256)
    text = "\n".join(lines)
    assert f"mfma_insts={mfma} expected={mfma}" in text
    assert "derived w4a4_gemm mfma_busy_cycles_per_mfma=32" in text
    assert "derived mfma_only mfma_busy_cycles_per_mfma=32" in text     # dispatch 2 chosen
    assert "mfma_busy_fraction=0.2500" in text
    assert "SQ_INSTS_VALU_per_element=2 " in text and "SQ_INSTS_SALU_per_element=1 " in text
    valu = 2 * M * Kp // 64
    assert f"valu_issue_fraction={valu / 1024000:.4f}" in text


def test_read_calibration(tmp_path):
    p = tmp_path / "c.txt"
    p.write_text("# x\ndevice=d; cus=256\n"
                 "inst=i8_32x32x32; waves_per_simd=2; grid=256; pops=4.9e+15; sclk_ghz_median=2.38\n"
                 "inst=fp4_32x32x64_scaled; waves_per_simd=2; grid=256; pops=7e+15; sclk_ghz_median=2.1\n")
    c = P.read_calibration(str(p))
    assert set(c) == {2} and c[2]["pops"] == 4.9e15 and c[2]["sclk_ghz_median"] == 2.38
    f = P.read_calibration(str(p), "fp4_32x32x64_scaled")
    assert f[2]["pops"] == 7e15


def test_source_hash_covers_device_headers():
    """A kernel's fingerprint changes with the header holding its body, not only its .hip."""
    one = P.source_sha256("w4a4_gemm.hip")
    both = P.source_sha256(P.GEMM_SRC)
    assert one != both and len(both) == 64
    assert P.KERNELS["w4a4_gemm"][1] == P.GEMM_SRC and "gemm_device.h" in P.GEMM_SRC
    assert "rht_quant_device.h" in P.RQ_SRC
