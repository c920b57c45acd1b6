"""The MFMA-only calibration kernel (needs a gfx950 GPU): a short launch returns a positive
rate below the published int8 peak scaled to its clock, and a shader clock between 0.5 and
3 GHz in every workgroup."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_calibration_kernel_rate_and_clock(kind):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    lib = C.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"\n[case] calibration kind={kind} grid={cus} block=512 iters=20000", flush=True)
    C.run(lib, cus, 512, 1000, kind)
    r = C.run(lib, cus, 512, 20000, kind)
    assert len(r["sclk_hz"]) == cus
    assert all(0.5e9 < hz < 3.0e9 for hz in r["sclk_hz"]), r["sclk_hz"][:8]
    clock = sorted(r["sclk_hz"])[cus // 2]
    # the published peak of the type is at 2.4 GHz; nothing can exceed it at the measured
    # clock (plus 5% for the launch-time spread between workgroups)
    peak = C.KINDS[kind][1]
    assert 0 < r["pops"] <= 1.05 * peak * clock / C.PEAK_CLOCK_HZ


def test_gemm_tiles_mode():
    """The GEMM tile-count timing: one row per shape, tile counts as stated, rates below the
    published int8 peak."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    print("\n[case] calibration gemm_tiles launches=5 batches=1", flush=True)
    rows = C.gemm_tiles(launches=5, batches=1, ramp_sec=0.01)
    assert [r["tiles"] for r in rows] == [64, 144, 216, 224, 255, 256]
    assert all(r["us"] > 0 and 0 < r["pops"] < C.PEAK_INT8_POPS / 1e15 for r in rows)


def test_reference_gemms_mode():
    """The reference GEMM timing: one row per GEMM, positive times, rates below the published
    peak of the GEMM's type (int8 5.0 POP/s, bf16 2.5 PFLOP/s)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    print("\n[case] calibration reference_gemms launches=5 batches=1", flush=True)
    rows = C.reference_gemms(launches=5, batches=1, ramp_sec=0.01)
    assert [r["gemm"] for r in rows] == [
        "vendor_int8_int32out_16q", "vendor_int8_int32out_int8_full", "vendor_int8_int32out_zeros",
        "vendor_bf16", "convrot_w4a4_bf16out_codes_-7_7"]
    for r in rows:
        peak = 2.5 if r["gemm"] == "vendor_bf16" else C.PEAK_INT8_POPS / 1e15
        assert r["us"] > 0 and 0 < r["pops"] < peak, r


def test_reference_copies_mode():
    """The reference copies: one row per size, rates below the published 8 TB/s."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    print("\n[case] calibration reference_copies launches=5 batches=1", flush=True)
    rows = C.reference_copies(launches=5, batches=1, ramp_sec=0.01)
    assert [r["copy_bytes_each_way"] for r in rows] == list(C.COPY_SIZES)
    assert all(r["us"] > 0 and 0 < r["tb_s"] < 8.0 for r in rows), rows
