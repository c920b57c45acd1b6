"""The MFMA-only calibration kernel (needs a gfx950 GPU): a short launch returns a positive
rate below the published int8 peak scaled to its clock, and a shader clock between 0.5 and
3 GHz in every workgroup."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_calibration_kernel_rate_and_clock():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    lib = C.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"\n[case] calibration grid={cus} block=512 iters=20000", flush=True)
    C.run(lib, cus, 512, 1000)
    r = C.run(lib, cus, 512, 20000)
    assert len(r["sclk_hz"]) == cus
    assert all(0.5e9 < hz < 3.0e9 for hz in r["sclk_hz"]), r["sclk_hz"][:8]
    clock = sorted(r["sclk_hz"])[cus // 2]
    # the published 5.0 POP/s is at 2.4 GHz; nothing can exceed it at the measured clock
    # (plus 5% for the launch-time spread between workgroups)
    assert 0 < r["pops"] <= 1.05 * C.PEAK_INT8_POPS * clock / C.PEAK_CLOCK_HZ
