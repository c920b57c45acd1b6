"""Full-size parity of the W8A8 and MXFP4 layers (needs a gfx950 GPU).

The int4 layer has the same check in test_gpu_parity.py.  Here every workload runs at its full
size, in the launch configuration the benchmark times with --codes int8 / mxfp4:
  * activation codes and scales of every row, and of every weight row, to the format's bars
    (test_gpu_w8a8.check_i8, test_gpu_mxfp4.check_mx);
  * the output rows (all of them for the attention projection, the padded proj_out variant
    and few tokens; a sample including every outlier row it picks for the MLP
    down-projection and the batch-2 proj_out) equal the GEMM of the GPU's own codes: bit for
    bit for int8, >= 99% of the bf16 outputs for MXFP4, whose sums are fp32;
  * with the oracle's own codes, the same output rows within 1e-2 relative Frobenius error.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O
from tests.test_gpu_mxfp4 import check_mx
from tests.test_gpu_parity import output_rows
from tests.test_gpu_w8a8 import check_i8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUT_FROB_MAX = 1e-2
FULL = ["rotate_quant", "attn_proj", "mlp_down", "proj_out", "proj_out_padded", "few_tokens"]


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


def _to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(DEV)


def _frob(y_bits, ref_bits):
    yo = O.bf16_bits_to_f32(ref_bits).astype(np.float64)
    yg = O.bf16_bits_to_f32(y_bits).astype(np.float64)
    return np.linalg.norm(yg - yo) / np.linalg.norm(yo)


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_w8a8_full_size(cr, name):
    wl = wk.WORKLOADS[name]
    print(f"\n[case] int8 full size {name}: M={wl.M} K={wl.K} N={wl.N} g={wl.g}", flush=True)
    x = wk.activations(wl)
    xd = _to_dev(x, wl.x_dtype)
    if wl.N is None:
        xq, xs, xr = cr.convrot_rotate_quant_act_i8(xd, wl.g, want_rotated=True)
        torch.cuda.synchronize()
        check_i8(xq, xs, xr, O.rotate_quantize_int8(x, wl.g), name)
        return
    w, b = wk.weights(wl), wk.bias(wl)
    wq, ws = cr.convrot_quant_weight_i8(_to_dev(w, wl.x_dtype), wl.g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_w8a8_linear(xd, wl.g, wq, ws, bias)
    xq, xs = cr.convrot_rotate_quant_act_i8(xd, wl.g)
    torch.cuda.synchronize()
    refx = O.rotate_quantize_int8(x, wl.g)
    check_i8(xq, xs, None, refx, name + " activations")
    refw = O.quantize_weight_int8(w, wl.g)
    check_i8(wq, ws, None, refw, name + " weights")
    rows = output_rows(name, x, wl.M, 12)
    own = O.w8a8_linear_from_codes(xq[rows].cpu().numpy(), xs[rows].cpu().numpy(),
                                   wq.cpu().numpy(), ws.cpu().numpy(), b)
    yr = y[rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(yr, own["out_bits"]), "output is not the GEMM of the GPU's codes"
    full = O.w8a8_linear_from_codes(refx["codes"][rows], refx["scale"][rows], refw["codes"],
                                    refw["scale"], b)
    frob = _frob(yr, full["out_bits"])
    assert frob <= OUT_FROB_MAX, f"rel Frobenius {frob:.2e}"


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_mxfp4_full_size(cr, name):
    wl = wk.WORKLOADS[name]
    print(f"\n[case] mxfp4 full size {name}: M={wl.M} K={wl.K} N={wl.N} g={wl.g}", flush=True)
    x = wk.activations(wl)
    xd = _to_dev(x, wl.x_dtype)
    kp = O.padded_k(wl.K, wl.g)
    nb = kp // 32
    if wl.N is None:
        xq, xbs, xr = cr.convrot_rotate_quant_act_mxfp4(xd, wl.g, want_rotated=True)
        torch.cuda.synchronize()
        check_mx(xq, xbs, xr, O.rotate_quantize_mxfp4(x, wl.g), name)
        return
    w, b = wk.weights(wl), wk.bias(wl)
    wq, wbs = cr.convrot_quant_weight_mxfp4(_to_dev(w, wl.x_dtype), wl.g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_mxfp4_linear(xd, wl.g, wq, wbs, bias)
    xq, xbs = cr.convrot_rotate_quant_act_mxfp4(xd, wl.g)
    torch.cuda.synchronize()
    refx = O.rotate_quantize_mxfp4(x, wl.g)
    check_mx(xq, xbs, None, refx, name + " activations")
    refw = O.quantize_weight_mxfp4(w, wl.g)
    check_mx(wq, wbs, None, refw, name + " weights")
    rows = output_rows(name, x, wl.M, 13)
    cw = O.unpack_int4(wq.cpu().numpy()) & 0xF
    ew = wbs.cpu().numpy()[:, :nb]
    own = O.mxfp4_linear_from_codes(O.unpack_int4(xq[rows].cpu().numpy()) & 0xF,
                                    xbs[rows].cpu().numpy()[:, :nb], cw, ew, b)
    yr = y[rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    same = np.mean(yr == own["out_bits"])
    assert same >= 0.99, f"only {same:.4f} of the outputs are the GEMM of the GPU's codes"
    full = O.mxfp4_linear_from_codes(refx["codes"][rows], refx["scales"][rows], refw["codes"],
                                     refw["scales"], b)
    frob = _frob(yr, full["out_bits"])
    assert frob <= OUT_FROB_MAX, f"rel Frobenius {frob:.2e}"
