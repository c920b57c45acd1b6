"""INT8 (W8A8) ConvRot on the GPU vs the CPU oracle, through the C ABI (needs a gfx950 GPU).

Same bars as the int4 path (see test_gpu_parity.py): scales bit-identical to
fp32(exact absmax / 127); codes off by at most one and only at fp32 near-ties of the
oracle's quotient, in at most 1e-4 of all codes; rotated activations within 1e-5 (row
relative); int32 sums and the bf16 GEMM output bit-identical given identical codes; the
end-to-end output within 1e-2 relative Frobenius error.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE_MISMATCH_MAX = 1e-4
ROT_REL_MAX = 1e-5
OUT_FROB_MAX = 1e-2


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


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check_i8(gpu_q, gpu_s, gpu_rot, ref, label="", max_frac=CODE_MISMATCH_MAX):
    s = gpu_s.cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["scale"].view(np.uint32)), \
        f"{label}: scales differ in {np.sum(s != ref['scale'])} rows"
    q = gpu_q.cpu().numpy()
    assert q.dtype == np.int8 and q.shape == ref["codes"].shape
    d = q.astype(np.int16) - ref["codes"].astype(np.int16)
    assert d.size == 0 or np.max(np.abs(d)) <= 1, f"{label}: code off by {np.max(np.abs(d))}"
    rows, cols = np.nonzero(d)
    if len(rows):
        z = np.abs((ref["yf"][rows, cols] / ref["scale"][rows]).astype(np.float32)).astype(np.float64)
        dist = np.abs(z - (np.floor(z) + 0.5))
        assert np.max(dist) <= 2.0 ** -13, f"{label}: a code differs away from a rounding tie"
    frac = np.count_nonzero(d) / max(d.size, 1)
    # every difference above sits at a near-tie; the rate bar allows at least one of them
    assert np.count_nonzero(d) <= max(max_frac * d.size, 1), f"{label}: {frac:.2e} codes differ"
    if gpu_rot is not None:
        r = gpu_rot.cpu().numpy()
        den = np.max(np.abs(ref["yf"]), axis=1)
        num = np.max(np.abs(r - ref["yf"]), axis=1)
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
        assert np.max(rel) <= ROT_REL_MAX, f"{label}: rotated rel err {np.max(rel):.2e}"


ROTATE_CASES = [
    # M, K, g, dtype
    (7, 200, 16, "f32"), (64, 256, 16, "f32"), (130, 1000, 64, "bf16"), (5, 100, 64, "f32"),
    (200, 3072, 256, "bf16"), (37, 3100, 256, "bf16"), (33, 777, 256, "f32"),
    (48, 12288, 1024, "bf16"), (23, 3000, 1024, "bf16"),
    (3, 53248, 1024, "bf16"), (2, 28672, 1024, "f32"), (2, 30720, 256, "f32"),
    (2, 30720, 64, "f32"), (2, 32768, 256, "bf16"), (2, 16384, 16, "f32"),
    # just past the on-chip limits: rejected
    (2, 55296, 1024, "bf16"), (2, 29696, 1024, "f32"), (2, 30976, 256, "f32"),
    (2, 30784, 64, "f32"),
]

# Longest K' held on chip with int8 codes, as include/convrot.h states.
MAX_KP_I8 = {(16, "bf16"): 16384, (16, "f32"): 16384, (64, "bf16"): 32768, (64, "f32"): 30720,
             (256, "bf16"): 32768, (256, "f32"): 30720, (1024, "bf16"): 53248,
             (1024, "f32"): 28672}


@pytest.mark.parametrize("M,K,g,dtype", ROTATE_CASES)
def test_rotate_quant_i8_parity(cr, M, K, g, dtype):
    _announce(f"rotate_quant_i8 M={M} K={K} g={g} {dtype}")
    if O.padded_k(K, g) > MAX_KP_I8[(g, dtype)]:
        with pytest.raises(cr.ConvRotError):
            cr.convrot_rotate_quant_act_i8(_to_dev(np.zeros((M, K)), dtype), g)
        return
    wl = wk.custom("t", M, K, None, g, x_dtype=dtype)
    x = wk.activations(wl)
    ref = O.rotate_quantize_int8(x, g)
    xq, xs, xr = cr.convrot_rotate_quant_act_i8(_to_dev(x, dtype), g, want_rotated=True)
    torch.cuda.synchronize()
    check_i8(xq, xs, xr, ref, f"M={M} K={K} g={g}")


@pytest.mark.parametrize("g", [16, 64, 256, 1024])
def test_rotate_quant_i8_edge_rows(cr, g):
    """Zero rows, constant rows, a single spike, negatives, tiny values."""
    _announce(f"i8 edge rows g={g}")
    K = 2 * g + g // 2
    x = np.zeros((6, K), dtype=np.float32)
    x[1, :] = 1.5
    x[2, :] = -0.375
    x[3, 5] = 1000.0
    x[4, :] = np.arange(K) % 9 - 4.0
    x[5, : g // 2] = 2.0 ** -20
    ref = O.rotate_quantize_int8(x, g)
    xq, xs = cr.convrot_rotate_quant_act_i8(_to_dev(x, "bf16"), g)
    torch.cuda.synchronize()
    check_i8(xq, xs, None, ref, "edge", max_frac=1.0)
    assert xs[0].item() == 0.0 and torch.all(xq[0] == 0)


GEMM_CASES = [
    # M, N, Kp, bias
    # M <= 256: the skinny kernel
    (1, 1, 16, False), (64, 64, 64, True), (100, 200, 512, True), (129, 257, 1040, False),
    (256, 3000, 3072, True), (16, 3072, 12288, False), (48, 300, 1040, True),
    # M > 256 with M N < 2^21 and at most one workgroup per CU: the skinny kernel
    (300, 500, 320, True), (1000, 1000, 512, False),
    # the tiled kernel (M N < 2^21 but more skinny workgroups than CUs; larger outputs)
    (600, 3000, 320, True), (1000, 2200, 1056, False), (4608, 3072, 256, True),
]


@pytest.mark.parametrize("M,N,Kp,with_bias", GEMM_CASES)
def test_w8a8_gemm_full_range(cr, M, N, Kp, with_bias):
    """Random codes over the whole int8 range: bit-exact sums and outputs."""
    _announce(f"w8a8 gemm M={M} N={N} Kp={Kp} bias={with_bias}")
    rng = np.random.default_rng(M + 3 * N + Kp)
    qx = rng.integers(-128, 128, size=(M, Kp)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, Kp)).astype(np.int8)
    sx = wk.random_scales(M, 1)
    sw = wk.random_scales(N, 2)
    b = wk.round_to_dtype(rng.standard_normal(N).astype(np.float32), "bf16") if with_bias else None
    ref = O.w8a8_linear_from_codes(qx, sx, qw, sw, b)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)  # noqa: E731
    xq, wq = dev(qx, torch.int8), dev(qw, torch.int8)
    xs, ws = dev(sx, torch.float32), dev(sw, torch.float32)
    bias = None if b is None else dev(b, torch.float32).to(torch.bfloat16)
    y, acc = cr.convrot_w8a8_gemm(xq, xs, wq, ws, bias, want_acc=True)
    y2 = cr.convrot_w8a8_gemm(xq, xs, wq, ws, bias)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])
    assert np.array_equal(y2.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])


def test_w8a8_gemm_extreme_scales(cr):
    """Bit-exact outputs for scales down to the subnormal range and up to overflow."""
    M, N, Kp = 300, 500, 320
    _announce(f"w8a8 gemm extreme scales M={M} N={N} Kp={Kp}")
    rng = np.random.default_rng(21)
    qx = rng.integers(-128, 128, size=(M, Kp)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, Kp)).astype(np.int8)
    sx, sw = wk.extreme_scales(M, 23), wk.extreme_scales(N, 24)
    b = wk.round_to_dtype(rng.standard_normal(N).astype(np.float32), "bf16")
    ref = O.w8a8_linear_from_codes(qx, sx, qw, sw, b)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)  # noqa: E731
    y = cr.convrot_w8a8_gemm(dev(qx, torch.int8), dev(sx, torch.float32), dev(qw, torch.int8),
                             dev(sw, torch.float32), dev(b, torch.float32).to(torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])


LINEAR_CASES = [
    # M, K, N, g, dtype, bias
    (64, 256, 256, 16, "f32", False), (200, 3072, 320, 256, "bf16", True),
    (130, 3100, 200, 256, "bf16", False), (70, 12288, 136, 1024, "bf16", False),
]


@pytest.mark.parametrize("M,K,N,g,dtype,with_bias", LINEAR_CASES)
def test_w8a8_linear_parity(cr, M, K, N, g, dtype, with_bias):
    _announce(f"w8a8 linear M={M} K={K} N={N} g={g} {dtype} bias={with_bias}")
    wl = wk.custom("t", M, K, N, g, x_dtype=dtype, bias_std=0.01 if with_bias else None)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    ref = O.convlinear8bit(x, w, b, g)
    wq, ws = cr.convrot_quant_weight_i8(_to_dev(w, dtype), g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_w8a8_linear(_to_dev(x, dtype), g, wq, ws, bias)
    torch.cuda.synchronize()
    check_i8(wq, ws, None, ref["w"], "weights")
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(y.float().cpu().numpy() - yo) / max(np.linalg.norm(yo), 1e-30)
    assert frob <= OUT_FROB_MAX, f"rel Frobenius {frob:.2e}"
    # with the oracle's own activation codes the GEMM output is bit-exact
    xq, xs = cr.convrot_rotate_quant_act_i8(_to_dev(x, dtype), g)
    check_i8(xq, xs, None, ref["x"], "activations")


def test_w8a8_empty(cr):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    xq, xs = cr.convrot_rotate_quant_act_i8(x, 16)
    assert xq.shape == (0, 64)
    wq = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    ws = torch.ones((8,), dtype=torch.float32, device=DEV)
    y = cr.convrot_w8a8_linear(x, 16, wq, ws)
    assert y.shape == (0, 8)
