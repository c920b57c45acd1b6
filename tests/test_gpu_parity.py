"""HIP path vs the CPU oracle, element by element, through the C ABI (needs a gfx950 GPU).

Bars (the stated tolerances, defined precisely here):
  * scales: bit-identical to the oracle's fp32(exact absmax / 7);
  * codes: differ only by one and only at fp32 near-ties of the quotient, in at most 1e-4
    of all codes (at least one code may differ: a small array can hold a single tie);
  * rotated activations: per row max|gpu - oracle| / max|oracle| <= 1e-5;
  * int32 accumulators: bit-identical given identical int4 operands;
  * GEMM output: bit-identical bf16 given identical operands (same fp32 op order);
  * end-to-end bf16 output: ||gpu - oracle||_F / ||oracle||_F <= 1e-2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu

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


DEV = "cuda:0"


def _to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(DEV)


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check_rotate_quant(gpu_q, gpu_s, gpu_rot, ref, label="", max_frac=CODE_MISMATCH_MAX):
    """Scales bit-exact; codes off by at most one, only at fp32 rounding near-ties of the
    oracle's quotient fp32(y / scale), and (for continuous data) in at most 1e-4 of codes,
    or one code."""
    s = gpu_s.cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["scale"].view(np.uint32)), \
        f"{label}: scales differ in {np.sum(s != ref['scale'])} rows"
    q = O.unpack_int4(gpu_q.cpu().numpy())
    d = q.astype(np.int16) - ref["codes"].astype(np.int16)
    assert d.size == 0 or np.max(np.abs(d)) <= 1, f"{label}: code off by {np.max(np.abs(d))}"
    rows, cols = np.nonzero(d)
    if len(rows):
        z = np.abs((ref["yf"][rows, cols] / ref["scale"][rows]).astype(np.float32)).astype(np.float64)
        dist = np.abs(z - (np.floor(z) + 0.5))
        assert np.max(dist) <= 2.0 ** -17, f"{label}: a code differs away from a rounding tie"
    frac = np.count_nonzero(d) / max(d.size, 1)
    # every difference above sits at a near-tie; the rate bar allows at least one of them
    assert np.count_nonzero(d) <= max(max_frac * d.size, 1), f"{label}: {frac:.2e} codes differ"
    if gpu_rot is not None:
        r = gpu_rot.cpu().numpy()
        den = np.max(np.abs(ref["yf"]), axis=1)
        num = np.max(np.abs(r - ref["yf"]), axis=1)
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
        assert np.max(rel) <= ROT_REL_MAX, f"{label}: rotated rel err {np.max(rel):.2e}"
    return frac


ROTATE_CASES = [
    # M, K, g, dtype
    (1, 16, 16, "f32"), (7, 200, 16, "f32"), (64, 256, 16, "f32"), (130, 37, 16, "bf16"),
    (63, 64, 64, "bf16"), (130, 1000, 64, "bf16"), (5, 100, 64, "f32"),
    (200, 3072, 256, "bf16"), (37, 3100, 256, "bf16"), (5, 300, 256, "bf16"),
    (33, 777, 256, "f32"), (17, 1001, 256, "bf16"),
    (48, 12288, 1024, "bf16"), (23, 3000, 1024, "bf16"), (9, 15360, 1024, "bf16"),
    (3, 5, 16, "bf16"), (4, 70000 // 64 * 64, 1024, "bf16"), (3, 61440, 1024, "bf16"),
    (2, 32768, 1024, "f32"), (2, 32768, 256, "bf16"), (2, 16384, 16, "f32"), (2, 32768, 64, "f32"),
]


@pytest.mark.parametrize("M,K,g,dtype", ROTATE_CASES)
def test_rotate_quant_parity(cr, M, K, g, dtype):
    _announce(f"rotate_quant M={M} K={K} g={g} {dtype}")
    if O.padded_k(K, g) > 61440:
        with pytest.raises(cr.ConvRotError):
            cr.convrot_rotate_quant_act(_to_dev(np.zeros((M, K)), dtype), g)
        return
    wl = wk.custom("t", M, K, None, g, x_dtype=dtype)
    x = wk.activations(wl)
    ref = O.rotate_quantize(x, g)
    xq, xs, xr = cr.convrot_rotate_quant_act(_to_dev(x, dtype), g, want_rotated=True)
    torch.cuda.synchronize()
    check_rotate_quant(xq, xs, xr, ref, f"M={M} K={K} g={g}")


@pytest.mark.parametrize("g", [16, 64, 256, 1024])
def test_rotate_quant_edge_rows(cr, g):
    """Zero rows, constant rows (every element ties for the max), a single spike, negatives."""
    _announce(f"edge rows g={g}")
    K = 3 * g + g // 2
    x = np.zeros((8, K), dtype=np.float32)
    x[1, :] = 1.5
    x[2, :] = -0.375
    x[3, 5] = 1000.0
    x[4, :] = np.arange(K) % 7 - 3.0
    x[5, : g // 2] = 2.0 ** -20
    x[6, :] = wk.round_to_dtype(np.random.default_rng(1).standard_normal(K).astype(np.float32) * 1e4,
                                "bf16")
    x[7, -1] = -3.0
    ref = O.rotate_quantize(x, g)
    xq, xs, xr = cr.convrot_rotate_quant_act(_to_dev(x, "bf16"), g, want_rotated=True)
    torch.cuda.synchronize()
    # small-integer rows put many quotients exactly on k + 1/2: only the tie rule may differ
    check_rotate_quant(xq, xs, xr, ref, "edge", max_frac=1.0)
    assert xs[0].item() == 0.0 and torch.all(xq[0] == 0)


def test_rotate_quant_strided_rows_and_streams(cr):
    """Row stride ldx > K (a column slice of a wider tensor) on a non-default stream."""
    _announce("strided rows + side stream")
    wl = wk.custom("t", 50, 700, None, 256)
    x = wk.activations(wl)
    wide = torch.zeros((50, 1024), dtype=torch.bfloat16, device=DEV)
    wide[:, :700] = _to_dev(x, "bf16")
    view = wide[:, :700]
    assert view.stride(0) == 1024
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xq, xs = cr.convrot_rotate_quant_act(view, 256)
    s.synchronize()
    check_rotate_quant(xq, xs, None, O.rotate_quantize(x, 256), "strided")


def test_rotate_quant_deterministic_and_canary(cr):
    _announce("determinism + canary")
    wl = wk.custom("t", 257, 3072, None, 256)
    x = _to_dev(wk.activations(wl), "bf16")
    Kp = 3072
    outs = []
    for fill in (0xAA, 0x55):
        xq = torch.full((257, Kp // 2), fill, dtype=torch.uint8, device=DEV)
        xs = torch.full((257,), float("nan"), dtype=torch.float32, device=DEV)
        xr = torch.full((257, Kp), float("nan"), dtype=torch.float32, device=DEV)
        cr.convrot_rotate_quant_act(x, 256, xq, xs, xr)
        outs.append((xq.clone(), xs.clone(), xr.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    assert torch.equal(outs[0][2].view(torch.int32), outs[1][2].view(torch.int32))
    assert not torch.isnan(outs[0][1]).any() and not torch.isnan(outs[0][2]).any()


def test_empty_inputs(cr):
    _announce("empty inputs")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    xq, xs = cr.convrot_rotate_quant_act(x, 16)
    assert xq.shape == (0, 32) and xs.shape == (0,)
    wq = torch.zeros((5, 32), dtype=torch.uint8, device=DEV)
    ws = torch.ones((5,), dtype=torch.float32, device=DEV)
    y = cr.convrot_w4a4_linear(x, 16, wq, ws)
    assert y.shape == (0, 5)
    y = cr.convrot_w4a4_gemm(xq, xs, wq[:0], ws[:0])
    assert y.shape == (0, 0)


GEMM_CASES = [
    # M, N, Kp, bias
    # K'/2 = 8 (mod 16), M <= 512: the skinny kernel with 8-byte row tails (32-, 64- and
    # 128-row workgroups, one and several K steps)
    (1, 1, 16, False), (17, 5, 48, True), (700, 300, 1040, True), (64, 700, 3088, True),
    (100, 33, 1552, False), (200, 300, 3088, False),
    # M <= 512: the skinny kernel (32, 64 and 128-row workgroups, ragged M, N and K)
    (1, 40, 128, True), (128, 128, 128, False), (200, 136, 1024, True), (129, 130, 256, True),
    (300, 257, 3072, False), (64, 256, 3328, True), (33, 96, 12288, False),
    (300, 7000, 3328, False), (512, 3072, 3072, True), (65, 200, 512, True),
    # M <= 64 (LDS-staged skinny kernel): one partial 1 KB batch with ragged N, exactly two
    # batches, three batches (an odd count, the last one half full), eight batches
    (63, 2, 1056, True), (32, 33, 4096, False), (64, 3000, 5120, True), (40, 1000, 16384, False),
    # M > 512 but M N < 2^21: the skinny kernel (128-row workgroups), ragged M and N
    (1000, 1000, 512, True), (4000, 500, 256, False), (600, 3000, 320, True), (513, 4087, 96, False),
    # K'/2 = 8 (mod 16): mid size (M N < 2^21, skinny with row tails) and large (M N >= 2^21,
    # the tiled kernel with 4-byte transfers; the last K step holds 8, 24, 40 or 56 bytes of
    # each row, one K step up to 25, ragged M and N)
    (1000, 1000, 528, True), (2100, 1100, 208, False), (4608, 3072, 3088, True),
    (1100, 2000, 16, True), (1500, 1500, 48, False), (2000, 1200, 496, True),
    (2500, 1001, 1552, False),
    # large-tile kernel (M N >= 2^21): ragged M and N, several tiles, K tails
    (600, 3500, 512, True), (1000, 2200, 1056, False), (4608, 3072, 256, True),
    (4607, 3071, 128, False), (1130, 1990, 576, True), (4000, 4090, 320, True),
    (4096, 4096, 128, False),
]


@pytest.mark.parametrize("M,N,Kp,with_bias", GEMM_CASES)
def test_gemm_parity_full_range_codes(cr, M, N, Kp, with_bias):
    """Random codes over the whole int4 range [-8, 7]: bit-exact sums and outputs."""
    _announce(f"gemm M={M} N={N} Kp={Kp} bias={with_bias}")
    qx = wk.random_codes(M, Kp, seed=M + Kp)
    qw = wk.random_codes(N, Kp, seed=N + 7 * Kp)
    sx = wk.random_scales(M, 1)
    sw = wk.random_scales(N, 2)
    b = wk.round_to_dtype(np.random.default_rng(3).standard_normal(N).astype(np.float32), "bf16") \
        if with_bias else None
    ref = O.w4a4_linear_from_codes(qx, sx, qw, sw, b)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)  # noqa: E731
    xq = dev(O.pack_int4(qx), torch.uint8)
    wq = dev(O.pack_int4(qw), torch.uint8)
    bias = None if b is None else dev(b, torch.float32).to(torch.bfloat16)
    y, acc = cr.convrot_w4a4_gemm(xq, dev(sx, torch.float32), wq, dev(sw, torch.float32), bias,
                                  want_acc=True)
    y2 = cr.convrot_w4a4_gemm(xq, dev(sx, torch.float32), wq, dev(sw, torch.float32), bias)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    ybits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ybits, ref["out_bits"])
    # without the integer sums requested (the production kernel instantiation)
    assert np.array_equal(y2.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])


@pytest.mark.parametrize("M,N,Kp", [(300, 500, 320), (4608, 3072, 256)])
def test_gemm_extreme_scales(cr, M, N, Kp):
    """Bit-exact outputs for scales down to the subnormal range and up to overflow."""
    _announce(f"gemm extreme scales M={M} N={N} Kp={Kp}")
    qx = wk.random_codes(M, Kp, seed=11)
    qw = wk.random_codes(N, Kp, seed=12)
    sx, sw = wk.extreme_scales(M, 13), wk.extreme_scales(N, 14)
    b = wk.round_to_dtype(np.random.default_rng(15).standard_normal(N).astype(np.float32), "bf16")
    ref = O.w4a4_linear_from_codes(qx, sx, qw, sw, b)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)  # noqa: E731
    y = cr.convrot_w4a4_gemm(dev(O.pack_int4(qx), torch.uint8), dev(sx, torch.float32),
                             dev(O.pack_int4(qw), torch.uint8), dev(sw, torch.float32),
                             dev(b, torch.float32).to(torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])


LINEAR_CASES = [
    # M, K, N, g, dtype, bias
    (64, 256, 256, 16, "f32", False),       # the tiny fp32 workload's shape
    (200, 3072, 320, 256, "bf16", True),
    (130, 3100, 200, 256, "bf16", False),   # ragged K, padded to 3328
    (70, 12288, 136, 1024, "bf16", False),
    (33, 1000, 130, 64, "bf16", True),
]


@pytest.mark.parametrize("M,K,N,g,dtype,with_bias", LINEAR_CASES)
def test_linear_parity(cr, M, K, N, g, dtype, with_bias):
    _announce(f"linear M={M} K={K} N={N} g={g} {dtype} bias={with_bias}")
    wl = wk.custom("t", M, K, N, g, x_dtype=dtype, bias_std=0.01 if with_bias else None)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    ref = O.convlinear4bit(x, w, b, g)
    wq, ws = cr.convrot_quant_weight(_to_dev(w, dtype), g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_w4a4_linear(_to_dev(x, dtype), g, wq, ws, bias)
    torch.cuda.synchronize()
    check_rotate_quant(wq, ws, None, ref["w"], "weights")
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    yg = y.float().cpu().numpy().astype(np.float64)
    frob = np.linalg.norm(yg - yo) / np.linalg.norm(yo)
    assert frob <= OUT_FROB_MAX, frob
    # With the GPU's own codes the whole epilogue is bit-exact against the oracle.
    xq, xs = cr.convrot_rotate_quant_act(_to_dev(x, dtype), g)
    own = O.w4a4_linear_from_codes(O.unpack_int4(xq.cpu().numpy()), xs.cpu().numpy(),
                                   O.unpack_int4(wq.cpu().numpy()), ws.cpu().numpy(), b)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), own["out_bits"])


def test_convlinear4bit_module(cr):
    _announce("ConvLinear4bit module")
    wl = wk.custom("t", 96, 512, 192, 64, bias_std=0.01)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    layer = cr.ConvLinear4bit.from_linear(_to_dev(w, "bf16"), _to_dev(b, "bf16"), group_size=64)
    y = layer(_to_dev(x, "bf16").reshape(2, 48, 512))
    assert y.shape == (2, 48, 192) and y.dtype == torch.bfloat16
    ref = O.convlinear4bit(x, w, b, 64)
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(y.reshape(96, 192).float().cpu().numpy() - yo) / np.linalg.norm(yo)
    assert frob <= OUT_FROB_MAX


@pytest.mark.parametrize("codes", ["int4", "int8", "mxfp4"])
def test_linear_modules_match_functional_api(cr, codes):
    """Each format's module: a 3-D input, bias; output bit-identical to the functional call on
    the same weights, and within the end-to-end bar of the oracle."""
    _announce(f"linear module {codes}")
    wl = wk.custom("m", 96, 700, 160, 256, bias_std=0.01)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    cls, quant, linear, oracle = {
        "int4": (cr.ConvLinear4bit, cr.convrot_quant_weight, cr.convrot_w4a4_linear,
                 O.convlinear4bit),
        "int8": (cr.ConvLinear8bit, cr.convrot_quant_weight_i8, cr.convrot_w8a8_linear,
                 O.convlinear8bit),
        "mxfp4": (cr.ConvLinearFP4, cr.convrot_quant_weight_mxfp4, cr.convrot_mxfp4_linear,
                  O.convlinear_fp4),
    }[codes]
    wd, bd, xd = _to_dev(w, "bf16"), _to_dev(b, "bf16").to(torch.bfloat16), _to_dev(x, "bf16")
    layer = cls.from_linear(wd, bd, group_size=256)
    y = layer(xd.reshape(2, 48, 700))
    assert y.shape == (2, 48, 160) and y.dtype == torch.bfloat16
    wq, ws = quant(wd, 256)
    y_f = linear(xd, 256, wq, ws, bd)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(96, 160).view(torch.int16), y_f.view(torch.int16))
    yo = O.bf16_bits_to_f32(oracle(x, w, b, 256)["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(y.reshape(96, 160).float().cpu().numpy() - yo) / np.linalg.norm(yo)
    assert frob <= OUT_FROB_MAX


# Full-size workloads in the launch configuration the benchmark times.  Codes and scales of
# every activation row and every weight row are checked against the oracle.  Outputs: every
# element where the oracle's GEMM is cheap (attention projection, the padded proj_out variant,
# few tokens); a sample of rows, including every outlier row it picks, for the MLP
# down-projection and the batch-2 proj_out (rows are independent).
FULL = ["rotate_quant", "attn_proj", "mlp_down", "proj_out", "proj_out_padded", "few_tokens"]
ALL_OUTPUTS = {"attn_proj", "proj_out_padded", "few_tokens"}


def output_rows(name, x, M, seed):
    if name in ALL_OUTPUTS:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    big = np.where(np.max(np.abs(x), axis=1) > 100)[0][:16]
    return np.unique(np.concatenate([rng.choice(M, min(M, 48), replace=False), big, [0, M - 1]]))


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size(cr, name):
    wl = wk.WORKLOADS[name]
    _announce(f"full size {name}: M={wl.M} K={wl.K} N={wl.N} g={wl.g}")
    x = wk.activations(wl)
    xd = _to_dev(x, wl.x_dtype)
    if wl.N is None:
        xq, xs, xr = cr.convrot_rotate_quant_act(xd, wl.g, want_rotated=True)
        torch.cuda.synchronize()
        check_rotate_quant(xq, xs, xr, O.rotate_quantize(x, wl.g), name)
        return
    w, b = wk.weights(wl), wk.bias(wl)
    wq, ws = cr.convrot_quant_weight(_to_dev(w, wl.x_dtype), wl.g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_w4a4_linear(xd, wl.g, wq, ws, bias)
    xq, xs = cr.convrot_rotate_quant_act(xd, wl.g)
    torch.cuda.synchronize()
    refx = O.rotate_quantize(x, wl.g)
    check_rotate_quant(xq, xs, None, refx, name + " activations")
    refw = O.quantize_weight(w, wl.g)
    check_rotate_quant(wq, ws, None, refw, name + " weights")
    rows = output_rows(name, x, wl.M, 11)
    # the output is exactly the GEMM + dequantization of the GPU's own codes ...
    own = O.w4a4_linear_from_codes(O.unpack_int4(xq[rows].cpu().numpy()), xs[rows].cpu().numpy(),
                                   O.unpack_int4(wq.cpu().numpy()), ws.cpu().numpy(), b)
    yr = y[rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(yr, own["out_bits"])
    # ... and within the tolerance of the output of the oracle's own codes
    full = O.w4a4_linear_from_codes(refx["codes"][rows], refx["scale"][rows], refw["codes"],
                                    refw["scale"], b)
    yo = O.bf16_bits_to_f32(full["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(O.bf16_bits_to_f32(yr).astype(np.float64) - yo) / np.linalg.norm(yo)
    assert frob <= OUT_FROB_MAX, frob
