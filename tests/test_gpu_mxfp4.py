"""MXFP4 ConvRot on the GPU vs the CPU oracle, through the C ABI (needs a gfx950 GPU).

Bars (derived from the arithmetic; the kernel's block maxima come from its fp32 rotation,
whose error is a few ulp of the row maximum, not from the exact rotation):
  * rotated activations within 1e-5 of the oracle (row relative);
  * a block's E8M0 byte may differ from the oracle's only by one, only where the oracle's
    block maximum lies within 2^-12 (in log2) of a power of two, in at most 1e-3 of blocks;
  * within blocks of equal scale a code may differ only where value / scale lies within the
    rotation's error of an E2M1 rounding tie, by one step, in at most 1e-3 of the codes
    (codes are compared by value: +0 and -0 are the same number).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROT_REL_MAX = 1e-5
BLOCK_MISMATCH_MAX = 1e-3
CODE_MISMATCH_MAX = 1e-3
TIES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


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


def check_mx(gpu_q, gpu_bs, gpu_rot, ref, label="", max_frac=CODE_MISMATCH_MAX):
    yf = ref["yf"].astype(np.float64)
    rows, kp = yf.shape
    bs_all = gpu_bs.cpu().numpy()
    nb = ref["scales"].shape[1]
    assert bs_all.dtype == np.uint8 and bs_all.shape == (rows, 4 * (-(-kp // 128)))
    assert np.all(bs_all[:, nb:] == 0), f"{label}: scale padding not zero"
    bs = bs_all[:, :nb]
    db = bs.astype(np.int64) - ref["scales"].astype(np.int64)
    bad = np.nonzero(db)
    if len(bad[0]):
        assert np.max(np.abs(db)) <= 1, f"{label}: block scale off by {np.max(np.abs(db))}"
        amax = np.abs(yf.reshape(rows, kp // 32, 32)).max(axis=2)[bad]
        l2 = np.log2(amax)
        assert np.all(np.abs(l2 - np.round(l2)) <= 2.0 ** -12), \
            f"{label}: a block scale differs away from a power of two"
    # each differing block sits at a power of two (checked above); at least one may differ
    assert len(bad[0]) <= max(BLOCK_MISMATCH_MAX * bs.size, 1), f"{label}: {len(bad[0])} blocks differ"
    q = O.unpack_int4(gpu_q.cpu().numpy()).astype(np.int64) & 0xF
    same = np.repeat(db == 0, 32, axis=1)
    vg = O.e2m1_decode(q)
    vo = O.e2m1_decode(ref["codes"])
    diff = (vg != vo) & same
    r_i, c_i = np.nonzero(diff)
    if len(r_i):
        grid = O.E2M1_GRID
        step = np.abs(np.searchsorted(grid, np.abs(vg[r_i, c_i])) -
                      np.searchsorted(grid, np.abs(vo[r_i, c_i])))
        assert np.all(step <= 1) and np.all(np.sign(vg[r_i, c_i]) * np.sign(vo[r_i, c_i]) >= 0), \
            f"{label}: a code differs by more than one step"
        x_scale = np.exp2(ref["scales"].astype(np.float64) - 127)[r_i, c_i // 32]
        t = np.abs(yf[r_i, c_i]) / x_scale
        rowmax = np.abs(yf).max(axis=1)[r_i]
        near = np.min(np.abs(t[:, None] - TIES[None, :]), axis=1)
        assert np.all(near <= 2.0 ** -14 * rowmax / x_scale + 1e-12), \
            f"{label}: a code differs away from a rounding tie"
    frac = len(r_i) / max(q.size, 1)
    # every difference above sits at a near-tie; the rate bar allows at least one of them
    assert len(r_i) <= max(max_frac * q.size, 1), f"{label}: {frac:.2e} codes differ"
    if gpu_rot is not None:
        r = gpu_rot.cpu().numpy()
        den = np.max(np.abs(yf), axis=1)
        num = np.max(np.abs(r - yf), axis=1)
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
        assert np.max(rel) <= ROT_REL_MAX, f"{label}: rotated rel err {np.max(rel):.2e}"


ROTATE_CASES = [
    # M, K, g, dtype
    (7, 200, 64, "f32"), (130, 1000, 64, "bf16"), (200, 3072, 256, "bf16"),
    (37, 3100, 256, "bf16"), (33, 777, 256, "f32"), (48, 12288, 1024, "bf16"),
    (23, 3000, 1024, "bf16"), (3, 61440, 1024, "bf16"), (2, 32768, 1024, "f32"),
    (2, 32768, 64, "bf16"), (9, 3000, 64, "bf16"), (5, 190, 64, "f32"),
]


@pytest.mark.parametrize("M,K,g,dtype", ROTATE_CASES)
def test_rotate_quant_mxfp4_parity(cr, M, K, g, dtype):
    _announce(f"rotate_quant_mxfp4 M={M} K={K} g={g} {dtype}")
    wl = wk.custom("t", M, K, None, g, x_dtype=dtype)
    x = wk.activations(wl)
    ref = O.rotate_quantize_mxfp4(x, g)
    xq, xbs, xr = cr.convrot_rotate_quant_act_mxfp4(_to_dev(x, dtype), g, want_rotated=True)
    torch.cuda.synchronize()
    check_mx(xq, xbs, xr, ref, f"M={M} K={K} g={g}")


@pytest.mark.parametrize("g", [64, 256, 1024])
def test_rotate_quant_mxfp4_edge_rows(cr, g):
    """Zero rows and blocks, constant rows, a single spike, tiny values, huge values."""
    _announce(f"mxfp4 edge rows g={g}")
    K = 2 * g + g // 2
    x = np.zeros((7, K), dtype=np.float32)
    x[1, :] = 1.5
    x[2, :] = -0.375
    x[3, 5] = 1000.0
    x[4, :] = np.arange(K) % 9 - 4.0
    x[5, : g // 2] = 2.0 ** -20
    x[6, :] = 3.0e38 / g
    ref = O.rotate_quantize_mxfp4(x, g)
    xq, xbs = cr.convrot_rotate_quant_act_mxfp4(_to_dev(x, "f32"), g)
    torch.cuda.synchronize()
    check_mx(xq, xbs, None, ref, "edge", max_frac=1.0)
    assert torch.all(xq[0] == 0) and torch.all(xbs[0] == 0)


def test_mxfp4_weights_and_strides(cr):
    _announce("mxfp4 weights, strided rows")
    wl = wk.custom("t", 50, 1100, 96, 256)
    w = wk.weights(wl)
    ref = O.quantize_weight_mxfp4(w, 256)
    wq, wbs = cr.convrot_quant_weight_mxfp4(_to_dev(w, "bf16"), 256)
    torch.cuda.synchronize()
    check_mx(wq, wbs, None, ref, "weights")
    x = wk.activations(wl)
    big = torch.zeros((50, 1200), dtype=torch.bfloat16, device=DEV)
    big[:, :1100] = _to_dev(x, "bf16")
    xq, xbs = cr.convrot_rotate_quant_act_mxfp4(big[:, :1100], 256)
    torch.cuda.synchronize()
    check_mx(xq, xbs, None, O.rotate_quantize_mxfp4(x, 256), "strided")


def test_mxfp4_rejects_group_16(cr):
    with pytest.raises(cr.ConvRotError):
        cr.convrot_rotate_quant_act_mxfp4(torch.zeros((2, 64), dtype=torch.bfloat16, device=DEV), 16)


def _pad_scales(e8, kp):
    out = np.zeros((e8.shape[0], 4 * (-(-kp // 128))), dtype=np.uint8)
    out[:, : e8.shape[1]] = e8
    return out


def check_mx_gemm(y, acc, ref, kp, bias, label=""):
    """fp32 sums within the accumulation bound; the bf16 output exactly the epilogue of the
    GPU's own sums; nearly all outputs bit-identical to the oracle's."""
    a = acc.cpu().numpy().astype(np.float64)
    # one rounding per 64-code instruction, plus the skinny kernel's sum of up to 16 per-wave
    # partial sums (the order of the fp32 additions is the implementation's)
    bound = (kp / 64 + 18) * 2.0 ** -23 * ref["abs_sum"] + 1e-30
    err = np.abs(a - ref["sum"])
    assert np.all(err <= bound), f"{label}: sum error {np.max(err / bound):.2f} x the bound"
    z = acc.cpu().numpy().astype(np.float32)
    if bias is not None:
        z = (z + bias[None, :].astype(np.float32)).astype(np.float32)
    ybits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ybits, O.f32_to_bf16_bits(z)), f"{label}: epilogue differs"
    same = np.mean(ybits == ref["out_bits"])
    assert same >= 0.99, f"{label}: only {same:.4f} of the outputs match the oracle's bits"


MX_GEMM_CASES = [
    # M, N, Kp, bias
    # M <= 256: the skinny kernel (32, 64 or 128 activation rows per workgroup)
    (1, 1, 64, False), (64, 64, 192, True), (129, 257, 1088, False), (200, 300, 12288, False),
    (33, 100, 1024, True), (40, 70, 64, False), (100, 90, 512, True), (256, 96, 256, False),
    # M > 256 with M N < 2^21 and at most one workgroup per CU: the skinny kernel
    (257, 64, 128, True), (300, 500, 320, True), (1000, 1000, 512, False),
    # the tiled kernel (M N < 2^21 but more skinny workgroups than CUs; larger outputs)
    (600, 3000, 320, True), (1000, 2200, 3008, True), (4608, 3072, 256, True),
]


@pytest.mark.parametrize("M,N,Kp,with_bias", MX_GEMM_CASES)
def test_mxfp4_gemm_parity(cr, M, N, Kp, with_bias):
    _mx_gemm_case(cr, M, N, Kp, with_bias)


# The tiled kernel runs K step 0 on its own, then eight steps per loop iteration, then the
# 0-7 steps left: K' = 128 n covers n K steps, every tail length and loop counts 0, 1 and 2,
# plus a ragged last step.
@pytest.mark.parametrize("nsteps", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 16, 17, 9.5])
def test_mxfp4_tiled_k_loop_lengths(cr, nsteps):
    _mx_gemm_case(cr, 600, 3000, int(128 * nsteps), int(nsteps) % 2 == 0)


def _mx_gemm_case(cr, M, N, Kp, with_bias):
    _announce(f"mxfp4 gemm M={M} N={N} Kp={Kp} bias={with_bias}")
    rng = np.random.default_rng(M + 5 * N + Kp)
    cx = rng.integers(0, 16, size=(M, Kp)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, Kp)).astype(np.uint8)
    ex = rng.integers(112, 142, size=(M, Kp // 32)).astype(np.uint8)
    ew = rng.integers(112, 142, size=(N, Kp // 32)).astype(np.uint8)
    b = wk.round_to_dtype(rng.standard_normal(N).astype(np.float32), "bf16") if with_bias else None
    ref = O.mxfp4_linear_from_codes(cx, ex, cw, ew, b)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    bias = None if b is None else torch.from_numpy(b).to(torch.bfloat16).to(DEV)
    args = (dev(O.pack_int4(cx)), dev(_pad_scales(ex, Kp)), dev(O.pack_int4(cw)),
            dev(_pad_scales(ew, Kp)), bias)
    y, acc = cr.convrot_mxfp4_gemm(*args, want_acc=True)
    y2 = cr.convrot_mxfp4_gemm(*args)
    torch.cuda.synchronize()
    check_mx_gemm(y, acc, ref, Kp, b, f"M={M} N={N} Kp={Kp}")
    assert torch.equal(y, y2), "the production instantiation differs from the debug one"


MX_LINEAR_CASES = [
    # M, K, N, g, dtype, bias
    (64, 256, 256, 64, "f32", False), (200, 3072, 320, 256, "bf16", True),
    (130, 3100, 200, 256, "bf16", False), (70, 12288, 136, 1024, "bf16", False),
    (33, 1000, 130, 64, "bf16", True),
]


@pytest.mark.parametrize("M,K,N,g,dtype,with_bias", MX_LINEAR_CASES)
def test_mxfp4_linear_parity(cr, M, K, N, g, dtype, with_bias):
    _announce(f"mxfp4 linear M={M} K={K} N={N} g={g} {dtype} bias={with_bias}")
    wl = wk.custom("t", M, K, N, g, x_dtype=dtype, bias_std=0.01 if with_bias else None)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    ref = O.convlinear_fp4(x, w, b, g)
    wq, wbs = cr.convrot_quant_weight_mxfp4(_to_dev(w, dtype), g)
    bias = None if b is None else _to_dev(b, "bf16")
    y = cr.convrot_mxfp4_linear(_to_dev(x, dtype), g, wq, wbs, bias)
    xq, xbs = cr.convrot_rotate_quant_act_mxfp4(_to_dev(x, dtype), g)
    torch.cuda.synchronize()
    check_mx(wq, wbs, None, ref["w"], "weights")
    check_mx(xq, xbs, None, ref["x"], "activations")
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(y.float().cpu().numpy() - yo) / max(np.linalg.norm(yo), 1e-30)
    assert frob <= 1e-2, f"rel Frobenius {frob:.2e}"
    # given the GPU's own codes, the output is the GEMM of those codes
    kp = O.padded_k(K, g)
    nb = kp // 32
    cx = O.unpack_int4(xq.cpu().numpy()) & 0xF
    cw = O.unpack_int4(wq.cpu().numpy()) & 0xF
    own = O.mxfp4_linear_from_codes(cx, xbs.cpu().numpy()[:, :nb], cw, wbs.cpu().numpy()[:, :nb], b)
    ybits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.mean(ybits == own["out_bits"]) >= 0.99


def test_mxfp4_empty_and_errors(cr):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros((8, 128), dtype=torch.uint8, device=DEV)
    wbs = torch.zeros((8, 8), dtype=torch.uint8, device=DEV)
    assert cr.convrot_mxfp4_linear(x, 256, wq, wbs).shape == (0, 8)
    with pytest.raises(cr.ConvRotError):
        cr.convrot_mxfp4_linear(torch.zeros((2, 64), dtype=torch.bfloat16, device=DEV), 16,
                                torch.zeros((8, 32), dtype=torch.uint8, device=DEV),
                                torch.zeros((8, 4), dtype=torch.uint8, device=DEV))
