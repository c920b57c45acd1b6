"""Rows of huge magnitude, and rows holding NaN or Inf, through rotate+quantize and the
layer, in every code format (needs a gfx950 GPU).

The rotation is an fp32 butterfly: a stage adds four values before halving, so its sums reach
up to 2^(k+1) times the largest input (k = log4 g), and 4 times the input for a row of equal
values.  Rows whose sums stay finite are quantized like any other: scales bit-identical to the
oracle's, codes and block bytes to the ordinary bars.  A row whose butterfly overflows, or that
holds a NaN or an Inf, is flagged rather than given a finite wrong result:
  * int4 and int8: its scale is NaN, so the layer's output row is NaN;
  * MXFP4: every block of a window that holds a non-finite value stores 0xFF, the E8M0 encoding
    of NaN, and the other windows of the row are quantized as usual.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import convrot_oracle as O
from tests.test_gpu_mxfp4 import check_mx
from tests.test_gpu_parity import check_rotate_quant
from tests.test_gpu_w8a8 import check_i8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32_MAX = float(np.finfo(np.float32).max)
BF16_MAX = 3.3895313892515355e38
GOOD = [0, 1, 2, 3, 4, 8]      # rows whose butterfly stays finite
OVERFLOW, NAN_ROW, INF_ROW = 5, 6, 7


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()
    return mod


def _rows(g, K, dtype, seed):
    """Nine rows: ordinary, equal values at 0.2 of the fp32 maximum, a spike at the type's
    largest finite value, random values up to FLT_MAX / 2^(k+2), a negative spike, equal
    values at half the fp32 maximum (their stage sums overflow), a NaN, an Inf, ordinary."""
    rng = np.random.default_rng(seed)
    k = int(round(np.log(g) / np.log(4)))
    x = rng.standard_normal((9, K))
    x /= np.max(np.abs(x), axis=1, keepdims=True)
    x[0] *= 1.0
    x[1] = 0.2 * F32_MAX
    x[2] = 0.0
    x[2, rng.integers(K)] = BF16_MAX if dtype == "bf16" else F32_MAX
    x[3] *= F32_MAX / 2.0 ** (k + 2)
    x[4, rng.integers(K)] = -0.25 * F32_MAX
    x[OVERFLOW] = 0.5 * F32_MAX
    nan_col, inf_col = int(rng.integers(K)), int(rng.integers(K))
    x[NAN_ROW, nan_col] = np.nan
    x[INF_ROW, inf_col] = np.inf
    x[8] *= 3.0
    t = torch.from_numpy(x).to(torch.float32 if dtype == "f32" else torch.bfloat16)
    return t.to(torch.float32).numpy().astype(np.float64), t, {NAN_ROW: nan_col, INF_ROW: inf_col}


def _flagged_scales(s):
    s = s.cpu().numpy()
    assert np.all(np.isnan(s[[OVERFLOW, NAN_ROW, INF_ROW]])), s[[OVERFLOW, NAN_ROW, INF_ROW]]
    assert np.all(np.isfinite(s[GOOD])), s[GOOD]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("g", [16, 64, 256, 1024])
@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_huge_rows_integer_codes(cr, fmt, g, dtype):
    K = 3 * g + g // 2
    print(f"\n[case] huge rows {fmt} g={g} K={K} {dtype}", flush=True)
    xh, xt, _ = _rows(g, K, dtype, seed=g)
    if fmt == "int4":
        q, s, xr = cr.convrot_rotate_quant_act(xt.to(DEV), g, want_rotated=True)
        torch.cuda.synchronize()
        check_rotate_quant(q[GOOD], s[GOOD], xr[GOOD], O.rotate_quantize(xh[GOOD], g),
                           f"int4 g={g} {dtype}")
    else:
        q, s, xr = cr.convrot_rotate_quant_act_i8(xt.to(DEV), g, want_rotated=True)
        torch.cuda.synchronize()
        check_i8(q[GOOD], s[GOOD], xr[GOOD], O.rotate_quantize_int8(xh[GOOD], g),
                 f"int8 g={g} {dtype}")
    _flagged_scales(s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("g", [64, 256, 1024])
def test_huge_rows_mxfp4(cr, g, dtype):
    K = 3 * g + g // 2
    print(f"\n[case] huge rows mxfp4 g={g} K={K} {dtype}", flush=True)
    xh, xt, bad_cols = _rows(g, K, dtype, seed=200 + g)
    q, bs = cr.convrot_rotate_quant_act_mxfp4(xt.to(DEV), g)
    torch.cuda.synchronize()
    check_mx(q[GOOD], bs[GOOD], None, O.rotate_quantize_mxfp4(xh[GOOD], g), f"mxfp4 g={g}")
    nb = (K + g - 1) // g * g // 32
    b = bs.cpu().numpy()[:, :nb]
    assert np.all(b[OVERFLOW] == 0xFF), b[OVERFLOW]
    # a NaN or an Inf spreads over its own window only: the other windows match the oracle's
    # on the same row with that element set to zero
    per_window = g // 32
    for row, col in bad_cols.items():
        w = col // g
        mine = np.arange(nb) // per_window == w
        assert np.all(b[row, mine] == 0xFF), (row, b[row, mine])
        clean = xh[row:row + 1].copy()
        clean[0, col] = 0.0
        ref = O.rotate_quantize_mxfp4(clean, g)
        assert np.array_equal(b[row, ~mine], ref["scales"][0, ~mine]), (row, b[row], ref["scales"])
    assert np.all(b[GOOD] != 0xFF)


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
def test_huge_rows_layer_output(cr, fmt):
    """The layer's output rows for flagged activation rows are NaN; those of the ordinary
    rows are finite (the huge rows' outputs may overflow to Inf, as their exact values do)."""
    g, K, N = 256, 1000, 96
    print(f"\n[case] huge rows layer {fmt} g={g} K={K} N={N}", flush=True)
    _, xt, _ = _rows(g, K, "bf16", seed=7)
    w = torch.from_numpy(np.random.default_rng(8).standard_normal((N, K))).to(torch.bfloat16).to(DEV)
    bias = torch.zeros(N, dtype=torch.bfloat16, device=DEV)
    if fmt == "int4":
        wq, ws = cr.convrot_quant_weight(w, g)
        y = cr.convrot_w4a4_linear(xt.to(DEV), g, wq, ws, bias)
    elif fmt == "int8":
        wq, ws = cr.convrot_quant_weight_i8(w, g)
        y = cr.convrot_w8a8_linear(xt.to(DEV), g, wq, ws, bias)
    else:
        wq, ws = cr.convrot_quant_weight_mxfp4(w, g)
        y = cr.convrot_mxfp4_linear(xt.to(DEV), g, wq, ws, bias)
    torch.cuda.synchronize()
    yf = y.float().cpu().numpy()
    assert np.all(np.isnan(yf[[OVERFLOW, NAN_ROW, INF_ROW]])), fmt
    assert np.all(np.isfinite(yf[[0, 8]])), fmt


@pytest.mark.parametrize("entry", ["two_kernel_tiled", "fused", "noalloc"])
def test_huge_rows_other_paths(cr, entry):
    """The same flag through the tiled GEMM (600 rows, 4096 outputs), the single-launch layer
    and the entry point without a workspace: flagged rows' outputs are NaN, the others finite
    and bit-identical to the two-kernel layer's."""
    g, K = 256, 1000
    M, N = (600, 4096) if entry == "two_kernel_tiled" else (64, 256)
    print(f"\n[case] huge rows {entry} M={M} K={K} N={N}", flush=True)
    _, xt, _ = _rows(g, K, "bf16", seed=11)
    x = torch.from_numpy(np.random.default_rng(12).standard_normal((M, K))).to(torch.bfloat16)
    x[:9] = xt
    x = x.to(DEV)
    w = torch.from_numpy(np.random.default_rng(13).standard_normal((N, K))).to(torch.bfloat16).to(DEV)
    bias = torch.zeros(N, dtype=torch.bfloat16, device=DEV)
    wq, ws = cr.convrot_quant_weight(w, g)
    ref = cr.convrot_w4a4_linear(x, g, wq, ws, bias)
    if entry == "fused":
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        y = cr.convrot_w4a4_linear_fused(x, g, wq, ws, bias, status=status)
    elif entry == "noalloc":
        y = cr.convrot_w4a4_linear_noalloc(x, g, wq, ws, bias)
    else:
        y = ref
    torch.cuda.synchronize()
    if entry == "fused":
        assert status.item() == 0
    yf = y.float().cpu().numpy()
    assert np.all(np.isnan(yf[[OVERFLOW, NAN_ROW, INF_ROW]])), entry
    rest = np.r_[0, 8, 9:M]
    assert np.all(np.isfinite(yf[rest])), entry
    assert torch.equal(y[rest].view(torch.int16), ref[rest].view(torch.int16)), entry


@pytest.mark.parametrize("g", [16, 256, 1024])
def test_huge_weight_rows(cr, g):
    """Weight rows go through the same kernel: huge rows in range match the oracle's weight
    quantization, flagged rows get NaN scales, and the layer's output columns for them are
    NaN while the others stay finite."""
    K = 3 * g + g // 2
    print(f"\n[case] huge weight rows g={g} K={K}", flush=True)
    wh, wt, _ = _rows(g, K, "bf16", seed=300 + g)
    wq, ws = cr.convrot_quant_weight(wt.to(DEV), g)
    torch.cuda.synchronize()
    check_rotate_quant(wq[GOOD], ws[GOOD], None, O.quantize_weight(wh[GOOD], g), f"weights g={g}")
    _flagged_scales(ws)
    x = torch.from_numpy(np.random.default_rng(301).standard_normal((5, K))).to(torch.bfloat16).to(DEV)
    y = cr.convrot_w4a4_linear(x, g, wq, ws, None)
    torch.cuda.synchronize()
    yf = y.float().cpu().numpy()
    assert np.all(np.isnan(yf[:, [OVERFLOW, NAN_ROW, INF_ROW]]))
    assert np.all(np.isfinite(yf[:, [0, 8]]))
