"""Rows of tiny magnitude through rotate+quantize, in every code format, against the oracle
(needs a gfx950 GPU).

A row whose largest rotated value is below q_max * 2^-126 has a subnormal scale: there the
reciprocal q_max / max overflows (int4 below ~2.1e-38, int8 below ~3.7e-37) or loses bits,
so the kernel divides by the row's fp32 scale instead (for every row below q_max * 2^-125, so
that the reciprocal it takes elsewhere always has a normal argument).  Each launch mixes such
rows with ordinary ones, so that waves holding both kinds are covered.

Bars:
  * scales (int4, int8): bit-identical to the oracle's fp32(exact absmax / q_max);
  * bf16 rows: bf16 subnormals are multiples of 2^-133 and the butterfly's sums and halvings
    stay on fp32's subnormal grid, so the rotation is exact; codes and rotated values meet
    the ordinary bars (codes differ only at near-ties, rotated values within 1e-5);
  * fp32 rows: values near 2^-149 carry few significant bits, so the butterfly's rounding is
    an absolute error of a few 2^-150 per stage; rotated values must lie within
    1e-5 max + 2^-138 of the oracle's, and every code must be one that a quotient within
    (that row's measured rotation error / scale + 2^-17) of the oracle's quotient rounds to;
    near 2^-149 that error is a few units of the scale, so codes may differ by more than one.
    A subnormal scale, rounded down by up to half of 2^-149, can also put quotients past
    q_max + 1/2: the codes clamp to the code range as the definition's do;
  * MXFP4: the block bytes and codes against the oracle with the same two readings.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ABS_FLOOR = 2.0 ** -138


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()
    return mod


# absmax of each row; 1.0 and 3.0 are ordinary rows sharing waves with the tiny ones
MAGS = {"bf16": [1.0, 2e-38, 1e-38, 1e-39, 3.0, 1e-39],
        "f32": [1.0, 5e-37, 1e-38, 1e-39, 1e-44, 3.0, 2e-45]}


def _rows(dtype, K, seed):
    rng = np.random.default_rng(seed)
    mags = MAGS[dtype]
    x = rng.standard_normal((len(mags), K))
    x /= np.max(np.abs(x), axis=1, keepdims=True)
    x *= np.array(mags)[:, None]
    t = torch.from_numpy(x).to(torch.float32 if dtype == "f32" else torch.bfloat16)
    return t.to(torch.float32).numpy().astype(np.float64), t


def _check_codes(q, s, xr, ref, strict, label, qmin, qmax):
    yf = ref["yf"].astype(np.float64)
    sc = ref["scale"].astype(np.float64)
    assert np.array_equal(s.view(np.uint32), ref["scale"].view(np.uint32)), \
        f"{label}: scales differ in rows {np.nonzero(s != ref['scale'])[0]}"
    err = np.max(np.abs(xr.astype(np.float64) - yf), axis=1)
    rowmax = np.max(np.abs(yf), axis=1)
    bound = (1e-5 * rowmax) if strict else (1e-5 * rowmax + ABS_FLOOR)
    assert np.all(err <= bound), f"{label}: rotated error {err} above {bound}"
    # every code must be one that a quotient within the rotation's error of the oracle's can
    # round to: k with k - 1/2 <= z + delta and k + 1/2 >= z - delta, clamped to the range
    live = sc > 0
    safe = np.where(live, sc, 1.0)
    z = np.where(live[:, None], yf / safe[:, None], 0.0)
    delta = 2.0 ** -17 + (np.zeros_like(err) if strict else np.where(live, err / safe, 0.0))
    delta = delta[:, None]
    lo = np.clip(np.ceil(z - delta - 0.5), qmin, qmax)
    hi = np.clip(np.floor(z + delta + 0.5), qmin, qmax)
    qi = q.astype(np.int64)
    bad = (qi < lo) | (qi > hi)
    assert not bad.any(), (f"{label}: {np.count_nonzero(bad)} codes outside the reachable "
                           f"range, rows {np.unique(np.nonzero(bad)[0])}")
    if strict:   # exact rotation: codes differ from the oracle's by one at most, at near-ties
        d = qi - ref["codes"].astype(np.int64)
        assert np.max(np.abs(d)) <= 1, f"{label}: a code is off by {np.max(np.abs(d))}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("g", [16, 64, 256, 1024])
@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_tiny_rows_integer_codes(cr, fmt, g, dtype):
    K = 3 * g + g // 2
    print(f"\n[case] tiny rows {fmt} g={g} K={K} {dtype}", flush=True)
    xh, xt = _rows(dtype, K, seed=g)
    if fmt == "int4":
        ref = O.rotate_quantize(xh, g)
        q, s, xr = cr.convrot_rotate_quant_act(xt.to(DEV), g, want_rotated=True)
        torch.cuda.synchronize()
        qh = O.unpack_int4(q.cpu().numpy())
    else:
        ref = O.rotate_quantize_int8(xh, g)
        q, s, xr = cr.convrot_rotate_quant_act_i8(xt.to(DEV), g, want_rotated=True)
        torch.cuda.synchronize()
        qh = q.cpu().numpy()
    # rows whose scale underflows to zero (2e-45 in both formats, 1e-44 with int8) have zero
    # codes, as an all-zero row; every other row has a positive scale
    assert np.all((ref["scale"] > 0) | (np.max(np.abs(xh), axis=1) < 1e-43))
    qmin, qmax = (-8, 7) if fmt == "int4" else (-128, 127)
    _check_codes(qh, s.cpu().numpy(), xr.cpu().numpy(), ref, dtype == "bf16", f"{fmt} g={g}",
                 qmin, qmax)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("g", [64, 256, 1024])
def test_tiny_rows_mxfp4(cr, g, dtype):
    K = 3 * g + g // 2
    print(f"\n[case] tiny rows mxfp4 g={g} K={K} {dtype}", flush=True)
    xh, xt = _rows(dtype, K, seed=100 + g)
    ref = O.rotate_quantize_mxfp4(xh, g)
    q, bs, xr = cr.convrot_rotate_quant_act_mxfp4(xt.to(DEV), g, want_rotated=True)
    torch.cuda.synchronize()
    yf = ref["yf"].astype(np.float64)
    r = xr.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(r - yf), axis=1)
    rowmax = np.max(np.abs(yf), axis=1)
    strict = dtype == "bf16"
    assert np.all(err <= 1e-5 * rowmax + (0.0 if strict else ABS_FLOOR)), err
    nb = ref["scales"].shape[1]
    b = bs.cpu().numpy()[:, :nb].astype(np.int64)
    # block bytes: a subnormal block maximum has exponent field 0, and E8M0 clamps at 0 too;
    # elsewhere they may differ only where the block maximum sits at a power of two
    db = b - ref["scales"].astype(np.int64)
    amax = np.abs(r.reshape(len(r), nb, 32)).max(axis=2)
    if np.any(db):
        l2 = np.log2(amax[db != 0])
        assert np.max(np.abs(db)) <= 1 and np.all(np.abs(l2 - np.round(l2)) <= 2.0 ** -12)
    # codes: those of the kernel's own rotated values under its block bytes (each E2M1
    # conversion is exact given them), and the oracle's codes wherever both agree
    scale = np.repeat(np.exp2(b.astype(np.float64) - 127), 32, axis=1)
    own = O.e2m1_encode(r / scale)
    qh = O.unpack_int4(q.cpu().numpy()).astype(np.int64) & 0xF
    assert np.array_equal(qh, own.astype(np.int64)), "codes are not the E2M1 codes of the values"
    if strict:
        same_block = np.repeat(db == 0, 32, axis=1)
        assert np.array_equal(qh[same_block], ref["codes"].astype(np.int64)[same_block])
