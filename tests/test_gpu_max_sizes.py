"""Maximum sizes (needs a gfx950 GPU with about 110 GB of free device memory).

Buffer loads and stores take 32-bit byte offsets from a base address, and a dispatch counts
its work-items in 32-bit fields.  These cases go past those limits and check sampled rows
and columns against the oracle:
  * the GEMM of every code format with M = 3 and N = 2^27 + 96 output columns, where the
    skinny grid would need more than 2^32 work-items (the library then takes the tiled
    kernel), and with N = 2^27 - 32, the widest output the skinny grid takes;
  * rotate+quantize of M = 2^29 + 256 rows (K = g = 64, bf16) in every format; the MXFP4
    block-scale rows alone then span more than 2 GiB;
  * rotate+quantize of rows 2 GiB apart (a strided view), in every format;
  * every format's GEMM at the largest depth accepted, K' = 65536, with int8 sums of 2^30.
Inputs are drawn on the device with torch's seeded generator; only the sampled rows and
columns come back to the host.  The bars are those of the format's own parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import convrot_oracle as O
from tests.test_gpu_mxfp4 import check_mx, check_mx_gemm
from tests.test_gpu_parity import check_rotate_quant
from tests.test_gpu_w8a8 import check_i8

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
SKINNY_WIDEST = (1 << 27) - 32
PAST_SKINNY = (1 << 27) + 96
M_TALL = (1 << 29) + 256


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


@pytest.fixture(autouse=True)
def _release_memory():
    torch.cuda.empty_cache()
    yield
    torch.cuda.empty_cache()


def _sample(n, rng, around=()):
    picks = [np.arange(min(n, 64)), np.arange(max(0, n - 64), n), rng.choice(n, 256, replace=False)]
    for c in around:
        picks.append(np.arange(max(0, c - 64), min(n, c + 64)))
    return np.unique(np.concatenate(picks))


@pytest.mark.parametrize("N", [SKINNY_WIDEST, PAST_SKINNY])
@pytest.mark.parametrize("codes", ["int4", "int8", "mxfp4"])
def test_gemm_wide_output(cr, codes, N):
    M, Kp = 3, 64
    print(f"\n[case] {codes} gemm M={M} N={N} Kp={Kp}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(N % 1000 + len(codes))
    if codes == "int8":
        xq = torch.randint(-128, 128, (M, Kp), dtype=torch.int8, device=DEV, generator=gen)
        wq = torch.randint(-128, 128, (N, Kp), dtype=torch.int8, device=DEV, generator=gen)
    else:
        xq = torch.randint(0, 256, (M, Kp // 2), dtype=torch.uint8, device=DEV, generator=gen)
        wq = torch.randint(0, 256, (N, Kp // 2), dtype=torch.uint8, device=DEV, generator=gen)
    bias = torch.randn(N, device=DEV, generator=gen).to(torch.bfloat16)
    if codes == "mxfp4":
        S = cr.mx_scale_stride(Kp)
        xf = torch.randint(118, 136, (M, S), dtype=torch.uint8, device=DEV, generator=gen)
        wf = torch.randint(118, 136, (N, S), dtype=torch.uint8, device=DEV, generator=gen)
        y, acc = cr.convrot_mxfp4_gemm(xq, xf, wq, wf, bias, want_acc=True)
    else:
        xf = torch.rand(M, device=DEV, generator=gen) * 0.01 + 1e-3
        wf = torch.rand(N, device=DEV, generator=gen) * 0.01 + 1e-3
        gemm = cr.convrot_w4a4_gemm if codes == "int4" else cr.convrot_w8a8_gemm
        y, acc = gemm(xq, xf, wq, wf, bias, want_acc=True)
    torch.cuda.synchronize()
    cols = _sample(N, np.random.default_rng(N), around=(1 << 26, 1 << 27))
    ct = torch.from_numpy(cols).to(DEV)
    b = bias[ct].float().cpu().numpy()
    xqh, wqh = xq.cpu().numpy(), wq[ct].cpu().numpy()
    if codes == "mxfp4":
        nb = Kp // 32
        ref = O.mxfp4_linear_from_codes(O.unpack_int4(xqh) & 0xF, xf.cpu().numpy()[:, :nb],
                                        O.unpack_int4(wqh) & 0xF, wf[ct].cpu().numpy()[:, :nb], b)
        check_mx_gemm(y[:, ct], acc[:, ct], ref, Kp, b, f"N={N}")
        return
    if codes == "int4":
        ref = O.w4a4_linear_from_codes(O.unpack_int4(xqh), xf.cpu().numpy(), O.unpack_int4(wqh),
                                       wf[ct].cpu().numpy(), b)
    else:
        ref = O.w8a8_linear_from_codes(xqh, xf.cpu().numpy(), wqh, wf[ct].cpu().numpy(), b)
    assert np.array_equal(acc[:, ct].cpu().numpy(), ref["acc"]), "int32 sums differ"
    ybits = y[:, ct].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ybits, ref["out_bits"]), "outputs differ"


def test_rotate_quant_tall_input(cr):
    K = g = 64
    print(f"\n[case] rotate_quant all formats M={M_TALL} K={K} g={g} bf16", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(29)
    x = torch.randn((M_TALL, K), device=DEV, dtype=torch.bfloat16, generator=gen)
    rows = _sample(M_TALL, np.random.default_rng(29), around=(1 << 28, 1 << 29))
    rt = torch.from_numpy(rows).to(DEV)
    xh = x[rt].float().cpu().numpy()

    q, s = cr.convrot_rotate_quant_act(x, g)
    torch.cuda.synchronize()
    check_rotate_quant(q[rt], s[rt], None, O.rotate_quantize(xh, g), "int4")
    del q, s
    torch.cuda.empty_cache()

    q, s = cr.convrot_rotate_quant_act_i8(x, g)
    torch.cuda.synchronize()
    check_i8(q[rt], s[rt], None, O.rotate_quantize_int8(xh, g), "int8")
    del q, s
    torch.cuda.empty_cache()

    kp = cr.convrot_padded_k(K, g)
    q = torch.empty((M_TALL, kp // 2), dtype=torch.uint8, device=DEV)
    bs = torch.full((M_TALL, cr.mx_scale_stride(kp)), 0xAA, dtype=torch.uint8, device=DEV)
    cr.convrot_rotate_quant_act_mxfp4(x, g, q, bs)
    torch.cuda.synchronize()
    check_mx(q[rt], bs[rt], None, O.rotate_quantize_mxfp4(xh, g), "mxfp4")
    assert not torch.any(bs == 0xAA), "block-scale bytes left unwritten"


def test_rotate_quant_row_stride_past_2gib(cr):
    """Rows 2^30 bf16 elements apart (a 2 GiB stride); the gaps hold a large sentinel, so a
    read past a row's K columns would change its scale."""
    M, K, g, ld = 3, 3100, 256, 1 << 30
    print(f"\n[case] rotate_quant all formats M={M} K={K} g={g} ldx={ld} bf16", flush=True)
    base = torch.full(((M - 1) * ld + K,), 1e4, dtype=torch.bfloat16, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(31)
    rows = torch.randn((M, K), device=DEV, dtype=torch.bfloat16, generator=gen)
    x = base.as_strided((M, K), (ld, 1))
    x.copy_(rows)
    xh = rows.float().cpu().numpy()
    q, s = cr.convrot_rotate_quant_act(x, g)
    q8, s8 = cr.convrot_rotate_quant_act_i8(x, g)
    qm, bm = cr.convrot_rotate_quant_act_mxfp4(x, g)
    torch.cuda.synchronize()
    check_rotate_quant(q, s, None, O.rotate_quantize(xh, g), "int4")
    check_i8(q8, s8, None, O.rotate_quantize_int8(xh, g), "int8")
    check_mx(qm, bm, None, O.rotate_quantize_mxfp4(xh, g), "mxfp4")


@pytest.mark.parametrize("M,N", [(40, 70), (1100, 2000)])
@pytest.mark.parametrize("codes", ["int4", "int8", "mxfp4"])
def test_gemm_max_depth(cr, codes, M, N):
    """K' = CONVROT_MAX_KP (65536), the skinny and the tiled kernel.  Row 0 of both operands
    holds the most negative code everywhere, so int8 sums reach 16384 K' = 2^30; the other
    rows are random full-range codes."""
    Kp = 65536
    print(f"\n[case] {codes} gemm max depth M={M} N={N} Kp={Kp}", flush=True)
    rng = np.random.default_rng(M + N)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    b = rng.standard_normal(N).astype(np.float32)
    b = O.bf16_bits_to_f32(O.f32_to_bf16_bits(b))
    bias = dev(b).to(torch.bfloat16)
    if codes == "int8":
        cx = rng.integers(-128, 128, size=(M, Kp)).astype(np.int8)
        cw = rng.integers(-128, 128, size=(N, Kp)).astype(np.int8)
        cx[0], cw[0] = -128, -128
        xq, wq = dev(cx), dev(cw)
    else:
        cx = rng.integers(-8, 8, size=(M, Kp)).astype(np.int8)
        cw = rng.integers(-8, 8, size=(N, Kp)).astype(np.int8)
        if codes == "mxfp4":
            cx, cw = cx & 0xF, cw & 0xF  # E2M1 codes 0..15; 0xF is -6, the largest magnitude
            cx[0], cw[0] = 0xF, 0xF
        else:
            cx[0], cw[0] = -8, -8
        xq, wq = dev(O.pack_int4(cx)), dev(O.pack_int4(cw))
    if codes == "mxfp4":
        S = cr.mx_scale_stride(Kp)
        ex = rng.integers(118, 136, size=(M, S)).astype(np.uint8)
        ew = rng.integers(118, 136, size=(N, S)).astype(np.uint8)
        y, acc = cr.convrot_mxfp4_gemm(xq, dev(ex), wq, dev(ew), bias, want_acc=True)
        torch.cuda.synchronize()
        nb = Kp // 32
        ref = O.mxfp4_linear_from_codes(cx.astype(np.uint8), ex[:, :nb], cw.astype(np.uint8),
                                        ew[:, :nb], b)
        check_mx_gemm(y, acc, ref, Kp, b, f"M={M} N={N}")
        return
    sx = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    sw = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    gemm = cr.convrot_w4a4_gemm if codes == "int4" else cr.convrot_w8a8_gemm
    y, acc = gemm(xq, dev(sx), wq, dev(sw), bias, want_acc=True)
    torch.cuda.synchronize()
    ref = O.w8a8_linear_from_codes(cx, sx, cw, sw, b)
    a = acc.cpu().numpy()
    assert a[0, 0] == (16384 if codes == "int8" else 64) * Kp
    assert np.array_equal(a, ref["acc"]), "int32 sums differ"
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref["out_bits"])
