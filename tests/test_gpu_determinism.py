"""Determinism and complete writes on the GPU, through the C ABI (needs a gfx950 GPU).

Every kernel runs twice on the same inputs, into output buffers pre-filled with two different
canary patterns. The two results must be bit-identical: a race would make them differ, and so
would any output element or padding byte that a kernel leaves unwritten (it keeps its canary).
The cases follow the kernel selection: the 256 x 256 tiled GEMM (also in its 4-byte transfer
form for packed rows of 8 (mod 16) bytes) and the skinny GEMM (also with 8-byte row tails),
for each code format, and the rotate+quantize kernels of each format.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CANARIES = (0xAA, 0x55)


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _filled(shape, dtype, byte):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(byte)
    return t


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


GEMM_CASES = [
    # codes, M, N, Kp, kernel chosen by the library for this shape
    ("int4", 1024, 2048, 512, "tiled"), ("int4", 4000, 4090, 256, "tiled"),
    ("int4", 100, 300, 512, "skinny"),
    ("int4", 70, 90, 48, "skinny-tail8"), ("int4", 2100, 1100, 208, "tiled-4-byte"),
    ("int8", 1024, 2048, 256, "tiled"), ("int8", 100, 300, 512, "skinny"),
    ("mxfp4", 1024, 2048, 512, "tiled"), ("mxfp4", 100, 300, 512, "skinny"),
]


@pytest.mark.parametrize("codes,M,N,Kp,path", GEMM_CASES)
def test_gemm_deterministic_and_complete(cr, codes, M, N, Kp, path):
    _announce(f"{codes} gemm {path} M={M} N={N} Kp={Kp}")
    rng = np.random.default_rng(M * 7 + N + Kp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    bias = dev(wk.round_to_dtype(rng.standard_normal(N).astype(np.float32), "bf16")).to(torch.bfloat16)
    if codes == "int8":
        xq = dev(rng.integers(-128, 128, size=(M, Kp)).astype(np.int8))
        wq = dev(rng.integers(-128, 128, size=(N, Kp)).astype(np.int8))
    else:
        xq = dev(rng.integers(0, 256, size=(M, Kp // 2)).astype(np.uint8))
        wq = dev(rng.integers(0, 256, size=(N, Kp // 2)).astype(np.uint8))
    if codes == "mxfp4":
        S = cr.mx_scale_stride(Kp)
        a = dev(rng.integers(118, 136, size=(M, S)).astype(np.uint8))
        b = dev(rng.integers(118, 136, size=(N, S)).astype(np.uint8))
        run = lambda y, acc: cr.convrot_mxfp4_gemm(xq, a, wq, b, bias, y=y, want_acc=acc)  # noqa: E731
        acc_dtype = torch.float32
    else:
        a = dev(wk.random_scales(M, 1))
        b = dev(wk.random_scales(N, 2))
        gemm = cr.convrot_w4a4_gemm if codes == "int4" else cr.convrot_w8a8_gemm
        run = lambda y, acc: gemm(xq, a, wq, b, bias, y=y, want_acc=acc)  # noqa: E731
        acc_dtype = torch.int32
    outs = []
    for byte in CANARIES:
        y = _filled((M, N), torch.bfloat16, byte)
        y2 = _filled((M, N), torch.bfloat16, byte)
        y_dbg, acc = run(y2, True)
        run(y, False)
        outs.append((y, y_dbg, acc))
    torch.cuda.synchronize()
    assert acc.dtype == acc_dtype
    assert _same_bits(outs[0][0], outs[1][0]), "production outputs differ between runs"
    assert _same_bits(outs[0][1], outs[1][1]), "debug outputs differ between runs"
    assert _same_bits(outs[0][2], outs[1][2]), "accumulators differ between runs"
    assert _same_bits(outs[0][0], outs[0][1]), "production and debug instantiations differ"


RQ_CASES = [
    # format, M, K, g
    ("int4", 37, 3100, 256), ("int4", 5, 3000, 1024), ("int8", 37, 3100, 256),
    ("int8", 9, 1000, 64), ("mxfp4", 37, 3100, 256), ("mxfp4", 9, 950, 64),
    ("mxfp4", 3, 2000, 1024),
]


@pytest.mark.parametrize("fmt,M,K,g", RQ_CASES)
def test_rotate_quant_deterministic_and_complete(cr, fmt, M, K, g):
    _announce(f"{fmt} rotate_quant M={M} K={K} g={g}")
    wl = wk.custom("t", M, K, None, g)
    x = torch.from_numpy(wk.activations(wl)).to(torch.bfloat16).to(DEV)
    Kp = cr.convrot_padded_k(K, g)
    outs = []
    for byte in CANARIES:
        xr = _filled((M, Kp), torch.float32, byte)
        if fmt == "int4":
            q = _filled((M, Kp // 2), torch.uint8, byte)
            s = _filled((M,), torch.float32, byte)
            cr.convrot_rotate_quant_act(x, g, q, s, xr)
        elif fmt == "int8":
            q = _filled((M, Kp), torch.int8, byte)
            s = _filled((M,), torch.float32, byte)
            cr.convrot_rotate_quant_act_i8(x, g, q, s, xr)
        else:
            q = _filled((M, Kp // 2), torch.uint8, byte)
            s = _filled((M, cr.mx_scale_stride(Kp)), torch.uint8, byte)
            cr.convrot_rotate_quant_act_mxfp4(x, g, q, s, xr)
        outs.append((q, s, xr))
    torch.cuda.synchronize()
    for i, name in enumerate(("codes", "scales", "rotated values")):
        assert _same_bits(outs[0][i], outs[1][i]), f"{name} differ between runs or are unwritten"
    if fmt == "mxfp4":  # the scale rows' padding bytes are written as zero
        nb = Kp // 32
        assert torch.all(outs[0][1][:, nb:] == 0)
