"""The single-launch ConvLinear4bit (convrot_w4a4_linear_fused) against the two-kernel path
(needs a gfx950 GPU).

Both run the same per-element arithmetic, so the fused call's activation codes and scales (in
its workspace) and its bf16 output must be bit-identical to convrot_rotate_quant_act +
convrot_w4a4_linear on the same input; the end-to-end output is also held to the oracle's bar
(1e-2 relative Frobenius).  Several calls in a row check that the grid barrier's counter is
back at zero after each call, and the status word stays zero (no barrier timed out).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # M, K, N, g, bias: the attention projection, an MLP down-projection slice, a padded
    # ragged layer (K' = 3328) and a layer with fewer row blocks and tiles than workgroups
    (4608, 3072, 3072, 256, True),
    (1000, 12288, 3072, 1024, False),
    (1130, 3100, 1990, 256, True),
    (100, 512, 200, 256, False),
    (9216, 15360, 3072, 1024, False),
]


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()
    return mod


def _layer(cr, M, K, N, g, with_bias, seed):
    wl = wk.custom(f"fused{seed}", M, K, N, g, bias_std=0.01 if with_bias else None)
    x = torch.from_numpy(wk.activations(wl)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(wk.weights(wl)).to(torch.bfloat16).to(DEV)
    b = wk.bias(wl)
    bias = None if b is None else torch.from_numpy(b).to(torch.bfloat16).to(DEV)
    wq, ws = cr.convrot_quant_weight(w, g)
    return wl, x, wq, ws, bias


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def test_fused_matches_two_kernel_path(cr):
    status = torch.zeros((1,), dtype=torch.int32, device=DEV)
    for i, (M, K, N, g, with_bias) in enumerate(CASES):
        print(f"\n[case] fused M={M} K={K} N={N} g={g} bias={with_bias}", flush=True)
        wl, x, wq, ws, bias = _layer(cr, M, K, N, g, with_bias, 20 + i)
        need = cr.convrot_w4a4_workspace_bytes(M, K, g)
        work = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        cr.convrot_w4a4_linear_fused(x, g, wq, ws, bias, y=y, workspace=work, status=status)
        y_ref = cr.convrot_w4a4_linear(x, g, wq, ws, bias)
        xq, xs = cr.convrot_rotate_quant_act(x, g)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "the grid barrier timed out"
        kp = cr.convrot_padded_k(K, g)
        codes = work[: M * kp // 2].view(M, kp // 2)
        off = -(-(M * kp // 2) // 256) * 256
        scales = work[off: off + 4 * M].view(torch.float32)
        assert torch.equal(codes, xq), "fused codes differ from rotate+quantize"
        assert torch.equal(scales.view(torch.int32), xs.view(torch.int32)), "fused scales differ"
        assert np.array_equal(_bits(y), _bits(y_ref)), "fused output differs from the two-kernel path"


def test_fused_end_to_end_against_oracle(cr):
    M, K, N, g = 1130, 3100, 1990, 256
    print(f"\n[case] fused vs oracle M={M} K={K} N={N} g={g}", flush=True)
    wl, x, wq, ws, bias = _layer(cr, M, K, N, g, True, 40)
    y = cr.convrot_w4a4_linear_fused(x, g, wq, ws, bias)
    torch.cuda.synchronize()
    ref = O.convlinear4bit(wk.activations(wl), wk.weights(wl), wk.bias(wl), g)
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(y.float().cpu().numpy() - yo) / np.linalg.norm(yo)
    assert frob <= 1e-2, f"rel. Frobenius error {frob:.2e}"


def test_fused_refuses_unsupported_shapes(cr):
    print("\n[case] fused unsupported", flush=True)
    w = torch.zeros((8, 256), dtype=torch.bfloat16, device=DEV)
    wq, ws = cr.convrot_quant_weight(w, 64)
    with pytest.raises(cr.ConvRotError):   # g = 64
        cr.convrot_w4a4_linear_fused(torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV),
                                     64, wq, ws)
    wq, ws = cr.convrot_quant_weight(w, 256)
    with pytest.raises(cr.ConvRotError):   # fp32 input
        cr.convrot_w4a4_linear_fused(torch.zeros((4, 256), dtype=torch.float32, device=DEV),
                                     256, wq, ws)
