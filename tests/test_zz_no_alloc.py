"""convrot_w4a4_linear_noalloc against convrot_w4a4_linear (needs a gfx950 GPU).

The no-allocation entry point runs the same two kernels with its activation codes in the
library's fixed device array instead of a caller workspace, so its output must be
bit-identical to convrot_w4a4_linear's on the same inputs.  Two calls in a row, the second
smaller, show that the array's leftover contents from the first call do not leak into the
second; a problem too large for the array is refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()
    return mod


def _layer(cr, M, K, N, g, seed, with_bias):
    wl = wk.custom(f"noalloc{seed}", M, K, N, g, bias_std=0.01 if with_bias else None)
    x = torch.from_numpy(wk.activations(wl)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(wk.weights(wl)).to(torch.bfloat16).to(DEV)
    b = wk.bias(wl)
    bias = None if b is None else torch.from_numpy(b).to(torch.bfloat16).to(DEV)
    wq, ws = cr.convrot_quant_weight(w, g)
    return wl, x, wq, ws, bias


def _bits(y):
    return y.view(torch.int16).cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice(cr):
    # large first call, then a smaller one with another g: the second must not see the first's
    # codes, and both must equal the workspace entry point's output bit for bit
    cases = [(2304, 3072, 1536, 256, 11, True), (100, 1000, 300, 64, 12, False)]
    for M, K, N, g, seed, with_bias in cases:
        print(f"\n[case] noalloc M={M} K={K} N={N} g={g} bias={with_bias}", flush=True)
        wl, x, wq, ws, bias = _layer(cr, M, K, N, g, seed, with_bias)
        y_ref = cr.convrot_w4a4_linear(x, g, wq, ws, bias)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        out = cr.convrot_w4a4_linear_noalloc(x, g, wq, ws, bias, y=y)
        torch.cuda.synchronize()
        assert out is y
        assert np.array_equal(_bits(y), _bits(y_ref)), "noalloc output differs"
        # and the end-to-end bar against the oracle
        ref = O.convlinear4bit(wk.activations(wl), wk.weights(wl), wk.bias(wl), g)
        yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
        frob = np.linalg.norm(y.float().cpu().numpy() - yo) / np.linalg.norm(yo)
        assert frob <= 1e-2, f"rel. Frobenius error {frob:.2e}"


def test_noalloc_refuses_oversize_and_keeps_output(cr):
    print("\n[case] noalloc oversize", flush=True)
    K, g = 3072, 256
    M = 49025        # one row past the fixed array (codes 1536 B + scale per row)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros((8, K // 2), dtype=torch.uint8, device=DEV)
    ws = torch.zeros((8,), dtype=torch.float32, device=DEV)
    y = torch.full((M, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(cr.ConvRotError) as e:
        cr.convrot_w4a4_linear_noalloc(x, g, wq, ws, None, y=y)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "an output was written by a refused call"
