"""Inputs at every alignment the API accepts (needs a gfx950 GPU).

x may start at any element boundary and have any row stride >= K.  bf16 rows that are not
4-byte aligned, or whose stride is odd, are read element by element; everything else with
16-byte loads, since buffer loads need dword alignment only.  Each case takes a column window
of a wider tensor (so the bytes around every row are other data), in every code format, and
checks codes and scales against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O
from tests.test_gpu_mxfp4 import check_mx
from tests.test_gpu_parity import check_rotate_quant
from tests.test_gpu_w8a8 import check_i8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


CASES = [
    # dtype, first column of the window, row stride (elements), K, g
    ("bf16", 1, 1024, 700, 256),   # 2-byte aligned rows
    ("bf16", 0, 1023, 700, 256),   # odd stride
    ("bf16", 3, 1023, 1000, 64),   # both, ragged window tail
    ("bf16", 2, 1026, 1024, 1024), # 4-byte aligned, stride not a multiple of 8 elements
    ("f32", 1, 1025, 700, 256),    # fp32: dword aligned, odd stride
    ("f32", 3, 3103, 3100, 256),
]


@pytest.mark.parametrize("codes", ["int4", "int8", "mxfp4"])
@pytest.mark.parametrize("dtype,c0,ld,K,g", CASES)
def test_rotate_quant_any_alignment(cr, codes, dtype, c0, ld, K, g):
    M = 37
    print(f"\n[case] {codes} rotate_quant {dtype} column {c0} stride {ld} K={K} g={g}", flush=True)
    wl = wk.custom("al", M, K, None, g, x_dtype=dtype)
    x = wk.activations(wl)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # the bytes around every row hold large values, so a read outside the row shows up
    wide = torch.full((M, ld), 3.0e4, dtype=tdt, device=DEV)
    view = wide[:, c0:c0 + K]
    view.copy_(torch.from_numpy(x).to(tdt))
    assert view.stride(0) == ld and view.data_ptr() % (4 if dtype == "f32" else 2) == 0
    torch.cuda.synchronize()
    if codes == "int4":
        q, s = cr.convrot_rotate_quant_act(view, g)
        torch.cuda.synchronize()
        check_rotate_quant(q, s, None, O.rotate_quantize(x, g), "int4")
    elif codes == "int8":
        q, s = cr.convrot_rotate_quant_act_i8(view, g)
        torch.cuda.synchronize()
        check_i8(q, s, None, O.rotate_quantize_int8(x, g), "int8")
    else:
        q, bs = cr.convrot_rotate_quant_act_mxfp4(view, g)
        torch.cuda.synchronize()
        check_mx(q, bs, None, O.rotate_quantize_mxfp4(x, g), "mxfp4")
