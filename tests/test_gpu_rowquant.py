"""The analysis helpers convrot_quant_rows_int4 / convrot_dequant_int4 against the oracle (needs
a gfx950 GPU): the layer's per-row int4 rule without the rotation (scale = fp32(max / 7), code =
clamp(rne(fp32(y / scale)), -8, 7), two codes per byte) and the exact fp64 dequantization.
Scales and codes are bit-exact: both sides divide in fp32 with IEEE rounding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

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


def _rows(M, K, seed):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, size=(M, 1)))
    y = y.astype(np.float32)
    y[1] = 0.0                                              # a zero row: scale 0, codes 0
    if K >= 7:                                              # exact ties: max 7 gives scale 1
        y[2, :7] = [7.0, 2.5, -2.5, 3.5, -0.5, 0.5, 1.5]
        y[2, 7:] = 0.0
    y[3] *= np.float32(1e-38)                               # scale and quotients near subnormal
    return y


def _oracle(y):
    s = O.row_scales(y)
    q = O.quantize(y, s)
    if q.shape[1] % 2:
        q = np.concatenate([q, np.zeros((q.shape[0], 1), dtype=q.dtype)], axis=1)
    return s, q


@pytest.mark.parametrize("M,K", [(8, 16), (37, 97), (300, 3072), (5, 1)])
def test_quant_rows_matches_oracle(cr, M, K):
    print(f"\n[case] quant_rows_int4 M={M} K={K}", flush=True)
    y = _rows(M, K, seed=M + K)
    q, s = cr.convrot_quant_rows_int4(torch.from_numpy(y).to(DEV))
    torch.cuda.synchronize()
    s_ref, q_ref = _oracle(y)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(O.unpack_int4(q.cpu().numpy()), q_ref)
    if M > 2 and K >= 7:
        assert list(O.unpack_int4(q.cpu().numpy())[2, :7]) == [7, 2, -2, 4, 0, 0, 2]


def test_quant_rows_strided(cr):
    print("\n[case] quant_rows_int4 strided rows", flush=True)
    wide = _rows(20, 300, seed=4)
    y = torch.from_numpy(wide).to(DEV)[:, 13:13 + 201]     # row stride 300, K = 201
    q, s = cr.convrot_quant_rows_int4(y)
    torch.cuda.synchronize()
    s_ref, q_ref = _oracle(np.ascontiguousarray(wide[:, 13:13 + 201]))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(O.unpack_int4(q.cpu().numpy()), q_ref)


@pytest.mark.parametrize("M,K", [(9, 64), (33, 97)])
def test_dequant_is_exact(cr, M, K):
    print(f"\n[case] dequant_int4 M={M} K={K}", flush=True)
    rng = np.random.default_rng(K)
    packed = rng.integers(0, 256, size=(M, (K + 1) // 2), dtype=np.int64).astype(np.uint8)
    s = (rng.standard_normal(M) * np.exp2(rng.integers(-100, 100, size=M))).astype(np.float32)
    out = cr.convrot_dequant_int4(torch.from_numpy(packed).to(DEV), torch.from_numpy(s).to(DEV), K)
    torch.cuda.synchronize()
    ref = O.unpack_int4(packed)[:, :K].astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.array_equal(out.cpu().numpy(), ref)
