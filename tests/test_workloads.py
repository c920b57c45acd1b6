"""Seeded synthetic inputs: deterministic, dtype-exact, outliers where stated (CPU only)."""
import numpy as np

import workloads as wk


def test_tiny_recipe():
    wl = wk.WORKLOADS["tiny"]
    x1, x2 = wk.activations(wl), wk.activations(wl)
    assert x1.shape == (64, 256) and x1.dtype == np.float32
    assert np.array_equal(x1, x2)
    big_rows = np.sum(np.median(np.abs(x1), axis=1) > 10)
    assert big_rows == 2
    w = wk.weights(wl)
    assert w.shape == (256, 256) and abs(float(w.std()) - 0.02) < 0.002
    assert wk.bias(wl) is None


def test_bf16_exact_and_outliers():
    wl = wk.custom("t", 200, 300, 64, 256)
    x = wk.activations(wl)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)            # bf16-exact values
    assert wl.Kp == 512
    assert np.sum(np.median(np.abs(x), axis=1) > 10) == wl.n_out_rows


def test_full_workload_table():
    t = wk.WORKLOADS
    assert (t["attn_proj"].M, t["attn_proj"].K, t["attn_proj"].N, t["attn_proj"].g) == (4608, 3072, 3072, 256)
    assert t["rotate_quant"].n_out_rows == 46
    assert t["mlp_down"].Kp == 12288 and t["mlp_down"].n_out_rows == 23
    assert t["proj_out"].n_out_rows == 92
    assert t["proj_out_padded"].Kp == 3328
    assert (t["few_tokens"].M, t["few_tokens"].N, t["few_tokens"].n_out_rows) == (64, 3072, 1)
