"""The C ABI from a plain C program (tests/native/convrot_client.c): no Python, C++ or torch in
the calling process.

Without a GPU: the client links against libconvrot.so and the HIP runtime, and every invalid
call it makes comes back as the status code include/convrot.h documents, before any device
work.  On the GPU: the client's ConvLinear4bit forward pass (weights quantized, workspace
sized and allocated, forward on its own stream, all through the header's entry points) is
bit-identical to the same calls made through the Python binding, and within the 1e-2
relative Frobenius bar of the oracle.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import workloads as wk
from oracle import convrot_oracle as O
from tests.native import build as native

CLIENT = native.CLIENT


def _client():
    if not os.path.exists(CLIENT):
        pytest.skip("C ABI client not built (tests/native/build.py)")
    return CLIENT


def _run(args, timeout=120):
    return subprocess.run([_client(), *args], capture_output=True, text=True, timeout=timeout)


def test_client_validation_without_device_work():
    r = _run(["errors"], timeout=60)
    assert r.returncode == 0, r.stderr
    assert "validation checks ok" in r.stdout


def test_client_usage_error():
    r = _run(["forward", "too", "few"], timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def _bf16_bits(a):
    return O.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


CASES = [
    # M, K, N, g, bias: the tiled GEMM with a ragged window tail, and the skinny GEMM
    (300, 3100, 200, 256, True),
    (64, 1024, 96, 64, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,g,with_bias", CASES)
def test_client_forward_matches_binding_and_oracle(tmp_path, M, K, N, g, with_bias):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as cr
    cr.load_library()  # raises if the HIP library is missing: no fallback
    print(f"\n[case] C client forward M={M} K={K} N={N} g={g} bias={with_bias}", flush=True)
    wl = wk.custom("c", M, K, N, g, x_dtype="bf16", bias_std=0.01 if with_bias else None)
    x, w, b = wk.activations(wl), wk.weights(wl), wk.bias(wl)
    paths = {k: str(tmp_path / f"{k}.bin") for k in ("x", "w", "b", "y")}
    _bf16_bits(x).tofile(paths["x"])
    _bf16_bits(w).tofile(paths["w"])
    if b is not None:
        _bf16_bits(b).tofile(paths["b"])
    r = _run(["forward", paths["x"], paths["w"], paths["b"] if b is not None else "-",
              str(M), str(K), str(N), str(g), paths["y"]])
    assert r.returncode == 0, r.stderr
    y_c = np.fromfile(paths["y"], dtype=np.uint16).reshape(M, N)

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev)  # noqa: E731
    wq, ws = cr.convrot_quant_weight(to(w), g)
    y_py = cr.convrot_w4a4_linear(to(x), g, wq, ws, None if b is None else to(b))
    torch.cuda.synchronize()
    y_py = y_py.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(y_c, y_py), "the C client and the Python binding disagree"

    ref = O.convlinear4bit(x, w, b, g)
    yo = O.bf16_bits_to_f32(ref["out_bits"]).astype(np.float64)
    frob = np.linalg.norm(O.bf16_bits_to_f32(y_c).astype(np.float64) - yo) / np.linalg.norm(yo)
    assert frob <= 1e-2, f"rel Frobenius {frob:.2e}"
