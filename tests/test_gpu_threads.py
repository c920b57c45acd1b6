"""Calls from several host threads at once (needs a gfx950 GPU).

The library's host code is re-entrant: four threads, each with a stream of its own, run the
forward pass of every code format on their own inputs concurrently (ctypes releases the
interpreter lock during each call).  Every result must be bit-identical to the same call made
alone from one thread.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import workloads as wk

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = 4
ROUNDS = 8


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


@pytest.mark.parametrize("codes", ["int4", "int8", "mxfp4"])
def test_concurrent_threads_match_single_thread(cr, codes):
    print(f"\n[case] {THREADS} host threads x {ROUNDS} rounds, {codes}", flush=True)
    quant_w, linear = {
        "int4": (cr.convrot_quant_weight, cr.convrot_w4a4_linear),
        "int8": (cr.convrot_quant_weight_i8, cr.convrot_w8a8_linear),
        "mxfp4": (cr.convrot_quant_weight_mxfp4, cr.convrot_mxfp4_linear),
    }[codes]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(DEV)  # noqa: E731
    # per thread: its own shape (tiled and skinny GEMMs, ragged windows) and inputs
    shapes = [(512, 3072, 1024, 256), (64, 1024, 512, 64), (300, 3100, 200, 256),
              (700, 2048, 768, 1024)]
    jobs = []
    for t, (M, K, N, g) in enumerate(shapes[:THREADS]):
        wl = wk.custom(f"th{t}", M, K, N, g, x_dtype="bf16", bias_std=0.01)
        wq, ws = quant_w(to(wk.weights(wl)), g)
        jobs.append((to(wk.activations(wl)), g, wq, ws, to(wk.bias(wl))))
    torch.cuda.synchronize()
    alone = [linear(x, g, wq, ws, b) for x, g, wq, ws, b in jobs]
    torch.cuda.synchronize()

    outs = [[None] * ROUNDS for _ in jobs]
    errors = []
    barrier = threading.Barrier(len(jobs))

    def work(t):
        try:
            x, g, wq, ws, b = jobs[t]
            stream = torch.cuda.Stream(device=DEV)  # default priority
            barrier.wait()
            with torch.cuda.stream(stream):
                for r in range(ROUNDS):
                    outs[t][r] = linear(x, g, wq, ws, b)
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=work, args=(t,)) for t in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for t, ref in enumerate(alone):
        for r in range(ROUNDS):
            assert torch.equal(outs[t][r].view(torch.int16), ref.view(torch.int16)), \
                f"thread {t}, round {r}: differs from the single-thread result"
