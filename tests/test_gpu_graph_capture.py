"""The forward pass captured in a HIP graph (needs a gfx950 GPU).

A caller may capture the library's calls with stream capture: every entry point only
enqueues kernels on the stream it is given (no allocation, no memset, no synchronisation).
Each format's forward pass is captured over several input buffers, with caller-owned
outputs and workspace, and the graph is replayed several times with eager work of the
program in between; every replay must be bit-identical to the eager result of the same
input, and inputs changed in place between replays must be picked up.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wk

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


def _variant(cr, codes):
    if codes == "int4":
        return cr.convrot_quant_weight, cr.convrot_w4a4_linear, cr.convrot_w4a4_workspace_bytes
    if codes == "int8":
        return cr.convrot_quant_weight_i8, cr.convrot_w8a8_linear, cr.convrot_w8a8_workspace_bytes
    return cr.convrot_quant_weight_mxfp4, cr.convrot_mxfp4_linear, cr.convrot_mxfp4_workspace_bytes


CASES = [
    # codes, M, K, N, g: the tiled GEMM, the skinny GEMM, and a ragged window tail
    ("int4", 1024, 3072, 2048, 256), ("int4", 64, 1024, 512, 64), ("int4", 300, 3100, 200, 256),
    ("int8", 1024, 3072, 2048, 256), ("int8", 64, 1024, 512, 64),
    ("mxfp4", 1024, 3072, 2048, 256), ("mxfp4", 64, 1024, 512, 64),
]


@pytest.mark.parametrize("codes,M,K,N,g", CASES)
def test_graph_replays_match_eager(cr, codes, M, K, N, g):
    print(f"\n[case] graph capture {codes} M={M} K={K} N={N} g={g}", flush=True)
    quant_w, linear, ws_bytes = _variant(cr, codes)
    wl = wk.custom("gc", M, K, N, g, x_dtype="bf16", bias_std=0.01)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(DEV)  # noqa: E731
    x = to(wk.activations(wl))
    xs = [x, x.flip(0).contiguous(), (x * 0.5).contiguous()]  # three different inputs
    wq, wsc = quant_w(to(wk.weights(wl)), g)
    bias = to(wk.bias(wl))
    work = torch.empty((ws_bytes(M, K, g),), dtype=torch.uint8, device=DEV)
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in xs]

    eager = [linear(xi, g, wq, wsc, bias, y=torch.empty_like(ys[0]), workspace=work).clone()
             for xi in xs]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
        for xi, yi in zip(xs, ys):
            linear(xi, g, wq, wsc, bias, y=yi, workspace=work)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for xi, yi in zip(xs, ys):
            linear(xi, g, wq, wsc, bias, y=yi, workspace=work)
    torch.cuda.synchronize()

    for rep in range(3):
        for yi in ys:
            yi.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (yi, ei) in enumerate(zip(ys, eager)):
            assert torch.equal(yi.view(torch.int16), ei.view(torch.int16)), \
                f"replay {rep}: output {i} differs from the eager result"
        # eager work of the program between replays, on the same buffers
        linear(xs[0], g, wq, wsc, bias, y=torch.empty_like(ys[0]), workspace=work)
        torch.cuda.synchronize()

    # inputs changed in place are read by the next replay
    xs[2].copy_(xs[1])
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(ys[2].view(torch.int16), eager[1].view(torch.int16))
