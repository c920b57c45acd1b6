"""The outlier-suppression tool on the GPU: its regular-transform statistics come from the
HIP kernels and must equal the oracle's; on inputs with same-sign row outliers it must show
Figure 2's direction (group-wise regular below the original, global Sylvester above it)."""
import numpy as np
import pytest
import torch

import workloads as wk
from oracle import convrot_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tool():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_w4a4_quantized_convrot_amd as mod
    from rotation_w4a4_quantized_convrot_amd import outliers
    mod.load_library()
    return outliers


def _inputs(M=96, K=1000, N=128):
    x = wk.offset_row_outliers(M, K, 3, 20.0, dtype="bf16")
    wl = wk.custom("t", M, K, N, 256)
    return x, wk.weights(wl)


def test_regular_statistics_match_oracle(tool):
    print("\n[case] outlier tool vs oracle, M=96 K=1000", flush=True)
    x, w = _inputs()
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).to(torch.bfloat16).cuda()
    res = tool.analyze(xd, (16, 256), wd)
    for r in res["transforms"]:
        if r["transform"] != "regular":
            continue
        ref = O.rotate_quantize(x, r["g"])
        assert r["column_discrepancy"] == np.sqrt(r["g"])
        assert r["max_abs"] == pytest.approx(float(np.max(np.abs(ref["yf"]))), rel=1e-6)
        deq = ref["codes"].astype(np.float64) * ref["scale"].astype(np.float64)[:, None]
        yf = ref["yf"].astype(np.float64)
        err = np.linalg.norm(deq - yf) / np.linalg.norm(yf)
        assert r["act_int4_rel_err"] == pytest.approx(err, rel=1e-4)
        exact = x.astype(np.float64) @ w.astype(np.float64).T
        refw = O.quantize_weight(w, r["g"])
        out = deq @ (refw["codes"].astype(np.float64) * refw["scale"].astype(np.float64)[:, None]).T
        e4 = np.linalg.norm(out - exact) / np.linalg.norm(exact)
        # a weight code off by one at a rounding tie moves this error measurably when it meets
        # an outlier activation, hence the loose bar against the oracle's codes ...
        assert r["w4a4_rel_err"] == pytest.approx(e4, rel=1e-2)
        assert r["w4a4_rel_err_kernel_bf16"] == pytest.approx(e4, rel=0.05)
        # ... and the exact one against the same arithmetic on the kernels' own codes
        import rotation_w4a4_quantized_convrot_amd as cr
        xq, xs = cr.convrot_rotate_quant_act(xd, r["g"])
        wq, ws = cr.convrot_quant_weight(wd, r["g"])
        dx = O.unpack_int4(xq.cpu().numpy()) * xs.cpu().numpy().astype(np.float64)[:, None]
        dw = O.unpack_int4(wq.cpu().numpy()) * ws.cpu().numpy().astype(np.float64)[:, None]
        ek = np.linalg.norm(dx @ dw.T - exact) / np.linalg.norm(exact)
        assert r["w4a4_rel_err"] == pytest.approx(ek, rel=1e-9)


def test_figure2_direction(tool):
    print("\n[case] outlier tool: figure 2 direction", flush=True)
    x, w = _inputs(M=256, K=3072, N=256)
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).to(torch.bfloat16).cuda()
    res = {(r["transform"], r["g"]): r for r in tool.analyze(xd, (256,), wd)["transforms"]}
    none = res[("none", None)]
    reg = res[("regular", 256)]
    glob = res[("sylvester_global", 4096)]
    assert reg["max_abs"] < none["max_abs"] < glob["max_abs"]
    assert reg["w4a4_rel_err"] < glob["w4a4_rel_err"]
    assert reg["w4a4_rel_err"] < none["w4a4_rel_err"]
