"""Outlier suppression by rotations: a measurement tool (not part of the ConvLinear4bit path).

It shows on synthetic inputs the mechanism behind the ConvRot paper's Figures 1 and 2
(arXiv 2512.03673): a global Sylvester-type Hadamard transform piles a row-wise outlier (a
token whose channels share a large same-sign value) into a single channel, while the
group-wise regular Hadamard transform spreads it evenly.  It also evaluates Definition 2.2's
column discrepancy, read as the largest absolute column sum of the +-1 matrix; by Theorem 2.1
(every H-matrix has squared column sums adding up to n^2) it is at least sqrt(n), with
equality exactly for regular matrices.

For each transform it reports the largest magnitude after the transform (the statistic of
Figure 2), the relative Frobenius error of symmetric per-token int4 quantization of the
transformed activations, and the relative Frobenius error of the whole W4A4 product against
the float64 X W^T (the transform applied to both operands, as the method does).

What runs where:
  * the group-wise regular transform, its int4 codes and scales, the weight codes and the
    ConvLinear4bit output: the HIP kernels, through the C ABI;
  * the comparison transforms the kernels do not implement (none, group-wise Sylvester,
    global Sylvester over the row zero-padded to a power of two): torch on the same device,
    with a fast Walsh-Hadamard transform.  Their int4 codes and scales come from the library's
    convrot_quant_rows_int4 (the layer's quantization rule without the rotation), and every
    dequantization from convrot_dequant_int4: no quantization arithmetic is repeated here.
  * every W4A4 error is evaluated the same way, as the float64 product of the dequantized
    codes; the kernels' own bf16 output error is reported beside it for the regular transform.

Usage: python -m rotation_w4a4_quantized_convrot_amd.outliers [--workload attn_proj]
       [--rows 1024] [--offset 20] [--json out.json]
"""
from __future__ import annotations

import argparse
import json
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _lib

GROUPS = (16, 64, 256, 1024)


def sylvester_pm1(n: int) -> np.ndarray:
    """The +-1 Sylvester-type Hadamard matrix of order n (a power of 2), by doubling."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"order must be a power of 2, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def column_discrepancy(h: np.ndarray) -> float:
    """Largest absolute column sum of a +-1 matrix (Definition 2.2, as read here)."""
    return float(np.max(np.abs(np.asarray(h, dtype=np.float64).sum(axis=0))))


def fwht(y: torch.Tensor) -> torch.Tensor:
    """Unnormalized Walsh-Hadamard transform along the last dimension (length a power of 2):
    y @ S_n^T with S_n the Sylvester matrix of sylvester_pm1."""
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError(f"length must be a power of 2, got {n}")
    lead = y.shape[:-1]
    out = y.reshape(-1, n)
    h = 1
    while h < n:
        v = out.view(-1, n // (2 * h), 2, h)
        out = torch.stack((v[:, :, 0] + v[:, :, 1], v[:, :, 0] - v[:, :, 1]), dim=2).reshape(-1, n)
        h *= 2
    return out.reshape(*lead, n)


def _pad_cols(x: torch.Tensor, width: int) -> torch.Tensor:
    return torch.nn.functional.pad(x, (0, width - x.shape[-1])) if width > x.shape[-1] else x


def sylvester_groups(x: torch.Tensor, g: int) -> torch.Tensor:
    """Group-wise orthonormal Sylvester transform of the rows of x (float64), windows of g."""
    kp = -(-x.shape[1] // g) * g
    y = _pad_cols(x.double(), kp).view(x.shape[0], kp // g, g)
    return (fwht(y) / math.sqrt(g)).reshape(x.shape[0], kp)


def sylvester_global(x: torch.Tensor) -> torch.Tensor:
    """Orthonormal Sylvester transform of each whole row, zero-padded to a power of 2."""
    n = 1 << max(0, (x.shape[1] - 1).bit_length())
    return fwht(_pad_cols(x.double(), n)) / math.sqrt(n)


def int4_dequantized(y: torch.Tensor) -> torch.Tensor:
    """Rows of y (a comparison transform's output, rounded to fp32) quantized to int4 per row
    and dequantized, by the library (fp64 result)."""
    from . import convrot_dequant_int4, convrot_quant_rows_int4
    q, s = convrot_quant_rows_int4(y.float().contiguous())
    return convrot_dequant_int4(q, s, y.shape[1])


def rel_frobenius(a: torch.Tensor, ref: torch.Tensor) -> float:
    den = torch.linalg.norm(ref.double())
    return float(torch.linalg.norm(a.double() - ref.double()) / den) if den > 0 else 0.0


def _row(name: str, g: Optional[int], disc: Optional[float], y: torch.Tensor,
         deq: torch.Tensor, w_deq: Optional[torch.Tensor], ref: Optional[torch.Tensor],
         bias: Optional[torch.Tensor]) -> dict:
    r = {"transform": name, "g": g, "column_discrepancy": disc,
         "max_abs": float(y.abs().max()), "act_int4_rel_err": rel_frobenius(deq, y)}
    if w_deq is not None:
        out = deq @ w_deq.T
        if bias is not None:
            out = out + bias.double()[None, :]
        r["w4a4_rel_err"] = rel_frobenius(out, ref)
    return r


def analyze(x: torch.Tensor, groups: Sequence[int] = GROUPS, w: Optional[torch.Tensor] = None,
            bias: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Every transform's statistics for X (device tensor [M, K], bf16 or fp32), and with a
    weight W [N, K] (same device) the W4A4 errors against float64 X W^T (+ bias)."""
    from . import (convrot_dequant_int4, convrot_quant_weight, convrot_rotate_quant_act,
                   convrot_w4a4_linear)
    rows = []
    ref = None
    if w is not None:
        ref = x.double() @ w.double().T
        if bias is not None:
            ref = ref + bias.double()[None, :]
    # no rotation
    wd = None if w is None else int4_dequantized(w.double())
    rows.append(_row("none", None, None, x.double(), int4_dequantized(x.double()), wd, ref,
                     bias))
    for g in groups:
        # regular, group-wise: the HIP kernels
        xq, xs, xr = convrot_rotate_quant_act(x, g, want_rotated=True)
        h = _lib.convrot_make_rht(g).numpy()
        wd = None
        if w is not None:
            wq, ws = convrot_quant_weight(w, g)
            wd = convrot_dequant_int4(wq, ws, 2 * wq.shape[1])
        r = _row("regular", g, column_discrepancy(h), xr.double(),
                 convrot_dequant_int4(xq, xs, 2 * xq.shape[1]), wd, ref, bias)
        if w is not None:
            r["w4a4_rel_err_kernel_bf16"] = rel_frobenius(convrot_w4a4_linear(x, g, wq, ws, bias),
                                                          ref)
        rows.append(r)
        # Sylvester, group-wise
        y = sylvester_groups(x, g)
        wd = None if w is None else int4_dequantized(sylvester_groups(w, g))
        rows.append(_row("sylvester", g, column_discrepancy(sylvester_pm1(g)), y,
                         int4_dequantized(y), wd, ref, bias))
    # Sylvester, global (one transform over the whole zero-padded row)
    y = sylvester_global(x)
    n = y.shape[1]
    wd = None if w is None else int4_dequantized(sylvester_global(w))
    rows.append(_row("sylvester_global", n, float(n), y, int4_dequantized(y), wd, ref, bias))
    return {"M": int(x.shape[0]), "K": int(x.shape[1]), "transforms": rows}


def _print(res: dict) -> None:
    print(f"M={res['M']} K={res['K']}")
    print(f"{'transform':>17} {'g':>6} {'col.disc':>9} {'max|y|':>9} {'act int4':>9} "
          f"{'W4A4':>9} {'kernel bf16':>11}")
    for r in res["transforms"]:
        d = "" if r["column_discrepancy"] is None else f"{r['column_discrepancy']:.0f}"
        print(f"{r['transform']:>17} {r['g'] or '':>6} {d:>9} {r['max_abs']:9.3f} "
              f"{r['act_int4_rel_err']:9.4f} {r.get('w4a4_rel_err', float('nan')):9.4f} "
              f"{r.get('w4a4_rel_err_kernel_bf16', float('nan')):11.4f}")


def main(argv=None) -> int:
    import workloads as wk
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="attn_proj")
    p.add_argument("--rows", type=int, default=1024, help="first rows of X to analyze")
    p.add_argument("--offset", type=float, default=20.0,
                   help="same-sign offset of the row-wise outlier tokens (0: the workload's X)")
    p.add_argument("--groups", default="16,64,256,1024")
    p.add_argument("--json", default=None)
    a = p.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the tool runs the HIP kernels: a GPU is required")
    wl = wk.WORKLOADS[a.workload]
    dt = torch.bfloat16 if wl.x_dtype == "bf16" else torch.float32
    rows = min(a.rows, wl.M)
    if a.offset:  # 1% of the tokens carry the offset, as the workloads' row outliers
        xn = wk.offset_row_outliers(rows, wl.K, max(1, rows // 100), a.offset, dtype=wl.x_dtype)
    else:
        xn = wk.activations(wl)[:rows]
    x = torch.from_numpy(xn).to(dt).cuda()
    w = b = None
    if wl.N is not None:
        w = torch.from_numpy(wk.weights(wl)).to(dt).cuda()
        bn = wk.bias(wl)
        b = None if bn is None else torch.from_numpy(bn).to(torch.bfloat16).cuda()
    res = analyze(x, [int(v) for v in a.groups.split(",")], w, b)
    res.update({"workload": wl.name, "offset": a.offset})
    _print(res)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
