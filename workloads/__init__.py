"""Seeded synthetic inputs for the ConvLinear4bit workloads.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds none of the method's arithmetic: only random draws, the
injection of row-wise and column-wise outliers, an optional GELU shaping of the
activation distribution, and the one-time cast of the drawn values to the input
dtype.

Why outliers: the ConvRot paper (arXiv 2512.03673, Abstract and Fig. 1/2)
targets diffusion-transformer activations that carry both row-wise (whole
token) and column-wise (fixed channel) outliers.  The FLUX.1-dev activations it
measures are not available, so these tensors stand in for them with the
FLUX-like layer shapes used below.

Recipe (seeds and picks are fixed so every consumer sees the same tensors):
  * X draws use numpy ``default_rng(seed_x)`` (seed 0), W draws seed 1, bias
    draws seed 2, outlier picks seed 3; draws are float32.
  * Outlier rows are the first ``n_out_rows`` entries of a permutation of the
    rows; outlier channels the first ``n_out_cols`` entries of a permutation of
    the columns (both from the seed-3 generator).  Row and column factors
    multiply where they meet.
  * Inputs declared bf16 are rounded once, round-to-nearest-even, after the
    outliers are applied (torch's float32 -> bfloat16 cast).  The float32 numpy
    copy returned alongside holds exactly the bf16 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_X, SEED_W, SEED_B, SEED_PICK = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic ConvLinear4bit problem: X [M x K] @ W[N x K]^T (+ bias)."""

    name: str
    M: int
    K: int
    N: Optional[int]          # None: rotate+quantize only (no weight / GEMM)
    g: int                    # rotation window (group) size
    x_dtype: str              # "f32" or "bf16" (weights and bias share it)
    x_dist: str = "normal"    # "normal" or "gelu" (GELU(N(0,1)), erf form)
    n_out_rows: int = 0       # number of row-wise outlier tokens
    row_scale: float = 1.0
    n_out_cols: int = 0       # number of column-wise outlier channels
    col_scale: float = 1.0
    w_std: float = 0.02
    bias_std: Optional[float] = None
    description: str = ""

    @property
    def Kp(self) -> int:
        """K rounded up to a whole number of windows (zero padding)."""
        return -(-self.K // self.g) * self.g


def _pct_rows(M: int, pct: float) -> int:
    return int(math.floor(pct * M))


# The five problems of the ConvLinear4bit hot path (FLUX.1-dev-like shapes).
WORKLOADS = {
    "tiny": Workload(
        "tiny", M=64, K=256, N=256, g=16, x_dtype="f32",
        n_out_rows=2, row_scale=40.0, n_out_cols=3, col_scale=20.0, w_std=0.02,
        description="tiny ConvLinear4bit, fp32 X[64x256], W[256x256], g=16"),
    "rotate_quant": Workload(
        "rotate_quant", M=4608, K=3072, N=None, g=256, x_dtype="bf16",
        n_out_rows=_pct_rows(4608, 0.01), row_scale=50.0, n_out_cols=8, col_scale=30.0,
        description="rotate+quantize only, bf16 X[4608x3072], g=256"),
    "attn_proj": Workload(
        "attn_proj", M=4608, K=3072, N=3072, g=256, x_dtype="bf16",
        n_out_rows=_pct_rows(4608, 0.01), row_scale=50.0, n_out_cols=8, col_scale=30.0,
        w_std=0.02, bias_std=0.01,
        description="attention projection, X[4608x3072] W[3072x3072] + bias, g=256"),
    "mlp_down": Workload(
        "mlp_down", M=4608, K=12288, N=3072, g=1024, x_dtype="bf16", x_dist="gelu",
        n_out_rows=_pct_rows(4608, 0.005), row_scale=50.0, w_std=0.01,
        description="MLP down-projection, GELU X[4608x12288] W[3072x12288], g=1024"),
    "proj_out": Workload(
        "proj_out", M=9216, K=15360, N=3072, g=1024, x_dtype="bf16",
        n_out_rows=_pct_rows(9216, 0.01), row_scale=50.0, n_out_cols=8, col_scale=30.0,
        w_std=0.01,
        description="single-stream proj_out batch 2, X[9216x15360] W[3072x15360], g=1024"),
    "few_tokens": Workload(
        "few_tokens", M=64, K=3072, N=3072, g=256, x_dtype="bf16",
        n_out_rows=1, row_scale=50.0, n_out_cols=8, col_scale=30.0, w_std=0.02, bias_std=0.01,
        description="few tokens (m <= 128), attention-projection weights, X[64x3072] + bias"),
    "proj_out_padded": Workload(
        "proj_out_padded", M=4608, K=3100, N=3072, g=256, x_dtype="bf16",
        n_out_rows=_pct_rows(4608, 0.01), row_scale=50.0, n_out_cols=8, col_scale=30.0,
        w_std=0.01,
        description="padded proj_out, X[4608x3100] W[3072x3100], g=256 (K'=3328)"),
}


def custom(name: str, M: int, K: int, N: Optional[int], g: int, x_dtype: str = "bf16",
           **kw) -> Workload:
    """A workload of arbitrary shape with the attention-projection outlier model."""
    base = dict(n_out_rows=max(1, _pct_rows(M, 0.01)) if M >= 2 else 0, row_scale=50.0,
                n_out_cols=min(8, K), col_scale=30.0, w_std=0.02)
    base.update(kw)
    return Workload(name, M=M, K=K, N=N, g=g, x_dtype=x_dtype, **base)


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    # Shapes the activation distribution only (input recipe, not the method).
    from scipy.special import erf
    z64 = z.astype(np.float64)
    return (0.5 * z64 * (1.0 + erf(z64 / math.sqrt(2.0)))).astype(np.float32)


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the input dtype (RNE), returned as float32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype}")
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def activations(wl: Workload) -> np.ndarray:
    """X [M x K] as float32 numpy holding values exact in ``wl.x_dtype``."""
    rng = np.random.default_rng(SEED_X)
    x = rng.standard_normal((wl.M, wl.K), dtype=np.float32)
    if wl.x_dist == "gelu":
        x = _gelu_erf(x)
    elif wl.x_dist != "normal":
        raise ValueError(wl.x_dist)
    pick = np.random.default_rng(SEED_PICK)
    rows = pick.permutation(wl.M)[: wl.n_out_rows]
    cols = pick.permutation(wl.K)[: wl.n_out_cols]
    if len(rows):
        x[rows, :] *= np.float32(wl.row_scale)
    if len(cols):
        x[:, cols] *= np.float32(wl.col_scale)
    return round_to_dtype(x, wl.x_dtype)


def weights(wl: Workload) -> np.ndarray:
    """W [N x K] ~ N(0, w_std^2) as float32 numpy exact in ``wl.x_dtype``."""
    assert wl.N is not None
    rng = np.random.default_rng(SEED_W)
    w = rng.standard_normal((wl.N, wl.K), dtype=np.float32) * np.float32(wl.w_std)
    return round_to_dtype(w, wl.x_dtype)


def bias(wl: Workload) -> Optional[np.ndarray]:
    """bias [N] ~ N(0, bias_std^2), bf16-exact, or None."""
    if wl.bias_std is None or wl.N is None:
        return None
    rng = np.random.default_rng(SEED_B)
    b = rng.standard_normal((wl.N,), dtype=np.float32) * np.float32(wl.bias_std)
    return round_to_dtype(b, "bf16")


def random_codes(rows: int, cols: int, seed: int, lo: int = -8, hi: int = 7) -> np.ndarray:
    """Uniform int4 codes in [lo, hi] (int8 array) for GEMM-only tests."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols), dtype=np.int64).astype(np.int8)


def random_scales(n: int, seed: int) -> np.ndarray:
    """Positive float32 scales spanning a few binades, for GEMM-only tests."""
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.5, 2.0, size=n) * np.exp2(rng.integers(-6, 2, size=n))).astype(np.float32)


def extreme_scales(n: int, seed: int) -> np.ndarray:
    """fp32 scales over the whole range the dequantization must handle bit-exactly: zero,
    values so small that the products are subnormal or vanish, huge values, negatives, and
    ordinary ones, interleaved so that some 32-row blocks are all ordinary."""
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, size=n)
    kind = rng.integers(0, 6, size=n)
    expo = np.select([kind == 0, kind == 1, kind == 2, kind == 3],
                     [rng.integers(-149, -110, size=n), rng.integers(-127, -117, size=n),
                      rng.integers(90, 100, size=n), rng.integers(-8, 2, size=n)],
                     rng.integers(-8, 2, size=n))
    s = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    s[kind == 4] *= -1
    s[rng.random(n) < 0.05] = 0.0
    s[:64] = (rng.uniform(0.5, 2.0, size=min(n, 64)) * 2.0 ** -5).astype(np.float32)
    return s


def offset_row_outliers(M: int, K: int, n_rows: int, offset: float, n_cols: int = 8,
                        col_scale: float = 30.0, seed: int = SEED_X,
                        dtype: str = "bf16") -> np.ndarray:
    """X [M x K] ~ N(0, 1) whose first ``n_rows`` rows of a permutation carry a common
    same-sign offset across every channel (a whole-token outlier that a global rotation
    accumulates), plus ``n_cols`` channel outliers scaled by ``col_scale``; rounded once to
    ``dtype``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    pick = np.random.default_rng(SEED_PICK)
    rows = pick.permutation(M)[:n_rows]
    cols = pick.permutation(K)[:n_cols]
    if len(rows):
        x[rows, :] += np.float32(offset)
    if len(cols):
        x[:, cols] *= np.float32(col_scale)
    return round_to_dtype(x, dtype)
