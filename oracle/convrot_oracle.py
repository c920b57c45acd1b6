"""CPU oracle for the ConvRot / ConvLinear4bit forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call this module.  The product
path (the HIP library and its Python binding) never does, and this module
imports nothing from it.  It shares no code, tables or helpers with the HIP
path.

Plain, slow and written for reading: numpy, float64 for the rotation, float32
exactly where the method's fp32 steps are, one library primitive per step
(``np.kron``, a matmul), no blocking, fusion or reordering.

Sources (the web pages this follows, cited by title and section):
  [AUTHOR]  ComfyUI issue #14735, comment by the ConvRot author: group-wise
            rotation on non-overlapping windows, the regular Hadamard matrix,
            group sizes that are powers of 4 (16, 64, 256, 1024), zero padding
            "inside the algorithm" when K is not a multiple of the group.
  [PAPER]   "ConvRot: Rotation-Based Plug-and-Play 4-bit Quantization for
            Diffusion Transformers" (arXiv 2512.03673, summary page): Abstract
            (ConvLinear4bit integrates rotation, quantization, GEMM and
            dequantization), Fig. 1-3, Definition 2.1 (Hadamard matrix),
            Theorem 2.1 (column-sum-squared property), Definition 2.2 (column
            discrepancy), Definition 2.3 (regular H-matrix), Theorem 2.3
            (Kronecker construction).  Only their titles are printed.
  [HSWQ]    HSWQ v2.3.4 release notes, "Krea2 ConvRot INT8 Quantization
            Release", section "Mathematical Formulation & Format Layout",
            sub-section "Hadamard Orthogonal Rotation": W_rot = W H^T,
            per-row scale = max|W_rot| / 127, W_q = round(W_rot / scale).
  [KITCHEN] comfy-kitchen PR #65 "Basic convrot int4 support", review
            comments: the integer-only power-of-4 size check (2^58 = 4^29),
            and int4_linear: unpack both int4 operands ("row major"),
            accumulate x @ w^T in fp32 (exact integers), multiply by the
            per-row x scale and per-column w scale, add the bias, cast last.

Readings taken where the pages are silent:
  * base matrix H4 = J4 - 2 I4 (symmetric; every row and column sums to +2);
    H_g = H4 (x) ... (x) H4 (k = log4 g factors); rotation = H_g / sqrt(g).
  * windows start at column 0; K is zero-padded to K' = ceil(K/g) g and the
    padded columns take part in the rotation and the GEMM (depth K').
  * int4 is symmetric: scale = absmax / 7 (the INT8 form with 127 -> 7),
    code = clamp(round_half_even(y / scale), -8, 7); a zero row has scale 0
    and codes 0.
  * the rotated value is the correctly rounded fp32 of the exact rotation.
  * packing: code 2j in the low nibble of byte j, code 2j+1 in the high
    nibble, two's complement; row stride K'/2 bytes.
  * dequant order: z = fp32(fp32(fp32(acc) * sx[m]) * sw[n]); z = fp32(z + b);
    output = bf16 round-to-nearest-even of z.

Every function is pinned in ``tests/oracle_pins.py`` (run by
``tests/test_oracle_pins.py``) against closed forms, invariants, brute force,
exact rational arithmetic or library routines; ``tests/test_oracle_mutations.py``
plants plausible mistakes in copies of it and checks that a pin fails.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

INT4_QMAX = 7       # symmetric int4: codes in [-8, 7], scale = absmax / 7
INT4_QMIN = -8
INT8_QMAX = 127     # symmetric int8 ([HSWQ]): codes in [-128, 127], scale = absmax / 127
INT8_QMIN = -128


# --------------------------------------------------------------------------
# Group size: a power of 4 ([AUTHOR]; [KITCHEN] review of the size check)
# --------------------------------------------------------------------------
def is_power_of_four(g) -> bool:
    """True iff g is an integer 4^k with k >= 1, decided with integers only."""
    if isinstance(g, bool) or not isinstance(g, (int, np.integer)):
        return False
    g = int(g)
    if g < 4 or (g & (g - 1)) != 0:
        return False
    return (g.bit_length() - 1) % 2 == 0


def check_group_size(g) -> None:
    if not is_power_of_four(g):
        raise ValueError(f"Regular Hadamard size must be a power of 4, got {g}")


def log4(g: int) -> int:
    check_group_size(g)
    return (int(g).bit_length() - 1) // 2


# --------------------------------------------------------------------------
# Regular Hadamard matrix ([PAPER] Def. 2.1, Def. 2.3, Thm. 2.3)
# --------------------------------------------------------------------------
def base_regular_hadamard() -> np.ndarray:
    """Order-4 regular Hadamard matrix J - 2I (entries +-1, row/col sums +2)."""
    return np.ones((4, 4), dtype=np.float64) - 2.0 * np.eye(4, dtype=np.float64)


def regular_hadamard(g: int) -> np.ndarray:
    """H_g = H4 (x) H4 (x) ... (x) H4, built by repeated Kronecker products."""
    k = log4(g)
    h = np.ones((1, 1), dtype=np.float64)
    for _ in range(k):
        h = np.kron(h, base_regular_hadamard())
    return h


# --------------------------------------------------------------------------
# Padding and group-wise rotation ([AUTHOR]; [PAPER] Fig. 3)
# --------------------------------------------------------------------------
def padded_k(K: int, g: int) -> int:
    check_group_size(g)
    return -(-int(K) // g) * g


def zero_pad_columns(a: np.ndarray, g: int) -> np.ndarray:
    """[A | 0] with K' = ceil(K/g) g columns, float64."""
    a = np.asarray(a, dtype=np.float64)
    rows, K = a.shape
    out = np.zeros((rows, padded_k(K, g)), dtype=np.float64)
    out[:, :K] = a
    return out


def rotate_groups(a: np.ndarray, g: int) -> np.ndarray:
    """Exact group-wise RHT in float64.

    Every non-overlapping window of g columns of the zero-padded row is
    multiplied by H_g^T / sqrt(g) (H_g is symmetric, so this is also H_g / sqrt(g)).
    sqrt(g) = 2^k is a power of two, so the normalisation is exact.  For bf16
    inputs the float64 sums are exact whenever a window's exponent spread is at
    most 35 binades (8 significand bits + log2(1024) growth <= 53).
    """
    h = regular_hadamard(g)
    ap = zero_pad_columns(a, g)
    rows, kp = ap.shape
    windows = ap.reshape(rows, kp // g, g)
    y = windows @ h.T
    return (y * 2.0 ** (-log4(g))).reshape(rows, kp)


def to_f32(y: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float64 -> float32 (the rotated activations)."""
    return np.asarray(y, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# Symmetric per-row int4 quantization ([HSWQ] "Hadamard Orthogonal Rotation",
# with q_max 127 -> 7 for int4; [PAPER] Abstract)
# --------------------------------------------------------------------------
def row_scales(yf: np.ndarray, qmax: int = INT4_QMAX) -> np.ndarray:
    """scale[m] = fp32(max_k |yf[m, k]| / qmax) with IEEE float32 division."""
    yf = np.asarray(yf, dtype=np.float32)
    amax = np.max(np.abs(yf), axis=1).astype(np.float32)
    return (amax / np.float32(qmax)).astype(np.float32)


def quantize(yf: np.ndarray, scale: np.ndarray, qmax: int = INT4_QMAX,
             qmin: int = INT4_QMIN) -> np.ndarray:
    """code = clamp(round_half_even(fp32(yf / scale)), qmin, qmax); 0 where scale == 0."""
    yf = np.asarray(yf, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    q = np.zeros(yf.shape, dtype=np.int8)
    live = scale > 0
    z = (yf[live] / scale[live, None]).astype(np.float32)
    q[live] = np.clip(np.rint(z), qmin, qmax).astype(np.int8)
    return q


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two codes per byte: column 2j -> low nibble, 2j+1 -> high nibble."""
    q = np.asarray(q, dtype=np.int64)
    rows, n = q.shape
    if n % 2:
        raise ValueError("packing needs an even number of columns")
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: sign-extended int8 codes [rows x 2*bytes]."""
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def rotate_quantize(a: np.ndarray, g: int) -> dict:
    """Pad, rotate, round to fp32, per-row scale, quantize, pack (one row = one token)."""
    yf = to_f32(rotate_groups(a, g))
    s = row_scales(yf)
    q = quantize(yf, s)
    return {"yf": yf, "scale": s, "codes": q, "packed": pack_int4(q)}


def quantize_weight(w: np.ndarray, g: int) -> dict:
    """Offline weight path: the same steps on the rows of W [N x K] (per output channel)."""
    return rotate_quantize(w, g)


def rotate_quantize_int8(a: np.ndarray, g: int) -> dict:
    """The INT8 variant ([HSWQ] "Hadamard Orthogonal Rotation": scale = max|rotated| / 127,
    codes = round(rotated / scale)) on the same group-wise regular rotation; one int8 code
    per element, rows of K' codes."""
    yf = to_f32(rotate_groups(a, g))
    s = row_scales(yf, INT8_QMAX)
    q = quantize(yf, s, INT8_QMAX, INT8_QMIN)
    return {"yf": yf, "scale": s, "codes": q}


def quantize_weight_int8(w: np.ndarray, g: int) -> dict:
    """Offline INT8 weight path (per output channel)."""
    return rotate_quantize_int8(w, g)


# --------------------------------------------------------------------------
# W4A4 GEMM and dequantization ([KITCHEN] review of int4_linear; [PAPER] Abstract)
# --------------------------------------------------------------------------
def int_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] qw[n, k] exactly (x @ w^T).

    The float64 matmul is exact: every partial sum is an integer of magnitude
    at most 64 K' (int4 codes) or 16384 K' (int8 codes), below 2^53.
    """
    acc = np.asarray(qx, dtype=np.float64) @ np.asarray(qw, dtype=np.float64).T
    return acc.astype(np.int64)


def f32_to_bf16_bits(z: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, round to nearest even (finite inputs)."""
    u = np.asarray(z, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def dequantize(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray,
               bias: Optional[np.ndarray] = None) -> np.ndarray:
    """out = bf16(fp32(fp32(fp32(acc) * sx[m]) * sw[n]) [+ fp32 bias[n]]), as bf16 bits.

    fp32(acc) is exact for int4 codes (|acc| <= 64 K' < 2^24); for int8 codes at large K' it
    is the round-to-nearest-even conversion of the exact integer."""
    z = np.asarray(acc, dtype=np.float32)
    z = (z * np.asarray(sx, dtype=np.float32)[:, None]).astype(np.float32)
    z = (z * np.asarray(sw, dtype=np.float32)[None, :]).astype(np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return f32_to_bf16_bits(z)


def w4a4_linear_from_codes(qx, sx, qw, sw, bias=None) -> dict:
    acc = int_gemm(qx, qw)
    return {"acc": acc, "out_bits": dequantize(acc, sx, sw, bias)}


def convlinear4bit(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], g: int) -> dict:
    """The whole forward pass: offline weight path, online activation path, GEMM, dequant."""
    xr = rotate_quantize(x, g)
    wr = quantize_weight(w, g)
    lin = w4a4_linear_from_codes(xr["codes"], xr["scale"], wr["codes"], wr["scale"], bias)
    return {"x": xr, "w": wr, **lin}


def w8a8_linear_from_codes(qx, sx, qw, sw, bias=None) -> dict:
    """INT8 GEMM (exact int32 sums: |acc| <= 16384 K' < 2^31 for K' <= 65536) + dequant."""
    acc = int_gemm(qx, qw)
    return {"acc": acc, "out_bits": dequantize(acc, sx, sw, bias)}


def convlinear8bit(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], g: int) -> dict:
    """The W8A8 forward pass: the same rotation, int8 codes on both sides."""
    xr = rotate_quantize_int8(x, g)
    wr = quantize_weight_int8(w, g)
    lin = w8a8_linear_from_codes(xr["codes"], xr["scale"], wr["codes"], wr["scale"], bias)
    return {"x": xr, "w": wr, **lin}


# --------------------------------------------------------------------------
# Floating-point 4-bit ConvRot.  [AUTHOR] says the method also suits floating-point
# quantization but fixes no format.  Reading: MXFP4 as the OCP Microscaling (MX)
# Specification v1.0 defines it (a published standard, not one of the pages): blocks of 32
# consecutive rotated values along K share an E8M0 scale 2^(floor(log2(block absmax)) - 2),
# 2 being the exponent of E2M1's largest normal value (6 = 1.5 * 2^2); each value becomes
# the E2M1 number nearest to value / scale, ties to the even mantissa, magnitudes beyond 6
# clamped to 6.  Same rotation, same row layouts as int4 (two codes per byte), plus one
# E8M0 byte per block.
# --------------------------------------------------------------------------
MX_BLOCK = 32
E2M1_EMAX = 2
E8M0_BIAS = 127


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa;
    exponent 0 is subnormal (0 or 0.5)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + 0.5 * m))
    return np.where(c & 8, -mag, mag)


E2M1_GRID = e2m1_decode(np.arange(8))  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(t: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code to t (exact float64 input), ties to the even code, so that
    magnitudes above 6 saturate at 6; the sign bit follows t's sign (-0.0 -> code 8)."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    d = np.abs(a[..., None] - E2M1_GRID)  # distance to each of the 8 magnitudes
    dmin = d.min(axis=-1, keepdims=True)
    tied = d == dmin
    idx = np.argmax(tied & (np.arange(8) % 2 == 0), axis=-1)  # an even code, if one is nearest
    has_even = np.any(tied & (np.arange(8) % 2 == 0), axis=-1)
    idx = np.where(has_even, idx, np.argmax(tied, axis=-1))
    return (idx | np.where(np.signbit(t), 8, 0)).astype(np.uint8)


def mx_block_exponents(yf: np.ndarray) -> np.ndarray:
    """Shared exponent of every 32-value block of each row: floor(log2(absmax)) - 2, clamped
    to E8M0's range [-127, 127]; an all-zero block takes -127."""
    yf = np.asarray(yf, dtype=np.float64)
    rows, n = yf.shape
    if n % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    amax = np.max(np.abs(yf.reshape(rows, n // MX_BLOCK, MX_BLOCK)), axis=2)
    _, ex = np.frexp(amax)  # amax = mant * 2^ex, mant in [0.5, 1): floor(log2) = ex - 1
    e = np.where(amax > 0, ex.astype(np.int64) - 1 - E2M1_EMAX, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def quantize_mxfp4(yf: np.ndarray):
    """(E2M1 codes [rows, n] as nibbles, E8M0 bytes [rows, n / 32])."""
    yf = np.asarray(yf, dtype=np.float64)
    e = mx_block_exponents(yf)
    scale = np.repeat(np.exp2(e.astype(np.float64)), MX_BLOCK, axis=1)
    return e2m1_encode(yf / scale), (e + E8M0_BIAS).astype(np.uint8)


def mxfp4_values(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """Decoded values: E2M1 value * 2^(E8M0 - 127) of its block (float64, exact)."""
    s = np.exp2(np.asarray(e8m0, dtype=np.float64) - E8M0_BIAS)
    return e2m1_decode(codes) * np.repeat(s, MX_BLOCK, axis=1)


def rotate_quantize_mxfp4(a: np.ndarray, g: int) -> dict:
    """Pad, rotate, round to fp32, MXFP4-quantize every 32-value block, pack."""
    yf = to_f32(rotate_groups(a, g))
    codes, e8m0 = quantize_mxfp4(yf)
    return {"yf": yf, "codes": codes, "scales": e8m0, "packed": pack_int4(codes)}


def quantize_weight_mxfp4(w: np.ndarray, g: int) -> dict:
    """Offline MXFP4 weight path (blocks along K of each output channel)."""
    return rotate_quantize_mxfp4(w, g)


def mxfp4_linear_from_codes(cx, ex, cw, ew, bias=None) -> dict:
    """sum_k x_k w_k of the decoded values in float64 (every product is exact; the sum is exact
    unless a row's block scales span more than ~45 binades), the same with magnitudes (for
    accumulation error bounds), and bf16(fp32(fp32(sum) + bias)) as bits."""
    vx, vw = mxfp4_values(cx, ex), mxfp4_values(cw, ew)
    z = vx @ vw.T
    mag = np.abs(vx) @ np.abs(vw).T
    zf = z.astype(np.float32)
    if bias is not None:
        zf = (zf + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return {"sum": z, "abs_sum": mag, "out_bits": f32_to_bf16_bits(zf)}


def convlinear_fp4(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], g: int) -> dict:
    """The MXFP4 forward pass: the same rotation, MXFP4 codes on both sides."""
    xr = rotate_quantize_mxfp4(x, g)
    wr = quantize_weight_mxfp4(w, g)
    lin = mxfp4_linear_from_codes(xr["codes"], xr["scales"], wr["codes"], wr["scales"], bias)
    return {"x": xr, "w": wr, **lin}
