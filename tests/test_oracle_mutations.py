"""Plant plausible mistakes in the oracle (CPU only) and check that the pins catch them.

Each mutation replaces one oracle function through monkeypatch for the duration
of one test; the designated pins must then fail.  This shows the pins are
sharp enough to catch a dropped term, a wrong sign, index or operand order.
"""
import numpy as np
import pytest

from oracle import convrot_oracle as O
from tests import oracle_pins as P

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _sylvester_base():
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    return np.kron(h2, h2)


def _one_entry_flipped():
    h = _orig["base_regular_hadamard"]().copy()
    h[0, 1] = -h[0, 1]
    return h


def _rotate_unnormalised(a, g):
    return _orig["rotate_groups"](a, g) * 2.0 ** _orig["log4"](g)


def _rotate_strided_windows(a, g):
    h = _orig["regular_hadamard"](g)
    ap = _orig["zero_pad_columns"](a, g)
    rows, kp = ap.shape
    win = ap.reshape(rows, g, kp // g).transpose(0, 2, 1)     # wrong: strided windows
    y = (win @ h.T * 2.0 ** -_orig["log4"](g)).transpose(0, 2, 1)
    return y.reshape(rows, kp)


def _padded_k_floor(K, g):
    return max(g, (int(K) // g) * g)


def _zero_pad_floor(a, g):
    a = np.asarray(a, dtype=np.float64)
    kp = _padded_k_floor(a.shape[1], g)
    out = np.zeros((a.shape[0], kp))
    n = min(kp, a.shape[1])
    out[:, :n] = a[:, :n]
    return out


def _row_scales_q8(yf, qmax=7):
    return _orig["row_scales"](yf, 8)


def _quantize_half_up(yf, scale, qmax=7, qmin=-8):
    yf = np.asarray(yf, dtype=np.float32)
    q = np.zeros(yf.shape, dtype=np.int8)
    live = scale > 0
    z = (yf[live] / scale[live, None]).astype(np.float32)
    q[live] = np.clip(np.floor(z + np.float32(0.5)), qmin, qmax).astype(np.int8)
    return q


def _pack_swapped(q):
    q = np.asarray(q, dtype=np.int64)
    return ((q[:, 1::2] & 0xF) | ((q[:, 0::2] & 0xF) << 4)).astype(np.uint8)


def _unpack_unsigned(b):
    b = np.asarray(b, dtype=np.int64)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = (b >> 4) & 0xF
    return out


def _gemm_bf16_accumulate(qx, qw):
    import torch
    a = torch.from_numpy(np.asarray(qx, dtype=np.float32)).to(torch.bfloat16)
    b = torch.from_numpy(np.asarray(qw, dtype=np.float32)).to(torch.bfloat16)
    out = torch.zeros((a.shape[0], b.shape[0]), dtype=torch.bfloat16)
    for k in range(a.shape[1]):  # bf16 running sum, as in the reviewed eager code
        out = (out + a[:, k:k + 1] * b[:, k][None, :]).to(torch.bfloat16)
    return out.to(torch.float64).numpy().astype(np.int64)


def _dequant_bias_first(acc, sx, sw, bias=None):
    z = np.asarray(acc, dtype=np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    z = (z * np.asarray(sx, dtype=np.float32)[:, None]).astype(np.float32)
    z = (z * np.asarray(sw, dtype=np.float32)[None, :]).astype(np.float32)
    return _orig["f32_to_bf16_bits"](z)


def _dequant_no_wscale(acc, sx, sw, bias=None):
    return _orig["dequantize"](acc, sx, np.ones_like(np.asarray(sw, dtype=np.float32)), bias)


def _bf16_truncate(z):
    u = np.asarray(z, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _rotate_quantize_int8_scale7(a, g):
    r = _orig["rotate_quantize_int8"](a, g)
    s = _orig["row_scales"](r["yf"], 7)
    return {"yf": r["yf"], "scale": s, "codes": _orig["quantize"](r["yf"], s, 127, -128)}


def _e2m1_ties_away(t):
    # nearest magnitude, ties to the larger one
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    d = np.abs(a[..., None] - O.E2M1_GRID)
    idx = 7 - np.argmin(d[..., ::-1], axis=-1)
    return (idx | np.where(np.signbit(t), 8, 0)).astype(np.uint8)


def _e2m1_no_negative_zero(t):
    c = _orig["e2m1_encode"](t)
    return np.where(c == 8, 0, c).astype(np.uint8)


def _to_f32_truncate(y):
    # drops the 29 low significand bits: rounds toward zero instead of to nearest even
    b = np.asarray(y, dtype=np.float64).view(np.uint64) & ~np.uint64((1 << 29) - 1)
    return b.view(np.float64).astype(np.float32)


def _to_f32_ties_away(y):
    # nearest, but exact midpoints go to the neighbour away from zero
    y = np.asarray(y, dtype=np.float64)
    r = y.astype(np.float32)
    away = np.nextafter(r, np.copysign(np.float32(np.inf), r))
    mid = (r.astype(np.float64) + away.astype(np.float64)) / 2.0
    return np.where(mid == y, away, r).astype(np.float32)


def _mx_values_unscaled(codes, e8m0):
    # decoded codes without their block scale
    return O.e2m1_decode(codes)


MUTATIONS = {
    "sylvester_base": ({"base_regular_hadamard": _sylvester_base}, ["pin_regular"]),
    "negated_base": ({"base_regular_hadamard": lambda: -_orig["base_regular_hadamard"]()},
                     ["pin_regular"]),
    "sign_flip_entry": ({"base_regular_hadamard": _one_entry_flipped},
                        ["pin_hadamard_definition"]),
    "unnormalised": ({"rotate_groups": _rotate_unnormalised}, ["pin_rotation_constant_row"]),
    "strided_windows": ({"rotate_groups": _rotate_strided_windows},
                        ["pin_rotation_brute_force_padded"]),
    "floor_padding": ({"zero_pad_columns": _zero_pad_floor, "padded_k": _padded_k_floor},
                      ["pin_rotation_brute_force_padded"]),
    "qmax_8": ({"row_scales": _row_scales_q8}, ["pin_quant_round_trip"]),
    "round_half_up": ({"quantize": _quantize_half_up}, ["pin_quant_ties_even"]),
    "swapped_nibbles": ({"pack_int4": _pack_swapped}, ["pin_pack_layout"]),
    "unsigned_unpack": ({"unpack_int4": _unpack_unsigned}, ["pin_pack_layout"]),
    "bf16_accumulation": ({"int_gemm": _gemm_bf16_accumulate}, ["pin_int_gemm_brute_force"]),
    "bias_before_scale": ({"dequantize": _dequant_bias_first}, ["pin_end_to_end_closed_form", "pin_int4_linear_semantics"]),
    "dropped_weight_scale": ({"dequantize": _dequant_no_wscale}, ["pin_int4_linear_semantics"]),
    "bf16_truncation": ({"f32_to_bf16_bits": _bf16_truncate}, ["pin_bf16_rounding_vs_torch"]),
    "int8_qmax_128": ({"INT8_QMAX": 128}, ["pin_int8_round_trip", "pin_int8_rotate_quantize"]),
    "int8_int4_scale": ({"rotate_quantize_int8": _rotate_quantize_int8_scale7},
                        ["pin_int8_rotate_quantize", "pin_int8_end_to_end_closed_form"]),
    "e2m1_ties_away": ({"e2m1_encode": _e2m1_ties_away}, ["pin_e2m1_rounding"]),
    "e2m1_lost_sign_of_zero": ({"e2m1_encode": _e2m1_no_negative_zero}, ["pin_e2m1_format"]),
    "mx_emax_3": ({"E2M1_EMAX": 3}, ["pin_mx_block_scale", "pin_mxfp4_round_trip",
                                     "pin_mxfp4_end_to_end_closed_form"]),
    "mx_block_16": ({"MX_BLOCK": 16}, ["pin_mx_block_scale"]),
    "to_f32_truncation": ({"to_f32": _to_f32_truncate}, ["pin_to_f32"]),
    "to_f32_ties_away": ({"to_f32": _to_f32_ties_away}, ["pin_to_f32"]),
    "mx_values_unscaled": ({"mxfp4_values": _mx_values_unscaled},
                           ["pin_mxfp4_gemm_brute_force", "pin_mxfp4_round_trip"]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    patches, pins = MUTATIONS[name]
    for attr, fn in patches.items():
        monkeypatch.setattr(O, attr, fn)
    for pin_name in pins:
        with pytest.raises((AssertionError, ValueError)):
            getattr(P, pin_name)(O)
