"""The Python binding checks every tensor argument on the host before it calls the library:
wrong shapes, dtypes or layouts raise ValueError / TypeError, so no kernel can read or write
past a buffer or read a sliced tensor with the wrong row stride.  CPU tensors are used
throughout: each case must be rejected by the shape and dtype checks, which run before the
device check (a CPU tensor that passed them would be rejected with "GPU")."""
import os

import pytest
import torch

import rotation_w4a4_quantized_convrot_amd as cr
from rotation_w4a4_quantized_convrot_amd import _lib

u8, i8, f32, bf16, i32 = torch.uint8, torch.int8, torch.float32, torch.bfloat16, torch.int32


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libconvrot.so not built")
    return _lib.load_library()


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def _raises(fn, *args, exc=(ValueError, TypeError), match=None, **kw):
    with pytest.raises(exc, match=match):
        fn(*args, **kw)


def _reaches_device_check(fn, *args, **kw):
    """Valid shapes: the call gets as far as the device check (CPU tensors are refused)."""
    with pytest.raises(ValueError, match="GPU"):
        fn(*args, **kw)


M, K, N, g = 5, 100, 7, 16          # K' = 112
KP = 112


def test_rotate_quant_outputs_checked():
    x = z((M, K), bf16)
    _reaches_device_check(cr.convrot_rotate_quant_act, x, g, z((M, KP // 2), u8), z((M,), f32),
                          z((M, KP), f32))
    _raises(cr.convrot_rotate_quant_act, x, g, z((M, KP // 2 - 1), u8), match="xq")
    _raises(cr.convrot_rotate_quant_act, x, g, z((M + 1, KP // 2), u8), match="xq")
    _raises(cr.convrot_rotate_quant_act, x, g, z((M, KP // 2), f32), match="xq")
    _raises(cr.convrot_rotate_quant_act, x, g, z((M, KP), u8)[:, ::2], match="xq")
    _raises(cr.convrot_rotate_quant_act, x, g, None, z((M - 1,), f32), match="xs")
    _raises(cr.convrot_rotate_quant_act, x, g, None, z((M,), bf16), match="xs")
    _raises(cr.convrot_rotate_quant_act, x, g, None, None, z((M, K), f32), match="xrot")
    _raises(cr.convrot_rotate_quant_act, z((M, K), torch.float16), g, match="bfloat16 or float32")
    _raises(cr.convrot_rotate_quant_act, z((M, K, 1), bf16), g, match="2-D")
    _raises(cr.convrot_rotate_quant_act, z((K, M), bf16).t(), g, match="unit column stride")
    # strided rows are accepted (the library takes the row stride)
    _reaches_device_check(cr.convrot_rotate_quant_act, z((M, 2 * K), bf16)[:, :K], g)


def test_rotate_quant_other_formats_checked():
    x = z((M, K), f32)
    _reaches_device_check(cr.convrot_rotate_quant_act_i8, x, g, z((M, KP), i8), z((M,), f32))
    _raises(cr.convrot_rotate_quant_act_i8, x, g, z((M, KP // 2), i8), match="xq")
    x64 = z((M, K), bf16)
    S = cr.mx_scale_stride(128)
    _reaches_device_check(cr.convrot_rotate_quant_act_mxfp4, x64, 64, z((M, 64), u8),
                          z((M, S), u8))
    _raises(cr.convrot_rotate_quant_act_mxfp4, x64, 64, z((M, 64), u8), z((M, S - 1), u8),
            match="scales")
    _raises(cr.convrot_rotate_quant_act_mxfp4, x64, 64, z((M, 64), u8), z((M,), f32),
            match="scales")


def test_quant_weight_checked():
    w = z((N, K), bf16)
    _reaches_device_check(cr.convrot_quant_weight, w, g, z((N, KP // 2), u8), z((N,), f32))
    _raises(cr.convrot_quant_weight, w, g, z((N, KP // 2 + 16), u8), match="wq")
    _raises(cr.convrot_quant_weight, w, g, None, z((N + 1,), f32), match="ws")
    _raises(cr.convrot_quant_weight, z((N, 2 * K), bf16)[:, :K], g, match="contiguous")
    _raises(cr.convrot_quant_weight_i8, w, g, z((N, KP // 2), i8), match="wq")
    _raises(cr.convrot_quant_weight_mxfp4, z((N, 128), bf16), 64, None, z((N, 3), u8),
            match="scales")


def _gemm_args(Mx=M, Nx=N, kp=KP, code_cols=lambda kp: kp // 2):
    return (z((Mx, code_cols(kp)), u8), z((Mx,), f32), z((Nx, code_cols(kp)), u8), z((Nx,), f32))


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_integer_gemm_checked(fmt):
    gemm = cr.convrot_w4a4_gemm if fmt == "int4" else cr.convrot_w8a8_gemm
    cols = (lambda kp: kp // 2) if fmt == "int4" else (lambda kp: kp)
    xq, xs, wq, ws = _gemm_args(code_cols=cols)
    _reaches_device_check(gemm, xq, xs, wq, ws, z((N,), bf16), z((M, N), bf16))
    _reaches_device_check(gemm, xq, xs.view(M, 1), wq, ws.view(N, 1))     # [rows, 1] scales
    _raises(gemm, xq, xs, wq[:, :-1].contiguous(), ws, match="same depth")
    _raises(gemm, xq, z((M - 1,), f32), wq, ws, match="xs")
    _raises(gemm, xq, xs, wq, z((N,), bf16), match="ws")
    _raises(gemm, xq, xs, wq, ws, z((N - 1,), bf16), match="bias")
    _raises(gemm, xq, xs, wq, ws, z((N,), f32), match="bias")
    _raises(gemm, xq, xs, wq, ws, None, z((M, N + 1), bf16), match="y")
    _raises(gemm, xq, xs, wq, ws, None, z((M, N), f32), match="y")
    _raises(gemm, xq, xs, wq, ws, None, z((N, M), bf16).t(), match="y")
    _raises(gemm, xq.to(f32), xs, wq, ws, match="xq")
    wide = z((M, 2 * xq.shape[1]), u8)[:, :xq.shape[1]]                   # sliced: wrong stride
    _raises(gemm, wide, xs, wq, ws, match="xq")
    _raises(gemm, xq.view(-1), xs, wq, ws, match="2-D")
    _raises(gemm, xq, xs.numpy(), wq, ws, match="Tensor")


def test_mxfp4_gemm_checked():
    xq, _, wq, _ = _gemm_args(kp=128)
    S = cr.mx_scale_stride(128)
    _reaches_device_check(cr.convrot_mxfp4_gemm, xq, z((M, S), u8), wq, z((N, S), u8))
    _raises(cr.convrot_mxfp4_gemm, xq, z((M, S + 4), u8), wq, z((N, S), u8), match="xbs")
    _raises(cr.convrot_mxfp4_gemm, xq, z((M, S), u8), wq, z((N - 1, S), u8), match="wbs")
    _raises(cr.convrot_mxfp4_gemm, xq, z((M, S), u8), wq, z((N, S), u8), z((N,), f32),
            match="bias")


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
def test_linear_checked(fmt):
    linear = {"int4": cr.convrot_w4a4_linear, "int8": cr.convrot_w8a8_linear,
              "mxfp4": cr.convrot_mxfp4_linear}[fmt]
    gg = 64 if fmt == "mxfp4" else g
    kp = cr.convrot_padded_k(K, gg)
    cols = kp if fmt == "int8" else kp // 2
    wq = z((N, cols), i8 if fmt == "int8" else u8)
    ws = z((N, cr.mx_scale_stride(kp)), u8) if fmt == "mxfp4" else z((N,), f32)
    x = z((M, K), bf16)
    _reaches_device_check(linear, x, gg, wq, ws, z((N,), bf16), z((M, N), bf16))
    # weights quantized for another K or group size
    _raises(linear, z((M, K + gg), bf16), gg, wq, ws, match="bytes per row")
    _raises(linear, x, gg, z((N, cols + 1), u8), ws, match="bytes per row")
    _raises(linear, x, gg, wq, ws, z((N + 1,), bf16), match="bias")
    _raises(linear, x, gg, wq, ws, None, z((M + 1, N), bf16), match="y")
    _raises(linear, z((M, 2 * K), bf16)[:, :K], gg, wq, ws, match="contiguous")
    if fmt == "mxfp4":
        _raises(linear, x, gg, wq, z((N, 1), u8), match="wbs")
    else:
        _raises(linear, x, gg, wq, z((N - 1,), f32), match="ws")
    ws_bad = z((64, 64), u8)[:, :8]
    _raises(linear, x, gg, wq, ws, workspace=ws_bad, match="workspace")


@pytest.mark.parametrize("cls", [cr.ConvLinear4bit, cr.ConvLinear8bit, cr.ConvLinearFP4])
def test_module_bias_is_a_buffer(cls):
    """The bias travels with state_dict() and .to(); a module built without bias has none."""
    mod = cls(K, N, 64, bias=True)
    mod.weight_packed.random_(0, 100)
    mod.weight_scale.random_(0, 100)
    mod.bias.copy_(torch.arange(N, dtype=f32).to(bf16))
    sd = mod.state_dict()
    assert set(sd) == {"weight_packed", "weight_scale", "bias"}
    other = cls(K, N, 64, bias=True)
    other.load_state_dict(sd)
    for name in sd:
        assert torch.equal(getattr(other, name), getattr(mod, name)), name
    assert other.bias.dtype == bf16
    assert "bias" in dict(mod.named_buffers())
    assert mod.to(torch.device("cpu")).bias is mod.bias
    plain = cls(K, N, 64)
    assert plain.bias is None and "bias" not in plain.state_dict()


def test_from_linear_checks_bias_length():
    with pytest.raises(ValueError, match="bias must have"):
        cr.ConvLinear4bit.from_linear(z((N, K), bf16), z((N + 1,), bf16), group_size=16)
    with pytest.raises(ValueError, match="2-D"):
        cr.ConvLinear4bit.from_linear(z((N * K,), bf16), None, group_size=16)


def test_row_quant_helpers_checked():
    y = z((M, K), f32)
    _reaches_device_check(cr.convrot_quant_rows_int4, y, z((M, (K + 1) // 2), u8), z((M,), f32))
    _raises(cr.convrot_quant_rows_int4, z((M, K), bf16), match="float32")
    _raises(cr.convrot_quant_rows_int4, y, z((M, K // 2 + 1), u8), match="q")
    _raises(cr.convrot_quant_rows_int4, y, None, z((M + 1,), f32), match="s")
    _reaches_device_check(cr.convrot_dequant_int4, z((M, 50), u8), z((M,), f32), 100)
    _raises(cr.convrot_dequant_int4, z((M, 50), u8), z((M,), f32), 102, match="bytes per row")
    _raises(cr.convrot_dequant_int4, z((M, 50), f32), z((M,), f32), 100, match="q")
    _raises(cr.convrot_dequant_int4, z((M, 50), u8), z((M,), f32), 100, z((M, 100), f32),
            match="out")
