"""ctypes binding of libconvrot (include/convrot.h): argument marshalling only.

Each function has the name of the C entry point it calls.  Torch tensors supply device
memory and the current HIP stream; every step of the computation runs in the HIP kernels
of libconvrot.  There is no fallback: if the library is not built the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconvrot.so")

CONVROT_OK = 0
CONVROT_ERR_GROUP = -1
CONVROT_ERR_UNSUPPORTED = -2
CONVROT_ERR_SHAPE = -3
CONVROT_ERR_NULL = -4
CONVROT_ERR_DTYPE = -5
CONVROT_ERR_ALIGN = -6
CONVROT_ERR_WORKSPACE = -7
CONVROT_ERR_HIP = -8
CONVROT_F32 = 0
CONVROT_BF16 = 1
CONVROT_MAX_KP = 65536

# (name, restype, argtypes) of every symbol include/convrot.h declares.
_c_int, _i32, _i64, _vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
SIGNATURES = {
    "convrot_status_string": (ctypes.c_char_p, [_c_int]),
    "convrot_version": (_c_int, []),
    "convrot_padded_k": (_i64, [_i64, _i64]),
    "convrot_is_power_of_4": (_c_int, [_i64]),
    "convrot_make_rht": (_c_int, [_i64, _vp, _i32]),
    "convrot_rotate_quant_act": (_c_int, [_vp, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "convrot_quant_weight": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_w4a4_gemm": (_c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_w4a4_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "convrot_w4a4_linear": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
    "convrot_rotate_quant_act_i8": (_c_int, [_vp, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                             _vp]),
    "convrot_quant_weight_i8": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_w8a8_gemm": (_c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_w8a8_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "convrot_w8a8_linear": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
    "convrot_rotate_quant_act_mxfp4": (_c_int, [_vp, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                                _vp]),
    "convrot_quant_weight_mxfp4": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_mxfp4_gemm": (_c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_mxfp4_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "convrot_mxfp4_linear": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libconvrot.so (once) and declares its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with rotation_w4a4_quantized_convrot_amd.build.build() "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class ConvRotError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _check(status: int, g=None) -> None:
    if status == CONVROT_OK:
        return
    if status == CONVROT_ERR_GROUP:
        raise ValueError(f"Regular Hadamard size must be a power of 4, got {g}")
    raise ConvRotError(status, convrot_status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CONVROT_BF16
    if t.dtype == torch.float32:
        return CONVROT_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _require_device(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU (the library has no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices")
    return dev


# ----------------------------------------------------------------- host helpers
def convrot_status_string(status: int) -> str:
    return load_library().convrot_status_string(int(status)).decode()


def convrot_version() -> int:
    return int(load_library().convrot_version())


def convrot_padded_k(K: int, g: int) -> int:
    r = int(load_library().convrot_padded_k(int(K), int(g)))
    if r < 0:
        _check(r, g)
    return r


def convrot_is_power_of_4(g: int) -> bool:
    return bool(load_library().convrot_is_power_of_4(int(g)))


def convrot_make_rht(g: int, normalized: bool = False) -> torch.Tensor:
    """Dense H_g (host fp32 tensor [g, g]) built by the library's closed form."""
    if not isinstance(g, int) or g < 1 or g > 4096:
        _check(CONVROT_ERR_GROUP if not convrot_is_power_of_4(int(g)) else CONVROT_ERR_UNSUPPORTED, g)
    h = torch.empty((g, g), dtype=torch.float32)
    _check(load_library().convrot_make_rht(g, h.data_ptr(), 1 if normalized else 0), g)
    return h


def convrot_w4a4_workspace_bytes(M: int, K: int, g: int) -> int:
    return int(load_library().convrot_w4a4_workspace_bytes(int(M), int(K), int(g)))


# ----------------------------------------------------------------- device entry points
def convrot_rotate_quant_act(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                             xs: Optional[torch.Tensor] = None, xrot: Optional[torch.Tensor] = None,
                             want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq uint8 [M, K'/2], xs fp32 [M][, xrot])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(x, xq, xs, xrot)
    if xq is None:
        xq = torch.empty((M, Kp // 2), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=dev)
    if xrot is None and want_rotated:
        xrot = torch.empty((M, Kp), dtype=torch.float32, device=dev)
    st = load_library().convrot_rotate_quant_act(
        _ptr(x), _dtype_code(x), M, K, x.stride(0), g, _ptr(xq), _ptr(xs), _ptr(xrot),
        _stream(dev))
    _check(st, g)
    return (xq, xs, xrot) if xrot is not None else (xq, xs)


def convrot_quant_weight(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq uint8 [N, K'/2], ws fp32 [N])."""
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    N, K = w.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(w, wq, ws)
    if wq is None:
        wq = torch.empty((N, Kp // 2), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = torch.empty((N,), dtype=torch.float32, device=dev)
    st = load_library().convrot_quant_weight(_ptr(w), _dtype_code(w), N, K, g, _ptr(wq), _ptr(ws),
                                             _stream(dev))
    _check(st, g)
    return wq, ws


def convrot_w4a4_gemm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      want_acc: bool = False):
    """Packed int4 GEMM + dequant: y bf16 [M, N] (and the int32 sums [M, N] if want_acc)."""
    M, half = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != half:
        raise ValueError("xq and wq must have the same packed depth")
    if bias is not None and bias.dtype != torch.bfloat16:
        raise TypeError("bias must be bfloat16")
    dev = _require_device(xq, xs, wq, ws, bias, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    st = load_library().convrot_w4a4_gemm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(bias), M, N,
                                          2 * half, _ptr(y), _ptr(acc), _stream(dev))
    _check(st)
    return (y, acc) if want_acc else y


def convrot_w4a4_linear(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ConvLinear4bit forward: x [M, K] contiguous -> y bf16 [M, N]."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    M, K = x.shape
    N = wq.shape[0]
    if bias is not None and bias.dtype != torch.bfloat16:
        raise TypeError("bias must be bfloat16")
    dev = _require_device(x, wq, ws, bias, y, workspace)
    need = convrot_w4a4_workspace_bytes(M, K, g)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = load_library().convrot_w4a4_linear(
        _ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(ws), N, _ptr(bias), _ptr(y),
        _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, g)
    return y


# ----------------------------------------------------------------- INT8 (W8A8) variant
def convrot_w8a8_workspace_bytes(M: int, K: int, g: int) -> int:
    return int(load_library().convrot_w8a8_workspace_bytes(int(M), int(K), int(g)))


def convrot_rotate_quant_act_i8(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                                xs: Optional[torch.Tensor] = None,
                                xrot: Optional[torch.Tensor] = None, want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq int8 [M, K'], xs fp32 [M][, xrot])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(x, xq, xs, xrot)
    if xq is None:
        xq = torch.empty((M, Kp), dtype=torch.int8, device=dev)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=dev)
    if xrot is None and want_rotated:
        xrot = torch.empty((M, Kp), dtype=torch.float32, device=dev)
    st = load_library().convrot_rotate_quant_act_i8(
        _ptr(x), _dtype_code(x), M, K, x.stride(0), g, _ptr(xq), _ptr(xs), _ptr(xrot),
        _stream(dev))
    _check(st, g)
    return (xq, xs, xrot) if xrot is not None else (xq, xs)


def convrot_quant_weight_i8(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq int8 [N, K'], ws fp32 [N])."""
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    N, K = w.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(w, wq, ws)
    if wq is None:
        wq = torch.empty((N, Kp), dtype=torch.int8, device=dev)
    if ws is None:
        ws = torch.empty((N,), dtype=torch.float32, device=dev)
    st = load_library().convrot_quant_weight_i8(_ptr(w), _dtype_code(w), N, K, g, _ptr(wq),
                                                _ptr(ws), _stream(dev))
    _check(st, g)
    return wq, ws


def convrot_w8a8_gemm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      want_acc: bool = False):
    """int8 GEMM + dequant: y bf16 [M, N] (and the int32 sums [M, N] if want_acc)."""
    M, Kp = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != Kp:
        raise ValueError("xq and wq must have the same depth")
    if bias is not None and bias.dtype != torch.bfloat16:
        raise TypeError("bias must be bfloat16")
    dev = _require_device(xq, xs, wq, ws, bias, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    st = load_library().convrot_w8a8_gemm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(bias), M, N,
                                          Kp, _ptr(y), _ptr(acc), _stream(dev))
    _check(st)
    return (y, acc) if want_acc else y


def convrot_w8a8_linear(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 ConvRot forward: x [M, K] contiguous -> y bf16 [M, N]."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    M, K = x.shape
    N = wq.shape[0]
    if bias is not None and bias.dtype != torch.bfloat16:
        raise TypeError("bias must be bfloat16")
    dev = _require_device(x, wq, ws, bias, y, workspace)
    need = convrot_w8a8_workspace_bytes(M, K, g)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = load_library().convrot_w8a8_linear(
        _ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(ws), N, _ptr(bias), _ptr(y),
        _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, g)
    return y


def mx_scale_stride(kp: int) -> int:
    """Bytes per row of MXFP4 block scales: K'/32 blocks padded to whole dwords."""
    return 4 * (-(-kp // 128))


def convrot_rotate_quant_act_mxfp4(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                                   xbs: Optional[torch.Tensor] = None,
                                   xrot: Optional[torch.Tensor] = None, want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq uint8 [M, K'/2] E2M1 codes,
    xbs uint8 [M, S] E8M0 block scales (S = 4 ceil(K'/128): K'/32 blocks, zero padding)
    [, xrot fp32 [M, K']])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(x, xq, xbs, xrot)
    if xq is None:
        xq = torch.empty((M, Kp // 2), dtype=torch.uint8, device=dev)
    if xbs is None:
        xbs = torch.empty((M, mx_scale_stride(Kp)), dtype=torch.uint8, device=dev)
    if xrot is None and want_rotated:
        xrot = torch.empty((M, Kp), dtype=torch.float32, device=dev)
    st = load_library().convrot_rotate_quant_act_mxfp4(
        _ptr(x), _dtype_code(x), M, K, x.stride(0), g, _ptr(xq), _ptr(xbs), _ptr(xrot),
        _stream(dev))
    _check(st, g)
    return (xq, xbs, xrot) if xrot is not None else (xq, xbs)


def convrot_quant_weight_mxfp4(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                               wbs: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq uint8 [N, K'/2], wbs uint8 [N, S])."""
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    N, K = w.shape
    Kp = convrot_padded_k(K, g)
    dev = _require_device(w, wq, wbs)
    if wq is None:
        wq = torch.empty((N, Kp // 2), dtype=torch.uint8, device=dev)
    if wbs is None:
        wbs = torch.empty((N, mx_scale_stride(Kp)), dtype=torch.uint8, device=dev)
    st = load_library().convrot_quant_weight_mxfp4(_ptr(w), _dtype_code(w), N, K, g, _ptr(wq),
                                                   _ptr(wbs), _stream(dev))
    _check(st, g)
    return wq, wbs


def convrot_mxfp4_gemm(xq: torch.Tensor, xbs: torch.Tensor, wq: torch.Tensor, wbs: torch.Tensor,
                       bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                       want_acc: bool = False):
    """MXFP4 GEMM: y bf16 [M, N] (and the fp32 sums [M, N] before the bias if want_acc)."""
    M, half = xq.shape
    N = wq.shape[0]
    Kp = 2 * half
    if wq.shape[1] != half:
        raise ValueError("xq and wq must have the same depth")
    if xbs.shape != (M, mx_scale_stride(Kp)) or wbs.shape != (N, mx_scale_stride(Kp)):
        raise ValueError("block scales must be [rows, 4 ceil(K'/128)]")
    if bias is not None and bias.dtype != torch.bfloat16:
        raise TypeError("bias must be bfloat16")
    dev = _require_device(xq, xbs, wq, wbs, bias, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.float32, device=dev) if want_acc else None
    st = load_library().convrot_mxfp4_gemm(_ptr(xq), _ptr(xbs), _ptr(wq), _ptr(wbs), _ptr(bias), M,
                                           N, Kp, _ptr(y), _ptr(acc), _stream(dev))
    _check(st)
    return (y, acc) if want_acc else y


def convrot_mxfp4_workspace_bytes(M: int, K: int, g: int) -> int:
    return int(load_library().convrot_mxfp4_workspace_bytes(M, K, g))


def convrot_mxfp4_linear(x: torch.Tensor, g: int, wq: torch.Tensor, wbs: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The MXFP4 ConvRot forward pass: x [M, K] contiguous -> y bf16 [M, N]."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    M, K = x.shape
    N = wq.shape[0]
    dev = _require_device(x, wq, wbs, bias, y, workspace)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    need = convrot_mxfp4_workspace_bytes(M, K, g)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    st = load_library().convrot_mxfp4_linear(_ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(wbs),
                                             N, _ptr(bias), _ptr(y), _ptr(workspace),
                                             workspace.numel(), _stream(dev))
    _check(st, g)
    return y
