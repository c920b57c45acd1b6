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
CONVROT_ERR_SCRATCH = -9
CONVROT_F32 = 0
CONVROT_BF16 = 1
CONVROT_MAX_KP = 65536
CONVROT_NOALLOC_SCRATCH_BYTES = 72 << 20

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
    "convrot_w4a4_linear_noalloc": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp,
                                             _vp, _vp]),
    "convrot_w4a4_linear_fused": (_c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp,
                                           _vp, ctypes.c_size_t, _vp, _vp]),
    "convrot_quant_rows_int4": (_c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "convrot_dequant_int4": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
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


_CODE_BYTES = (torch.uint8, torch.int8)   # code tensors: one byte per element, either signedness


def _is_tensor(t, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")


def _mat(t: Optional[torch.Tensor], name: str, rows: int, cols: int, dtypes) -> None:
    """A caller-supplied 2-D buffer: contiguous, shape (rows, cols), one of dtypes (None passes:
    the binding allocates it)."""
    if t is None:
        return
    _is_tensor(t, name)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _vec(t: Optional[torch.Tensor], name: str, n: int, dtype: torch.dtype) -> None:
    """A per-row or per-column vector: contiguous, n elements as (n,) or (n, 1), dtype."""
    if t is None:
        return
    _is_tensor(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) not in ((n,), (n, 1)):
        raise ValueError(f"{name} must have {n} elements as ({n},) or ({n}, 1), got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _codes_2d(t: torch.Tensor, name: str) -> Tuple[int, int]:
    _is_tensor(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got {t.dim()} dimensions")
    return int(t.shape[0]), int(t.shape[1])


def _activations(x: torch.Tensor, contiguous: bool, name: str = "x") -> Tuple[int, int]:
    """x [M, K], bf16 or fp32; rows may be strided unless the entry point needs row stride K."""
    _is_tensor(x, name)
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got {x.dim()} dimensions")
    if contiguous and not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    _dtype_code(x)
    return int(x.shape[0]), int(x.shape[1])


def _workspace(ws: torch.Tensor) -> int:
    """Bytes of a caller-supplied workspace (contiguous; any dtype)."""
    _is_tensor(ws, "workspace")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


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
# Every entry point checks each tensor argument on the host first (device, dtype, contiguity
# and the exact shape implied by M, N and K'), so that no kernel reads or writes past a buffer.
def _rotate(fn, x, g, xq, xs, xrot, want_rotated, code_cols, code_dtype, scale_shape,
            scale_dtype):
    M, K = _activations(x, contiguous=False)
    Kp = convrot_padded_k(K, g)
    cols = code_cols(Kp)
    _mat(xq, "xq", M, cols, _CODE_BYTES)
    sshape = scale_shape(M, Kp)
    if len(sshape) == 1:
        _vec(xs, "xs", M, scale_dtype)
    else:
        _mat(xs, "scales", sshape[0], sshape[1], (scale_dtype,))
    _mat(xrot, "xrot", M, Kp, (torch.float32,))
    dev = _require_device(x, xq, xs, xrot)
    if xq is None:
        xq = torch.empty((M, cols), dtype=code_dtype, device=dev)
    if xs is None:
        xs = torch.empty(sshape, dtype=scale_dtype, device=dev)
    if xrot is None and want_rotated:
        xrot = torch.empty((M, Kp), dtype=torch.float32, device=dev)
    st = fn(_ptr(x), _dtype_code(x), M, K, x.stride(0), g, _ptr(xq), _ptr(xs), _ptr(xrot),
            _stream(dev))
    _check(st, g)
    return (xq, xs, xrot) if xrot is not None else (xq, xs)


def _quant_weight(fn, w, g, wq, ws, code_cols, code_dtype, scale_shape, scale_dtype):
    N, K = _activations(w, contiguous=True, name="w")
    Kp = convrot_padded_k(K, g)
    cols = code_cols(Kp)
    _mat(wq, "wq", N, cols, _CODE_BYTES)
    sshape = scale_shape(N, Kp)
    if len(sshape) == 1:
        _vec(ws, "ws", N, scale_dtype)
    else:
        _mat(ws, "scales", sshape[0], sshape[1], (scale_dtype,))
    dev = _require_device(w, wq, ws)
    if wq is None:
        wq = torch.empty((N, cols), dtype=code_dtype, device=dev)
    if ws is None:
        ws = torch.empty(sshape, dtype=scale_dtype, device=dev)
    st = fn(_ptr(w), _dtype_code(w), N, K, g, _ptr(wq), _ptr(ws), _stream(dev))
    _check(st, g)
    return wq, ws


def _row_scale_shape(rows: int, kp: int):
    return (rows,)


def _mx_scale_shape(rows: int, kp: int):
    return (rows, mx_scale_stride(kp))


def _half(kp: int) -> int:
    return kp // 2


def _full(kp: int) -> int:
    return kp


def _gemm_checks(xq, xs, wq, ws, bias, y, cols_per_kp, mx: bool):
    """Shapes of a GEMM call from its code operands; returns (M, N, K')."""
    M, cols = _codes_2d(xq, "xq")
    N, wcols = _codes_2d(wq, "wq")
    if wcols != cols:
        raise ValueError(f"xq and wq must have the same depth, got {cols} and {wcols} bytes")
    Kp = cols * cols_per_kp
    _mat(xq, "xq", M, cols, _CODE_BYTES)
    _mat(wq, "wq", N, cols, _CODE_BYTES)
    if mx:
        _mat(xs, "xbs", M, mx_scale_stride(Kp), (torch.uint8,))
        _mat(ws, "wbs", N, mx_scale_stride(Kp), (torch.uint8,))
    else:
        _is_tensor(xs, "xs")
        _is_tensor(ws, "ws")
        _vec(xs, "xs", M, torch.float32)
        _vec(ws, "ws", N, torch.float32)
    _vec(bias, "bias", N, torch.bfloat16)
    _mat(y, "y", M, N, (torch.bfloat16,))
    return M, N, Kp


def _gemm(fn, xq, xs, wq, ws, bias, y, want_acc, cols_per_kp, mx, acc_dtype):
    M, N, Kp = _gemm_checks(xq, xs, wq, ws, bias, y, cols_per_kp, mx)
    dev = _require_device(xq, xs, wq, ws, bias, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=acc_dtype, device=dev) if want_acc else None
    st = fn(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(bias), M, N, Kp, _ptr(y), _ptr(acc),
            _stream(dev))
    _check(st)
    return (y, acc) if want_acc else y


def _linear(fn, need_fn, x, g, wq, ws, bias, y, workspace, code_cols, mx):
    M, K = _activations(x, contiguous=True)
    Kp = convrot_padded_k(K, g)
    N, cols = _codes_2d(wq, "wq")
    if cols != code_cols(Kp):
        raise ValueError(f"wq must have {code_cols(Kp)} bytes per row for K={K}, g={g} "
                         f"(K' = {Kp}), got {cols}")
    _mat(wq, "wq", N, cols, _CODE_BYTES)
    if mx:
        _mat(ws, "wbs", N, mx_scale_stride(Kp), (torch.uint8,))
    else:
        _is_tensor(ws, "ws")
        _vec(ws, "ws", N, torch.float32)
    _vec(bias, "bias", N, torch.bfloat16)
    _mat(y, "y", M, N, (torch.bfloat16,))
    if workspace is not None:
        _workspace(workspace)
    dev = _require_device(x, wq, ws, bias, y, workspace)
    if workspace is None:
        workspace = torch.empty((max(need_fn(M, K, g), 1),), dtype=torch.uint8, device=dev)
    nbytes = _workspace(workspace)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = fn(_ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(ws), N, _ptr(bias), _ptr(y),
            _ptr(workspace), nbytes, _stream(dev))
    _check(st, g)
    return y


def convrot_rotate_quant_act(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                             xs: Optional[torch.Tensor] = None, xrot: Optional[torch.Tensor] = None,
                             want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq uint8 [M, K'/2], xs fp32 [M][, xrot])."""
    return _rotate(load_library().convrot_rotate_quant_act, x, g, xq, xs, xrot, want_rotated,
                   _half, torch.uint8, _row_scale_shape, torch.float32)


def convrot_quant_weight(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq uint8 [N, K'/2], ws fp32 [N])."""
    return _quant_weight(load_library().convrot_quant_weight, w, g, wq, ws, _half, torch.uint8,
                         _row_scale_shape, torch.float32)


def convrot_w4a4_gemm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      want_acc: bool = False):
    """Packed int4 GEMM + dequant: y bf16 [M, N] (and the int32 sums [M, N] if want_acc)."""
    return _gemm(load_library().convrot_w4a4_gemm, xq, xs, wq, ws, bias, y, want_acc, 2, False,
                 torch.int32)


def convrot_w4a4_linear(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ConvLinear4bit forward: x [M, K] contiguous -> y bf16 [M, N]."""
    return _linear(load_library().convrot_w4a4_linear, convrot_w4a4_workspace_bytes, x, g, wq,
                   ws, bias, y, workspace, _half, False)


def convrot_w4a4_linear_fused(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                              bias: Optional[torch.Tensor] = None,
                              y: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None,
                              status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ConvLinear4bit forward in one kernel launch (rotate + quantize, grid barrier, GEMM):
    x [M, K] bf16 contiguous -> y bf16 [M, N], bit-identical to convrot_w4a4_linear.
    status: int32 [1] device tensor, zero on entry; the kernel sets it nonzero if its grid
    barrier timed out (y then incomplete).  Unsupported shapes raise ConvRotError."""
    M, K = _activations(x, contiguous=True)
    Kp = convrot_padded_k(K, g)
    N, cols = _codes_2d(wq, "wq")
    if cols != Kp // 2:
        raise ValueError(f"wq must have {Kp // 2} bytes per row for K={K}, g={g} (K' = {Kp}), "
                         f"got {cols}")
    _mat(wq, "wq", N, cols, _CODE_BYTES)
    _is_tensor(ws, "ws")
    _vec(ws, "ws", N, torch.float32)
    _vec(bias, "bias", N, torch.bfloat16)
    _mat(y, "y", M, N, (torch.bfloat16,))
    if status is not None:
        _vec(status, "status", 1, torch.int32)
    if workspace is not None:
        _workspace(workspace)
    dev = _require_device(x, wq, ws, bias, y, workspace, status)
    if workspace is None:
        workspace = torch.empty((max(convrot_w4a4_workspace_bytes(M, K, g), 1),),
                                dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.zeros((1,), dtype=torch.int32, device=dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = load_library().convrot_w4a4_linear_fused(
        _ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(ws), N, _ptr(bias), _ptr(y),
        _ptr(workspace), _workspace(workspace), _ptr(status), _stream(dev))
    _check(st, g)
    return y


def convrot_w4a4_linear_noalloc(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                                bias: Optional[torch.Tensor] = None,
                                y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ConvLinear4bit forward without a workspace: the library keeps the activation codes in a
    fixed device array of CONVROT_NOALLOC_SCRATCH_BYTES per device (calls that overlap in
    time on one device race on it).  Pass y to keep the call free of allocations."""
    M, K = _activations(x, contiguous=True)
    Kp = convrot_padded_k(K, g)
    N, cols = _codes_2d(wq, "wq")
    if cols != Kp // 2:
        raise ValueError(f"wq must have {Kp // 2} bytes per row for K={K}, g={g} (K' = {Kp}), "
                         f"got {cols}")
    _mat(wq, "wq", N, cols, _CODE_BYTES)
    _is_tensor(ws, "ws")
    _vec(ws, "ws", N, torch.float32)
    _vec(bias, "bias", N, torch.bfloat16)
    _mat(y, "y", M, N, (torch.bfloat16,))
    dev = _require_device(x, wq, ws, bias, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = load_library().convrot_w4a4_linear_noalloc(
        _ptr(x), _dtype_code(x), M, K, g, _ptr(wq), _ptr(ws), N, _ptr(bias), _ptr(y),
        _stream(dev))
    _check(st, g)
    return y


# ----------------------------------------------------------------- INT8 (W8A8) variant
def convrot_w8a8_workspace_bytes(M: int, K: int, g: int) -> int:
    return int(load_library().convrot_w8a8_workspace_bytes(int(M), int(K), int(g)))


def convrot_rotate_quant_act_i8(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                                xs: Optional[torch.Tensor] = None,
                                xrot: Optional[torch.Tensor] = None, want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq int8 [M, K'], xs fp32 [M][, xrot])."""
    return _rotate(load_library().convrot_rotate_quant_act_i8, x, g, xq, xs, xrot, want_rotated,
                   _full, torch.int8, _row_scale_shape, torch.float32)


def convrot_quant_weight_i8(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq int8 [N, K'], ws fp32 [N])."""
    return _quant_weight(load_library().convrot_quant_weight_i8, w, g, wq, ws, _full, torch.int8,
                         _row_scale_shape, torch.float32)


def convrot_w8a8_gemm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      want_acc: bool = False):
    """int8 GEMM + dequant: y bf16 [M, N] (and the int32 sums [M, N] if want_acc)."""
    return _gemm(load_library().convrot_w8a8_gemm, xq, xs, wq, ws, bias, y, want_acc, 1, False,
                 torch.int32)


def convrot_w8a8_linear(x: torch.Tensor, g: int, wq: torch.Tensor, ws: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 ConvRot forward: x [M, K] contiguous -> y bf16 [M, N]."""
    return _linear(load_library().convrot_w8a8_linear, convrot_w8a8_workspace_bytes, x, g, wq,
                   ws, bias, y, workspace, _full, False)


def mx_scale_stride(kp: int) -> int:
    """Bytes per row of MXFP4 block scales: K'/32 blocks padded to whole dwords."""
    return 4 * (-(-kp // 128))


def convrot_rotate_quant_act_mxfp4(x: torch.Tensor, g: int, xq: Optional[torch.Tensor] = None,
                                   xbs: Optional[torch.Tensor] = None,
                                   xrot: Optional[torch.Tensor] = None, want_rotated: bool = False):
    """x [M, K] (bf16/fp32, row stride x.stride(0)) -> (xq uint8 [M, K'/2] E2M1 codes,
    xbs uint8 [M, S] E8M0 block scales (S = 4 ceil(K'/128): K'/32 blocks, zero padding)
    [, xrot fp32 [M, K']])."""
    return _rotate(load_library().convrot_rotate_quant_act_mxfp4, x, g, xq, xbs, xrot,
                   want_rotated, _half, torch.uint8, _mx_scale_shape, torch.uint8)


def convrot_quant_weight_mxfp4(w: torch.Tensor, g: int, wq: Optional[torch.Tensor] = None,
                               wbs: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [N, K] contiguous (bf16/fp32) -> (wq uint8 [N, K'/2], wbs uint8 [N, S])."""
    return _quant_weight(load_library().convrot_quant_weight_mxfp4, w, g, wq, wbs, _half,
                         torch.uint8, _mx_scale_shape, torch.uint8)


def convrot_mxfp4_gemm(xq: torch.Tensor, xbs: torch.Tensor, wq: torch.Tensor, wbs: torch.Tensor,
                       bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                       want_acc: bool = False):
    """MXFP4 GEMM: y bf16 [M, N] (and the fp32 sums [M, N] before the bias if want_acc)."""
    return _gemm(load_library().convrot_mxfp4_gemm, xq, xbs, wq, wbs, bias, y, want_acc, 2, True,
                 torch.float32)


def convrot_mxfp4_workspace_bytes(M: int, K: int, g: int) -> int:
    return int(load_library().convrot_mxfp4_workspace_bytes(M, K, g))


def convrot_mxfp4_linear(x: torch.Tensor, g: int, wq: torch.Tensor, wbs: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The MXFP4 ConvRot forward pass: x [M, K] contiguous -> y bf16 [M, N]."""
    return _linear(load_library().convrot_mxfp4_linear, convrot_mxfp4_workspace_bytes, x, g, wq,
                   wbs, bias, y, workspace, _half, True)


# ----------------------------------------------------------------- analysis helpers
def convrot_quant_rows_int4(y: torch.Tensor, q: Optional[torch.Tensor] = None,
                            s: Optional[torch.Tensor] = None):
    """Per-row int4 codes of already-transformed rows (no rotation): y fp32 [M, K] (rows may be
    strided) -> (q uint8 [M, ceil(K/2)], s fp32 [M]), the layer's quantization rule."""
    _is_tensor(y, "y")
    if y.dim() != 2:
        raise ValueError(f"y must be 2-D, got {y.dim()} dimensions")
    if y.dtype != torch.float32:
        raise TypeError(f"y must be torch.float32, got {y.dtype}")
    if y.stride(1) != 1 and y.shape[1] > 1:
        raise ValueError("y must be 2-D with unit column stride")
    M, K = int(y.shape[0]), int(y.shape[1])
    cols = (K + 1) // 2
    _mat(q, "q", M, cols, _CODE_BYTES)
    _vec(s, "s", M, torch.float32)
    dev = _require_device(y, q, s)
    if q is None:
        q = torch.empty((M, cols), dtype=torch.uint8, device=dev)
    if s is None:
        s = torch.empty((M,), dtype=torch.float32, device=dev)
    _check(load_library().convrot_quant_rows_int4(_ptr(y), M, K, y.stride(0), _ptr(q), _ptr(s),
                                                  _stream(dev)))
    return q, s


def convrot_dequant_int4(q: torch.Tensor, s: torch.Tensor, K: int,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed int4 codes q [M, ceil(K/2)] and row scales s [M] -> fp64 [M, K], code * scale."""
    M, cols = _codes_2d(q, "q")
    if q.dtype not in _CODE_BYTES:
        raise TypeError(f"q must be torch.uint8 or torch.int8, got {q.dtype}")
    if cols != (K + 1) // 2:
        raise ValueError(f"q must have {(K + 1) // 2} bytes per row for K = {K}, got {cols}")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _vec(s, "s", M, torch.float32)
    _mat(out, "out", M, K, (torch.float64,))
    dev = _require_device(q, s, out)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float64, device=dev)
    _check(load_library().convrot_dequant_int4(_ptr(q), _ptr(s), M, K, _ptr(out), _stream(dev)))
    return out

