"""ConvLinear4bit: plug-and-play W4A4 replacement for a linear layer, and its W8A8 and MXFP4
siblings.

ConvRot paper (arXiv 2512.03673), Abstract and Fig. 3: the module integrates rotation,
quantization, GEMM and dequantization.  Weights are rotated and quantized once, offline
(per output channel); activations are rotated and quantized per token on every call.  The
other two code formats keep the same rotation: int8 codes with scale absmax / 127 (the HSWQ
release notes' "Hadamard Orthogonal Rotation" form), and MXFP4 (E2M1 codes with one E8M0
scale per 32 values; the ConvRot author notes that the rotation suits floating-point
quantization too).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class _ConvLinearBase(torch.nn.Module):
    """Shared module logic; subclasses name the code format's entry points and buffers."""

    # per format: the entry points, the code dtype, codes per weight row given K', and the
    # scale buffer's shape and dtype
    _code_dtype = torch.uint8
    _quant_weight = None
    _workspace_bytes = None
    _linear = None

    def __init__(self, in_features: int, out_features: int, group_size: int = 256,
                 bias: bool = False, device=None):
        super().__init__()
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.group_size = int(group_size)
        self.padded_in = _lib.convrot_padded_k(self.in_features, self.group_size)
        self.register_buffer("weight_packed", torch.zeros(
            (self.out_features, self._code_bytes(self.padded_in)), dtype=self._code_dtype,
            device=device))
        shape, dtype = self._scale_layout(self.out_features, self.padded_in)
        self.register_buffer("weight_scale", torch.zeros(shape, dtype=dtype, device=device))
        # bf16 [N], or None; a buffer, so that state_dict() and .to() carry it with the weights
        self.register_buffer("bias", torch.zeros((self.out_features,), dtype=torch.bfloat16,
                                                 device=device) if bias else None)

    @staticmethod
    def _code_bytes(kp: int) -> int:
        return kp // 2

    @staticmethod
    def _scale_layout(n: int, kp: int):
        return (n,), torch.float32

    @classmethod
    def from_linear(cls, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    group_size: int = 256):
        """Builds the layer from a dense weight [N, K] (bf16 or fp32, on the GPU) and an
        optional bias of N elements."""
        if weight.dim() != 2:
            raise ValueError(f"weight must be 2-D [N, K], got shape {tuple(weight.shape)}")
        n, k = weight.shape
        if bias is not None and bias.numel() != n:
            raise ValueError(f"bias must have {n} elements (one per output), got {bias.numel()}")
        mod = cls(k, n, group_size, bias=bias is not None, device=weight.device)
        type(mod)._quant_weight(weight.contiguous(), group_size, mod.weight_packed,
                                mod.weight_scale)
        if bias is not None:
            mod.bias.copy_(bias.detach().reshape(n).to(torch.bfloat16))
        return mod

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        # The activation codes live in a workspace from the caching allocator, per call: it is
        # stream-ordered, so forward passes on different streams never share one.
        return type(self)._linear(x2, self.group_size, self.weight_packed, self.weight_scale,
                                  self.bias).reshape(*lead, self.out_features)


class ConvLinear4bit(_ConvLinearBase):
    """y = dequant(int4(RHT(x)) @ int4(RHT(W))^T) + bias, output bf16."""

    _quant_weight = staticmethod(_lib.convrot_quant_weight)
    _workspace_bytes = staticmethod(_lib.convrot_w4a4_workspace_bytes)
    _linear = staticmethod(_lib.convrot_w4a4_linear)


class ConvLinear8bit(_ConvLinearBase):
    """The W8A8 form: int8 codes, per-token / per-channel scale absmax / 127, output bf16."""

    _code_dtype = torch.int8
    _quant_weight = staticmethod(_lib.convrot_quant_weight_i8)
    _workspace_bytes = staticmethod(_lib.convrot_w8a8_workspace_bytes)
    _linear = staticmethod(_lib.convrot_w8a8_linear)

    @staticmethod
    def _code_bytes(kp: int) -> int:
        return kp


class ConvLinearFP4(_ConvLinearBase):
    """The MXFP4 form: E2M1 codes with E8M0 block scales on both operands, output bf16.
    group_size must be 64, 256 or 1024."""

    _quant_weight = staticmethod(_lib.convrot_quant_weight_mxfp4)
    _workspace_bytes = staticmethod(_lib.convrot_mxfp4_workspace_bytes)
    _linear = staticmethod(_lib.convrot_mxfp4_linear)

    @staticmethod
    def _scale_layout(n: int, kp: int):
        return (n, _lib.mx_scale_stride(kp)), torch.uint8
