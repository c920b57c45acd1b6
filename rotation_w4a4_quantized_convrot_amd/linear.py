"""ConvLinear4bit: plug-and-play W4A4 replacement for a linear layer.

ConvRot paper (arXiv 2512.03673), Abstract and Fig. 3: the module integrates rotation,
quantization, GEMM and dequantization.  Weights are rotated and quantized once, offline
(per output channel); activations are rotated and quantized per token on every call.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class ConvLinear4bit(torch.nn.Module):
    """y = dequant(int4(RHT(x)) @ int4(RHT(W))^T) + bias, output bf16."""

    def __init__(self, in_features: int, out_features: int, group_size: int = 256,
                 device=None):
        super().__init__()
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.group_size = int(group_size)
        self.padded_in = _lib.convrot_padded_k(self.in_features, self.group_size)
        self.register_buffer("weight_packed", torch.zeros(
            (self.out_features, self.padded_in // 2), dtype=torch.uint8, device=device))
        self.register_buffer("weight_scale", torch.zeros(
            (self.out_features,), dtype=torch.float32, device=device))
        self.bias: Optional[torch.Tensor] = None
        self._workspace: Optional[torch.Tensor] = None

    @classmethod
    def from_linear(cls, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    group_size: int = 256) -> "ConvLinear4bit":
        """Builds the layer from a dense weight [N, K] (bf16 or fp32, on the GPU)."""
        n, k = weight.shape
        mod = cls(k, n, group_size, device=weight.device)
        _lib.convrot_quant_weight(weight.contiguous(), group_size, mod.weight_packed,
                                  mod.weight_scale)
        if bias is not None:
            mod.bias = bias.detach().to(torch.bfloat16).contiguous()
        return mod

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        need = _lib.convrot_w4a4_workspace_bytes(x2.shape[0], self.in_features, self.group_size)
        if self._workspace is None or self._workspace.numel() < need or \
                self._workspace.device != x2.device:
            self._workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x2.device)
        y = _lib.convrot_w4a4_linear(x2, self.group_size, self.weight_packed, self.weight_scale,
                                     self.bias, workspace=self._workspace)
        return y.reshape(*lead, self.out_features)
