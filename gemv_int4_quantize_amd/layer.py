"""Frozen int4 linear layer with autograd, for QLoRA-style fine-tuning.

Forward ``Y = X @ w^T (+ bias)`` runs the W4A16 GEMV / GEMM; backward
``dX = dY @ w`` runs the transposed GEMM on the same packed buffer, with no
repacking and no reshaping of scales or zeros.  The base weight is frozen: no
gradient is produced for it (nor for the base bias).  Source: "Re-write HQQ Fused
Gemm Transpose" (pytorch/ao #185), which fine-tunes a frozen 4-bit base with LoRA
adapters and needs exactly these two products of one packed weight.

The library's matmul accumulates and returns fp32.  bf16 and fp16 activations enter
it as they are (fp16 activations multiply the fp16 weight operand); other dtypes
are converted to bf16.  The incoming gradient takes the activations' 16-bit dtype
(fp16 gradients need the caller's loss scaling, as in any fp16 training).  A
dtype conversion here is argument marshalling; the products run in the gfx950
kernels.  A bias that requires grad gets the sum of the incoming gradient over
the rows.
"""

from __future__ import annotations

import torch

from . import ops
from .ops import QuantizedWeight


def _operand(t: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return (t if t.dtype == dtype else t.to(dtype)).contiguous()


class _W4A16Matmul(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, qw: QuantizedWeight, bias: torch.Tensor | None):
        lead = x.shape[:-1]
        adt = x.dtype if x.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
        y = ops.mm(_operand(x.reshape(-1, x.shape[-1]), adt), qw,
                   bias=None if bias is None else _operand(bias, torch.float32))
        ctx.qw = qw
        ctx.x_dtype = x.dtype
        ctx.a_dtype = adt
        ctx.lead = lead
        return y.view(*lead, qw.N)

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        qw: QuantizedWeight = ctx.qw
        g2 = gy.reshape(-1, qw.N)
        dx = None
        if ctx.needs_input_grad[0]:
            dx = ops.mm(_operand(g2, ctx.a_dtype), qw, transposed=True).view(*ctx.lead, qw.K).to(ctx.x_dtype)
        db = g2.sum(0) if ctx.needs_input_grad[2] else None
        return dx, None, db


def w4a16_linear(x: torch.Tensor, qw: QuantizedWeight, bias: torch.Tensor | None = None) -> torch.Tensor:
    """Differentiable ``x @ w^T (+ bias)`` over a packed int4 weight (fp32 result)."""
    return _W4A16Matmul.apply(x, qw, bias)


class W4A16Linear(torch.nn.Module):
    """A frozen int4 base linear layer: ``forward(x) = x @ w^T (+ bias)``, fp32 output."""

    def __init__(self, qw: QuantizedWeight, bias: torch.Tensor | None = None):
        super().__init__()
        self.qw = qw
        if bias is not None:
            bias = bias.detach().to(torch.float32).contiguous()
        self.register_buffer("bias", bias)

    @classmethod
    def from_weight(cls, weight: torch.Tensor, mode: str = "rowwise", group: int | None = None,
                    bias: torch.Tensor | None = None) -> "W4A16Linear":
        """Quantize a [N][K] fp32 / fp16 / bf16 device weight and wrap it."""
        return cls(ops.quantize_pack(weight, mode, group), bias)

    @property
    def in_features(self) -> int:
        return self.qw.K

    @property
    def out_features(self) -> int:
        return self.qw.N

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return w4a16_linear(x, self.qw, self.bias)
