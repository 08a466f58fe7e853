"""Frozen int4 linear layer with autograd, for QLoRA-style fine-tuning.

Forward ``Y = X @ w^T (+ bias)`` runs the W4A16 GEMV / GEMM; backward
``dX = dY @ w`` runs the transposed GEMM on the same packed buffer, with no
repacking and no reshaping of scales or zeros.  The base weight is frozen: no
gradient is produced for it (nor for the base bias).  Source: "Re-write HQQ Fused
Gemm Transpose" (pytorch/ao #185), which fine-tunes a frozen 4-bit base with LoRA
adapters and needs exactly these two products of one packed weight.

The library's matmul accumulates in fp32.  The forward output is fp32 unless
``out_dtype`` asks for bfloat16 / float16 (the fp32 sum, bias included, rounded
once to nearest even in the kernel's epilogue; the bias then has that dtype, as
"[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560) ties the
bias type to the output type).  bf16 and
fp16 activations enter as they are (fp16 activations multiply the fp16 weight
operand); other dtypes are converted to bf16.  The incoming gradient takes the
activations' 16-bit dtype (fp16 gradients need the caller's loss scaling, as in
any fp16 training), and dX is written by the kernel directly in the dtype of x
when that is bf16 / fp16 (the same single rounding as converting its fp32 result).
A dtype conversion here is argument marshalling; the products run in the gfx950
kernels.  A bias that requires grad gets the sum of the incoming gradient over
the rows.
"""

from __future__ import annotations

import torch

from . import ops
from .ops import QuantizedWeight

_OUT_DTYPES = (None, torch.float32, torch.bfloat16, torch.float16)
_HALF = (torch.bfloat16, torch.float16)


def _operand(t: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return (t if t.dtype == dtype else t.to(dtype)).contiguous()


class _W4A16Matmul(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, qw: QuantizedWeight, bias: torch.Tensor | None,
                out_dtype: torch.dtype | None):
        lead = x.shape[:-1]
        adt = x.dtype if x.dtype in _HALF else torch.bfloat16
        odt = torch.float32 if out_dtype is None else out_dtype
        y = ops.mm(_operand(x.reshape(-1, x.shape[-1]), adt), qw,
                   bias=None if bias is None else _operand(bias, odt), out_dtype=odt)
        ctx.qw = qw
        ctx.x_dtype = x.dtype
        ctx.a_dtype = adt
        ctx.lead = lead
        ctx.bias_dtype = None if bias is None else bias.dtype
        return y.view(*lead, qw.N)

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        qw: QuantizedWeight = ctx.qw
        g2 = gy.reshape(-1, qw.N)
        dx = None
        if ctx.needs_input_grad[0]:
            gdt = ctx.x_dtype if ctx.x_dtype in _HALF else torch.float32
            dx = ops.mm(_operand(g2, ctx.a_dtype), qw, transposed=True, out_dtype=gdt).view(*ctx.lead, qw.K)
            if dx.dtype != ctx.x_dtype:
                dx = dx.to(ctx.x_dtype)
        db = g2.float().sum(0).to(ctx.bias_dtype) if ctx.needs_input_grad[2] else None
        return dx, None, db, None


def w4a16_linear(x: torch.Tensor, qw: QuantizedWeight, bias: torch.Tensor | None = None,
                 out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """Differentiable ``x @ w^T (+ bias)`` over a packed int4 weight: fp32 result, or
    ``out_dtype`` (bfloat16 / float16) rounded once from the fp32 sum."""
    if out_dtype not in _OUT_DTYPES:
        raise ValueError(f"out_dtype must be None, float32, bfloat16 or float16, not {out_dtype}")
    return _W4A16Matmul.apply(x, qw, bias, out_dtype)


class W4A16Linear(torch.nn.Module):
    """A frozen int4 base linear layer: ``forward(x) = x @ w^T (+ bias)``; fp32 output, or
    ``out_dtype`` (bfloat16 / float16, the bias held in that dtype)."""

    def __init__(self, qw: QuantizedWeight, bias: torch.Tensor | None = None, out_dtype: torch.dtype | None = None):
        super().__init__()
        if out_dtype not in _OUT_DTYPES:
            raise ValueError(f"out_dtype must be None, float32, bfloat16 or float16, not {out_dtype}")
        self.qw = qw
        self.out_dtype = out_dtype
        if bias is not None:
            bias = bias.detach().to(torch.float32 if out_dtype is None else out_dtype).contiguous()
        self.register_buffer("bias", bias)

    @classmethod
    def from_weight(cls, weight: torch.Tensor, mode: str = "rowwise", group: int | None = None,
                    bias: torch.Tensor | None = None, out_dtype: torch.dtype | None = None) -> "W4A16Linear":
        """Quantize a [N][K] fp32 / fp16 / bf16 device weight and wrap it."""
        return cls(ops.quantize_pack(weight, mode, group), bias, out_dtype)

    @property
    def in_features(self) -> int:
        return self.qw.K

    @property
    def out_features(self) -> int:
        return self.qw.N

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return w4a16_linear(x, self.qw, self.bias, self.out_dtype)
