"""GPU parity of the frozen int4 autograd layer: forward = W4A16 GEMM / GEMV, backward dX =
transposed GEMM on the same packed buffer, both against the oracle."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_mm_close, assert_rounded_close, dev_weight, host

pytestmark = pytest.mark.gpu


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 64)], ids=["rowwise", "g64"])
@pytest.mark.parametrize("lead", [(3,), (2, 96)], ids=["decode3", "batch2x96"])
def test_layer_forward_backward(mode, g, lead):
    N, K = 768, 1024
    M = int(np.prod(lead))
    print(f"[case] layer {mode}{g or ''} lead={lead}", flush=True)
    wb = synth.weight(709, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(wb, "bf16"), O.ROWWISE if mode == "rowwise" else O.GROUPWISE, g)
    bias = synth.bias_f32(709, 1, N)
    layer = w4.W4A16Linear.from_weight(dev_weight(wb, "bf16"), mode, g, torch.from_numpy(bias).to(DEV))
    xb = synth.activations_bf16(709, 2, M, K)
    gb = synth.activations_bf16(709, 3, M, N, tensor_id=synth.T_DY)
    # fp32 tensors holding bf16 values: the layer's conversions to bf16 are then exact
    x = torch.from_numpy(_bf16_to_f32(xb)).to(DEV).view(*lead, K).requires_grad_(True)
    y = layer(x)
    assert y.shape == (*lead, N) and y.dtype == torch.float32
    assert_mm_close(host(y.detach()).reshape(M, N), O.matmul(xb, *ref, K, bias=bias), f"layer forward {mode}")
    gy = torch.from_numpy(_bf16_to_f32(gb)).to(DEV).view(*lead, N)
    y.backward(gy)
    assert x.grad is not None and x.grad.shape == x.shape
    assert_mm_close(host(x.grad).reshape(M, K), O.matmul(gb, *ref, K, transposed=True), f"layer dX {mode}")
    # the base weight is frozen: no tensor of the packed operand takes part in autograd
    assert not any(t.requires_grad for t in (layer.qw.packed, layer.qw.scales, layer.qw.zeros))


def test_layer_fp16_and_trainable_bias():
    """fp16 activations and gradients take the fp16 path (fp16 weight operand) end to end,
    against the oracle's fp16 matmul; a bias that requires grad gets the row sum of dY."""
    N, K, M = 520, 1024, 130
    print("[case] layer fp16", flush=True)
    wb = synth.weight(713, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(wb, "bf16"), O.GROUPWISE, 64)
    qw = w4.quantize_pack(dev_weight(wb, "bf16"), "groupwise", 64)
    x16 = synth.activations_bf16(713, 1, M, K)  # draws; stored below as fp16
    xf = _bf16_to_f32(x16).astype(np.float16)
    gf = _bf16_to_f32(synth.activations_bf16(713, 2, M, N, tensor_id=synth.T_DY)).astype(np.float16)
    bias = torch.from_numpy(synth.bias_f32(713, 3, N)).to(DEV).requires_grad_(True)
    x = torch.from_numpy(xf).to(DEV).requires_grad_(True)
    y = w4.w4a16_linear(x, qw, bias)
    assert y.dtype == torch.float32
    xb = xf.view(np.uint16)
    assert_mm_close(host(y.detach()), O.matmul(xb, *ref, K, bias=host(bias.detach()), a_dtype="f16"),
                    "layer fp16 forward")
    y.backward(torch.from_numpy(gf.astype(np.float32)).to(DEV))
    assert x.grad.dtype == torch.float16
    assert_mm_close(host(x.grad.float()), O.matmul(gf.view(np.uint16), *ref, K, transposed=True, a_dtype="f16"),
                    "layer fp16 dX (fp16 stored)")
    want_db = gf.astype(np.float64).sum(0)
    np.testing.assert_allclose(host(bias.grad).astype(np.float64), want_db, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("M", [4, 640], ids=["gemv", "gemm"])
def test_layer_bf16_output(M):
    """out_dtype=bfloat16: forward output and bias in bf16, rounded once from the fp32 sum;
    bf16 gradients in, dX written in bf16 by the kernel; both against the oracle's float64
    products rounded to bf16, and bit-identical to rounding the fp32 layer's results."""
    N, K = 1024, 2048
    print(f"[case] layer bf16 output M={M}", flush=True)
    wb = synth.weight(714, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(wb, "bf16"), O.ROWWISE, None)
    qw = w4.quantize_pack(dev_weight(wb, "bf16"), "rowwise")
    b16 = O.bf16_rne_bits(synth.bias_f32(714, 1, N))
    bias = torch.from_numpy(b16.view(np.int16)).to(DEV).view(torch.bfloat16)
    xb = synth.activations_bf16(714, 2, M, K)
    gb = synth.activations_bf16(714, 3, M, N, tensor_id=synth.T_DY)
    x = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16).requires_grad_(True)
    layer = w4.W4A16Linear(qw, bias, out_dtype=torch.bfloat16)
    y = layer(x)
    assert y.dtype == torch.bfloat16 and layer.bias.dtype == torch.bfloat16
    b64 = O.bf16_bits_to_f64(b16)
    assert_rounded_close(host(y.detach().float()).astype(np.float64), O.matmul(xb, *ref, K, bias=b64), "bf16",
                         "layer bf16 forward")
    gy = torch.from_numpy(gb.view(np.int16)).to(DEV).view(torch.bfloat16)
    y.backward(gy)
    assert x.grad.dtype == torch.bfloat16
    assert_rounded_close(host(x.grad.float()).astype(np.float64), O.matmul(gb, *ref, K, transposed=True), "bf16",
                         "layer bf16 dX")
    # the same products through the fp32 layer, rounded afterwards: the same bits
    x32 = x.detach().clone().requires_grad_(True)
    y32 = w4.w4a16_linear(x32, qw, bias.float())
    y32.backward(gy.float())
    assert torch.equal(y.detach(), y32.detach().to(torch.bfloat16))
    assert torch.equal(x.grad, x32.grad)
