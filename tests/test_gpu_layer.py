"""GPU parity of the frozen int4 autograd layer: forward = W4A16 GEMM / GEMV, backward dX =
transposed GEMM on the same packed buffer, both against the oracle."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_mm_close, dev_weight, host

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
