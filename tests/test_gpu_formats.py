"""GPU parity of the format variants: integer zero points (AWQ style) and INT8-word packing."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_mm_close, assert_quant_equal, dev_bf16, dev_f32, dev_weight, host

pytestmark = pytest.mark.gpu

OMODE = {"global": O.GLOBAL, "rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}
MODES = [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 64), ("groupwise", 128),
         ("groupwise", 1024)]


def _special_weight(N, K, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, :] = 0.0                       # all-zero row
    w[1, : K // 2] = 0.75               # constant half row
    w[2, :] = np.abs(w[2, :]) + 0.1     # all positive: the zero point clamps at 0
    w[3, :] = -np.abs(w[3, :]) - 0.1    # all negative: the zero point clamps at 15
    w[4, 5] = 3.0                       # outliers
    w[5, 17] = -2.5
    w[6, ::7] = 0.0                     # exact zeros inside a normal row
    return w


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode,g", MODES, ids=[f"{m}{g or ''}" for m, g in MODES])
def test_int_zero_quantize_bit_exact(dtype, mode, g):
    print(f"[case] int-zero quantize dtype={dtype} mode={mode} g={g}", flush=True)
    N, K = 37, 4096
    w = synth.weight(730, 0, N, K, dtype) if dtype != "f32" else _special_weight(N, K, 730)
    w32 = O.to_f32(w, dtype)
    ref = O.quantize_pack(w32, OMODE[mode], g, int_zero=True)
    qw = w4.quantize_pack(dev_weight(w, dtype), mode, g, zero="int")
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"int zero {dtype} {mode}{g}")
    z = host(qw.zeros.float())
    assert np.all(z == np.round(z)) and z.min() >= 0 and z.max() <= 15


@pytest.mark.parametrize("M,tr", [(1, False), (4, False), (200, False), (200, True)])
@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 128)], ids=["rowwise", "g128"])
def test_int_zero_matmul(M, tr, mode, g):
    """Integer zero points need no matmul change: parity on the GEMV, GEMM and transposed paths."""
    N, K = 520, 2048
    print(f"[case] int-zero matmul M={M} t={tr} {mode}{g or ''}", flush=True)
    w = synth.weight(731, M, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g, int_zero=True)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g, zero="int")
    a = synth.activations_bf16(731, M, M, N if tr else K)
    bias = synth.bias_f32(731, M, K if tr else N)
    y = w4.mm(dev_bf16(a), qw, transposed=tr, bias=dev_f32(bias))
    assert_mm_close(host(y), O.matmul(a, *ref, K, tr, bias=bias), f"int zero M={M} t={tr} {mode}{g}")


def test_int_zero_fused_qkv():
    K = 1024
    sizes = (256, 128, 128)
    ws = [synth.weight(732, i, n, K, "bf16", tensor_id=synth.T_Q + i) for i, n in enumerate(sizes)]
    fused = w4.quantize_fused([dev_weight(w, "bf16") for w in ws], "groupwise", 128, zero="int")
    refs = [O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, 128, int_zero=True) for w in ws]
    assert_quant_equal(fused, *O.fuse_rows(refs), what="fused int zero")


def test_int8_word_view_and_wrap():
    """INT8 packing: the packed weight viewed as bytes equals the oracle's two-codes-per-byte
    packing, and a weight wrapped from such bytes (uploaded from the oracle) multiplies to
    the oracle's product."""
    N, K, M = 136, 1024, 3
    w = synth.weight(733, 0, N, K, "f16")
    w32 = O.to_f32(w, "f16")
    q, s, z = O.quantize(w32, O.GROUPWISE, 64)
    qw = w4.quantize_pack(dev_weight(w, "f16"), "groupwise", 64)
    np.testing.assert_array_equal(host(qw.packed_bytes()), O.pack_bytes(q))
    u8 = torch.from_numpy(O.pack_bytes(q)).to(DEV)
    wrapped = w4.QuantizedWeight.from_bytes(u8, torch.from_numpy(s).to(DEV), torch.from_numpy(z).to(DEV),
                                            "groupwise", 64)
    x = synth.activations_bf16(733, 0, M, K)
    assert_mm_close(host(w4.mm(dev_bf16(x), wrapped)), O.matmul(x, O.pack(q), s, z, K), "int8-wrapped weight")


def _acts_f16(cfg, idx, M, L):
    """Synthetic activations as fp16 bits (the bf16 draw, rounded to fp16)."""
    a = O.bf16_bits_to_f64(synth.activations_bf16(cfg, idx, M, L))
    return a.astype(np.float16).view(np.uint16)


def _dev_f16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.float16)


@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 64), ("groupwise", 16)],
                         ids=["rowwise", "g64", "g16"])
def test_dequantize_f16_bit_exact(mode, g):
    N, K = 300, 2048
    w = synth.weight(734, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    got = w4.dequantize(qw, torch.float16).view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, O.dequantize_f16_bits(*ref, K))


F16_CASES = [(1, False), (2, False), (3, False), (4, False), (37, False), (300, False), (128, True), (300, True)]


@pytest.mark.parametrize("M,tr", F16_CASES, ids=[f"{m}{'t' if t else ''}" for m, t in F16_CASES])
@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 64), ("groupwise", 16)],
                         ids=["rowwise", "g64", "g16"])
def test_f16_activations(M, tr, mode, g):
    """fp16 activations times the fp16 weight operand, fp32 accumulation, on every path."""
    N, K = 264, 2048
    print(f"[case] f16 activations M={M} t={tr} {mode}{g or ''}", flush=True)
    w = synth.weight(735, M, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    a = _acts_f16(735, M, M, N if tr else K)
    bias = synth.bias_f32(735, M, K if tr else N)
    y = w4.mm(_dev_f16(a), qw, transposed=tr, bias=dev_f32(bias))
    assert_mm_close(host(y), O.matmul(a, *ref, K, tr, bias=bias, a_dtype="f16"), f"f16 M={M} t={tr} {mode}{g}")


def test_f16_activations_split_k_and_bf16_out():
    """fp16 activations on a split-K GEMM, written as bf16 through the epilogue."""
    M, N, K = 128, 2048, 8192
    w = synth.weight(736, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, 128)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), "groupwise", 128)
    assert "splitk" in w4.kernel_for(M, N, K, "groupwise", 128)
    a = _acts_f16(736, 0, M, K)
    y = w4.mm(_dev_f16(a), qw)
    ref64 = O.matmul(a, *ref, K, a_dtype="f16")
    assert_mm_close(host(y), ref64, "f16 split-K")
    yb = w4.mm(_dev_f16(a), qw, out_dtype=torch.bfloat16)
    assert torch.equal(yb, y.to(torch.bfloat16))


def test_serialized_weight_round_trip(tmp_path):
    """A weight quantized on the GPU, saved and loaded back, multiplies bit-identically."""
    N, K, M = 520, 2048, 300
    w = synth.weight(737, 0, N, K, "bf16")
    qw = w4.quantize_pack(dev_weight(w, "bf16"), "groupwise", 128, zero="int")
    path = str(tmp_path / "w.w4")
    w4.save(qw, path)
    back = w4.load(path, device=DEV)
    assert back.zero == "int" and (back.N, back.K, back.group) == (N, K, 128)
    x = dev_bf16(synth.activations_bf16(737, 0, M, K))
    assert torch.equal(w4.mm(x, back), w4.mm(x, qw))
    ref = O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, 128, int_zero=True)
    assert_quant_equal(back, *ref, what="loaded weight")
