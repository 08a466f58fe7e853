"""GPU parity of quantize-and-pack and dequantize: bit-exact with the oracle."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_quant_equal, dev_weight, host, host_bits16

pytestmark = pytest.mark.gpu

MODES = [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 32), ("groupwise", 64),
         ("groupwise", 128), ("groupwise", 256), ("groupwise", 512), ("groupwise", 1024), ("groupwise", 4096)]
OMODE = {"global": O.GLOBAL, "rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}


def _special_weight(N, K, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, :] = 0.0                       # all-zero row
    w[1, : K // 2] = 0.75               # constant half row
    w[2, :] = np.abs(w[2, :]) + 0.1     # all positive
    w[3, :] = -np.abs(w[3, :]) - 0.1    # all negative
    w[4, 5] = 3.0                       # outliers
    w[5, 17] = -2.5
    w[6, :] += 100.0                    # narrow range far from 0: zero points near -1e4
    return w


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode,g", MODES, ids=[f"{m}{g or ''}" for m, g in MODES])
def test_quantize_bit_exact_small(dtype, mode, g):
    print(f"[case] quantize small dtype={dtype} mode={mode} g={g}", flush=True)
    N, K = 37, 4096          # ragged N, several groups per row for every g
    w = _special_weight(N, K, 10)
    if dtype == "f16":
        w = w.astype(np.float16)
    elif dtype == "bf16":
        w = synth.f32_to_bf16_bits(w)
    w32 = O.to_f32(w, dtype)
    ref = O.quantize_pack(w32, OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, dtype), mode, g)
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"{dtype} {mode} {g}")


@pytest.mark.parametrize("N,K,mode,g", [(1, 8, "rowwise", None), (3, 24, "rowwise", None), (5, 1376, "rowwise", None),
                                        (2, 11008, "rowwise", None), (4, 16384, "rowwise", None),
                                        (7, 48, "groupwise", 16), (1, 4096, "groupwise", 4096),
                                        (9, 2056, "global", None)])
def test_quantize_odd_shapes(N, K, mode, g):
    print(f"[case] quantize odd N={N} K={K} mode={mode} g={g}", flush=True)
    w = synth.weight(500, N * 7 + K, N, K, "f16")
    w32 = O.to_f32(w, "f16")
    ref = O.quantize_pack(w32, OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "f16"), mode, g)
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"N={N} K={K} {mode} {g}")


@pytest.mark.parametrize("mode,g", [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 32),
                                    ("groupwise", 64), ("groupwise", 128), ("groupwise", 256), ("groupwise", 512),
                                    ("groupwise", 1024), ("groupwise", 2048)])
def test_quantize_full_size(mode, g, full_quant_weight):
    """fp16 W [128256][2048] with 0.1% outliers: the whole packed tensor and every scale and
    zero, bit-exact with the oracle on the full tensor."""
    print(f"[case] quantize full 128256x2048 mode={mode} g={g}", flush=True)
    w32, wd = full_quant_weight
    qw = w4.quantize_pack(wd, mode, g)
    torch.cuda.synchronize()
    ref = O.quantize_pack(w32, OMODE[mode], g)
    assert_quant_equal(qw, *ref, what=f"full {mode} {g}")


@pytest.fixture(scope="module")
def full_quant_weight():
    N, K = 128256, 2048
    w = synth.weight_with_outliers(5, 0, N, K)
    wd = dev_weight(w, "f16")
    yield O.to_f32(w, "f16"), wd
    del wd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode,g", [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 128),
                                    ("groupwise", 2048)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_bit_exact(mode, g, out):
    print(f"[case] dequantize mode={mode} g={g} out={out}", flush=True)
    N, K = 33, 2048
    w = _special_weight(N, K, 11)
    p, s, z = O.quantize_pack(w, OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "f32"), mode, g)
    if out == "bf16":
        d = w4.dequantize(qw, torch.bfloat16)
        np.testing.assert_array_equal(host_bits16(d), O.dequantize_bf16_bits(p, s, z, K))
    else:
        d = w4.dequantize(qw, torch.float32)
        np.testing.assert_array_equal(host(d).view(np.uint32), O.dequantize_f32(p, s, z, K).view(np.uint32))


def test_dequantize_tiny_zero_order():
    """Zeros so small that q - z is inexact in fp32: the export keeps subtract-then-multiply."""
    N, K = 4, 64
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    p = O.pack(q)
    s = np.array([[0.0276336669921875], [0.0026454925537109375], [0.04571533203125], [0.5]], dtype=np.float16)
    z = np.array([[0.00046753883361816406], [-0.0003650188446044922], [0.0003650188446044922], [3.0]],
                 dtype=np.float16)
    qw = w4.QuantizedWeight(packed=torch.from_numpy(p).to(DEV), scales=torch.from_numpy(s).to(DEV),
                            zeros=torch.from_numpy(z).to(DEV), N=N, K=K, mode=1, group=0)
    d = w4.dequantize(qw, torch.float32)
    np.testing.assert_array_equal(host(d).view(np.uint32), O.dequantize_f32(p, s, z, K).view(np.uint32))


def test_quantize_into_row_slices_matches_separate():
    """Fused-QKV construction: quantizing Q, K, V into one operand equals the oracle's row concatenation."""
    K = 1024
    parts = [synth.weight(6, i, n, K, "bf16", tensor_id=synth.T_Q + i) for i, n in enumerate((256, 128, 128))]
    for mode, g in [("rowwise", None), ("groupwise", 64)]:
        ref = O.fuse_rows([O.quantize_pack(O.to_f32(p, "bf16"), OMODE[mode], g) for p in parts])
        qw = w4.quantize_fused([dev_weight(p, "bf16") for p in parts], mode, g)
        torch.cuda.synchronize()
        assert_quant_equal(qw, *ref, what=f"fused {mode}")
    with pytest.raises(ValueError):
        w4.quantize_fused([dev_weight(p, "bf16") for p in parts], "global", None)


def _tie_weight(N, K, g, dtype, seed):
    """Groups whose every interior value lands exactly on a rounding tie: with
    c = m 2^e (m odd, few significant bits, so every value below is exact in the dtype),
    the group holds lo = -u c and hi = (15 - u) c, so s = c and z = u exactly, and the other
    values are (k + 1/2 - u) c (u an integer: w / s + z = k + 1/2) or (k - u + 1/2) c with
    u = v + 1/2 (z fractional, w / s an integer, w / s + z = k + 1/2 again)."""
    r = np.random.default_rng(seed)
    mmax = 7 if dtype == "bf16" else 63
    w = np.empty((N, K), dtype=np.float32)
    for n in range(N):
        for g0 in range(0, K, g):
            c = float(r.choice(np.arange(3, mmax + 1, 2))) * 2.0 ** int(r.integers(-12, -5))
            if r.integers(2):
                u = float(r.integers(0, 8))                 # integer zero
                vals = (np.arange(14) + 0.5 - u) * c
            else:
                u = float(r.integers(0, 7)) + 0.5           # fractional zero
                vals = (np.arange(14) - u + 0.5) * c
            grp = np.resize(vals, g)
            grp[:2] = (-u * c, (15.0 - u) * c)
            w[n, g0:g0 + g] = r.permutation(grp)
    return w


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode,g,zero", [("groupwise", 16, "fp16"), ("groupwise", 128, "fp16"),
                                         ("rowwise", None, "fp16"), ("groupwise", 32, "int"),
                                         ("rowwise", None, "int")])
def test_quantize_exact_ties(dtype, mode, g, zero):
    """Every code decided by a tie (w / s + z exactly k + 1/2, or w / s exactly k + 1/2 for
    integer zeros): the kernel must take the correctly rounded, half-to-even decision."""
    print(f"[case] quantize ties dtype={dtype} mode={mode} g={g} zero={zero}", flush=True)
    N, K = 24, 2048
    w = _tie_weight(N, K, g or K, dtype, 31)
    if dtype == "f16":
        w = w.astype(np.float16)
    elif dtype == "bf16":
        w = synth.f32_to_bf16_bits(w)
    w32 = O.to_f32(w, dtype)
    ref = O.quantize_pack(w32, OMODE[mode], g, int_zero=zero == "int")
    # the construction does produce ties in the oracle's own arithmetic
    q, s16, z16 = O.quantize(w32, OMODE[mode], g, int_zero=zero == "int")
    s_f = np.repeat(s16.astype(np.float32), g or K, axis=1)
    z_f = np.repeat(z16.astype(np.float32), g or K, axis=1)
    t = w32 / s_f if zero == "int" else w32 / s_f + z_f
    assert np.mean(t - np.floor(t) == 0.5) > 0.4
    qw = w4.quantize_pack(dev_weight(w, dtype), mode, g, zero=zero)
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"ties {dtype} {mode} {g} {zero}")


@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 16), ("groupwise", 128), ("global", None)])
def test_quantize_zero_overflow(mode, g):
    """fp32 groups whose fp16 zero point would overflow (range below 15 |min| / 65504, e.g.
    [1.0, 1.0001]) are quantized as constant groups (s = 1, z = fp16(0 - min)), bit-exact
    with the oracle, and dequantize to finite values."""
    print(f"[case] quantize zero overflow mode={mode} g={g}", flush=True)
    N, K = 12, 1024
    r = np.random.default_rng(77)
    w = (np.float32(1.0) + np.float32(1e-4) * r.random((N, K), dtype=np.float32)).astype(np.float32)
    w[:, 0], w[:, 1] = 1.0, 1.0001
    w[3, :] = np.float32(-1000.0) - np.float32(0.01) * r.random(K, dtype=np.float32)
    w[5, :] = (r.standard_normal(K) * 0.02).astype(np.float32)   # an ordinary row among them
    ref = O.quantize_pack(w, OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "f32"), mode, g)
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"zero overflow {mode} {g}")
    d = host(w4.dequantize(qw, torch.float32))
    assert np.all(np.isfinite(d))
    np.testing.assert_array_equal(d.view(np.uint32), O.dequantize_f32(*ref, K).view(np.uint32))
