"""Pins of the oracle's matmul (CPU only): exact brute force, one-hot layout pins,
closed forms, linearity, bias and the fused-QKV identities."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth


def _case(N, K, mode, g, seed, M=3, dtype="f32"):
    w = synth.weight(200 + seed, 0, N, K, dtype)
    w32 = O.to_f32(w, dtype)
    packed, s, z = O.quantize_pack(w32, mode, g)
    return packed, s, z


def _exact_product(a_bits, wbits, transposed, bias):
    a = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(a_bits)]
    w = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(wbits)]
    N, K = len(w), len(w[0])
    M = len(a)
    if transposed:
        out = [[sum(a[m][n] * w[n][k] for n in range(N)) for k in range(K)] for m in range(M)]
    else:
        out = [[sum(a[m][k] * w[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    if bias is not None:
        out = [[v + Fraction(float(bias[j])) for j, v in enumerate(row)] for row in out]
    return np.array([[float(v) for v in row] for row in out])


@pytest.mark.parametrize("transposed", [False, True])
@pytest.mark.parametrize("mode,g", [(O.GLOBAL, None), (O.ROWWISE, None), (O.GROUPWISE, 16)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_bruteforce_tiny(transposed, mode, g, with_bias):
    N, K, M = 8, 32, 3
    packed, s, z = _case(N, K, mode, g, 1)
    a = synth.activations_bf16(201, 0, M, N if transposed else K)
    bias = synth.bias_f32(201, 1, K if transposed else N) if with_bias else None
    y = O.matmul(a, packed, s, z, K, transposed, bias)
    wbits = O.dequantize_bf16_bits(packed, s, z, K)
    ye = _exact_product(a, wbits, transposed, bias)
    assert np.allclose(y, ye, rtol=1e-13, atol=1e-13)


def _f16_bits_fraction(b: int) -> Fraction:
    """Exact value of an fp16 bit pattern, decoded from the format's fields (1 sign bit,
    5 exponent bits with bias 15, 10 fraction bits; exponent 0 is subnormal)."""
    sign = -1 if b >> 15 else 1
    e, f = (b >> 10) & 31, b & 1023
    assert e != 31, "finite values only"
    if e == 0:
        return sign * Fraction(f, 1024) * Fraction(1, 2**14)
    return sign * (1 + Fraction(f, 1024)) * Fraction(2) ** (e - 15)


@pytest.mark.parametrize("transposed", [False, True])
@pytest.mark.parametrize("mode,g", [(O.ROWWISE, None), (O.GROUPWISE, 16)])
def test_bruteforce_tiny_f16(transposed, mode, g):
    """fp16 activations: every product of the fp16 operand fp16_rne(fp32(q - z) * s) with
    hand-decoded fp16 activations, summed exactly, against matmul(a_dtype="f16")."""
    from exact import round_fmt
    N, K, M = 8, 32, 3
    packed, s, z = _case(N, K, mode, g, 7)
    q = O.unpack(packed)
    gs = K if mode == O.ROWWISE else g
    wq = [[round_fmt(round_fmt(round_fmt(Fraction(int(q[n, k])) - Fraction(float(z[n, k // gs])), "f32")
                               * Fraction(float(s[n, k // gs])), "f32"), "f16") for k in range(K)]
          for n in range(N)]
    L = N if transposed else K
    a = (np.random.default_rng(8).standard_normal((M, L)) * 2).astype(np.float16).view(np.uint16)
    a[0, 0] = 0x0001  # the smallest fp16 subnormal
    a[1, 1] = 0x8400  # -2^-14, the smallest normal, negative
    af = [[_f16_bits_fraction(int(v)) for v in row] for row in a]
    if transposed:
        ye = [[sum(af[m][n] * wq[n][k] for n in range(N)) for k in range(K)] for m in range(M)]
    else:
        ye = [[sum(af[m][k] * wq[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    y = O.matmul(a, packed, s, z, K, transposed, a_dtype="f16")
    assert np.allclose(y, np.array([[float(v) for v in row] for row in ye]), rtol=1e-13, atol=1e-13)


def _bf16_onehot(M, L, idx):
    x = np.zeros((M, L), dtype=np.uint16)
    x[0, idx] = 0x3F80  # 1.0
    return x


@pytest.mark.parametrize("mode,g", [(O.ROWWISE, None), (O.GROUPWISE, 32)])
def test_onehot_layout(mode, g):
    N, K = 24, 96
    packed, s, z = _case(N, K, mode, g, 2)
    wd = O.bf16_bits_to_f64(O.dequantize_bf16_bits(packed, s, z, K))
    for k in (0, 7, 8, 31, 32, 95):
        y = O.matmul(_bf16_onehot(2, K, k), packed, s, z, K, False)
        assert np.array_equal(y[0], wd[:, k]) and np.all(y[1] == 0)
    for n in (0, 1, 23):
        y = O.matmul(_bf16_onehot(2, N, n), packed, s, z, K, True)
        assert np.array_equal(y[0], wd[n, :]) and np.all(y[1] == 0)


def test_constant_codes_closed_form():
    # every code equal to c: Y[m, n] = sum over groups of bf16((c - z) s) * (sum of X over the group)
    N, K, g, c = 5, 64, 16, 9
    q = np.full((N, K), c, dtype=np.uint8)
    packed = O.pack(q)
    r = np.random.default_rng(3)
    s = r.uniform(0.001, 0.02, (N, K // g)).astype(np.float16)
    z = r.uniform(0, 15, (N, K // g)).astype(np.float16)
    x = synth.activations_bf16(203, 0, 2, K)
    y = O.matmul(x, packed, s, z, K, False)
    x64 = O.bf16_bits_to_f64(x)
    for n in range(N):
        for m in range(2):
            want = 0.0
            for gi in range(K // g):
                val = (np.float32(c) - np.float32(z[n, gi])) * np.float32(s[n, gi])
                val = O.bf16_bits_to_f64(O.bf16_rne_bits(np.array([val], dtype=np.float32)))[0]
                want += val * x64[m, gi * g:(gi + 1) * g].sum()
            assert abs(y[m, n] - want) <= 1e-12 * max(1.0, abs(want))


def test_linearity_and_bias():
    N, K = 16, 64
    packed, s, z = _case(N, K, O.GROUPWISE, 16, 4)
    r = np.random.default_rng(5)
    # small integers are exact in bf16 and so are their sums
    x1 = r.integers(-8, 8, (3, K)).astype(np.float32)
    x2 = r.integers(-8, 8, (3, K)).astype(np.float32)
    b = synth.f32_to_bf16_bits
    y1 = O.matmul(b(x1), packed, s, z, K)
    y2 = O.matmul(b(x2), packed, s, z, K)
    y12 = O.matmul(b(x1 + x2), packed, s, z, K)
    assert np.allclose(y12, y1 + y2, rtol=1e-14, atol=1e-14)
    bias = synth.bias_f32(204, 0, N)
    yb = O.matmul(b(x1), packed, s, z, K, bias=bias)
    assert np.array_equal(yb - y1, np.broadcast_to(bias.astype(np.float64), yb.shape))


@pytest.mark.parametrize("mode,g", [(O.ROWWISE, None), (O.GROUPWISE, 64)])
def test_fused_qkv_identities(mode, g):
    K = 128
    parts = []
    for i, n in enumerate((32, 16, 16)):
        w = synth.weight(205, i, n, K, "bf16", tensor_id=synth.T_Q + i)
        parts.append(O.quantize_pack(O.to_f32(w, "bf16"), mode, g))
    fused = O.fuse_rows(parts)
    x = synth.activations_bf16(205, 9, 3, K)
    y_f = O.matmul(x, *fused, K)
    y_s = np.concatenate([O.matmul(x, *p, K) for p in parts], axis=1)
    assert np.array_equal(y_f, y_s)
    dy = synth.activations_bf16(205, 10, 3, 64)
    dx_f = O.matmul(dy, *fused, K, transposed=True)
    offs = [0, 32, 48, 64]
    dx_s = sum(O.matmul(dy[:, offs[i]:offs[i + 1]].copy(), *parts[i], K, transposed=True) for i in range(3))
    assert np.allclose(dx_f, dx_s, rtol=1e-12, atol=1e-12)


def test_fuse_rejects_global():
    K = 64
    parts = [O.quantize_pack(synth.weight(206, i, 8, K, "f32"), O.GLOBAL) for i in range(3)]
    with pytest.raises(ValueError):
        O.fuse_rows(parts)


def test_round_output_pins():
    """Output rounding of the epilogue: values whose bf16 / fp16 roundings follow from the
    formats' definitions (8 and 11 significant bits, ties to even)."""
    y = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-8 + 2.0**-20, -3.0 - 2.0**-7,
                  65504.0, 1e-3])
    # bf16: 1 + 2^-8 is the tie between 1 and 1 + 2^-7 -> even (1); 1 + 3*2^-8 ties -> 1 + 2^-6;
    # just above the tie rounds up; -3 - 2^-7 ties between -3 and -3 - 2^-6 -> even (-3)
    want_bf16 = [1.0, 1.0, 1.0 + 2.0**-6, 1.0 + 2.0**-7, -3.0, 65536.0, None]
    got = O.round_output(y, "bf16")
    for g, w in zip(got, want_bf16):
        if w is not None:
            assert g == w
    # 1e-3 in bf16: the nearest 8-bit significand times 2^-10 (1e-3 = 1.024 * 2^-10)
    assert got[-1] == round(1.024 * 128) / 128 * 2.0**-10
    # fp16 keeps 1 + 2^-8 (11 significant bits) and tops out at 65504
    got16 = O.round_output(y, "f16")
    assert got16[1] == 1.0 + 2.0**-8 and got16[5] == 65504.0
    assert got16[3] == 1.0 + 2.0**-8  # 2^-20 is below half an fp16 ulp at 1
    np.testing.assert_array_equal(O.round_output(y, "f32"), y.astype(np.float32).astype(np.float64))
