"""Pins of the oracle's packing and dequantization (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from exact import bf16_from_fraction_bits, frac, round_fmt


def test_pack_layout_hand_words():
    # code k = 8c + j sits at bits 4j of word c: 0..7 -> 0x76543210, 8..15 -> 0xFEDCBA98
    q = np.arange(16, dtype=np.uint8).reshape(1, 16)
    p = O.pack(q)
    assert p.view(np.uint32)[0].tolist() == [0x76543210, 0xFEDCBA98]
    # byte view: two codes per byte, low nibble first (the INT8-word layout)
    assert p.view(np.uint8)[0].tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]


def test_pack_unpack_bijection():
    r = np.random.default_rng(7)
    q = r.integers(0, 16, size=(13, 256), dtype=np.uint8)
    assert np.array_equal(O.unpack(O.pack(q)), q)
    words = r.integers(-2**31, 2**31, size=(5, 40), dtype=np.int64).astype(np.int32)
    assert np.array_equal(O.pack(O.unpack(words)), words)


def _exact_deq_bits(q, s16, z16):
    """bf16_rne(fp32(fp32(q - z) * s)) with exact rationals and the independent rounding."""
    d = round_fmt(Fraction(q) - frac(z16), "f32")
    p = round_fmt(d * frac(s16), "f32")
    b = round_fmt(p, "bf16")
    return bf16_from_fraction_bits(b)


def _meta_samples():
    r = np.random.default_rng(11)
    s = list(r.uniform(1e-4, 0.05, 20)) + [6.1e-8, 1e-6, 0.5, 1.0, 3.0, 1000.0]
    z = list(r.uniform(0.0, 15.0, 20)) + [0.0, -3.25, 15.0, 40.0, 1e-3, 7.4990234375]
    # zeros so small that q - z is not exact in fp32 (pins the order of the two fp32 ops)
    s += [0.0276336669921875, 0.0026454925537109375, 0.04571533203125]
    z += [0.00046753883361816406, -0.0003650188446044922, 0.0003650188446044922]
    return [(np.float16(a), np.float16(b)) for a, b in zip(s, z)]


@pytest.mark.parametrize("s16,z16", _meta_samples())
def test_dequant_all_codes_exact(s16, z16):
    q = np.arange(16, dtype=np.uint8).reshape(2, 8)
    packed = O.pack(q)
    scales = np.array([[s16]], dtype=np.float16)
    zeros = np.array([[z16]], dtype=np.float16)
    bits = O.dequantize_bf16_bits(packed, scales, zeros, 8).reshape(-1)
    f32 = O.dequantize_f32(packed, scales, zeros, 8).reshape(-1)
    for c in range(16):
        assert int(bits[c]) == _exact_deq_bits(c, s16, z16), (c, s16, z16)
        d = round_fmt(Fraction(c) - frac(z16), "f32")
        assert Fraction(float(f32[c])) == round_fmt(d * frac(s16), "f32"), (c, s16, z16)
    # the fp16 operand: the same fp32 value rounded once more, to fp16
    b16 = O.dequantize_f16_bits(packed, scales, zeros, 8).reshape(-1)
    for c in range(16):
        d = round_fmt(Fraction(c) - frac(z16), "f32")
        want = round_fmt(round_fmt(d * frac(s16), "f32"), "f16")
        got = O.f16_bits_to_f64(np.array([b16[c]]))[0]
        assert (Fraction(got) if np.isfinite(got) else got) == want, (c, s16, z16)


def test_bf16_rounding_ties_and_specials():
    # a value exactly halfway between two bf16 values rounds to the even significand
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.40e38, 0.0, -0.0,
                     1e-40], dtype=np.float32)
    got = O.bf16_rne_bits(vals)
    exp = [bf16_from_fraction_bits(round_fmt(frac(v), "bf16")) for v in vals]
    assert got.tolist() == exp[:5] + [0x8000] + exp[6:]


def test_meta_expansion_per_mode():
    # one-hot codes pin which scale/zero each element uses, for every mode
    N, K = 4, 64
    q = np.zeros((N, K), dtype=np.uint8)
    packed = O.pack(q + 1)
    for mode, g in [(O.GLOBAL, None), (O.ROWWISE, None), (O.GROUPWISE, 16)]:
        shp = O.meta_shape(N, K, mode, g)
        s = (np.arange(np.prod(shp)).reshape(shp) + 1).astype(np.float16)
        z = np.zeros(shp, dtype=np.float16)
        deq = O.dequantize_f32(packed, s, z, K)   # (1 - 0) * s = s
        for n in range(N):
            for k in range(K):
                if mode == O.GLOBAL:
                    want = 1.0
                elif mode == O.ROWWISE:
                    want = n + 1.0
                else:
                    want = n * (K // 16) + k // 16 + 1.0
                assert deq[n, k] == want


def test_pack_bytes_golden_and_word_view():
    """INT8 packing: two codes per byte, low nibble first (written out by hand), and the
    int32 words of the INT32 packing viewed as little-endian bytes are the same bytes."""
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 0, 0, 15, 9, 10, 11, 12]], dtype=np.uint8)
    want = np.array([[0x21, 0x43, 0x65, 0x87, 0x0F, 0xF0, 0xA9, 0xCB]], dtype=np.uint8)
    np.testing.assert_array_equal(O.pack_bytes(q), want)
    r = np.random.default_rng(5).integers(0, 16, size=(7, 64), dtype=np.uint8)
    np.testing.assert_array_equal(O.pack(r).view(np.uint8).reshape(7, 32), O.pack_bytes(r))
