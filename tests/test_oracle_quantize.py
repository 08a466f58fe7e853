"""Pins of the oracle's quantizer (CPU only).

The oracle is checked against things other than itself:
* a hand-derived golden group (tests/golden/quant_row.txt);
* an exact-rational brute force of every rounding step (tests/exact.py) on
  tiny matrices, for every mode and several group sizes;
* invariants that any correct min-max asymmetric quantizer satisfies.
"""

import os

import numpy as np
import pytest

import oracle as O
import synth
from exact import frac, rint_clamp_0_15, round_fmt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("mode,g", [(O.GROUPWISE, 16), (O.ROWWISE, None)])
def test_golden_row(dtype, mode, g):
    gd = _read_golden("quant_row.txt")
    w = np.array([float(v) for v in gd["w"]], dtype=np.float32).reshape(1, 16)
    if dtype == "f16":
        w = w.astype(np.float16)
    w32 = O.to_f32(w, dtype)
    packed, s, z = O.quantize_pack(w32, mode, g)
    assert int(s.view(np.uint16)[0, 0]) == int(gd["scale_bits"][0], 16)
    assert int(z.view(np.uint16)[0, 0]) == int(gd["zero_bits"][0], 16)
    q = O.unpack(packed)
    assert q[0].tolist() == [int(v) for v in gd["q"]]
    words = [int(v, 16) for v in gd["words_hex"]]
    assert packed.view(np.uint32)[0].tolist() == words
    deq = O.dequantize_f32(packed, s, z, 16)
    assert deq[0].tolist() == [float(v) for v in gd["deq"]]
    bits = O.dequantize_bf16_bits(packed, s, z, 16)
    assert np.array_equal(O.bf16_bits_to_f64(bits), deq.astype(np.float64))


def _brute_quantize(w32, mode, g):
    """Every step in exact rationals, rounded with the independent IEEE rounding of tests/exact.py."""
    N, K = w32.shape
    if mode == O.GLOBAL:
        groups = [[(n, k) for n in range(N) for k in range(K)]]
    elif mode == O.ROWWISE:
        groups = [[(n, k) for k in range(K)] for n in range(N)]
    else:
        groups = [[(n, k) for k in range(c * g, (c + 1) * g)] for n in range(N) for c in range(K // g)]
    q = np.zeros((N, K), dtype=np.uint8)
    ss, zz = [], []
    for grp in groups:
        vals = [frac(w32[n, k]) for n, k in grp]
        lo, hi = min(vals), max(vals)
        d = round_fmt(hi - lo, "f32")
        s32 = round_fmt(d / 15, "f32")
        s16 = round_fmt(s32, "f16")
        if s16 == 0 or isinstance(s16, float):
            s16 = 1
        z32 = round_fmt((0 - lo) / s16, "f32")
        z16 = round_fmt(z32, "f16")
        if isinstance(z16, float):  # an fp16 zero beyond 65504: the group is treated as constant
            s16 = 1
            z16 = round_fmt(round_fmt(0 - lo, "f32"), "f16")
        assert not isinstance(z16, float), "test data must keep |min| <= 65504"
        for (n, k), v in zip(grp, vals):
            a = round_fmt(v / s16, "f32")
            t = round_fmt(a + z16, "f32")
            q[n, k] = rint_clamp_0_15(t)
        ss.append(float(s16))
        zz.append(float(z16))
    shp = O.meta_shape(N, K, mode, g)
    return q, np.array(ss).reshape(shp), np.array(zz).reshape(shp)


def _tiny_inputs():
    r = np.random.default_rng(1234)
    cases = []
    cases.append(("normal", r.standard_normal((3, 64)).astype(np.float32) * np.float32(0.02)))
    cases.append(("positive", np.abs(r.standard_normal((2, 64))).astype(np.float32) + np.float32(0.5)))
    cases.append(("negative", -np.abs(r.standard_normal((2, 32))).astype(np.float32) - np.float32(0.25)))
    w = r.standard_normal((2, 64)).astype(np.float32)
    w[0, :16] = 0.0          # an all-zero group
    w[1, 16:32] = 0.3        # a constant group
    w[1, 40] = 7.0           # an outlier
    cases.append(("special", w))
    cases.append(("fp16grid", r.standard_normal((2, 64)).astype(np.float16).astype(np.float32)))
    cases.append(("wide", (r.standard_normal((2, 32)) * 300).astype(np.float32)))
    # groups whose range is tiny next to their offset: the fp16 zero -min/s would overflow
    n = np.float32(1.0) + np.float32(1e-4) * r.random((2, 32), dtype=np.float32)
    n[1, :16] = np.float32(-1000.0) - np.float32(0.01) * r.random(16, dtype=np.float32)
    cases.append(("narrow", n))
    return cases


@pytest.mark.parametrize("name,w", _tiny_inputs(), ids=[c[0] for c in _tiny_inputs()])
def test_bruteforce_all_modes(name, w):
    K = w.shape[1]
    configs = [(O.GLOBAL, None), (O.ROWWISE, None), (O.GROUPWISE, 16), (O.GROUPWISE, 32), (O.GROUPWISE, K)]
    for mode, g in configs:
        q, s, z = O.quantize(w, mode, g)
        qb, sb, zb = _brute_quantize(w, mode, g)
        assert np.array_equal(s.astype(np.float64), sb), (name, mode, g)
        assert np.array_equal(z.astype(np.float64), zb), (name, mode, g)
        assert np.array_equal(q, qb), (name, mode, g)


def _expand(meta, N, K):
    rows, groups = meta.shape
    m = meta.astype(np.float64)
    if rows == 1 and groups == 1:
        return np.full((N, K), m[0, 0])
    return np.repeat(m, K // groups, axis=1)


@pytest.mark.parametrize("mode,g", [(O.GLOBAL, None), (O.ROWWISE, None), (O.GROUPWISE, 16),
                                    (O.GROUPWISE, 64), (O.GROUPWISE, 128), (O.GROUPWISE, 1024)])
def test_invariants(mode, g):
    N, K = 64, 1024
    w = synth.weight(99, 0, N, K, "f32")
    packed, s, z = O.quantize_pack(w, mode, g)
    q = O.unpack(packed)
    assert q.min() >= 0 and q.max() <= 15
    deq = O.dequantize_f32(packed, s, z, K).astype(np.float64)
    S = _expand(s, N, K)
    # |deq - w| <= s/2, up to the fp16 rounding of scale and zero (relative 2^-11 each)
    err = np.abs(deq - w.astype(np.float64))
    assert np.all(err <= S * (0.5 + 16 * 2.0 ** -10) + 1e-12)
    # the group minimum codes to 0 and the maximum to 15
    gsize = N * K if mode == O.GLOBAL else (K if mode == O.ROWWISE else g)
    qg = q.reshape(-1, gsize)
    wg = w.reshape(-1, gsize)
    rows = np.arange(qg.shape[0])
    assert np.all(qg[rows, wg.argmin(axis=1)] == 0)
    assert np.all(qg[rows, wg.argmax(axis=1)] == 15)


def test_rowwise_equals_groupwise_k():
    w = synth.weight(99, 1, 16, 512, "f16")
    w32 = O.to_f32(w, "f16")
    a = O.quantize_pack(w32, O.ROWWISE)
    b = O.quantize_pack(w32, O.GROUPWISE, 512)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_constant_and_zero_groups():
    w = np.zeros((2, 32), dtype=np.float32)
    w[1, :16] = 0.75
    w[1, 16:] = -2.5
    packed, s, z = O.quantize_pack(w, O.GROUPWISE, 16)
    assert np.all(s.astype(np.float32) == 1.0)
    assert z.view(np.uint16)[0, 0] == 0x0000          # +0, not -0
    deq = O.dequantize_f32(packed, s, z, 32)
    assert np.array_equal(deq, w)


def test_bf16_input_is_exact():
    b = synth.weight(99, 2, 8, 64, "bf16")
    w32 = O.to_f32(b, "bf16")
    assert np.array_equal(synth.f32_to_bf16_bits(w32), b)


def _brute_quantize_int_zero(w32, mode, g):
    """Exact-rational brute force of the integer-zero (AWQ order) quantizer."""
    from exact import rint_half_even
    N, K = w32.shape
    if mode == O.GLOBAL:
        groups = [[(n, k) for n in range(N) for k in range(K)]]
    elif mode == O.ROWWISE:
        groups = [[(n, k) for k in range(K)] for n in range(N)]
    else:
        groups = [[(n, k) for k in range(c * g, (c + 1) * g)] for n in range(N) for c in range(K // g)]
    q = np.zeros((N, K), dtype=np.uint8)
    ss, zz = [], []
    for grp in groups:
        vals = [frac(w32[n, k]) for n, k in grp]
        lo, hi = min(vals), max(vals)
        s16 = round_fmt(round_fmt(round_fmt(hi - lo, "f32") / 15, "f32"), "f16")
        if s16 == 0 or isinstance(s16, float):
            s16 = 1
        z = min(max(rint_half_even(round_fmt((0 - lo) / s16, "f32")), 0), 15)
        for (n, k), v in zip(grp, vals):
            q[n, k] = min(max(rint_half_even(round_fmt(v / s16, "f32")) + z, 0), 15)
        ss.append(float(s16))
        zz.append(float(z))
    shp = O.meta_shape(N, K, mode, g)
    return q, np.array(ss).reshape(shp), np.array(zz).reshape(shp)


@pytest.mark.parametrize("name,w", _tiny_inputs(), ids=[c[0] for c in _tiny_inputs()])
def test_bruteforce_int_zero(name, w):
    K = w.shape[1]
    for mode, g in [(O.GLOBAL, None), (O.ROWWISE, None), (O.GROUPWISE, 16), (O.GROUPWISE, 32), (O.GROUPWISE, K)]:
        q, s, z = O.quantize(w, mode, g, int_zero=True)
        qb, sb, zb = _brute_quantize_int_zero(w, mode, g)
        assert np.array_equal(s.astype(np.float64), sb), (name, mode, g)
        assert np.array_equal(z.astype(np.float64), zb), (name, mode, g)
        assert np.array_equal(q, qb), (name, mode, g)


def test_int_zero_order_matters_at_ties():
    """Rounding w/s before adding the integer zero (AWQ's order) differs from rounding
    w/s + z when w/s is a half-integer and z is odd: pin one such element."""
    # group [-1.5, ..., 6.0]: s = fp16(7.5 / 15) = 0.5, z = rint(1.5 / 0.5) = 3 (odd);
    # w = 0.25 -> w / s = 0.5 -> rint = 0 -> q = 3, whereas rint(0.5 + 3) = 4
    w = np.array([[-1.5, 6.0, 0.25, 0.0] + [0.0] * 12], dtype=np.float32)
    q, s, z = O.quantize(w, O.GROUPWISE, 16, int_zero=True)
    assert float(s[0, 0]) == 0.5 and float(z[0, 0]) == 3.0
    assert q[0, 2] == 3 and q[0, 3] == 3 and q[0, 0] == 0 and q[0, 1] == 15


@pytest.mark.parametrize("mode,g", [(O.ROWWISE, None), (O.GROUPWISE, 32), (O.GROUPWISE, 128)])
def test_int_zero_invariants(mode, g):
    w = synth.weight(11, 0, 48, 256, "f32")
    w[3, :40] = 0.0
    q, s, z = O.quantize(w, mode, g, int_zero=True)
    zf = z.astype(np.float64)
    assert np.all(zf == np.round(zf)) and zf.min() >= 0 and zf.max() <= 15
    # an exact zero weight (with min <= 0 <= max in its group) gets code z and dequantizes to 0
    deq = O.dequantize_f32(O.pack(q), s, z, w.shape[1])
    zero_pos = w == 0.0
    assert np.all(deq[zero_pos] == 0.0)
    # every in-range weight is within half a step of its dequantized value (up to rounding)
    sx = _expand(s, *w.shape)
    assert np.all(np.abs(deq - w) <= 0.5 * sx * (1 + 1e-3) + 1e-7)


def test_zero_overflow_group():
    """fp32 [1.0, 1.0001]: s = fp16(1e-4 / 15) is an fp16 subnormal and -min/s ~ -1.5e5 is
    beyond fp16, so the group is quantized as a constant group: s = 1, z = -1, every code 0
    and the dequantized values exactly 1.0 (finite).  Only fp32 weights reach this: an fp16
    or bf16 group's range is at least one unit of its min's last place, so |min| / range is
    at most 2^11 and -min/s stays below 15 * 2^11 < 65504."""
    w = np.array([[1.0, 1.0001] + [1.00005] * 14], dtype=np.float32)
    for mode, g in [(O.ROWWISE, None), (O.GROUPWISE, 16), (O.GLOBAL, None)]:
        packed, s, z = O.quantize_pack(w, mode, g)
        assert int(s.view(np.uint16)[0, 0]) == 0x3C00
        assert int(z.view(np.uint16)[0, 0]) == 0xBC00  # -1.0
        assert np.all(O.unpack(packed) == 0)
        assert np.all(O.dequantize_f32(packed, s, z, 16) == 1.0)


def test_zero_overflow_bound():
    """The fallback applies exactly when fp16(-min / s) overflows: a group with a finite
    zero point just below 65504 keeps its min-max scale."""
    lo = np.float32(-1.0)
    # s = 2^-14 (fp16 normal): -lo / s = 16384, finite; the group keeps s
    w = np.array([[lo, lo + np.float32(15 * 2.0 ** -14)]], dtype=np.float32)
    _, s, z = O.quantize_pack(np.repeat(w, 8, axis=1), O.ROWWISE)
    assert float(s[0, 0]) == 2.0 ** -14 and float(z[0, 0]) == 16384.0
    # s = 2^-17 (fp16 subnormal): -lo / s = 131072 overflows fp16; s falls back to 1
    w = np.array([[lo, lo + np.float32(15 * 2.0 ** -17)]], dtype=np.float32)
    _, s, z = O.quantize_pack(np.repeat(w, 8, axis=1), O.ROWWISE)
    assert float(s[0, 0]) == 1.0 and float(z[0, 0]) == 1.0
