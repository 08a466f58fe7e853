"""Pins of the oracle's reported quantities: compression (closed form, and the
page's printed column) and MAE (a hand-derived value on two golden rows, and the
page's trend; the page's own MAE values stay unpinned, their data being unstated)."""

import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_table():
    rows = []
    with open(os.path.join(GOLDEN, "page_quant_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            mode, g, mae, comp = line.split()
            rows.append((mode, None if g == "-" else int(g), float(mae), float(comp)))
    return rows


def test_page_compression_column_reproduced():
    # The page's column is 16 bits of metadata per group on a 4096 x 4096 matrix.
    N = K = 4096
    for mode, g, _, comp in _page_table():
        pairs = 1 if mode == "GLOBAL" else (N if mode == "ROWWISE" else N * K // g)
        assert round(O.page_compression_ratio(N, K, pairs), 6) == pytest.approx(comp, abs=1.5e-6)


@pytest.mark.parametrize("g", [16, 32, 64, 128, 256, 512, 1024, 2048])
def test_compression_closed_form(g):
    N, K = 128, 4096
    assert O.compression_ratio(N, K, N * K // g) == pytest.approx(16.0 / (4.0 + 32.0 / g), rel=1e-15)


def test_mae_trend_matches_page():
    # The page's MAE grows with the group size and GLOBAL is the worst; the data it was
    # measured on is unstated, so only the ordering is pinned.
    N, K = 256, 4096
    w = synth.weight(300, 0, N, K, "f16", std=1.0)
    w32 = O.to_f32(w, "f16")
    maes = {}
    for g in (16, 32, 64, 128, 256, 512, 1024, 2048, 4096):
        maes[g] = O.mae(w32, *O.quantize_pack(w32, O.GROUPWISE, g))
    glob = O.mae(w32, *O.quantize_pack(w32, O.GLOBAL))
    row = O.mae(w32, *O.quantize_pack(w32, O.ROWWISE))
    seq = [maes[g] for g in sorted(maes)]
    assert all(a < b for a, b in zip(seq, seq[1:]))
    assert glob > max(seq)
    assert row == pytest.approx(maes[4096], rel=1e-12)


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.split()
    return out


def test_mae_hand_derived_rows():
    """MAE of two ROWWISE rows derived by hand (tests/golden/mae_rows.txt).  A signed mean, a
    squared error, a sum instead of a mean, or the bf16 operand in place of the fp32
    dequantization each gives a different value."""
    gd = _golden("mae_rows.txt")
    a = np.array([float(v) for v in gd["row_a"]], dtype=np.float32)
    b = np.array([float(v) for v in gd["row_b"]], dtype=np.float32)
    # the decimal inputs of row A are within 3e-7 of their fp32 values: 1e-7 on a mean of 16
    for row, key in ((a, "mae_a"), (b, "mae_b")):
        w = row.reshape(1, 16)
        assert O.mae(w, *O.quantize_pack(w, O.ROWWISE)) == pytest.approx(float(gd[key][0]), abs=1e-7)
    w = np.stack([a, b])
    packed, s, z = O.quantize_pack(w, O.ROWWISE)
    assert int(s.view(np.uint16)[1, 0]) == int(gd["scale_bits_b"][0], 16)
    assert int(z.view(np.uint16)[1, 0]) == int(gd["zero_bits_b"][0], 16)
    assert O.mae(w, packed, s, z) == pytest.approx(float(gd["mae_both"][0]), abs=1e-7)
    # row B alone is exact: every value involved is a dyadic rational
    wb = b.reshape(1, 16)
    assert O.mae(wb, *O.quantize_pack(wb, O.ROWWISE)) == 105.0 / 16384.0
