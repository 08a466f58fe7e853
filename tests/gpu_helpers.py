"""Helpers for the GPU parity tests: host <-> device transfers and the tolerance check.

Inputs always come from ``synth`` on the host; the expected values always come
from ``oracle`` on the same host arrays.  Nothing computed by the HIP path is
ever fed back into the oracle.
"""

import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")

# matmul tolerance: relative Frobenius error and an elementwise bound
FRO_TOL = 1e-3
ELEM_ATOL = 1e-2
ELEM_RTOL = 1e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_weight(w: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(w, dtype=np.float16)).to(DEV)
    return dev_bf16(w)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_quant_equal(qw, packed, scales, zeros, rows=None, what=""):
    """Packed words, scales and zeros must be bit-exact with the oracle."""
    gp = host(qw.packed)
    gs = host_bits16(qw.scales)
    gz = host_bits16(qw.zeros)
    if rows is not None:
        gp = gp[rows]
        if gs.shape[0] > 1:
            gs, gz = gs[rows], gz[rows]
    np.testing.assert_array_equal(gp, packed, err_msg=f"packed {what}")
    np.testing.assert_array_equal(gs, scales.view(np.uint16), err_msg=f"scales {what}")
    np.testing.assert_array_equal(gz, zeros.view(np.uint16), err_msg=f"zeros {what}")


def assert_mm_close(y: np.ndarray, ref: np.ndarray, what=""):
    """Relative Frobenius error <= 1e-3 and |y - ref| <= 1e-2 |ref| + 1e-2 for every element."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape, what)
    assert np.all(np.isfinite(y)), f"non-finite output {what}"
    nref = np.linalg.norm(ref)
    fro = np.linalg.norm(y - ref) / (nref if nref > 0 else 1.0)
    assert fro <= FRO_TOL, f"relative Frobenius error {fro:.3e} > {FRO_TOL} {what}"
    bad = np.abs(y - ref) > ELEM_RTOL * np.abs(ref) + ELEM_ATOL
    assert not bad.any(), f"{int(bad.sum())} elements outside the elementwise bound {what}"
    return fro


def assert_rounded_close(y: np.ndarray, ref64: np.ndarray, dt: str, what: str):
    """y (stored in dt) against the oracle sum rounded to dt: the fp32 accumulation may put
    the sum on the other side of a rounding boundary, so allow one unit in the last place
    of dt on top of the matmul bounds."""
    want = O.round_output(ref64, dt)
    ulp = np.abs(want) * (2.0**-7 if dt == "bf16" else 2.0**-10 if dt == "f16" else 0.0)
    bad = np.abs(y - want) > ELEM_RTOL * np.abs(want) + ELEM_ATOL + ulp
    assert not bad.any(), f"{int(bad.sum())} elements outside the bound {what}"
    fro = np.linalg.norm(y - want) / max(np.linalg.norm(want), 1e-30)
    assert fro <= FRO_TOL, f"relative Frobenius error {fro:.3e} {what}"


def oracle_rows_global(w32: np.ndarray, rows: np.ndarray):
    """Oracle GLOBAL quantization of selected rows, exactly as if the whole tensor were quantized.

    GLOBAL scale / zero depend only on the tensor's min and max, and a row's codes only on
    those and its own values; so quantizing the selected rows together with the rows that
    hold the global min and max reproduces the full-tensor result for those rows.
    """
    flat_min = np.unravel_index(np.argmin(w32), w32.shape)[0]
    flat_max = np.unravel_index(np.argmax(w32), w32.shape)[0]
    sel = np.concatenate([rows, [flat_min, flat_max]])
    p, s, z = O.quantize_pack(w32[sel], O.GLOBAL)
    return p[: len(rows)], s, z
