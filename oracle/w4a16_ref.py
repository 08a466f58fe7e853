"""Reference (oracle) semantics of W4A16 quantize-and-pack and the int4 matmul.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (web pages; cited by title and section):

* "Quantized LLM Inference with Triton Kernels" (anaaaiva/llm-quantization),
  Objectives 1-3: FP16 -> INT4 quantization with global / rowwise / groupwise
  modes, packed into INT8 or INT32 words; its quantization table (MAE and
  compression per mode and group size); the matmul ``Y = X_bf16 @ W_int4^T``.
* "Re-write HQQ Fused Gemm Transpose" (pytorch/ao #185): the reference path is
  ``dequantize()`` followed by a bf16 matmul; the transposed kernel reads the
  same packed weights, scales and zeros (``transposed=True``).
* "Add fused QKV HQQ triton_mm test" (pytorch/ao #306): Q, K and V weights are
  quantized, packed and fused into one operand; the fused result must equal the
  separate ones in both modes.
* "Modify small-batched weight only quantization" (TensorRT-LLM #2213): 4-bit
  weights with group size 128 along K for batched decode GEMV.
* "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560):
  an fp32 bias added in the matmul epilogue.

Readings where the pages are silent:

1. Scale and zero are min-max asymmetric: ``s = (max-min)/15``, ``z = -min/s``,
   computed in fp32 and stored as fp16 (round to nearest even); ``z`` is not
   rounded to an integer.  A zero or non-finite fp16 scale is replaced by 1.
7. A group whose fp16 zero would be infinite (its range below 15 |min| / 65504,
   e.g. [1.0, 1.0001] in fp32) is quantized like a constant group: s = 1 and
   ``z = fp16(0 - min)``, so its values dequantize to within its range of min.
   Only when |min| > 65504 (possible for fp32 / bf16 weights) does that zero
   overflow too; it is then left infinite.
2. Codes: ``q = clamp(rint(w/s + z), 0, 15)`` with fp32 divide and add and
   round-half-to-even.
3. Packing: row-major ``[N][K/8]`` int32 words; code ``k = 8c + j`` of row n
   sits in bits ``[4j, 4j+3]`` of word c (LSB first; byte-identical to two
   codes per byte, low nibble first).
4. Scales and zeros are two fp16 arrays ``[rows][K/g]`` (group index fastest);
   ROWWISE keeps one pair per row, GLOBAL one pair for the whole tensor.
5. Dequantization is ``bf16_rne(fp32(fp32(q) - z) * s)``: the weight operand of
   the matmul is bf16, as in the dequantize-then-bf16-matmul reference path.
6. Products accumulate in float64 here; the output is fp32 on the GPU.

Pins (tests/test_oracle_*.py, run with ``-m "not gpu"``):

* quantize: exact-rational brute force of every rounding step on tiny inputs,
  a hand-derived golden row (tests/golden/quant_row.txt), invariants
  (code range, min->0 / max->15, error bound, ROWWISE == GROUPWISE(g=K)).
* pack / unpack: the golden word of the LSB-first layout, bijection both ways.
* pack_bytes (INT8 packing): golden bytes of the same codes; the int32 words
  viewed as little-endian bytes equal it.
* quantize with integer zero points: the same exact-rational brute force in
  AWQ's order (round, then add the integer zero), and invariants (integer zero
  in [0, 15], exact zero maps to code z and dequantizes to exactly 0).
* dequantize: all 16 codes against an exact-rational bf16 rounding (and fp16
  rounding for the fp16 operand).
* matmul: exact-rational triple loop on tiny shapes (bf16 activations, and fp16
  activations decoded by hand from their bit fields against the fp16 operand),
  one-hot pins of the layout in both modes, constant-code closed form,
  linearity and bias.
* fused QKV: column concatenation (non-transposed) and sum (transposed).
* round_output: hand-derived bf16 / fp16 roundings (ties to even, 8 and 11
  significant bits, the fp16 maximum).
* compression: the page's printed column reproduced by its closed form.
* MAE: a hand-derived value on two golden rows (tests/golden/mae_rows.txt) that
  tells the fp32 dequantization from the bf16 one and an absolute mean from a
  signed or squared one; the page's own MAE values stay unpinned (its data
  distribution is unstated), only their trends are checked.
* zero overflow (reading 7): a group built so that -min/s overflows fp16, and
  the exact-rational brute force over such groups.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "GLOBAL", "ROWWISE", "GROUPWISE", "MODE_NAMES",
    "meta_shape", "to_f32", "quantize", "pack", "unpack", "quantize_pack", "pack_bytes",
    "dequantize_f32", "bf16_rne_bits", "bf16_bits_to_f64", "dequantize_bf16_bits", "f16_bits_to_f64",
    "dequantize_f16_bits",
    "matmul", "round_output", "fuse_rows", "mae", "compression_ratio", "page_compression_ratio",
]

GLOBAL, ROWWISE, GROUPWISE = 0, 1, 2
MODE_NAMES = {GLOBAL: "global", ROWWISE: "rowwise", GROUPWISE: "groupwise"}

_F32 = np.float32
_F16 = np.float16


def meta_shape(N: int, K: int, mode: int, g: int | None = None) -> tuple[int, int]:
    """Shape of the scales (and zeros) array: GLOBAL (1,1), ROWWISE (N,1), GROUPWISE (N, K/g).

    Group modes as in the quantization table of "Quantized LLM Inference with
    Triton Kernels" (GLOBAL, ROWWISE, GROUPWISE with a group size along K).
    """
    if mode == GLOBAL:
        return (1, 1)
    if mode == ROWWISE:
        return (N, 1)
    if mode == GROUPWISE:
        assert g is not None and K % g == 0
        return (N, K // g)
    raise ValueError(mode)


def to_f32(W: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 view of a weight stored as 'f32', 'f16' or 'bf16' (uint16 bits)."""
    if dtype == "f32":
        return np.asarray(W, dtype=_F32)
    if dtype == "f16":
        return np.asarray(W, dtype=_F16).astype(_F32)
    if dtype == "bf16":
        return (np.asarray(W, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(_F32)
    raise ValueError(dtype)


def _grouped(w32: np.ndarray, mode: int, g: int | None) -> np.ndarray:
    """View [N][K] as [rows][groups][elements per group]."""
    N, K = w32.shape
    if mode == GLOBAL:
        return w32.reshape(1, 1, N * K)
    if mode == ROWWISE:
        return w32.reshape(N, 1, K)
    return w32.reshape(N, K // g, g)


def quantize(w32: np.ndarray, mode: int, g: int | None = None, int_zero: bool = False):
    """Asymmetric uint4 codes with an fp16 scale and zero per group.

    Follows Objective 1 of "Quantized LLM Inference with Triton Kernels"
    (FP16 -> INT4, global / rowwise / groupwise) with readings 1 and 2 of the
    module docstring.  Returns ``(q uint8 [N][K], scales fp16, zeros fp16)``.

    ``int_zero``: the integer zero point of the AWQ format named by "Modify
    small-batched weight only quantization" (W4A16 AWQ, g = 128), in AWQ's order:
    ``z = clamp(rint((0 - min) / s), 0, 15)`` and ``q = clamp(rint(w / s) + z, 0, 15)``
    (rounding before the integer add; the two orders differ at ties).  The zero is
    stored as the fp16 value of that integer.
    """
    w32 = np.asarray(w32, dtype=_F32)
    N, K = w32.shape
    assert np.all(np.isfinite(w32)), "the oracle is defined for finite weights"
    grp = _grouped(w32, mode, g)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        lo = grp.min(axis=-1)                      # exact
        hi = grp.max(axis=-1)                      # exact
        s32 = (hi - lo) / _F32(15.0)               # fp32 subtract, fp32 divide (RNE)
        s16 = s32.astype(_F16)                     # fp16 RNE
        s16 = np.where((s16 == 0) | ~np.isfinite(s16), _F16(1.0), s16)
        s_f = s16.astype(_F32)
        z32 = (_F32(0.0) - lo) / s_f               # 0 - lo keeps an all-zero group's zero at +0
        if int_zero:
            z_f = np.clip(np.rint(z32), 0, 15).astype(_F32)   # an integer in [0, 15]
            z16 = z_f.astype(_F16)                             # exact
            t = np.rint(grp / s_f[..., None]) + z_f[..., None]  # round, then the exact integer add
        else:
            z16 = z32.astype(_F16)
            # A zero point beyond the fp16 range (the group's range is below 15 |min| / 65504,
            # tiny next to its offset) makes the group degenerate like a zero scale: s = 1
            # and z = fp16(0 - min), so its values dequantize to min (reading 7).
            wide = ~np.isfinite(z16)
            if np.any(wide):
                s16 = np.where(wide, _F16(1.0), s16)
                s_f = s16.astype(_F32)
                z16 = np.where(wide, ((_F32(0.0) - lo) / s_f).astype(_F16), z16)
            z_f = z16.astype(_F32)
            t = grp / s_f[..., None] + z_f[..., None]  # two fp32 ops, each rounded
    assert not np.any(np.isnan(t)), "code argument is NaN (zero overflowed fp16)"
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8)  # rint: round half to even (a no-op for int_zero)
    return q.reshape(N, K), s16.reshape(meta_shape(N, K, mode, g)), z16.reshape(meta_shape(N, K, mode, g))


def pack(q: np.ndarray) -> np.ndarray:
    """Pack 8 codes per int32 word, LSB first (reading 3).

    Objective 1 of "Quantized LLM Inference with Triton Kernels" packs the int4
    matrix into INT8 or INT32 words; code ``k = 8c + j`` goes to bits 4j..4j+3.
    """
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    assert K % 8 == 0
    q32 = q.reshape(N, K // 8, 8).astype(np.uint32)
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        word |= (q32[:, :, j] & np.uint32(0xF)) << np.uint32(4 * j)
    return word.view(np.int32)


def unpack(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack`: int32 ``[N][K/8]`` -> uint8 codes ``[N][K]``."""
    w = np.asarray(packed).view(np.uint32)
    N, C = w.shape
    q = np.empty((N, C, 8), dtype=np.uint8)
    for j in range(8):
        q[:, :, j] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    return q.reshape(N, C * 8)


def quantize_pack(w32: np.ndarray, mode: int, g: int | None = None, int_zero: bool = False):
    """Quantize then pack: returns ``(packed int32 [N][K/8], scales fp16, zeros fp16)``."""
    q, s, z = quantize(w32, mode, g, int_zero)
    return pack(q), s, z


def pack_bytes(q: np.ndarray) -> np.ndarray:
    """INT8 packing of Objective 1 of "Quantized LLM Inference with Triton Kernels":
    two codes per byte, code ``k = 2b + j`` in bits 4j..4j+3 of byte b (uint8 [N][K/2])."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    assert K % 2 == 0
    q2 = q.reshape(N, K // 2, 2)
    return ((q2[:, :, 0] & 0xF) | ((q2[:, :, 1] & 0xF) << 4)).astype(np.uint8)


def _expand_meta(meta: np.ndarray, N: int, K: int) -> np.ndarray:
    """Broadcast a [rows][groups] fp16 array to one fp32 value per element [N][K]."""
    rows, groups = meta.shape
    m = meta.astype(_F32)
    if rows == 1 and groups == 1:
        return np.broadcast_to(m.reshape(1, 1), (N, K))
    assert rows == N and K % groups == 0
    return np.repeat(m, K // groups, axis=1)


def dequantize_f32(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int) -> np.ndarray:
    """fp32 ``(q - z) * s`` (two fp32 ops, each rounded); the inverse of the quantizer.

    "Re-write HQQ Fused Gemm Transpose": the reference path dequantizes the
    packed weights with their scales and zeros before a bf16 matmul.
    """
    q = unpack(packed)
    N = q.shape[0]
    assert q.shape[1] == K
    s = _expand_meta(scales, N, K)
    z = _expand_meta(zeros, N, K)
    with np.errstate(over="ignore", invalid="ignore"):
        return (q.astype(_F32) - z) * s


def bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=_F32).view(np.uint32)
    nan = np.isnan(np.ascontiguousarray(x32, dtype=_F32))
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(_F32).astype(np.float64)


def dequantize_bf16_bits(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int) -> np.ndarray:
    """The bf16 weight operand ``bf16_rne((q - z) * s)`` as uint16 bits (reading 5)."""
    return bf16_rne_bits(dequantize_f32(packed, scales, zeros, K))


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64 (exact)."""
    return np.asarray(b, dtype=np.uint16).view(_F16).astype(np.float64)


def dequantize_f16_bits(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int) -> np.ndarray:
    """The fp16 weight operand ``fp16_rne((q - z) * s)`` (the fp32 two-op sequence, then one
    rounding to fp16) as uint16 bits: the operand of fp16 activations."""
    with np.errstate(over="ignore"):
        return dequantize_f32(packed, scales, zeros, K).astype(_F16).view(np.uint16)


def matmul(a_bf16: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int,
           transposed: bool = False, bias: np.ndarray | None = None, a_dtype: str = "bf16") -> np.ndarray:
    """float64 result of the W4A16 matmul.

    Non-transposed (Objective 2 of "Quantized LLM Inference with Triton
    Kernels"): ``Y[m, n] = sum_k X[m, k] * w[n, k] (+ bias[n])`` with X bf16 [M][K].
    Transposed ("Re-write HQQ Fused Gemm Transpose", same packed buffer):
    ``dX[m, k] = sum_n dY[m, n] * w[n, k] (+ bias[k])`` with dY bf16 [M][N].
    ``w`` is the bf16 dequantized weight; the bias is fp32 ("[Kernel] Adding
    bias epilogue support for cutlass_scaled_mm").  Accumulates in float64.
    ``a_dtype="f16"``: the activations are fp16 bits and the weight operand is
    ``dequantize_f16_bits`` (the fp16 path of a W4A16 kernel).
    """
    if a_dtype == "f16":
        w64 = f16_bits_to_f64(dequantize_f16_bits(packed, scales, zeros, K))
        a64 = f16_bits_to_f64(a_bf16)
    else:
        w64 = bf16_bits_to_f64(dequantize_bf16_bits(packed, scales, zeros, K))   # [N][K]
        a64 = bf16_bits_to_f64(a_bf16)
    y = a64 @ w64 if transposed else a64 @ w64.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return y


def round_output(y: np.ndarray, dtype: str) -> np.ndarray:
    """The matmul output in its storage dtype, as float64.

    "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560) gives
    the bias the output dtype and adds it before the one conversion of the sum to
    that dtype.  Here the sum (bias included, see ``matmul``) is rounded to fp32 and
    then to ``dtype`` ("f32", "bf16" or "f16"), round to nearest, ties to even; the
    fp32 step only differs from a direct rounding on exact double-rounding ties.
    """
    y32 = np.asarray(y, dtype=np.float64).astype(_F32)
    if dtype == "f32":
        return y32.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(bf16_rne_bits(y32))
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return y32.astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def fuse_rows(parts):
    """Fuse per-projection (packed, scales, zeros) triples by row concatenation.

    "Add fused QKV HQQ triton_mm test": Q, K and V weights are quantized and
    packed separately and then fused into one operand.  Only defined for
    ROWWISE / GROUPWISE metadata (one pair per row or per row-group): a GLOBAL
    pair belongs to one tensor, so it is rejected.
    """
    for p, s, z in parts:
        if s.shape == (1, 1) and p.shape[0] != 1:
            raise ValueError("GLOBAL scale/zero cannot be fused by rows")
    packed = np.concatenate([p for p, _, _ in parts], axis=0)
    scales = np.concatenate([s for _, s, _ in parts], axis=0)
    zeros = np.concatenate([z for _, _, z in parts], axis=0)
    return packed, scales, zeros


def mae(w32: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> float:
    """Mean absolute error of the fp32 dequantization against the fp32 weight (float64 mean).

    The quantity tabulated per mode in "Quantized LLM Inference with Triton Kernels".
    """
    K = w32.shape[1]
    d = dequantize_f32(packed, scales, zeros, K).astype(np.float64)
    return float(np.mean(np.abs(d - np.asarray(w32, dtype=np.float64))))


def compression_ratio(N: int, K: int, pairs: int) -> float:
    """fp16 bytes over (packed codes + fp16 scale and fp16 zero per pair)."""
    return (N * K * 2.0) / (N * K / 2.0 + 4.0 * pairs)


def page_compression_ratio(N: int, K: int, pairs: int) -> float:
    """The convention of the page's compression column: 16 bits of metadata per group."""
    return (N * K * 2.0) / (N * K / 2.0 + 2.0 * pairs)
