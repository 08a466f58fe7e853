"""PyTorch-facing binding of the W4A16 library.

Argument marshalling only: tensors supply device memory and the current HIP
stream; every step of quantization, dequantization and the matmul runs in the
library's gfx950 kernels (see include/w4a16.h for the contract).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import DT_BF16, DT_F16, DT_F32, MODE_GLOBAL, MODE_GROUPWISE, MODE_ROWWISE, W4Desc, check, lib

_MODES = {"global": MODE_GLOBAL, "rowwise": MODE_ROWWISE, "groupwise": MODE_GROUPWISE}
_WDT = {torch.float32: DT_F32, torch.float16: DT_F16, torch.bfloat16: DT_BF16}


def mode_id(mode) -> int:
    if isinstance(mode, str):
        return _MODES[mode.lower()]
    return int(mode)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    """The current HIP stream of `device` (the raw handle; about 2 us cheaper per call than
    building torch's stream object)."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(idx).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _as_bf16(a: torch.Tensor) -> torch.Tensor:
    """Accept bf16 or fp16 activations, or 16-bit integer tensors holding bf16 bits."""
    if a.dtype in (torch.bfloat16, torch.float16):
        return a
    if a.dtype in (torch.int16, torch.uint16):
        return a.view(torch.bfloat16)
    raise TypeError(f"activations must be bfloat16 (got {a.dtype})")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")


@dataclass
class QuantizedWeight:
    """Packed int4 weight W[N][K]: packed int32 [N][K/8], fp16 scales / zeros."""

    packed: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    N: int
    K: int
    mode: int
    group: int
    zero: str = "fp16"  # "fp16" zero points, or "int" (integer zero points in [0, 15])

    def desc(self) -> W4Desc:
        return W4Desc(self.N, self.K, self.mode, self.group if self.mode == MODE_GROUPWISE else 0)

    def packed_bytes(self) -> torch.Tensor:
        """The packed codes as INT8 words: uint8 [N][K/2], two codes per byte, low nibble
        first -- the same bytes as the int32 words (a view, no copy)."""
        return self.packed.view(torch.uint8)

    @classmethod
    def from_bytes(cls, packed_u8: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, mode, group=None):
        """Wrap INT8-packed codes (uint8 [N][K/2], 4-byte aligned, contiguous) without a copy."""
        if packed_u8.dtype != torch.uint8 or packed_u8.dim() != 2 or not packed_u8.is_contiguous():
            raise ValueError("packed_u8 must be a contiguous uint8 [N][K/2] tensor")
        if packed_u8.shape[1] % 4 or packed_u8.data_ptr() % 4:
            raise ValueError("INT8-packed rows must hold a multiple of 8 codes and be 4-byte aligned")
        N, K = packed_u8.shape[0], packed_u8.shape[1] * 2
        m = mode_id(mode)
        return cls(packed_u8.view(torch.int32), scales, zeros, N, K, m, int(group) if m == MODE_GROUPWISE else 0)

    def mm(self, x: torch.Tensor, bias: torch.Tensor | None = None, out: torch.Tensor | None = None):
        """Y = X @ w^T (+ bias)."""
        return mm(x, self, transposed=False, bias=bias, out=out)

    def mm_t(self, dy: torch.Tensor, bias: torch.Tensor | None = None, out: torch.Tensor | None = None):
        """dX = dY @ w (+ bias), on the same packed buffer."""
        return mm(dy, self, transposed=True, bias=bias, out=out)


def meta_shape(N: int, K: int, mode: int, group: int) -> tuple[int, int]:
    if mode == MODE_GLOBAL:
        return (1, 1)
    if mode == MODE_ROWWISE:
        return (N, 1)
    return (N, K // group)


def empty_quantized(N: int, K: int, mode, group: int | None, device) -> QuantizedWeight:
    """Allocate the buffers of a packed weight (contents undefined)."""
    m = mode_id(mode)
    g = int(group) if m == MODE_GROUPWISE else 0
    shp = meta_shape(N, K, m, g)
    return QuantizedWeight(
        packed=torch.empty((N, K // 8), dtype=torch.int32, device=device),
        scales=torch.empty(shp, dtype=torch.float16, device=device),
        zeros=torch.empty(shp, dtype=torch.float16, device=device),
        N=N, K=K, mode=m, group=g)


_ZERO = {"fp16": _lib.ZERO_FP16, "int": _lib.ZERO_INT}


def quantize_pack_into(W: torch.Tensor, qw: QuantizedWeight, row0: int = 0, zero: str = "fp16") -> None:
    """Quantize W [n][K] into rows row0 .. row0+n of an existing packed weight.

    Used to fuse projections (for example Q, K and V) into one packed operand
    without a copy: each part is quantized straight into its row slice.
    zero="int" rounds each zero point to an integer in [0, 15] (AWQ style).
    """
    _need_cuda(W, qw.packed)
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D tensor")
    n, K = W.shape
    if K != qw.K or row0 < 0 or row0 + n > qw.N:
        raise ValueError("W does not fit the packed weight")
    if qw.mode == MODE_GLOBAL and (row0 != 0 or n != qw.N):
        raise ValueError("a GLOBAL scale / zero cannot be shared by row slices")
    dt = _WDT.get(W.dtype)
    if dt is None:
        raise TypeError(f"unsupported weight dtype {W.dtype}")
    desc = W4Desc(n, K, qw.mode, qw.group)
    L = lib()
    ws_bytes = ctypes.c_size_t(0)
    check(L.w4_workspace_bytes(ctypes.byref(desc), _lib.OP_QUANTIZE, 0, ctypes.byref(ws_bytes)))
    ws = torch.empty(max(ws_bytes.value, 1), dtype=torch.uint8, device=W.device) if ws_bytes.value else None
    gpr = qw.scales.shape[1]
    mrow = 0 if qw.mode == MODE_GLOBAL else row0
    packed = qw.packed[row0:row0 + n]
    scales = qw.scales[mrow:mrow + (1 if qw.mode == MODE_GLOBAL else n)]
    zeros = qw.zeros[mrow:mrow + (1 if qw.mode == MODE_GLOBAL else n)]
    assert scales.shape[1] == gpr
    check(L.w4_quantize_pack_zp(_ptr(W), dt, ctypes.byref(desc), _ZERO[zero], _ptr(packed), _ptr(scales),
                                _ptr(zeros), _ptr(ws), ws_bytes.value, _stream(W.device)))


def quantize_pack(W: torch.Tensor, mode="groupwise", group: int | None = 128, zero: str = "fp16") -> QuantizedWeight:
    """Quantize and pack W [N][K] (fp32, fp16 or bf16) to asymmetric uint4; zero="int" gives
    integer zero points (AWQ style)."""
    N, K = W.shape
    qw = empty_quantized(N, K, mode, group, W.device)
    qw.zero = zero
    quantize_pack_into(W, qw, 0, zero)
    return qw


def quantize_fused(parts, mode="groupwise", group: int | None = 128, zero: str = "fp16") -> QuantizedWeight:
    """Quantize several [n_i][K] weights into one row-concatenated packed operand (fused QKV)."""
    K = parts[0].shape[1]
    N = sum(p.shape[0] for p in parts)
    if mode_id(mode) == MODE_GLOBAL:
        raise ValueError("GLOBAL scale / zero cannot be fused by rows")
    qw = empty_quantized(N, K, mode, group, parts[0].device)
    qw.zero = zero
    r = 0
    for p in parts:
        quantize_pack_into(p, qw, r, zero)
        r += p.shape[0]
    return qw


def serialize(qw: QuantizedWeight) -> bytes:
    """The packed weight in the library's serialized form (w4_serial_header, then the packed
    words, scales and zeros at 64-byte aligned offsets); device tensors are copied to host."""
    hdr = _lib.W4SerialHeader()
    check(lib().w4_serial_layout(ctypes.byref(qw.desc()), _ZERO[qw.zero], ctypes.byref(hdr)))
    buf = bytearray(hdr.total_bytes)
    buf[:ctypes.sizeof(hdr)] = bytes(hdr)
    for off, t, n in ((hdr.packed_offset, qw.packed, hdr.packed_bytes), (hdr.scales_offset, qw.scales, hdr.meta_bytes),
                      (hdr.zeros_offset, qw.zeros, hdr.meta_bytes)):
        b = t.contiguous().cpu().view(torch.uint8).numpy().tobytes()
        assert len(b) == n
        buf[off:off + n] = b
    return bytes(buf)


def deserialize(data: bytes, device="cuda") -> QuantizedWeight:
    """Inverse of :func:`serialize`: validate the header and upload the sections to `device`."""
    data = bytes(data)
    desc = W4Desc()
    zk = ctypes.c_int(0)
    cbuf = ctypes.create_string_buffer(data, len(data))
    check(lib().w4_serial_parse(cbuf, len(data), ctypes.byref(desc), ctypes.byref(zk)))
    hdr = _lib.W4SerialHeader.from_buffer_copy(data[:ctypes.sizeof(_lib.W4SerialHeader)])
    N, K, m = desc.N, desc.K, desc.mode
    g = desc.group if m == MODE_GROUPWISE else 0
    shp = meta_shape(N, K, m, g)

    def section(off, n, dtype, shape):
        return torch.frombuffer(bytearray(data[off:off + n]), dtype=dtype).reshape(shape).to(device)

    return QuantizedWeight(
        packed=section(hdr.packed_offset, hdr.packed_bytes, torch.int32, (N, K // 8)),
        scales=section(hdr.scales_offset, hdr.meta_bytes, torch.float16, shp),
        zeros=section(hdr.zeros_offset, hdr.meta_bytes, torch.float16, shp),
        N=N, K=K, mode=m, group=g, zero={v: k for k, v in _ZERO.items()}[zk.value])


def save(qw: QuantizedWeight, path: str) -> None:
    with open(path, "wb") as f:
        f.write(serialize(qw))


def load(path: str, device="cuda") -> QuantizedWeight:
    with open(path, "rb") as f:
        return deserialize(f.read(), device)


def dequantize(qw: QuantizedWeight, dtype=torch.bfloat16) -> torch.Tensor:
    """w = bf16_rne((q - z) * s) (bfloat16), fp16_rne((q - z) * s) (float16) or fp32 (q - z) * s
    (float32), [N][K]."""
    _need_cuda(qw.packed)
    out = torch.empty((qw.N, qw.K), dtype=dtype, device=qw.packed.device)
    odt = {torch.bfloat16: DT_BF16, torch.float16: DT_F16, torch.float32: DT_F32}[dtype]
    desc = qw.desc()
    check(lib().w4_dequantize(_ptr(qw.packed), _ptr(qw.scales), _ptr(qw.zeros), ctypes.byref(desc), _ptr(out), odt,
                              _stream(out.device)))
    return out


_ODT = {torch.float32: DT_F32, torch.float16: DT_F16, torch.bfloat16: DT_BF16}


def _workspace(qw: QuantizedWeight, M: int, transposed: bool, split_k: bool, device):
    if not transposed and 0 <= M <= 4:
        return None, 0  # the decode GEMV takes no workspace (w4_workspace_bytes reports 0)
    ws_bytes = ctypes.c_size_t(0)
    if split_k:
        op = _lib.OP_MM_T if transposed else _lib.OP_MM
        check(lib().w4_workspace_bytes(ctypes.byref(qw.desc()), op, M, ctypes.byref(ws_bytes)))
    ws = torch.empty(ws_bytes.value, dtype=torch.uint8, device=device) if ws_bytes.value else None
    return ws, ws_bytes.value


def _mm_out(a: torch.Tensor, qw: QuantizedWeight, transposed: bool, bias, outs, split_k: bool):
    """Marshal one w4a16_mm_out call: `outs` are 2-D [M][cols_i] tensors of one dtype
    (rows contiguous, any row stride) covering the output columns in order."""
    a = _as_bf16(a)
    _need_cuda(a, qw.packed, bias, *outs)
    if a.dim() != 2 or not a.is_contiguous():
        raise ValueError("activations must be a contiguous 2-D tensor")
    M, L = a.shape
    if L != (qw.N if transposed else qw.K):
        raise ValueError(f"activation width {L} does not match the weight ({qw.N}x{qw.K}, transposed={transposed})")
    dt = outs[0].dtype
    if dt not in _ODT or any(o.dtype != dt for o in outs):
        raise ValueError("outputs must share one dtype among float32, float16 and bfloat16")
    outc = qw.K if transposed else qw.N
    if bias is not None and (bias.dtype != dt or bias.numel() != outc or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous {dt} vector of length {outc}")
    segs = (_lib.W4OutSeg * len(outs))()
    for i, o in enumerate(outs):
        if o.dim() != 2 or o.shape[0] != M or o.stride(1) != 1:
            raise ValueError("each output must be a 2-D [M][cols] tensor with contiguous rows")
        segs[i].Y = o.data_ptr()
        segs[i].cols = o.shape[1]
        segs[i].ld = o.stride(0) if M > 1 else o.shape[1]
    ws, ws_bytes = _workspace(qw, M, transposed, split_k, a.device)
    desc = qw.desc()
    adt = DT_F16 if a.dtype == torch.float16 else DT_BF16
    check(lib().w4a16_mm_out(_ptr(a), adt, M, _ptr(qw.packed), _ptr(qw.scales), _ptr(qw.zeros), ctypes.byref(desc),
                             1 if transposed else 0, _ptr(bias), _ODT[dt], segs, len(outs), _ptr(ws), ws_bytes,
                             _stream(a.device)))


def mm(a: torch.Tensor, qw: QuantizedWeight, transposed: bool = False, bias: torch.Tensor | None = None,
       out: torch.Tensor | None = None, split_k: bool = True, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """W4A16 matmul: Y = A @ w^T (+bias) or, transposed, dX = A @ w (+bias), fp32 accumulation.

    A is bfloat16 (the weight operand bf16_rne((q - z) * s)) or float16 (an fp16 weight operand).

    The output is fp32 unless `out_dtype` (or `out`) asks for bfloat16 / float16, rounded once
    to nearest even; the bias, when given, has the output dtype.  split_k lets a GEMM with few
    output tiles split its contraction over a workspace (allocated here from torch's caching
    allocator; the sum order is fixed)."""
    a = _as_bf16(a)
    M = a.shape[0] if a.dim() == 2 else -1
    outc = qw.K if transposed else qw.N
    dt = out_dtype if out_dtype is not None else (out.dtype if out is not None else torch.float32)
    if out is None:
        out = torch.empty((max(M, 0), outc), dtype=dt, device=a.device)
    elif out.shape != (M, outc) or out.dtype != dt or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the output shape and dtype")
    if (dt is torch.float32 and a.dtype is torch.bfloat16 and (bias is None or bias.dtype is torch.float32)
            and M >= 0):
        _mm_f32(a, qw, transposed, bias, out, split_k)  # the common case: w4a16_mm itself
    else:
        _mm_out(a, qw, transposed, bias, [out], split_k)
    return out


def _mm_f32(a: torch.Tensor, qw: QuantizedWeight, transposed: bool, bias, out: torch.Tensor, split_k: bool):
    """bf16 activations, fp32 output and bias: one w4a16_mm call (the checks of _mm_out)."""
    _need_cuda(a, qw.packed, bias, out)
    if not a.is_contiguous():
        raise ValueError("activations must be a contiguous 2-D tensor")
    M, L = a.shape
    if L != (qw.N if transposed else qw.K):
        raise ValueError(f"activation width {L} does not match the weight ({qw.N}x{qw.K}, transposed={transposed})")
    outc = out.shape[1]
    if bias is not None and (bias.numel() != outc or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous torch.float32 vector of length {outc}")
    ws, ws_bytes = _workspace(qw, M, transposed, split_k, a.device)
    check(lib().w4a16_mm(_ptr(a), M, _ptr(qw.packed), _ptr(qw.scales), _ptr(qw.zeros), ctypes.byref(qw.desc()),
                         1 if transposed else 0, _ptr(bias), _ptr(out), _ptr(ws), ws_bytes, _stream(a.device)))


def mm_split(a: torch.Tensor, qw: QuantizedWeight, outs: list[torch.Tensor], bias: torch.Tensor | None = None,
             transposed: bool = False, split_k: bool = True) -> list[torch.Tensor]:
    """One product written to separate outputs in one launch: outs[i] [M][n_i] receives the
    next n_i output columns (for a fused Q/K/V weight, non-transposed: Q, K and V).
    Outputs share a dtype (fp32, bf16 or fp16) and may be row-strided views; the bias, if
    any, spans all output columns in that dtype."""
    if sum(o.shape[1] for o in outs) != (qw.K if transposed else qw.N):
        raise ValueError("the outputs' columns must sum to the output width")
    _mm_out(a, qw, transposed, bias, list(outs), split_k)
    return list(outs)


def kernel_for(M: int, N: int, K: int, mode="groupwise", group: int | None = 128, transposed=False) -> str | None:
    """Name of the kernel the library dispatches for this shape (host-side query)."""
    m = mode_id(mode)
    desc = W4Desc(N, K, m, int(group) if m == MODE_GROUPWISE else 0)
    r = lib().w4a16_mm_kernel(M, ctypes.byref(desc), 1 if transposed else 0)
    return r.decode() if r is not None else None


def mm_plan(M: int, N: int, K: int, mode="groupwise", group: int | None = 128, transposed=False,
            ws_bytes: int = 0) -> dict:
    """The launch a matmul makes with a workspace of ``ws_bytes`` (host-side query):
    ``{"kernel", "lds_bytes", "workspace_bytes"}``; raises W4Error as the matmul would."""
    m = mode_id(mode)
    desc = W4Desc(N, K, m, int(group) if m == MODE_GROUPWISE else 0)
    out = _lib.W4MmPlan()
    _lib.check(lib().w4a16_mm_plan(M, ctypes.byref(desc), 1 if transposed else 0, ws_bytes, ctypes.byref(out)))
    return {"kernel": out.kernel.decode(), "lds_bytes": int(out.lds_bytes), "workspace_bytes": int(out.workspace_bytes)}
