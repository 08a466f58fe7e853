"""ctypes view of the C ABI in include/w4a16.h (libw4a16.so, built in-tree).

Loading fails loudly when the library is missing: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")

W4_OK = 0
W4_ERR_INVALID = -1
W4_ERR_UNSUPPORTED = -2
W4_ERR_ALIGN = -3
W4_ERR_RESOURCE = -4
W4_ERR_LAUNCH = -5

MODE_GLOBAL, MODE_ROWWISE, MODE_GROUPWISE = 0, 1, 2
DT_F32, DT_F16, DT_BF16 = 0, 1, 2
OP_QUANTIZE, OP_MM, OP_MM_T, OP_DEQUANTIZE = 0, 1, 2, 3
ZERO_FP16, ZERO_INT = 0, 1

# every entry point declared in include/w4a16.h
EXPORTS = (
    "w4_meta_pairs", "w4_workspace_bytes", "w4_quantize_pack", "w4_quantize_pack_zp", "w4_dequantize", "w4a16_mm",
    "w4a16_mm_out", "w4a16_mm_noalloc", "w4a16_mm_kernel", "w4a16_mm_plan", "w4_serial_layout", "w4_serial_parse",
    "w4_status_string", "w4_last_error", "w4_version",
)


class W4Desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("mode", ctypes.c_int32), ("group", ctypes.c_int32)]


class W4OutSeg(ctypes.Structure):
    _fields_ = [("Y", ctypes.c_void_p), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64)]


class W4MmPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("lds_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


class W4SerialHeader(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_char * 8), ("version", ctypes.c_uint32), ("header_bytes", ctypes.c_uint32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("mode", ctypes.c_int32), ("group", ctypes.c_int32),
                ("zero_kind", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("packed_offset", ctypes.c_uint64), ("packed_bytes", ctypes.c_uint64),
                ("scales_offset", ctypes.c_uint64), ("zeros_offset", ctypes.c_uint64), ("meta_bytes", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64), ("reserved", ctypes.c_uint8 * 32)]


class W4Error(RuntimeError):
    """A negative status returned by the library, with its detail message."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4a16.so once (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m gemv_int4_quantize_amd.build` "
                          "(the W4A16 ops have no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    pdesc = ctypes.POINTER(W4Desc)
    L.w4_meta_pairs.argtypes = [pdesc, ctypes.POINTER(ctypes.c_int64)]
    L.w4_workspace_bytes.argtypes = [pdesc, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    L.w4_quantize_pack.argtypes = [vp, i32, pdesc, vp, vp, vp, vp, sz, vp]
    L.w4_quantize_pack_zp.argtypes = [vp, i32, pdesc, i32, vp, vp, vp, vp, sz, vp]
    L.w4_dequantize.argtypes = [vp, vp, vp, pdesc, vp, i32, vp]
    L.w4a16_mm.argtypes = [vp, i64, vp, vp, vp, pdesc, i32, vp, vp, vp, sz, vp]
    L.w4a16_mm_noalloc.argtypes = [vp, i64, vp, vp, vp, pdesc, i32, vp, vp, vp]
    L.w4a16_mm_out.argtypes = [vp, i32, i64, vp, vp, vp, pdesc, i32, vp, i32, ctypes.POINTER(W4OutSeg), i32, vp, sz,
                               vp]
    L.w4_serial_layout.argtypes = [pdesc, i32, ctypes.POINTER(W4SerialHeader)]
    L.w4_serial_parse.argtypes = [vp, sz, pdesc, ctypes.POINTER(ctypes.c_int)]
    L.w4a16_mm_kernel.argtypes = [i64, pdesc, i32]
    L.w4a16_mm_kernel.restype = ctypes.c_char_p
    L.w4a16_mm_plan.argtypes = [i64, pdesc, i32, sz, ctypes.POINTER(W4MmPlan)]
    L.w4_status_string.argtypes = [i32]
    L.w4_status_string.restype = ctypes.c_char_p
    L.w4_last_error.argtypes = []
    L.w4_last_error.restype = ctypes.c_char_p
    L.w4_version.argtypes = []
    L.w4_version.restype = ctypes.c_char_p
    for name in ("w4_meta_pairs", "w4_workspace_bytes", "w4_quantize_pack", "w4_quantize_pack_zp", "w4_dequantize",
                 "w4a16_mm", "w4a16_mm_out", "w4a16_mm_noalloc", "w4a16_mm_plan", "w4_serial_layout",
                 "w4_serial_parse"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().w4_status_string(status).decode()


def last_error() -> str:
    return lib().w4_last_error().decode()


def check(status: int) -> None:
    """Raise W4Error for a negative status."""
    if status != W4_OK:
        raise W4Error(status, last_error())
