"""The serialized packed-weight format (host only, no GPU): header layout against the
documented byte layout, validation of corrupted headers, and a save / load round trip of
oracle-made weights through CPU tensors."""

import ctypes
import struct

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gemv_int4_quantize_amd import _lib
import gemv_int4_quantize_amd as w4


def _up64(x):
    return (x + 63) // 64 * 64


def _expected_header(N, K, mode, g, zero_kind):
    """The 128-byte header written out from the format's documentation with struct."""
    pairs = 1 if mode == _lib.MODE_GLOBAL else N if mode == _lib.MODE_ROWWISE else N * (K // g)
    packed_off = _up64(128)
    packed_bytes = N * (K // 8) * 4
    meta = pairs * 2
    scales_off = _up64(packed_off + packed_bytes)
    zeros_off = _up64(scales_off + meta)
    total = _up64(zeros_off + meta)
    return struct.pack("<8sIIqqiiii6Q32s", b"W4A16PK\0", 1, 128, N, K, mode,
                       g if mode == _lib.MODE_GROUPWISE else 0, zero_kind, 0,
                       packed_off, packed_bytes, scales_off, zeros_off, meta, total, bytes(32))


@pytest.mark.parametrize("N,K,mode,g,zk", [(37, 4096, _lib.MODE_GROUPWISE, 128, 0), (5, 64, _lib.MODE_ROWWISE, 0, 1),
                                          (16, 1024, _lib.MODE_GLOBAL, 0, 0), (3, 8, _lib.MODE_ROWWISE, 0, 0)])
def test_layout_matches_documented_bytes(N, K, mode, g, zk):
    h = _lib.W4SerialHeader()
    assert _lib.lib().w4_serial_layout(ctypes.byref(_lib.W4Desc(N, K, mode, g)), zk, ctypes.byref(h)) == 0
    assert ctypes.sizeof(h) == 128
    assert bytes(h) == _expected_header(N, K, mode, g, zk)


def _oracle_weight(zero):
    w = synth.weight(740, 0, 24, 512, "f32")
    p, s, z = O.quantize_pack(w, O.GROUPWISE, 64, int_zero=(zero == "int"))
    return w4.QuantizedWeight(torch.from_numpy(p), torch.from_numpy(s), torch.from_numpy(z), 24, 512,
                              _lib.MODE_GROUPWISE, 64, zero)


@pytest.mark.parametrize("zero", ["fp16", "int"])
def test_round_trip(zero, tmp_path):
    qw = _oracle_weight(zero)
    path = str(tmp_path / "w.w4")
    w4.save(qw, path)
    back = w4.load(path, device="cpu")
    assert (back.N, back.K, back.mode, back.group, back.zero) == (qw.N, qw.K, qw.mode, qw.group, zero)
    for a, b in ((back.packed, qw.packed), (back.scales, qw.scales), (back.zeros, qw.zeros)):
        assert a.dtype == b.dtype and torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                                                  b.view(torch.int16) if b.dtype == torch.float16 else b)
    data = open(path, "rb").read()
    hdr = _lib.W4SerialHeader.from_buffer_copy(data[:128])
    # the packed section read as bytes is the INT8 packing of the same codes
    q = O.unpack(qw.packed.numpy())
    sec = np.frombuffer(data[hdr.packed_offset:hdr.packed_offset + hdr.packed_bytes], dtype=np.uint8)
    np.testing.assert_array_equal(sec.reshape(24, 256), O.pack_bytes(q))


def test_parse_rejects_corruption():
    data = bytearray(w4.serialize(_oracle_weight("fp16")))
    L = _lib.lib()

    def parse(b, n=None):
        d, z = _lib.W4Desc(), ctypes.c_int(0)
        buf = ctypes.create_string_buffer(bytes(b), len(b))
        return L.w4_serial_parse(buf, len(b) if n is None else n, ctypes.byref(d), ctypes.byref(z))

    assert parse(data) == _lib.W4_OK
    for off, val in ((0, 0x58), (8, 2), (12, 64), (40, 3), (48, 9), (64, 0x11), (112, 1)):
        bad = bytearray(data)
        bad[off] = val            # magic, version, header size, mode, zero kind, an offset, reserved
        assert parse(bad) == _lib.W4_ERR_INVALID, off
    assert parse(data, len(data) - 1) == _lib.W4_ERR_INVALID     # truncated
    assert parse(data[:100]) == _lib.W4_ERR_INVALID              # shorter than the header
