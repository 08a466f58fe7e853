"""The allocation-free matmul entry point (w4a16_mm_noalloc): through the C ABI, its
output equals w4a16_mm's with the workspace w4_workspace_bytes reports, bit for bit,
on calls in a row whose second input is smaller; a plan whose split-K planes exceed
the static scratch is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gemv_int4_quantize_amd import _lib
from gpu_helpers import DEV, assert_mm_close, dev_bf16, dev_f32, dev_weight, host

SCRATCH_BYTES = 64 << 20


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _ws_bytes(qw, M, transposed):
    b = ctypes.c_size_t(0)
    _lib.check(_lib.lib().w4_workspace_bytes(ctypes.byref(qw.desc()), _lib.OP_MM_T if transposed else _lib.OP_MM, M,
                                             ctypes.byref(b)))
    return b.value


def _both(a, qw, transposed, bias):
    """(w4a16_mm with its reported workspace, w4a16_mm_noalloc) outputs of one product."""
    L = _lib.lib()
    M = a.shape[0]
    outc = qw.K if transposed else qw.N
    ws_bytes = _ws_bytes(qw, M, transposed)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    y_ref = torch.full((M, outc), float("nan"), device=DEV)
    y_na = torch.full((M, outc), float("nan"), device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    d = qw.desc()
    _lib.check(L.w4a16_mm(_ptr(a), M, _ptr(qw.packed), _ptr(qw.scales), _ptr(qw.zeros), ctypes.byref(d),
                          int(transposed), _ptr(bias), _ptr(y_ref), _ptr(ws), ws_bytes, st))
    _lib.check(L.w4a16_mm_noalloc(_ptr(a), M, _ptr(qw.packed), _ptr(qw.scales), _ptr(qw.zeros), ctypes.byref(d),
                                  int(transposed), _ptr(bias), _ptr(y_na), st))
    torch.cuda.synchronize()
    return y_ref, y_na, ws_bytes


# calls in a row, each smaller than the one before (scratch planes 4, 4, 3, 0.5 (the mid-M
# kernel's split) and 0.375 MiB, then none)
CALLS = [(64, 4096, 4096, "groupwise", 128, True), (64, 4096, 4096, "groupwise", 128, False),
         (33, 3000, 8192, "groupwise", 256, False), (16, 4096, 16384, "groupwise", 128, False),
         (24, 2048, 2048, "rowwise", None, True), (3, 1000, 2048, "groupwise", 128, False)]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    for i, (M, N, K, mode, g, t) in enumerate(CALLS):
        print(f"[case] noalloc M={M} N={N} K={K} {mode}{g or ''} t={t}", flush=True)
        w = synth.weight(714, i, N, K, "bf16")
        ref = O.quantize_pack(O.to_f32(w, "bf16"), {"rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}[mode], g)
        qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
        a = synth.activations_bf16(714, i, M, N if t else K)
        bias = synth.bias_f32(714, i, K if t else N)
        y_ref, y_na, ws_bytes = _both(dev_bf16(a), qw, t, dev_f32(bias))
        assert ws_bytes <= SCRATCH_BYTES
        assert (ws_bytes > 0) == (i < 5), (i, ws_bytes)
        assert torch.equal(y_ref, y_na), f"call {i}: noalloc differs from w4a16_mm"
        assert_mm_close(host(y_na), O.matmul(a, *ref, K, t, bias), f"noalloc call {i}")


def test_noalloc_refuses_planes_past_the_scratch():
    """Host-side refusal: no pointer is touched and nothing is enqueued."""
    L = _lib.lib()
    M, N, K = 768, 16384, 32768  # a split-K plan with 192 MiB of partial planes
    d = _lib.W4Desc(N, K, _lib.MODE_ROWWISE, 0)
    b = ctypes.c_size_t(0)
    assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM, M, ctypes.byref(b)) == 0
    if b.value <= SCRATCH_BYTES:
        pytest.skip("the planner no longer splits this shape past the scratch")
    a16 = ctypes.c_void_p(0x10000)
    st = L.w4a16_mm_noalloc(a16, M, a16, a16, a16, ctypes.byref(d), 0, None, a16, None)
    assert st == _lib.W4_ERR_RESOURCE
    assert "static scratch" in _lib.last_error()
    # argument checks come first, as for w4a16_mm
    assert L.w4a16_mm_noalloc(None, M, a16, a16, a16, ctypes.byref(d), 0, None, a16, None) == _lib.W4_ERR_INVALID
    assert L.w4a16_mm_noalloc(a16, 0, a16, a16, a16, ctypes.byref(d), 0, None, a16, None) == _lib.W4_OK
