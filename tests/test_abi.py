"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-only entry points and argument validation behave
as documented (no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import gemv_int4_quantize_amd as w4
from gemv_int4_quantize_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "w4a16.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(w4\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = w4.lib()
    names = _declared()
    assert len(names) >= 9
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert _lib.lib().w4_version().decode().startswith("w4a16-gfx950")
    for code, name in [(0, "W4_OK"), (-1, "W4_ERR_INVALID"), (-2, "W4_ERR_UNSUPPORTED"), (-3, "W4_ERR_ALIGN"),
                       (-4, "W4_ERR_RESOURCE"), (-5, "W4_ERR_LAUNCH")]:
        assert _lib.status_string(code) == name


def _pairs(N, K, mode, g=0):
    out = ctypes.c_int64(-1)
    st = _lib.lib().w4_meta_pairs(ctypes.byref(_lib.W4Desc(N, K, mode, g)), ctypes.byref(out))
    return st, out.value


def test_meta_pairs():
    assert _pairs(128256, 2048, _lib.MODE_GLOBAL) == (0, 1)
    assert _pairs(128256, 2048, _lib.MODE_ROWWISE) == (0, 128256)
    assert _pairs(128256, 2048, _lib.MODE_GROUPWISE, 16) == (0, 128256 * 128)
    assert _pairs(4096, 11008, _lib.MODE_GROUPWISE, 64) == (0, 4096 * 172)


@pytest.mark.parametrize("N,K,mode,g,why", [
    (0, 64, 1, 0, "N = 0"),
    (4, 12, 1, 0, "K not a multiple of 8"),
    (4, 64, 2, 24, "group not a power of two"),
    (4, 64, 2, 8, "group below 16"),
    (4, 64, 2, 128, "group larger than K"),
    (4, 96, 2, 64, "group does not divide K"),
    (4, 8192, 2, 8192, "group above 4096"),
    (4, 64, 7, 0, "unknown mode"),
])
def test_invalid_descriptors(N, K, mode, g, why):
    st, _ = _pairs(N, K, mode, g)
    assert st == _lib.W4_ERR_INVALID, why
    assert _lib.last_error()


def test_workspace_bytes():
    L = _lib.lib()
    b = ctypes.c_size_t(123)
    d = _lib.W4Desc(1024, 2048, _lib.MODE_GLOBAL, 0)
    assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_QUANTIZE, 0, ctypes.byref(b)) == 0 and b.value > 0
    d = _lib.W4Desc(1024, 2048, _lib.MODE_GROUPWISE, 128)
    assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_QUANTIZE, 0, ctypes.byref(b)) == 0 and b.value == 0
    assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM, 4, ctypes.byref(b)) == 0 and b.value == 0
    # a GEMM with few output tiles plans a split-K over fp32 partial planes [S][M][out]
    d = _lib.W4Desc(4096, 4096, _lib.MODE_GROUPWISE, 128)
    for op, name in ((_lib.OP_MM, "gemm_nt_"), (_lib.OP_MM_T, "gemm_t_")):
        assert L.w4_workspace_bytes(ctypes.byref(d), op, 64, ctypes.byref(b)) == 0
        k = w4.kernel_for(64, 4096, 4096, "groupwise", 128, transposed=op == _lib.OP_MM_T)
        assert k.startswith(name) and "_splitk" in k
        S = int(k.rsplit("_splitk", 1)[1])
        assert S >= 2 and b.value == S * 64 * 4096 * 4
        # enough output tiles: no split, no workspace
        assert L.w4_workspace_bytes(ctypes.byref(d), op, 8192, ctypes.byref(b)) == 0 and b.value == 0
        assert "_splitk" not in w4.kernel_for(8192, 4096, 4096, "groupwise", 128, transposed=op == _lib.OP_MM_T)
    assert L.w4_workspace_bytes(ctypes.byref(d), 99, 4, ctypes.byref(b)) == _lib.W4_ERR_INVALID
    # the mid-M kernel (5 <= M <= 32, forward) splits rows longer than one block covers
    # (64 units of 128 columns at M <= 16, 32 at M <= 32) over planes [S][M][N]
    d = _lib.W4Desc(4096, 16384, _lib.MODE_GROUPWISE, 128)
    for M, S in ((16, 2), (32, 4)):
        assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM, M, ctypes.byref(b)) == 0
        assert w4.kernel_for(M, 4096, 16384, "groupwise", 128) == f"skinny_m{16 if M <= 16 else 32}_splitk{S}"
        assert b.value == S * M * 4096 * 4
    d = _lib.W4Desc(4096, 8192, _lib.MODE_GROUPWISE, 128)
    assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM, 8, ctypes.byref(b)) == 0 and b.value == 0
    # a partial last round: whole rounds of tile columns unsplit, the last columns split
    # into compact planes [S][M][columns past the unsplit ones]
    d = _lib.W4Desc(4096, 11008, _lib.MODE_ROWWISE, 0)
    for M in (3072, 8192):  # dX [M][11008]: 128- or 256-column tiles, 11008 = 86 x 128 = 43 x 256
        assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM_T, M, ctypes.byref(b)) == 0
        k = w4.kernel_for(M, 4096, 11008, "rowwise", None, transposed=True)
        assert "_tail" in k and "_splitk" in k, k
        bn = int(k.split("_tail", 1)[0].rsplit("x", 1)[1])
        tail_cols = int(k.split("_tail", 1)[1].split("_", 1)[0])
        S = int(k.rsplit("_splitk", 1)[1])
        pw = 11008 - (11008 // bn - tail_cols) * bn
        assert 0 < tail_cols < 11008 // bn and S >= 2 and b.value == S * M * pw * 4


def _mm(A, M, packed, s, z, desc, transposed=0, bias=None, Y=1024):
    return _lib.lib().w4a16_mm(A, M, packed, s, z, ctypes.byref(desc), transposed, bias, Y, None, 0, None)


def test_mm_validation_before_launch():
    d = _lib.W4Desc(64, 128, _lib.MODE_GROUPWISE, 32)
    a16 = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    assert _mm(None, 4, a16, a16, a16, d) == _lib.W4_ERR_INVALID
    assert _mm(a16, -1, a16, a16, a16, d) == _lib.W4_ERR_INVALID
    assert _mm(ctypes.c_void_p(0x10008), 4, a16, a16, a16, d) == _lib.W4_ERR_ALIGN
    assert _mm(a16, 4, ctypes.c_void_p(0x10004), a16, a16, d) == _lib.W4_ERR_ALIGN
    assert _mm(a16, 4, a16, ctypes.c_void_p(0x10001), a16, d) == _lib.W4_ERR_ALIGN
    assert _mm(a16, 4, a16, a16, a16, d, Y=ctypes.c_void_p(0x10002)) == _lib.W4_ERR_ALIGN
    d40 = _lib.W4Desc(64, 40, _lib.MODE_ROWWISE, 0)
    assert _mm(a16, 4, a16, a16, a16, d40) == _lib.W4_ERR_UNSUPPORTED
    dn = _lib.W4Desc(60, 128, _lib.MODE_ROWWISE, 0)
    assert _mm(a16, 4, a16, a16, a16, dn, transposed=1) == _lib.W4_ERR_UNSUPPORTED
    # transposed: 32-bit buffer offsets bound N and K
    assert _mm(a16, 4, a16, a16, a16, _lib.W4Desc(1 << 22, 128, _lib.MODE_ROWWISE, 0), transposed=1) == \
        _lib.W4_ERR_UNSUPPORTED
    assert _mm(a16, 4, a16, a16, a16, _lib.W4Desc(64, (1 << 21) + 32, _lib.MODE_ROWWISE, 0), transposed=1) == \
        _lib.W4_ERR_UNSUPPORTED
    # M == 0 is a successful no-op and never touches the pointers
    assert _mm(a16, 0, a16, a16, a16, d) == _lib.W4_OK


def test_quantize_validation_before_launch():
    L = _lib.lib()
    a16 = ctypes.c_void_p(0x10000)
    d = _lib.W4Desc(64, 128, _lib.MODE_GROUPWISE, 32)
    q = L.w4_quantize_pack
    assert q(a16, 5, ctypes.byref(d), a16, a16, a16, None, 0, None) == _lib.W4_ERR_INVALID
    assert q(ctypes.c_void_p(0x10008), 1, ctypes.byref(d), a16, a16, a16, None, 0, None) == _lib.W4_ERR_ALIGN
    dg = _lib.W4Desc(64, 128, _lib.MODE_GLOBAL, 0)
    assert q(a16, 1, ctypes.byref(dg), a16, a16, a16, None, 0, None) == _lib.W4_ERR_RESOURCE
    assert q(a16, 1, ctypes.byref(dg), a16, a16, a16, a16, 16, None) == _lib.W4_ERR_RESOURCE
    qz = L.w4_quantize_pack_zp
    assert qz(a16, 1, ctypes.byref(d), 7, a16, a16, a16, None, 0, None) == _lib.W4_ERR_INVALID
    assert qz(a16, 1, ctypes.byref(d), _lib.ZERO_INT, ctypes.c_void_p(0x10002), a16, a16, None, 0, None) == \
        _lib.W4_ERR_ALIGN
    dq = L.w4_dequantize
    assert dq(a16, a16, a16, ctypes.byref(d), a16, 7, None) == _lib.W4_ERR_INVALID
    assert dq(a16, a16, a16, ctypes.byref(d), ctypes.c_void_p(0x10004), _lib.DT_BF16, None) == _lib.W4_ERR_ALIGN


def test_dispatch_names():
    # decode shapes go to the GEMV, 5 <= M <= 32 forward to the mid-M kernel, prefill /
    # fine-tune shapes and the transposed mode to the MFMA GEMM
    for M in (1, 2, 3, 4):
        assert w4.kernel_for(M, 4096, 4096, "groupwise", 128) == f"gemv_m{M}"
    assert w4.kernel_for(5, 4096, 4096, "groupwise", 128) == "skinny_m16"
    assert w4.kernel_for(32, 4096, 4096, "groupwise", 128) == "skinny_m32"
    assert w4.kernel_for(33, 4096, 4096, "groupwise", 128).startswith("gemm_nt_")
    assert w4.kernel_for(2048, 12288, 4096, "rowwise", None).startswith("gemm_nt_")
    assert w4.kernel_for(2048, 12288, 4096, "groupwise", 64, transposed=True).startswith("gemm_t_")
    assert w4.kernel_for(4, 4096, 4096, "groupwise", 128, transposed=True).startswith("gemm_t_")
    assert w4.kernel_for(4, 4096, 40, "rowwise", None) is None


def test_mm_out_validation_before_launch():
    """w4a16_mm_out rejects bad output specifications before touching any pointer."""
    L = _lib.lib()
    d = _lib.W4Desc(64, 128, _lib.MODE_ROWWISE, 0)
    a16 = ctypes.c_void_p(0x10000)

    def call(segs, nsegs, dt=_lib.DT_BF16, M=4, bias=None, transposed=0, adt=_lib.DT_BF16):
        arr = (_lib.W4OutSeg * max(1, len(segs)))(*[_lib.W4OutSeg(*s) for s in segs]) if segs else None
        return L.w4a16_mm_out(a16, adt, M, a16, a16, a16, ctypes.byref(d), transposed, bias, dt, arr, nsegs,
                              None, 0, None)

    ok3 = [(0x20000, 32, 32), (0x30000, 16, 16), (0x40000, 16, 20)]
    assert call(ok3, 3, dt=7) == _lib.W4_ERR_INVALID                       # unknown dtype
    assert call(ok3, 3, adt=_lib.DT_F32) == _lib.W4_ERR_INVALID            # activations bf16 or fp16 only
    assert call(ok3, 0) == _lib.W4_ERR_INVALID                             # no segments
    assert call(ok3 + [(0x50000, 1, 1)] * 2, 5) == _lib.W4_ERR_INVALID     # more than four
    assert call([(0x20000, 32, 32), (0x30000, 16, 16)], 2) == _lib.W4_ERR_INVALID  # 48 != N
    assert call([(0x20000, 64, 63)], 1) == _lib.W4_ERR_INVALID             # ld < cols
    assert call([(0x20000, 0, 0), (0x30000, 64, 64)], 2) == _lib.W4_ERR_INVALID    # empty segment
    assert call([(0x20001, 64, 64)], 1) == _lib.W4_ERR_ALIGN               # bf16 output at an odd address
    assert call([(0x20002, 64, 64)], 1, dt=_lib.DT_F32) == _lib.W4_ERR_ALIGN  # fp32 needs 4 bytes
    assert call([(0x20000, 64, 64)], 1, bias=ctypes.c_void_p(0x60001)) == _lib.W4_ERR_ALIGN
    assert call([(None, 64, 64)], 1) == _lib.W4_ERR_INVALID                # NULL output
    # M == 0: structure still checked, pointers never touched
    assert call([(None, 64, 64)], 1, M=0) == _lib.W4_OK
    assert call([(None, 32, 32)], 1, M=0) == _lib.W4_ERR_INVALID


def test_mm_plan_follows_the_launch():
    """w4a16_mm_plan reports the launch a matmul makes for a given workspace: the split
    plan and its bytes only when the workspace holds them, the unsplit tile otherwise."""
    L = _lib.lib()
    for t, name in ((False, "gemm_nt_"), (True, "gemm_t_")):
        d = _lib.W4Desc(4096, 4096, _lib.MODE_GROUPWISE, 128)
        need = ctypes.c_size_t(0)
        assert L.w4_workspace_bytes(ctypes.byref(d), _lib.OP_MM_T if t else _lib.OP_MM, 64, ctypes.byref(need)) == 0
        full = w4.mm_plan(64, 4096, 4096, "groupwise", 128, transposed=t, ws_bytes=need.value)
        assert full["kernel"] == w4.kernel_for(64, 4096, 4096, "groupwise", 128, transposed=t)
        assert "_splitk" in full["kernel"] and full["workspace_bytes"] == need.value
        for ws in (0, need.value - 1):
            p = w4.mm_plan(64, 4096, 4096, "groupwise", 128, transposed=t, ws_bytes=ws)
            assert p["kernel"].startswith(name) and "_splitk" not in p["kernel"] and p["workspace_bytes"] == 0
            assert 0 < p["lds_bytes"] <= 160 * 1024
    g = w4.mm_plan(4, 16384, 16384, "groupwise", 128)
    assert g["kernel"] == "gemv_m4" and g["workspace_bytes"] == 0 and 0 < g["lds_bytes"] <= 160 * 1024
    assert w4.mm_plan(0, 64, 64, "rowwise", None)["kernel"] == "none"
    with pytest.raises(w4.W4Error):
        w4.mm_plan(4, 64, 40, "rowwise", None)


def _forced_plan(cfg, M, N, K, transposed, ws):
    """The plan under W4A16_GEMM_CFG=cfg, queried in a fresh process (the override is read once)."""
    import json
    import subprocess
    import sys
    code = ("import json, sys; sys.path.insert(0, %r); import gemv_int4_quantize_amd as w4; "
            "print(json.dumps(w4.mm_plan(%d, %d, %d, 'rowwise', None, %r, %d)))"
            % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))), M, N, K, transposed, ws))
    env = dict(os.environ, W4A16_GEMM_CFG=str(cfg))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("cfg,name,transposed,N,K", [(0, "gemm_t_256x256", True, 4096, 4096),
                                                     (1, "gemm_t_256x128", True, 4096, 4096),
                                                     (5, "gemm_nt_lds_256x256", False, 64, (1 << 21) + 64)])
def test_forced_tile_footprint(cfg, name, transposed, N, K):
    """A tile forced through W4A16_GEMM_CFG is the one reported and launched, split or not,
    with its LDS footprint: two stages of (BM + BN) rows of BK + 8 bf16 values.  (The
    non-transposed LDS tile serves contractions longer than 2^21 only.)"""
    bm, bn = (int(v) for v in name.rsplit("_", 1)[1].split("x"))
    want = 2 * (bm + bn) * (64 + 8) * 2
    for M, ws in ((64, 1 << 30), (64, 0), (4096, 1 << 30)):
        p = _forced_plan(cfg, M, N, K, transposed, ws)
        assert p["kernel"].startswith(name), p
        assert p["lds_bytes"] == want, p
        assert (p["workspace_bytes"] > 0) == ("_splitk" in p["kernel"]), p


def test_layer_rejects_unsupported_output_dtypes():
    """The layer's out_dtype is fp32 (None), bfloat16 or float16; anything else is rejected
    on the host before any tensor is touched."""
    import torch
    with pytest.raises(ValueError):
        w4.w4a16_linear(torch.zeros(2, 64), None, out_dtype=torch.int8)
    with pytest.raises(ValueError):
        w4.W4A16Linear(None, out_dtype=torch.float64)
