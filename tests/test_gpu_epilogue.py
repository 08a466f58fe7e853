"""GPU parity of the matmul output epilogue: bf16 / fp16 outputs with a bias in the output
dtype, and one product written to several output segments (fused Q/K/V)."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_mm_close, assert_rounded_close, dev_bf16, dev_weight, host

pytestmark = pytest.mark.gpu

OMODE = {"rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _bias_in(b32: np.ndarray, dt: str) -> np.ndarray:
    """The synthetic fp32 bias as values representable in the output dtype (float64)."""
    if dt == "bf16":
        return O.bf16_bits_to_f64(O.bf16_rne_bits(b32))
    if dt == "f16":
        return b32.astype(np.float16).astype(np.float64)
    return b32.astype(np.float64)


def _dev_vec(v: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(v.astype(np.float32)).to(DEV).to(TDT[dt])


def _host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


# (M, N, K, transposed, expected kernel prefix)
CASES = [(1, 1000, 2048, False, "gemv_m1"), (3, 520, 4096, False, "gemv_m3"),
         (16, 1000, 4096, False, "skinny_m16"), (24, 520, 8192, False, "skinny_m32_splitk"),
         (200, 1000, 2048, False, "gemm_nt"), (96, 4096, 8192, False, "gemm_nt"),
         (256, 1000, 2048, True, "gemm_t"), (64, 2048, 4096, True, "gemm_t"),
         (1000, 4096, 4096, False, "gemm_nt"), (1000, 4096, 4096, True, "gemm_t")]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ci", range(len(CASES)), ids=[f"{c[0]}x{c[1]}x{c[2]}{'t' if c[3] else ''}" for c in CASES])
@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 64)], ids=["rowwise", "g64"])
def test_output_dtype_and_bias(dt, ci, mode, g):
    M, N, K, tr, kern = CASES[ci]
    print(f"[case] epilogue {dt} M={M} N={N} K={K} t={tr} {mode}{g or ''}", flush=True)
    w = synth.weight(720, ci, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    assert w4.kernel_for(M, N, K, mode, g, tr).startswith(kern)
    outc = K if tr else N
    a = synth.activations_bf16(720, ci, M, N if tr else K)
    b = _bias_in(synth.bias_f32(720, ci, outc), dt)
    y = w4.mm(dev_bf16(a), qw, transposed=tr, bias=_dev_vec(b, dt), out_dtype=TDT[dt])
    assert y.dtype == TDT[dt] and y.shape == (M, outc)
    ref64 = O.matmul(a, *ref, K, tr, bias=b)
    assert_rounded_close(_host64(y), ref64, dt, f"{dt} {mode} M={M} t={tr}")
    # invariant: the rounding happens once, on the fp32 epilogue value the same kernel
    # computes (same plan, same summation order): out == dt(fp32 output with the same bias)
    y32 = w4.mm(dev_bf16(a), qw, transposed=tr, bias=_dev_vec(b, "f32"))
    assert torch.equal(y, y32.to(TDT[dt]))


@pytest.mark.parametrize("M", [1, 4, 16, 130, 512])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_qkv_segments(M, dt):
    """One launch over a fused Q/K/V weight writes Q, K and V to separate tensors."""
    K = 2048
    sizes = (1024, 256, 256)
    ws_ = [synth.weight(721, i, n, K, "bf16", tensor_id=synth.T_Q + i) for i, n in enumerate(sizes)]
    parts = [O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, 128) for w in ws_]
    fused = w4.quantize_fused([dev_weight(w, "bf16") for w in ws_], "groupwise", 128)
    x = synth.activations_bf16(721, M, M, K)
    b = _bias_in(synth.bias_f32(721, M, sum(sizes)), dt)
    outs = [torch.empty((M, n), dtype=TDT[dt], device=DEV) for n in sizes]
    w4.mm_split(dev_bf16(x), fused, outs, bias=_dev_vec(b, dt))
    offs = np.cumsum((0,) + sizes)
    for i, (o, p) in enumerate(zip(outs, parts)):
        ref64 = O.matmul(x, *p, K, bias=b[offs[i]:offs[i + 1]])
        if dt == "f32":
            assert_mm_close(host(o), ref64, f"segment {i} M={M}")
        else:
            assert_rounded_close(_host64(o), ref64, dt, f"segment {i} M={M}")
    # invariant: the segments are exactly the column slices of the single-output product
    whole = w4.mm(dev_bf16(x), fused, bias=_dev_vec(b, dt), out_dtype=TDT[dt])
    for i, o in enumerate(outs):
        assert torch.equal(o, whole[:, offs[i]:offs[i + 1]])


@pytest.mark.parametrize("M,tr", [(2, False), (24, False), (256, False), (128, True)])
def test_segments_into_strided_views(M, tr):
    """Segments with row strides wider than their columns (views into a padded buffer):
    every output lands in place and the padding is left untouched."""
    N, K = 768, 1024
    w = synth.weight(722, M, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), O.ROWWISE)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), "rowwise")
    outc = K if tr else N
    a = synth.activations_bf16(722, M, M, N if tr else K)
    cols = (outc // 4, outc // 2, outc - outc // 4 - outc // 2)
    pad = 40
    buf = torch.full((M, outc + 3 * pad), -7.25, dtype=torch.float32, device=DEV)
    views, c = [], 0
    for i, n in enumerate(cols):
        views.append(buf[:, c + (i + 1) * pad: c + (i + 1) * pad + n])
        c += n
    w4.mm_split(dev_bf16(a), qw, views, transposed=tr)
    ref64 = O.matmul(a, *ref, K, tr)
    got = np.concatenate([host(v) for v in views], axis=1)
    assert_mm_close(got, ref64, f"strided segments M={M} t={tr}")
    hb = host(buf)
    mask = np.ones(hb.shape, dtype=bool)
    c = 0
    for i, n in enumerate(cols):
        mask[:, c + (i + 1) * pad: c + (i + 1) * pad + n] = False
        c += n
    assert np.all(hb[mask] == -7.25)


@pytest.mark.parametrize("M,tr", [(300, False), (1024, False), (300, True), (1024, True)])
def test_fp32_output_layouts(M, tr):
    """An unsplit fp32 output is stored four columns at a time when its rows are 16-byte
    aligned (a lane-quad transpose of the MFMA result), else one value at a time.  Every
    layout gives the same bits as the contiguous output, with and without a bias, and
    leaves the memory around a view untouched."""
    N, K = 1024, 2048
    w = synth.weight(723, M, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), O.ROWWISE)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), "rowwise")
    outc = K if tr else N
    a_bits = synth.activations_bf16(723, M, M, N if tr else K)
    a = dev_bf16(a_bits)
    b32 = synth.bias_f32(723, M, outc)
    ref64 = O.matmul(a_bits, *ref, K, tr)
    for bias in (None, _dev_vec(b32, "f32")):
        want = w4.mm(a, qw, transposed=tr, bias=bias, split_k=False)
        bref = np.zeros(outc) if bias is None else b32.astype(np.float64)
        assert_mm_close(host(want), ref64 + bref, f"contiguous M={M} t={tr}")
        # (first column offset in floats, row stride): aligned rows with padding, a base one
        # float past alignment, and a row stride that is not a multiple of four
        for off, ld in ((4, outc + 8), (1, outc + 8), (0, outc + 1)):
            buf = torch.full((M, ld), -7.25, dtype=torch.float32, device=DEV)
            view = buf[:, off:off + outc]
            w4.mm_split(a, qw, [view], bias=bias, transposed=tr, split_k=False)
            assert torch.equal(view, want), (off, ld, bias is None)
            hb = host(buf)
            mask = np.ones(hb.shape, dtype=bool)
            mask[:, off:off + outc] = False
            assert np.all(hb[mask] == -7.25), (off, ld)
