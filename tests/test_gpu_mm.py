"""GPU parity of the W4A16 matmul (GEMV and MFMA GEMM, both directions) against the oracle."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import (DEV, ELEM_ATOL, ELEM_RTOL, assert_mm_close, assert_quant_equal, dev_bf16, dev_f32,
                         dev_weight, host, oracle_rows_global)

pytestmark = pytest.mark.gpu

OMODE = {"global": O.GLOBAL, "rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}


def _setup(cfg, idx, N, K, mode, g, wdtype="bf16"):
    w = synth.weight(cfg, idx, N, K, wdtype)
    w32 = O.to_f32(w, wdtype)
    ref = O.quantize_pack(w32, OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, wdtype), mode, g)
    return w32, ref, qw


# ------------------------------------------------------------------ small shapes, every mode


SMALL_MODES = [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 32), ("groupwise", 64),
               ("groupwise", 128), ("groupwise", 2048)]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("mode,g", SMALL_MODES, ids=[f"{m}{g or ''}" for m, g in SMALL_MODES])
@pytest.mark.parametrize("N,K", [(37, 2048), (300, 4096), (64, 11008)])
def test_gemv_small(M, mode, g, N, K):
    if g is not None and K % g:
        pytest.skip("group does not divide K")
    print(f"[case] gemv M={M} N={N} K={K} mode={mode} g={g}", flush=True)
    _, ref, qw = _setup(700, N + K, N, K, mode, g)
    x = synth.activations_bf16(700, N + K, M, K)
    bias = synth.bias_f32(700, N + K, N) if M % 2 else None
    assert w4.kernel_for(M, N, K, mode, g) == f"gemv_m{M}"
    y = w4.mm(dev_bf16(x), qw, bias=None if bias is None else dev_f32(bias))
    assert_mm_close(host(y), O.matmul(x, *ref, K, bias=bias), f"gemv M={M} {mode}{g}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("mode,g", [("groupwise", 128), ("rowwise", None), ("groupwise", 16)],
                         ids=["groupwise128", "rowwise", "groupwise16"])
def test_gemv_long_k(M, mode, g):
    """K long enough that X is staged into LDS in several phases (K = 47104 + 1024 ragged)."""
    N, K = 300, 48128
    print(f"[case] gemv long K M={M} N={N} K={K} mode={mode} g={g}", flush=True)
    _, ref, qw = _setup(707, M, N, K, mode, g)
    x = synth.activations_bf16(707, M, M, K)
    bias = synth.bias_f32(707, M, N)
    assert w4.kernel_for(M, N, K, mode, g) == f"gemv_m{M}"
    y = w4.mm(dev_bf16(x), qw, bias=dev_f32(bias))
    assert_mm_close(host(y), O.matmul(x, *ref, K, bias=bias), f"gemv long K M={M} {mode}{g}")


GEMM_MODES = [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 64), ("groupwise", 256)]


@pytest.mark.parametrize("M", [5, 17, 128, 129, 300])
@pytest.mark.parametrize("mode,g", GEMM_MODES, ids=[f"{m}{g or ''}" for m, g in GEMM_MODES])
@pytest.mark.parametrize("transposed", [False, True], ids=["nt", "t"])
def test_gemm_small(M, mode, g, transposed):
    N, K = 264, 1024  # ragged against every tile size in both directions
    print(f"[case] gemm M={M} N={N} K={K} mode={mode} g={g} t={transposed}", flush=True)
    _, ref, qw = _setup(701, M, N, K, mode, g)
    a = synth.activations_bf16(701, M, M, N if transposed else K)
    bias = synth.bias_f32(701, M, K if transposed else N)
    y = w4.mm(dev_bf16(a), qw, transposed=transposed, bias=dev_f32(bias))
    assert_mm_close(host(y), O.matmul(a, *ref, K, transposed, bias), f"gemm M={M} {mode}{g} t={transposed}")


# (g, K): the forward kernel's wide scale / zero loads cover 2, 4 or 8 contraction steps
# depending on g and on K modulo 128 / 256 / 512
WIDE_META_CASES = [(32, 1024), (32, 1152), (64, 1024), (64, 1280), (64, 1152), (128, 1536), (128, 1152)]


@pytest.mark.parametrize("g,K", WIDE_META_CASES, ids=[f"g{g}-K{K}" for g, K in WIDE_META_CASES])
def test_gemm_wide_meta_spans(g, K):
    M, N = 160, 264
    print(f"[case] gemm wide meta M={M} N={N} K={K} g={g}", flush=True)
    _, ref, qw = _setup(709, g + K, N, K, "groupwise", g)
    a = synth.activations_bf16(709, g + K, M, K)
    bias = synth.bias_f32(709, g + K, N)
    for split in (True, False):
        y = w4.mm(dev_bf16(a), qw, bias=dev_f32(bias), split_k=split)
        assert_mm_close(host(y), O.matmul(a, *ref, K, False, bias), f"wide meta g={g} K={K} split={split}")


@pytest.mark.parametrize("M", [2, 8, 200])
@pytest.mark.parametrize("transposed", [False, True], ids=["nt", "t"])
def test_onehot_exact(M, transposed):
    """A one-hot activation row selects one dequantized weight row or column exactly (bit-exact)."""
    N, K = 136, 512
    _, ref, qw = _setup(702, M, N, K, "groupwise", 32)
    wd = O.bf16_bits_to_f64(O.dequantize_bf16_bits(*ref, K))
    L = N if transposed else K
    a = np.zeros((M, L), dtype=np.uint16)
    hot = [(m * 37 + 5) % L for m in range(M)]
    for m in range(M):
        a[m, hot[m]] = 0x3F80
    y = host(w4.mm(dev_bf16(a), qw, transposed=transposed)).astype(np.float64)
    for m in range(M):
        want = wd[hot[m], :] if transposed else wd[:, hot[m]]
        np.testing.assert_array_equal(y[m], want)


def test_single_matmul_case():
    """X bf16 [4][2048], W fp32 [2048][2048] ~ N(0, 0.02), groupwise g=128, seed 0."""
    x, w = synth.single_matmul_case()
    ref = O.quantize_pack(w, O.GROUPWISE, 128)
    qw = w4.quantize_pack(dev_weight(w, "f32"), "groupwise", 128)
    y = w4.mm(dev_bf16(x), qw)
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what="single matmul")
    assert_mm_close(host(y), O.matmul(x, *ref, 2048), "single matmul")


def test_deterministic_and_empty():
    N, K = 512, 2048
    _, ref, qw = _setup(703, 0, N, K, "groupwise", 128)
    for M, t in [(3, False), (256, False), (256, True)]:
        a = dev_bf16(synth.activations_bf16(703, M, M, N if t else K))
        y1 = w4.mm(a, qw, transposed=t)
        y2 = w4.mm(a, qw, transposed=t)
        assert torch.equal(y1, y2)
    e = w4.mm(torch.empty((0, K), dtype=torch.bfloat16, device=DEV), qw)
    assert e.shape == (0, N)


def test_bias_on_minus_off():
    N, K, M = 384, 2048, 130
    _, ref, qw = _setup(704, 0, N, K, "rowwise", None)
    x = dev_bf16(synth.activations_bf16(704, 1, M, K))
    b = synth.bias_f32(704, 2, N)
    d = host(w4.mm(x, qw, bias=dev_f32(b))).astype(np.float64) - host(w4.mm(x, qw)).astype(np.float64)
    assert np.allclose(d, np.broadcast_to(b.astype(np.float64), d.shape), rtol=0, atol=2e-6)


def test_fused_qkv_equivalence():
    """One fused QKV operand equals separate Q, K, V in both directions."""
    K = 1024
    sizes = (512, 256, 256)
    ws = [synth.weight(705, i, n, K, "bf16", tensor_id=synth.T_Q + i) for i, n in enumerate(sizes)]
    for mode, g in [("rowwise", None), ("groupwise", 64)]:
        fused = w4.quantize_fused([dev_weight(w, "bf16") for w in ws], mode, g)
        parts = [w4.quantize_pack(dev_weight(w, "bf16"), mode, g) for w in ws]
        for M in (4, 256):
            x = dev_bf16(synth.activations_bf16(705, M, M, K))
            yf = host(w4.mm(x, fused))
            ys = np.concatenate([host(w4.mm(x, p)) for p in parts], axis=1)
            assert_mm_close(yf, ys, f"fused NT {mode} M={M}")
            dy = synth.activations_bf16(705, M + 1, M, sum(sizes))
            dxf = host(w4.mm(dev_bf16(dy), fused, transposed=True))
            offs = np.cumsum((0,) + sizes)
            dxs = sum(host(w4.mm(dev_bf16(np.ascontiguousarray(dy[:, offs[i]:offs[i + 1]])), parts[i],
                                 transposed=True)).astype(np.float64) for i in range(3))
            assert_mm_close(dxf, dxs, f"fused T {mode} M={M}")


SHORT_M_CASES = [(8, 4096, 2048, False, "skinny_m16"), (40, 4096, 2048, False, "gemm_nt_32x128"),
                 (96, 8192, 4096, False, "gemm_nt_64x128"), (24, 8192, 2048, True, "gemm_t_32x128"),
                 (64, 12288, 4096, True, "gemm_t_32x128")]


@pytest.mark.parametrize("ci", range(len(SHORT_M_CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{'t' if c[3] else 'nt'}" for c in SHORT_M_CASES])
def test_short_m_tiles(ci):
    """5 <= M < 128 runs the mid-M kernel (forward, M <= 32) or the 32- and 64-row tiles (with
    split-K); parity with the oracle."""
    M, N, K, t, name = SHORT_M_CASES[ci]
    print(f"[case] short M={M} N={N} K={K} t={t}", flush=True)
    assert w4.kernel_for(M, N, K, "groupwise", 128, transposed=t).startswith(name)
    _, ref, qw = _setup(708, ci, N, K, "groupwise", 128)
    a = synth.activations_bf16(708, ci, M, N if t else K)
    bias = synth.bias_f32(708, ci, K if t else N)
    y = w4.mm(dev_bf16(a), qw, transposed=t, bias=dev_f32(bias))
    assert_mm_close(host(y), O.matmul(a, *ref, K, t, bias), f"short M {ci}")


# (M, N, K, mode, g, f16, epi): every M block count, both units-per-wave forms, one-group and
# two-group lane chunks (g = 16), ragged rows (N % 16), a ragged last unit (K % 128), idle
# waves (K / 128 < 16 units or a short last split), splits of 2, 3 and 4, fp16 activations and
# the bf16-output epilogue with a bf16 bias
MIDM_CASES = [(5, 264, 1024, "groupwise", 16, False, False), (8, 300, 4096, "groupwise", 128, False, False),
              (13, 37, 2080, "groupwise", 32, False, True), (16, 1000, 4128, "rowwise", None, True, False),
              (17, 264, 1056, "global", None, False, True), (24, 520, 8192, "groupwise", 64, True, True),
              (32, 4104, 16384, "groupwise", 256, False, False), (32, 48, 11040, "groupwise", 32, False, True),
              (7, 130, 256, "groupwise", 256, False, False), (31, 2056, 4096, "groupwise", 16, True, False)]


@pytest.mark.parametrize("ci", range(len(MIDM_CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4] or ''}" for c in MIDM_CASES])
def test_mid_m_kernel(ci):
    """5 <= M <= 32, forward: the mid-M kernel matches the oracle on every output and is
    deterministic; so does the launch without a workspace (the mid-M kernel unsplit when a
    row fits one block, else the tiles)."""
    M, N, K, mode, g, f16, epi = MIDM_CASES[ci]
    print(f"[case] mid-M M={M} N={N} K={K} {mode}{g or ''} f16={f16} epi={epi}", flush=True)
    assert w4.kernel_for(M, N, K, mode, g).startswith("skinny_m16" if M <= 16 else "skinny_m32")
    _, ref, qw = _setup(713, ci, N, K, mode, g)
    a = synth.activations_bf16(713, ci, M, K)
    if f16:
        a = O.bf16_bits_to_f64(a).astype(np.float16).view(np.uint16)  # the bf16 draw, rounded to fp16
        ad = torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.float16)
    else:
        ad = dev_bf16(a)
    kw = {}
    if epi:
        bias = O.bf16_bits_to_f64(O.bf16_rne_bits(synth.bias_f32(713, ci, N)))
        kw = dict(bias=torch.from_numpy(bias.astype(np.float32)).to(DEV).to(torch.bfloat16), out_dtype=torch.bfloat16)
    else:
        bias = synth.bias_f32(713, ci, N)
        kw = dict(bias=dev_f32(bias))
    want = O.matmul(a, *ref, K, bias=bias, a_dtype="f16" if f16 else "bf16")
    y1 = w4.mm(ad, qw, **kw)
    assert torch.equal(y1, w4.mm(ad, qw, **kw))
    y0 = w4.mm(ad, qw, split_k=False, **kw)
    for y, what in ((y1, "split"), (y0, "unsplit")):
        got = host(y.float()).astype(np.float64)
        if epi:
            w_ = O.round_output(want, "bf16")
            bad = np.abs(got - w_) > ELEM_RTOL * np.abs(w_) + ELEM_ATOL + np.abs(w_) * 2.0**-7
            assert not bad.any(), f"{int(bad.sum())} elements outside the bound, mid-M case {ci} {what}"
        else:
            assert_mm_close(got, want, f"mid-M {ci} {what}")


SPLITK_CASES = [(64, 4104, 4096, True, "groupwise", 128), (64, 4096, 4128, False, "groupwise", 32),
                (160, 4096, 4096, False, "rowwise", None), (300, 2056, 4096, True, "groupwise", 64),
                (96, 8200, 2048, True, "global", None), (33, 3000, 8192, False, "groupwise", 256)]


@pytest.mark.parametrize("ci", range(len(SPLITK_CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{'t' if c[3] else 'nt'}" for c in SPLITK_CASES])
def test_splitk_gemm(ci):
    """Few output tiles: the contraction is split over a workspace (ragged last slice
    included); the result matches the oracle, is deterministic, and agrees with the
    unsplit launch."""
    M, N, K, t, mode, g = SPLITK_CASES[ci]
    print(f"[case] splitk M={M} N={N} K={K} t={t} {mode}{g or ''}", flush=True)
    assert "_splitk" in w4.kernel_for(M, N, K, mode, g, transposed=t)
    _, ref, qw = _setup(706, ci, N, K, mode, g)
    a = synth.activations_bf16(706, ci, M, N if t else K)
    bias = synth.bias_f32(706, ci, K if t else N)
    ad, bd = dev_bf16(a), dev_f32(bias)
    y1 = w4.mm(ad, qw, transposed=t, bias=bd)
    y2 = w4.mm(ad, qw, transposed=t, bias=bd)
    y0 = w4.mm(ad, qw, transposed=t, bias=bd, split_k=False)
    assert torch.equal(y1, y2)
    want = O.matmul(a, *ref, K, t, bias)
    assert_mm_close(host(y1), want, f"splitk {ci}")
    assert_mm_close(host(y0), want, f"unsplit {ci}")


TAIL_CASES = [(1536, 2048, 11008, True, "rowwise", None, False), (1536, 11008, 2048, False, "rowwise", None, True),
              (768, 2048, 11008, True, "groupwise", 64, True), (1536, 11008, 2048, False, "groupwise", 128, False)]


@pytest.mark.parametrize("ci", range(len(TAIL_CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{'t' if c[3] else 'nt'}{c[4]}" for c in TAIL_CASES])
def test_split_tail_gemm(ci):
    """A partial last round of workgroups: the whole-round tile columns run unsplit and the
    rest with a split contraction (compact partial planes, reduction over the tail columns
    through the epilogue).  Sampled rows match the oracle, with fp32 bias and bf16 output
    in two cases; results are deterministic; the unsplit launch matches too."""
    M, N, K, t, mode, g, epi = TAIL_CASES[ci]
    print(f"[case] split tail M={M} N={N} K={K} t={t} {mode}{g or ''} epi={epi}", flush=True)
    assert "_tail" in w4.kernel_for(M, N, K, mode, g, transposed=t)
    w = synth.weight(707, ci, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    wdq = O.bf16_bits_to_f64(O.dequantize_bf16_bits(*ref, K))
    outc = K if t else N
    a = synth.activations_bf16(707, ci, M, N if t else K)
    # bias in the output dtype: bf16 values (as float64 for the oracle)
    bias = O.bf16_bits_to_f64(O.bf16_rne_bits(synth.bias_f32(707, ci, outc))) if epi else None
    ad = dev_bf16(a)
    if epi:
        bd = torch.from_numpy(bias.astype(np.float32)).to(DEV)
        kw = dict(transposed=t, bias=bd.to(torch.bfloat16), out_dtype=torch.bfloat16)
    else:
        kw = dict(transposed=t)
    y1 = w4.mm(ad, qw, **kw)
    y2 = w4.mm(ad, qw, **kw)
    y0 = w4.mm(ad, qw, split_k=False, **kw)
    assert torch.equal(y1, y2)
    if epi:
        # the bf16 output is the fp32 epilogue value of the same plan, rounded once
        y32 = w4.mm(ad, qw, transposed=t, bias=bd)
        assert torch.equal(y1, y32.to(torch.bfloat16))
    ms = _edge_idx(M, np.random.default_rng(ci), 16)
    msd = torch.from_numpy(ms).to(DEV)
    want = O.bf16_bits_to_f64(a[ms]) @ (wdq if t else wdq.T)
    if epi:
        want = O.round_output(want + bias, "bf16")
    for y, what in ((y1, "tail"), (y0, "unsplit")):
        got = host(y[msd].float()).astype(np.float64)
        if epi:
            ulp = np.abs(want) * 2.0**-7
            bad = np.abs(got - want) > ELEM_RTOL * np.abs(want) + ELEM_ATOL + ulp
            assert not bad.any(), f"{int(bad.sum())} elements outside the bound, {what} {ci}"
        else:
            assert_mm_close(got, want, f"{what} {ci}")


EIGHT_WAVE_CASES = [  # (M, N, K, transposed, mode, g, fp16 activations, bf16 output with bias, expected kernel)
    (1500, 8200, 256, False, "groupwise", 16, False, False, "gemm_nt_256x256"),
    (1500, 8200, 2080, False, "groupwise", 32, False, True, "gemm_nt_256x256"),
    (300, 20000, 256, False, "groupwise", 64, True, False, "gemm_nt_128x256"),
    (300, 20000, 320, False, "global", None, False, True, "gemm_nt_128x256"),
    (1024, 4096, 11008, False, "rowwise", None, False, False, "gemm_nt_256x256_splitk4"),
    (700, 1024, 12320, True, "groupwise", 16, False, False, "gemm_t_w8_256x256"),
    (500, 8200, 2080, True, "groupwise", 32, True, True, "gemm_t_w8_256x256_splitk8"),
    (1000, 4104, 2080, True, "global", None, False, True, "gemm_t_w8_256x256_splitk4"),
]


@pytest.mark.parametrize("ci", range(len(EIGHT_WAVE_CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{'t' if c[3] else 'nt'}{c[4]}{c[5] or ''}" for c in EIGHT_WAVE_CASES])
def test_eight_wave_tiles(ci):
    """The tiles with eight waves on one workgroup's LDS tiles: forward 256 x 256 and
    128 x 256 (one activation tile across 256 output columns) and transposed 256 x 256 (2 x 4
    waves of 128 x 64).  Ragged M and output columns, a partial last contraction step, two
    groups per lane chunk (g = 16), a contraction that is not a whole number of 64-wide
    steps on the forward register route, fp16 activations, bf16 output with bias, split
    contractions.  Sampled rows (tile edges included) match the oracle; the results are
    deterministic."""
    M, N, K, t, mode, g, f16, epi, kern = EIGHT_WAVE_CASES[ci]
    print(f"[case] eight-wave M={M} N={N} K={K} t={t} {mode}{g or ''} f16={f16} epi={epi}", flush=True)
    assert w4.kernel_for(M, N, K, mode, g, transposed=t) == kern
    w = synth.weight(712, ci, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    outc = K if t else N
    a = synth.activations_bf16(712, ci, M, N if t else K)
    if f16:
        a = O.bf16_bits_to_f64(a).astype(np.float16).view(np.uint16)  # the bf16 draw, rounded to fp16
        ad = torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.float16)
    else:
        ad = dev_bf16(a)
    bias = O.bf16_bits_to_f64(O.bf16_rne_bits(synth.bias_f32(712, ci, outc))) if epi else None
    kw = dict(transposed=t)
    if epi:
        kw.update(bias=torch.from_numpy(bias.astype(np.float32)).to(DEV).to(torch.bfloat16), out_dtype=torch.bfloat16)
    y1 = w4.mm(ad, qw, **kw)
    assert torch.equal(y1, w4.mm(ad, qw, **kw))
    ms = _edge_idx(M, np.random.default_rng(ci), 12)
    got = host(y1[torch.from_numpy(ms).to(DEV)].float()).astype(np.float64)
    want = O.matmul(a[ms], *ref, K, transposed=t, a_dtype="f16" if f16 else "bf16")
    if epi:
        want = O.round_output(want + bias, "bf16")
        ulp = np.abs(want) * 2.0**-7
        bad = np.abs(got - want) > ELEM_RTOL * np.abs(want) + ELEM_ATOL + ulp
        assert not bad.any(), f"{int(bad.sum())} elements outside the bound, case {ci}"
    else:
        assert_mm_close(got, want, f"eight-wave {ci}")


# ------------------------------------------------------------------ full-size workloads, sampled outputs

DECODE_SHAPES = [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008), (2048, 2048), (8192, 8192),
                 (16384, 16384)]


@pytest.mark.parametrize("si", range(len(DECODE_SHAPES)), ids=[f"{n}x{k}" for n, k in DECODE_SHAPES])
def test_decode_gemv_full(si):
    """Decode batched GEMV, Llama-2-7B-like layers, g=128, M = 1..4, at full size: the
    packed codes, scales and zeros bit-exact with the oracle, and every output of Y; the
    same weights at the mid-M sizes M = 8, 16, 32 (the mid-M kernel, split as the bench
    launches it) and M = 64 (tiles)."""
    N, K = DECODE_SHAPES[si]
    print(f"[case] decode full N={N} K={K}", flush=True)
    w = synth.weight(2, si, N, K, "bf16")
    qw = w4.quantize_pack(dev_weight(w, "bf16"), "groupwise", 128)
    ref = O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, 128)
    del w
    torch.cuda.synchronize()
    assert_quant_equal(qw, *ref, what=f"decode {N}x{K}")
    wdq = O.bf16_bits_to_f64(O.dequantize_bf16_bits(*ref, K))  # the oracle's weight operand [N][K]
    for M in (1, 2, 3, 4, 8, 16, 32, 64):
        x = synth.activations_bf16(2, si * 10 + M, M, K)
        y = host(w4.mm(dev_bf16(x), qw))
        assert_mm_close(y, O.bf16_bits_to_f64(x) @ wdq.T, f"decode {N}x{K} M={M}")


def _edge_idx(n, rng, k):
    """k random indices below n plus the tile edges every planner route has: the first and
    last index, and both sides of each multiple of 32, 64, 128 and 256 near the ends."""
    edges = {0, 1, n - 2, n - 1}
    for t in (32, 64, 128, 256):
        for b in (t, 2 * t, (n // t) * t, (n // t - 1) * t):
            edges.update((b - 1, b))
    pick = set(rng.choice(n, min(n, k), replace=False).tolist())
    return np.array(sorted(i for i in edges | pick if 0 <= i < n))


PREFILL_SHAPES = [(2048, 2048), (8192, 2048), (2048, 8192), (512, 2048), (128256, 2048)]


@pytest.mark.parametrize("si", range(len(PREFILL_SHAPES)), ids=[f"{n}x{k}" for n, k in PREFILL_SHAPES])
def test_prefill_gemm_full(si):
    """Prefill GEMM, Llama-3.2-1B-like shapes, M in {128, 512, 2048}, three modes, fp32 bias: sampled outputs."""
    N, K = PREFILL_SHAPES[si]
    w = synth.weight(3, si, N, K, "bf16")
    w32 = O.to_f32(w, "bf16")
    wd = dev_weight(w, "bf16")
    bias = synth.bias_f32(3, si, N)
    rows = _edge_idx(N, np.random.default_rng(100 + si), 40)
    for mode, g in [("global", None), ("rowwise", None), ("groupwise", 64)]:
        print(f"[case] prefill full N={N} K={K} mode={mode}", flush=True)
        qw = w4.quantize_pack(wd, mode, g)
        if mode == "global":
            ref = oracle_rows_global(w32, rows)
        else:
            ref = O.quantize_pack(w32[rows], OMODE[mode], g)
        for M in (128, 512, 2048):
            x = synth.activations_bf16(3, si * 10 + M, M, K)
            y = w4.mm(dev_bf16(x), qw, bias=dev_f32(bias))
            ms = _edge_idx(M, np.random.default_rng(M), 24)
            ys = host(y[torch.from_numpy(ms).to(DEV)][:, torch.from_numpy(rows).to(DEV)])
            del y
            assert_mm_close(ys, O.matmul(x[ms], *ref, K, bias=bias[rows]), f"prefill {N}x{K} {mode} M={M}")


QLORA_SHAPES = [(12288, 4096), (11008, 4096), (4096, 11008)]


@pytest.mark.parametrize("si", range(len(QLORA_SHAPES)), ids=[f"{n}x{k}" for n, k in QLORA_SHAPES])
def test_qlora_pair_full(si):
    """QLoRA pair on one packed buffer: Y = X w^T and dX = dY w, rowwise and g=64: sampled outputs."""
    N, K = QLORA_SHAPES[si]
    if si == 0:  # fused QKV packed from separate Q, K, V
        ws = [synth.weight(4, 0, 4096, K, "bf16", tensor_id=synth.T_Q + i) for i in range(3)]
        w = np.concatenate(ws, axis=0)
    else:
        ws = None
        w = synth.weight(4, si, N, K, "bf16")
    w32 = O.to_f32(w, "bf16")
    for mode, g in [("rowwise", None), ("groupwise", 64)]:
        print(f"[case] qlora full N={N} K={K} mode={mode}", flush=True)
        if ws is not None:
            qw = w4.quantize_fused([dev_weight(p, "bf16") for p in ws], mode, g)
        else:
            qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
        ref_full = O.quantize_pack(w32, OMODE[mode], g)
        wdq = O.bf16_bits_to_f64(O.dequantize_bf16_bits(*ref_full, K))  # oracle weight operand [N][K]
        rows = _edge_idx(N, np.random.default_rng(200 + si), 32)
        for M in (1024, 2048, 4096):
            ms = _edge_idx(M, np.random.default_rng(M + si), 12)
            msd = torch.from_numpy(ms).to(DEV)
            x = synth.activations_bf16(4, si * 10 + M, M, K)
            y = w4.mm(dev_bf16(x), qw)
            ys = host(y[msd][:, torch.from_numpy(rows).to(DEV)])
            del y
            yref = O.bf16_bits_to_f64(x[ms]) @ wdq[rows].T
            assert_mm_close(ys, yref, f"qlora NT {N}x{K} {mode} M={M}")
            dy = synth.activations_bf16(4, si * 10 + M, M, N, tensor_id=synth.T_DY)
            dx = w4.mm(dev_bf16(dy), qw, transposed=True)
            dxs = host(dx[msd])
            del dx
            dxref = O.bf16_bits_to_f64(dy[ms]) @ wdq
            assert_mm_close(dxs, dxref, f"qlora T {N}x{K} {mode} M={M}")
