"""GPU parity of the decode GEMV (M <= 4) at the edges of its layout: rows of one partial
2048-column iteration, several iterations with a ragged last one, X staged in one or
several phases, scale / zero arrays at any 2-byte alignment, tiny N; plus the
non-transposed LDS tile on contractions past 2^21 with a ragged last step."""

import numpy as np
import pytest
import torch

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import DEV, assert_mm_close, assert_quant_equal, dev_bf16, dev_f32, dev_weight, host

pytestmark = pytest.mark.gpu

OMODE = {"global": O.GLOBAL, "rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}

# (N, K): one partial 2048-column iteration, several with a ragged last one, long rows
# whose X fills the LDS in one phase or needs several (M = 4 at K = 32768 and 33792)
EDGE_SHAPES = [(1, 32), (5, 1024), (257, 6144), (64, 30720), (33, 32768), (19, 33792), (700, 2080)]
EDGE_MODES = [("global", None), ("rowwise", None), ("groupwise", 16), ("groupwise", 32), ("groupwise", 128),
               ("groupwise", 1024)]


@pytest.mark.parametrize("N,K", EDGE_SHAPES, ids=[f"{n}x{k}" for n, k in EDGE_SHAPES])
@pytest.mark.parametrize("mode,g", EDGE_MODES, ids=[f"{m}{g or ''}" for m, g in EDGE_MODES])
def test_gemv_edges(N, K, mode, g):
    if g is not None and K % g:
        pytest.skip("group does not divide K")
    print(f"[case] gemv edges N={N} K={K} mode={mode} g={g}", flush=True)
    w = synth.weight(710, N + K, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    for M in (1, 2, 3, 4):
        assert w4.kernel_for(M, N, K, mode, g) == f"gemv_m{M}"
        x = synth.activations_bf16(710, N + K + M, M, K)
        bias = synth.bias_f32(710, N + M, N) if M % 2 == 0 else None
        y = w4.mm(dev_bf16(x), qw, bias=None if bias is None else dev_f32(bias))
        assert_mm_close(host(y), O.matmul(x, *ref, K, bias=bias), f"gemv edges {N}x{K} {mode}{g} M={M}")


def _offset_copy(t: torch.Tensor, off: int) -> torch.Tensor:
    """A copy of t that starts `off` elements into a larger buffer (2-byte aligned only)."""
    buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("mode,g", [("groupwise", 128), ("groupwise", 16), ("rowwise", None), ("groupwise", 2048)],
                         ids=["g128", "g16", "rowwise", "g2048"])
@pytest.mark.parametrize("offs", [(1, 7), (3, 0), (6, 5)], ids=["s1z7", "s3z0", "s6z5"])
def test_gemv_meta_any_alignment(mode, g, offs):
    """Scales and zeros at 2-, 6-, 12- and 14-byte offsets from 16-byte alignment (the
    boundary asks for 2-byte alignment only)."""
    N, K = 300, 4096
    print(f"[case] gemv meta alignment {mode}{g} offs={offs}", flush=True)
    w = synth.weight(711, 0, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    q0 = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    qw = w4.QuantizedWeight(packed=q0.packed, scales=_offset_copy(q0.scales, offs[0]),
                            zeros=_offset_copy(q0.zeros, offs[1]), N=N, K=K, mode=q0.mode, group=q0.group)
    assert qw.scales.data_ptr() % 16 == 2 * offs[0] % 16 or offs[0] == 0
    assert_quant_equal(qw, *ref, what="offset copy")
    for M in (1, 4):
        x = synth.activations_bf16(711, M, M, K)
        y = host(w4.mm(dev_bf16(x), qw))
        assert_mm_close(y, O.matmul(x, *ref, K), f"meta alignment {mode}{g} {offs} M={M}")


@pytest.mark.parametrize("K", [(1 << 21) + 32, (1 << 21) + 64], ids=["ragged", "whole"])
@pytest.mark.parametrize("mode,g", [("rowwise", None), ("groupwise", 32)], ids=["rowwise", "g32"])
def test_nt_lds_tile_long_contraction(K, mode, g):
    """M = 8 past K = 2^21: without a workspace the non-transposed LDS tile runs; with K % 64 ==
    32 its last step reads half a step: the columns past K must count as zero and no word past a
    row is read.  With a workspace the mid-M kernel runs, its contraction split into 257 ranges
    (the last one a single ragged unit)."""
    M, N = 8, 64
    print(f"[case] nt lds tile M={M} N={N} K={K} {mode}{g}", flush=True)
    assert w4.mm_plan(M, N, K, mode, g, ws_bytes=0)["kernel"] == "gemm_nt_lds_256x256"
    assert w4.kernel_for(M, N, K, mode, g) == "skinny_m16_splitk257"
    w = synth.weight(712, K % 128, N, K, "bf16")
    ref = O.quantize_pack(O.to_f32(w, "bf16"), OMODE[mode], g)
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    del w
    x = synth.activations_bf16(712, K % 128, M, K)
    bias = synth.bias_f32(712, 0, N)
    for split in (False, True):
        y = host(w4.mm(dev_bf16(x), qw, bias=dev_f32(bias), split_k=split))
        assert_mm_close(y, O.matmul(x, *ref, K, bias=bias), f"nt lds K={K} {mode}{g} split={split}")
