"""GPU parity over seeded random shapes: M from 1 to 2100 (GEMV, short-M and prefill
plans, split and unsplit), N a multiple of 8, K a multiple of 64, rowwise or groupwise
(g = 64, 128, 256), both directions, with and without the fp32 bias.  The planner picks
the kernel for each shape, so this covers tile / split combinations that the fixed
shapes of the other tests may not reach.  Sampled outputs against the oracle."""

import numpy as np
import pytest

import gemv_int4_quantize_amd as w4
import oracle as O
import synth
from gpu_helpers import assert_mm_close, dev_bf16, dev_f32, dev_weight, host

pytestmark = pytest.mark.gpu

OMODE = {"rowwise": O.ROWWISE, "groupwise": O.GROUPWISE}


def _case(seed: int):
    r = np.random.default_rng(seed)
    M = int(r.integers(1, 2100)) if seed % 2 else int(r.integers(1, 128))
    N = int(r.integers(1, 512)) * 8
    K = int(r.integers(1, 64)) * 64
    tr = bool(r.integers(0, 2)) and M > 4
    mode = ("rowwise", "groupwise")[int(r.integers(0, 2))]
    g = (64, 128, 256)[int(r.integers(0, 3))] if mode == "groupwise" else None
    if g is not None and K % g:
        g = 64
    return r, M, N, K, tr, mode, g, bool(r.integers(0, 2))


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    r, M, N, K, tr, mode, g, use_b = _case(seed)
    print(f"[case] seed={seed} M={M} N={N} K={K} t={tr} {mode}{g or ''} bias={use_b} "
          f"{w4.kernel_for(M, N, K, mode, g, tr)}", flush=True)
    w = synth.weight(901, seed, N, K, "bf16")
    w32 = O.to_f32(w, "bf16")
    qw = w4.quantize_pack(dev_weight(w, "bf16"), mode, g)
    outc = K if tr else N
    a = synth.activations_bf16(901, seed, M, N if tr else K)
    b = synth.bias_f32(901, seed, outc) if use_b else None
    y = host(w4.mm(dev_bf16(a), qw, transposed=tr, bias=None if b is None else dev_f32(b)))
    ms = np.sort(r.choice(M, min(M, 16), replace=False))
    cs = np.sort(r.choice(outc, min(outc, 24), replace=False))
    if tr:
        want = O.matmul(a[ms], *O.quantize_pack(w32, OMODE[mode], g), K, True, bias=b)[:, cs]
    else:
        want = O.matmul(a[ms], *O.quantize_pack(w32[cs], OMODE[mode], g), K, bias=None if b is None else b[cs])
    assert_mm_close(y[ms][:, cs], want, f"seed {seed}")
