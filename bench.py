#!/usr/bin/env python3
"""Benchmark of the W4A16 hot path on one MI355X.

Headline workload (one "step"): the decode batched GEMV sweep at Llama-2-7B-like
layer shapes, groupwise g=128 along K, M in {1, 2, 3, 4}; (N, K) in
{(12288,4096) fused QKV, (4096,4096) o_proj, (22016,4096) fused gate+up,
(4096,11008) down, (2048,2048), (8192,8192), (16384,16384)}; X bf16 ~ N(0,1),
W ~ N(0,0.02) quantized on the GPU before timing.  28 launches per step.

value = algorithmic bytes of a step / GPU time of a step (GB/s), where a launch
moves N*K/2 (codes) + 4*N*K/g (fp16 scale + zero) + 2*M*K (X) + 4*M*N (Y) bytes.
Weights rotate through >= 1 GiB of distinct copies so no launch finds its
weights in the 256 MB Infinity Cache.

Also reported in the same JSON line (context, not `value`):
  prefill   forward GEMM at Llama-3.2-1B-like shapes: M in {128, 512, 2048},
            (N,K) in {(2048,2048), (8192,2048), (2048,8192), (512,2048), (128256,2048)},
            global / rowwise / g=64, fp32 bias; TFLOP/s overall, by M, and the minimum
            at M >= 512.
  gemm      QLoRA pair at Llama-2-7B layer shapes: M in {1024, 2048, 4096},
            (N,K) in {(12288,4096) fused QKV, (11008,4096), (4096,11008)}, rowwise
            and g=64, forward Y = X w^T and transposed dX = dY w on one packed buffer;
            TFLOP/s = 2MNK / kernel time, fraction of the 2.5 PFLOP/s bf16 peak.
  quantize  fp16 W [128256][2048] ~ N(0,0.02) with 0.1% outliers ~ N(0,0.5), ten
            modes: packed GB/s, MAE of the fp32 dequantization, compression ratio.
  single_matmul the single-matmul workload (X [4][2048], W fp32 2048x2048, g=128): GPU
            time per call and the host's enqueue cost per call.
  midm      M in {8, 16, 32, 64, 100} at the decode shapes, both directions, TFLOP/s.
  cpu_baseline  the CPU oracle timed on a bounded sample of the GEMV sweep (matmul), and its
            quantizer on rows of the quantize workload; host CPU model and threads.

Timing: the GPU is parked on a spin kernel while the host enqueues the whole
batch, so the two HIP events around the timed part measure back-to-back GPU
execution, not host overhead.  Every timed region is preceded, on the GPU
timeline and with no gap, by an untimed lead-in of the same work (`warmup` steps
of the sweep; >= 25 ms of the same launches elsewhere, at most 1000 calls): for about the first 10 ms
of work after an idle period the GPU's power management holds the rate 10-20%
below its sustained value, and the lead-in takes the timed region past that
transient.  The rate right after idle is reported beside `value` as context.
The timed region is `steps` steps of the sweep; per-shape figures come from
separate batches of 20 launches of one shape, each with its own lead-in.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

DECODE_SHAPES = [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008), (2048, 2048), (8192, 8192),
                 (16384, 16384)]
DECODE_G = 128
QLORA_SHAPES = [(12288, 4096), (11008, 4096), (4096, 11008)]
QLORA_M = [1024, 2048, 4096]
QUANT_MODES = [("global", None), ("rowwise", None)] + [("groupwise", g) for g in (16, 32, 64, 128, 256, 512, 1024,
                                                                                   2048)]
POOL_BYTES = 1 << 30
POINT_POOL_BYTES = 640 << 20  # per-shape batches: well above the 256 MB last-level cache


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(M: int, N: int, K: int, g: int) -> int:
    return N * K // 2 + 4 * N * (K // g) + 2 * M * K + 4 * M * N


def source_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gemv_int4_quantize_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


WARM_MS = 25.0  # untimed lead-in before every timed region, ms of GPU work


def run_batch(torch, fns, warm=(), per_fn_s: float = 30e-6) -> float:
    """Run `warm` then `fns` back-to-back behind a GPU spin (so the host enqueues ahead of
    the GPU); returns the GPU time in ms of `fns` alone (two events after `warm`).

    The spin is sized from a per-launch host budget; if the host took longer to enqueue than
    the spin lasted, the GPU may have waited on it, so the batch is run again with a longer spin."""
    n = len(warm) + len(fns)
    for _ in range(4):
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        s0.record()
        torch.cuda._sleep(int(2.4e9 * per_fn_s * n) + 2_000_000)
        s1.record()
        h0 = time.perf_counter()
        for fn in warm:
            fn()
        a.record()
        for fn in fns:
            fn()
        b.record()
        host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        if host_ms < 0.9 * s0.elapsed_time(s1):
            return a.elapsed_time(b)
        per_fn_s *= 4
    raise RuntimeError("the host could not enqueue the batch within the spin")


# While the spin runs, the launch queue takes about 2000 packets before the host blocks
# (measured: 1000 calls of a split-K GEMM, two kernels each, enqueue at ~15 us per call;
# 2000 such calls block until the spin ends).
MAX_LEAD_CALLS = 1000


def timed(torch, fns, warm_ms: float = WARM_MS) -> float:
    """GPU ms of `fns`, run after an untimed lead-in of the same list repeated for >= warm_ms
    (or for MAX_LEAD_CALLS calls, whichever is shorter)."""
    est = run_batch(torch, fns)
    reps = max(1, min(math.ceil(warm_ms / max(est, 1e-3)), MAX_LEAD_CALLS // len(fns)))
    return run_batch(torch, fns, warm=list(fns) * reps)


def clone_qw(w4, qw):
    return w4.QuantizedWeight(qw.packed.clone(), qw.scales.clone(), qw.zeros.clone(), qw.N, qw.K, qw.mode, qw.group)


MALL_BYTES = 256 << 20  # MI355X Infinity Cache (last-level cache)


def weight_pool(w4, qw, pool_bytes: int = POOL_BYTES):
    """Copies of a packed weight that together exceed the last-level cache several times, so a
    launch rotating through them finds its weight in HBM (a single copy when it is already
    larger than the cache)."""
    nb = qw.packed.numel() * 4 + 2 * (qw.scales.numel() + qw.zeros.numel()) * 2
    n = 1 if nb >= MALL_BYTES else max(2, math.ceil(pool_bytes / nb))
    return [qw] + [clone_qw(w4, qw) for _ in range(n - 1)]


def rotating(pool):
    """A callable returning the pool's weights in turn."""
    ctr = [0]

    def nxt():
        q = pool[ctr[0] % len(pool)]
        ctr[0] += 1
        return q
    return nxt


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bench_gemv(torch, w4, synth, args):
    """The headline sweep: returns (result dict, per-launch records)."""
    import numpy as np
    per_copy = sum(N * K // 2 + 4 * N * (K // DECODE_G) for N, K in DECODE_SHAPES)
    copies = max(4, math.ceil(POOL_BYTES / per_copy))
    log(f"GEMV sweep: {len(DECODE_SHAPES)} shapes x M=1..4, pool of {copies} weight copies "
        f"({copies * per_copy / 2**30:.2f} GiB)")
    layers = []
    for si, (N, K) in enumerate(DECODE_SHAPES):
        w = synth.weight(2, si, N, K, "bf16")
        qw = w4.quantize_pack(dev_bf16(torch, w), "groupwise", DECODE_G)
        del w
        pool = [qw] + [clone_qw(w4, qw) for _ in range(copies - 1)]
        xs = {M: dev_bf16(torch, synth.activations_bf16(2, si * 10 + M, M, K)) for M in (1, 2, 3, 4)}
        ys = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in (1, 2, 3, 4)}
        layers.append((N, K, pool, xs, ys))
    torch.cuda.synchronize()

    launches = []   # (M, N, K) in step order
    for (N, K, pool, xs, ys) in layers:
        for M in (1, 2, 3, 4):
            launches.append((M, N, K))
    step_bytes = sum(gemv_bytes(M, N, K, DECODE_G) for M, N, K in launches)

    counter = [0]

    def make_step():
        fns = []
        for (N, K, pool, xs, ys) in layers:
            for M in (1, 2, 3, 4):
                def fn(N=N, K=K, pool=pool, x=xs[M], y=ys[M]):
                    qw = pool[counter[0] % len(pool)]
                    counter[0] += 1
                    w4.mm(x, qw, out=y)
                fns.append(fn)
        return fns

    run_batch(torch, make_step())  # first launches: code objects loaded, kernel arguments set up
    warm = []
    for _ in range(args.warmup):
        warm += make_step()
    fns = []
    for _ in range(args.steps):
        fns += make_step()
    # the timed region: `steps` steps, launches back-to-back, right behind `warmup` untimed steps
    span = run_batch(torch, fns, warm=warm)
    n = len(launches)
    ms_per_step = span / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    if args.sweep_only:
        return {"value": value, "ms_per_step": ms_per_step, "step_bytes": step_bytes, "per_point_gbs": None,
                "after_idle_gbs": None, "mean_launch_us": ms_per_step * 1e3 / n, "launches_per_step": n,
                "points": [], "pool_copies": copies}
    # context: the same number of steps timed right after an idle period, with no lead-in
    idle_fns = []
    for _ in range(args.steps):
        idle_fns += make_step()
    after_idle_gbs = step_bytes * args.steps / (run_batch(torch, idle_fns) * 1e-3) / 1e9
    # per-shape figures: 20 back-to-back launches of one point, rotating over enough
    # copies of that one weight that they cannot stay in the 256 MB last-level cache
    points = []
    point_ms = []
    for (N, K, pool, xs, ys) in layers:
        b1 = N * K // 2 + 4 * N * (K // DECODE_G)
        extra = [clone_qw(w4, pool[0]) for _ in range(max(0, math.ceil(POINT_POOL_BYTES / b1) - len(pool)))]
        ppool = pool + extra
        pctr = [0]
        for M in (1, 2, 3, 4):
            def one(x=xs[M], y=ys[M], ppool=ppool):
                qw = ppool[pctr[0] % len(ppool)]
                pctr[0] += 1
                w4.mm(x, qw, out=y)
            t = timed(torch, [one] * 20) / 20
            point_ms.append(t)
            b = gemv_bytes(M, N, K, DECODE_G)
            points.append({"M": M, "N": N, "K": K, "us": round(t * 1e3, 3), "GBps": round(b / (t * 1e-3) / 1e9, 1),
                           "kernel": w4.kernel_for(M, N, K, "groupwise", DECODE_G)})
        del extra, ppool
        torch.cuda.empty_cache()
    per_point_gbs = step_bytes / (sum(point_ms) * 1e-3) / 1e9
    return {
        "value": value, "ms_per_step": ms_per_step, "step_bytes": step_bytes, "per_point_gbs": per_point_gbs,
        "after_idle_gbs": after_idle_gbs,
        "mean_launch_us": ms_per_step * 1e3 / n, "launches_per_step": n, "points": points,
        "pool_copies": copies,
    }


def bench_gemm(torch, w4, synth, reps: int):
    import numpy as np
    log("QLoRA GEMM pair: 3 shapes x {rowwise, g64} x M in {1024, 2048, 4096} x {NT, T}")
    pts = []
    layer = []
    for si, (N, K) in enumerate(QLORA_SHAPES):
        if si == 0:
            parts = [dev_bf16(torch, synth.weight(4, 0, 4096, K, "bf16", tensor_id=synth.T_Q + i)) for i in range(3)]
        else:
            parts = None
            wd = dev_bf16(torch, synth.weight(4, si, N, K, "bf16"))
        for mode, g in [("rowwise", None), ("groupwise", 64)]:
            qw = w4.quantize_fused(parts, mode, g) if parts is not None else w4.quantize_pack(wd, mode, g)
            pool = weight_pool(w4, qw)
            nxt = rotating(pool)
            for M in QLORA_M:
                x = dev_bf16(torch, synth.activations_bf16(4, si * 10 + M, M, K))
                dy = dev_bf16(torch, synth.activations_bf16(4, si * 10 + M, M, N, tensor_id=synth.T_DY))
                y = torch.empty((M, N), dtype=torch.float32, device="cuda")
                dx = torch.empty((M, K), dtype=torch.float32, device="cuda")
                t_nt = timed(torch, [lambda: w4.mm(x, nxt(), out=y)] * reps) / reps * 1e-3
                t_t = timed(torch, [lambda: w4.mm(dy, nxt(), transposed=True, out=dx)] * reps) / reps * 1e-3
                fl = 2.0 * M * N * K
                pts.append({"M": M, "N": N, "K": K, "mode": mode if g is None else f"g{g}",
                            "nt_tflops": round(fl / t_nt / 1e12, 1), "t_tflops": round(fl / t_t / 1e12, 1),
                            "t_over_nt": round(t_t / t_nt, 3), "nt_us": round(t_nt * 1e6, 1),
                            "t_us": round(t_t * 1e6, 1),
                            "nt_kernel": w4.kernel_for(M, N, K, mode, g), "t_kernel": w4.kernel_for(M, N, K, mode, g,
                                                                                                   True)})
                if g is None:
                    # the QLoRA layer step (forward + backward dX) against the reference path of the
                    # page: dequantize the frozen weight to bf16 every step, then two bf16 matmuls
                    # (torch / hipBLASLt); also the two bf16 matmuls alone, as if W were stored in bf16
                    F = torch.nn.functional
                    wd16 = w4.dequantize(qw, torch.bfloat16)
                    dense_pool = [wd16] + [wd16.clone() for _ in range(max(1, math.ceil(POOL_BYTES / (
                        wd16.numel() * 2))) - 1)] if wd16.numel() * 2 < MALL_BYTES else [wd16]
                    dctr = [0]

                    # like the reference route (bf16 in, bf16 out), the fused layer writes its
                    # forward output and dX in bf16: the kernels round the fp32 sums once
                    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                    dx16 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")

                    def fused_pair():
                        q = nxt()
                        w4.mm(x, q, out=y16)
                        w4.mm(dy, q, transposed=True, out=dx16)

                    def fused_pair_f32():
                        q = nxt()
                        w4.mm(x, q, out=y)
                        w4.mm(dy, q, transposed=True, out=dx)

                    def ref_step():
                        # the page's reference path: dequantize the frozen weight, then two bf16 matmuls
                        wd = w4.dequantize(nxt(), torch.bfloat16)
                        F.linear(x, wd)
                        torch.mm(dy, wd)

                    def dense_step():
                        wd = dense_pool[dctr[0] % len(dense_pool)]
                        dctr[0] += 1
                        F.linear(x, wd)
                        torch.mm(dy, wd)
                    fused, ref, dense = [fused_pair], [ref_step], [dense_step]
                    t_f = timed(torch, fused * reps) / reps * 1e-3
                    t_f32 = timed(torch, [fused_pair_f32] * reps) / reps * 1e-3
                    t_r = timed(torch, ref * reps) / reps * 1e-3
                    t_d = timed(torch, dense * reps) / reps * 1e-3
                    layer.append({"M": M, "N": N, "K": K, "fused_us": round(t_f * 1e6, 1),
                                  "fused_f32_out_us": round(t_f32 * 1e6, 1),
                                  "dequant_ref_us": round(t_r * 1e6, 1), "dense_bf16_us": round(t_d * 1e6, 1)})
                    del wd16, dense_pool, y16, dx16
                del x, dy, y, dx
            del qw, pool, nxt
        torch.cuda.empty_cache()
    fl = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pts)
    t_nt = sum(p["nt_us"] for p in pts) * 1e-6
    t_t = sum(p["t_us"] for p in pts) * 1e-6
    big = [p for p in pts if p["M"] >= 512]
    return {
        "workload": "QLoRA pair, Llama-2-7B layer shapes, one packed buffer per weight",
        "nt_tflops": round(fl / t_nt / 1e12, 1), "t_tflops": round(fl / t_t / 1e12, 1),
        "nt_frac_of_peak": round(fl / t_nt / 1e12 / BF16_PEAK_TFLOPS, 4),
        "t_frac_of_peak": round(fl / t_t / 1e12 / BF16_PEAK_TFLOPS, 4),
        "t_over_nt_total": round(t_t / t_nt, 3),
        "t_over_nt_max": max(p["t_over_nt"] for p in pts),
        "min_tflops_m_ge_512": min(min(p["nt_tflops"], p["t_tflops"]) for p in big),
        "qlora_layer_step": {
            "workload": "forward + backward dX of a frozen rowwise int4 layer at the same shapes and M, "
                        "bf16 activations, gradients and outputs on both routes",
            "fused_ms": round(sum(p["fused_us"] for p in layer) * 1e-3, 3),
            "fused_f32_out_ms": round(sum(p["fused_f32_out_us"] for p in layer) * 1e-3, 3),
            "dequant_ref_ms": round(sum(p["dequant_ref_us"] for p in layer) * 1e-3, 3),
            "dense_bf16_ms": round(sum(p["dense_bf16_us"] for p in layer) * 1e-3, 3),
            "speedup_vs_dequant_ref": round(sum(p["dequant_ref_us"] for p in layer) /
                                            sum(p["fused_us"] for p in layer), 3),
        },
        "points": pts,
        "layer_points": layer,
    }


PREFILL_SHAPES = [(2048, 2048), (8192, 2048), (2048, 8192), (512, 2048), (128256, 2048)]
PREFILL_M = [128, 512, 2048]


def bench_prefill(torch, w4, synth, reps: int):
    """Prefill GEMM at Llama-3.2-1B-like shapes, three scale modes, fp32 bias epilogue."""
    log("prefill GEMM: 5 shapes x {global, rowwise, g64} x M in {128, 512, 2048}, fp32 bias")
    pts = []
    for si, (N, K) in enumerate(PREFILL_SHAPES):
        wd = dev_bf16(torch, synth.weight(3, si, N, K, "bf16"))
        bias = torch.from_numpy(synth.bias_f32(3, si, N)).cuda()
        for mode, g in [("global", None), ("rowwise", None), ("groupwise", 64)]:
            qw = w4.quantize_pack(wd, mode, g)
            pool = weight_pool(w4, qw)
            nxt = rotating(pool)
            for M in PREFILL_M:
                x = dev_bf16(torch, synth.activations_bf16(3, si * 10 + M, M, K))
                y = torch.empty((M, N), dtype=torch.float32, device="cuda")
                t = timed(torch, [lambda: w4.mm(x, nxt(), bias=bias, out=y)] * reps) / reps * 1e-3
                fl = 2.0 * M * N * K
                pts.append({"M": M, "N": N, "K": K, "mode": mode if g is None else f"g{g}", "us": round(t * 1e6, 1),
                            "tflops": round(fl / t / 1e12, 1), "kernel": w4.kernel_for(M, N, K, mode, g)})
                del x, y
            del qw, pool, nxt
        del wd, bias
        torch.cuda.empty_cache()
    fl = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pts)
    t = sum(p["us"] for p in pts) * 1e-6
    by_m = {}
    for M in PREFILL_M:
        sel = [p for p in pts if p["M"] == M]
        by_m[str(M)] = round(sum(2.0 * p["M"] * p["N"] * p["K"] for p in sel) / (sum(p["us"] for p in sel) * 1e-6)
                             / 1e12, 1)
    big = [p for p in pts if p["M"] >= 512]
    return {
        "workload": "prefill GEMM, Llama-3.2-1B-like shapes, global / rowwise / g64, fp32 bias",
        "tflops": round(fl / t / 1e12, 1), "frac_of_peak": round(fl / t / 1e12 / BF16_PEAK_TFLOPS, 4),
        "tflops_by_M": by_m,
        "min_tflops_m_ge_512": min(p["tflops"] for p in big),
        "points": pts,
    }


def bench_single(torch, w4, synth):
    """The single W4A16 matmul (X bf16 [4][2048], W fp32 [2048][2048] ~ N(0,0.02) quantized with
    g=128, seed 0): GPU time per call with cold weights, and the host's enqueue cost per call
    through the C ABI (the GPU parked on a spin meanwhile)."""
    import numpy as np
    x, w = synth.single_matmul_case()
    qw = w4.quantize_pack(torch.from_numpy(w).cuda(), "groupwise", 128)
    xd = dev_bf16(torch, x)
    y = torch.empty((4, 2048), dtype=torch.float32, device="cuda")
    nxt = rotating(weight_pool(w4, qw))
    n = 200
    t = timed(torch, [lambda: w4.mm(xd, nxt(), out=y)] * n) / n
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.05))
    h0 = time.perf_counter()
    for _ in range(n):
        w4.mm(xd, nxt(), out=y)
    host_us = (time.perf_counter() - h0) * 1e6 / n
    torch.cuda.synchronize()
    b = gemv_bytes(4, 2048, 2048, 128)
    return {"workload": "single W4A16 matmul: X bf16 [4][2048], W fp32 [2048][2048] g=128, seed 0",
            "kernel": w4.kernel_for(4, 2048, 2048, "groupwise", 128), "us": round(t * 1e3, 3),
            "GBps": round(b / (t * 1e-3) / 1e9, 1), "host_enqueue_us_per_call": round(host_us, 2)}


MIDM_M = [8, 16, 32, 64, 100]


def bench_midm(torch, w4, synth, reps: int):
    """Mid-M (5 <= M < 128) at the decode layer shapes, g=128, both directions: TFLOP/s per point
    with cold weights."""
    log(f"mid-M GEMM: M in {MIDM_M} x {len(DECODE_SHAPES)} decode shapes x {{NT, T}}")
    pts = []
    for si, (N, K) in enumerate(DECODE_SHAPES):
        qw = w4.quantize_pack(dev_bf16(torch, synth.weight(2, si, N, K, "bf16")), "groupwise", DECODE_G)
        pool = weight_pool(w4, qw)
        nxt = rotating(pool)
        for M in MIDM_M:
            x = dev_bf16(torch, synth.activations_bf16(6, si * 10 + M, M, K))
            dy = dev_bf16(torch, synth.activations_bf16(6, si * 10 + M, M, N, tensor_id=synth.T_DY))
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            dx = torch.empty((M, K), dtype=torch.float32, device="cuda")
            t_nt = timed(torch, [lambda: w4.mm(x, nxt(), out=y)] * reps) / reps * 1e-3
            t_t = timed(torch, [lambda: w4.mm(dy, nxt(), transposed=True, out=dx)] * reps) / reps * 1e-3
            fl = 2.0 * M * N * K
            b = N * K // 2 + 4 * N * (K // DECODE_G)
            pts.append({"M": M, "N": N, "K": K, "nt_us": round(t_nt * 1e6, 2), "t_us": round(t_t * 1e6, 2),
                        "nt_tflops": round(fl / t_nt / 1e12, 1), "t_tflops": round(fl / t_t / 1e12, 1),
                        "nt_weight_GBps": round(b / t_nt / 1e9, 1),
                        "nt_kernel": w4.kernel_for(M, N, K, "groupwise", DECODE_G),
                        "t_kernel": w4.kernel_for(M, N, K, "groupwise", DECODE_G, True)})
            del x, dy, y, dx
        del qw, pool, nxt
        torch.cuda.empty_cache()
    fl = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pts)

    def wbytes(p):  # algorithmic bytes: weights, scales and zeros, activations, fp32 output
        return p["N"] * p["K"] // 2 + 4 * p["N"] * (p["K"] // DECODE_G) + 2 * p["M"] * p["K"] + 4 * p["M"] * p["N"]

    by_m = {}
    for M in MIDM_M:
        sel = [p for p in pts if p["M"] == M]
        f = sum(2.0 * p["M"] * p["N"] * p["K"] for p in sel)
        t_nt = sum(p["nt_us"] for p in sel) * 1e-6
        by_m[str(M)] = {"nt_tflops": round(f / t_nt / 1e12, 1),
                        "t_tflops": round(f / (sum(p["t_us"] for p in sel) * 1e-6) / 1e12, 1),
                        "nt_GBps": round(sum(wbytes(p) for p in sel) / t_nt / 1e9, 1)}
    sel = [p for p in pts if p["M"] <= 32]
    nt_gbps = sum(wbytes(p) for p in sel) / (sum(p["nt_us"] for p in sel) * 1e-6) / 1e9
    return {"workload": "mid-M GEMM at the decode layer shapes, g=128, M in {8, 16, 32, 64, 100}",
            "nt_tflops": round(fl / (sum(p["nt_us"] for p in pts) * 1e-6) / 1e12, 1),
            "t_tflops": round(fl / (sum(p["t_us"] for p in pts) * 1e-6) / 1e12, 1),
            "nt_m_le_32": {"GBps": round(nt_gbps, 1), "frac_of_hbm_peak": round(nt_gbps / HBM_PEAK_GBS, 4)},
            "by_M": by_m, "points": pts}


def bench_quantize(torch, w4, synth, reps: int):
    import numpy as np
    N, K = 128256, 2048
    log(f"quantize-pack: fp16 [{N}][{K}] with 0.1% outliers, {len(QUANT_MODES)} modes")
    wd = torch.from_numpy(synth.weight_with_outliers(5, 0, N, K)).cuda()
    w64 = None
    out = []
    for mode, g in QUANT_MODES:
        qw = w4.quantize_pack(wd, mode, g)
        t = timed(torch, [lambda: w4.quantize_pack(wd, mode, g)] * reps) / reps * 1e-3
        pairs = 1 if mode == "global" else (N if mode == "rowwise" else N * K // g)
        reads = 2 if mode == "global" else 1
        nbytes = reads * N * K * 2 + N * K // 2 + 4 * pairs
        deq = w4.dequantize(qw, torch.float32)
        if w64 is None:
            w64 = wd.to(torch.float64)
        mae = float((deq.to(torch.float64) - w64).abs().mean())
        del deq
        comp = (N * K * 2.0) / (N * K / 2.0 + 4.0 * pairs)
        out.append({"mode": mode if g is None else f"g{g}", "us": round(t * 1e6, 1),
                    "GBps": round(nbytes / t / 1e9, 1), "frac_of_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                    "mae": round(mae, 6), "compression": round(comp, 6)})
    del wd, w64
    torch.cuda.empty_cache()
    return {"workload": "fp16 W [128256][2048] ~ N(0,0.02) + 0.1% N(0,0.5) outliers", "points": out}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, budget_s: float):
    """The CPU oracle on bounded samples: the matmul on the GEMV sweep (algorithmic GB/s, the
    headline's unit) and, separately, the quantizer on rows of the quantize workload."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas_threads = os.cpu_count() or 1
    # shapes of the sweep in order, every M; stops once the budget of oracle time is spent
    sample = [(si, M) for si in (1, 0, 3, 2, 5) for M in (1, 2, 3, 4)]
    done, total_bytes, t_total = [], 0, 0.0
    cache = {}
    for si, M in sample:
        N, K = DECODE_SHAPES[si]
        if si not in cache:
            cache.clear()
            w = synth.weight(2, si, N, K, "bf16")
            cache[si] = O.quantize_pack(O.to_f32(w, "bf16"), O.GROUPWISE, DECODE_G)
            del w
        p, s, z = cache[si]
        x = synth.activations_bf16(2, si * 10 + M, M, K)
        t0 = time.perf_counter()
        O.matmul(x, p, s, z, K)
        dt = time.perf_counter() - t0
        t_total += dt
        total_bytes += gemv_bytes(M, N, K, DECODE_G)
        done.append(f"{N}x{K}/M{M}")
        if t_total > budget_s:
            break
    # the quantizer (numpy elementwise, one thread) on the first 8192 rows of the quantize
    # workload, g=128 and rowwise; GB/s counts the bytes the GPU kernel moves for those rows
    wq = synth.weight_with_outliers(5, 0, 128256, 2048)[:8192]
    w32 = O.to_f32(wq, "f16")
    qt, qb = 0.0, 0
    for mode, g in ((O.GROUPWISE, 128), (O.ROWWISE, None)):
        t0 = time.perf_counter()
        O.quantize_pack(w32, mode, g)
        qt += time.perf_counter() - t0
        pairs = w32.shape[0] * (w32.shape[1] // g if g else 1)
        qb += w32.size * 2 + w32.size // 2 + 4 * pairs
    return {"value": round(total_bytes / t_total / 1e9, 3), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": "oracle matmul (bf16 dequantize + float64 BLAS product) on " + ", ".join(done) +
                      f" of the decode sweep, {t_total:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "quantize": {"GBps": round(qb / qt / 1e9, 3), "cores": 1, "seconds": round(qt, 2),
                         "sample": "oracle quantize_pack (numpy fp32, one thread) of fp16 [8192][2048] rows of "
                                   "the quantize workload, g=128 and rowwise"}}


def load_traffic(step_bytes_per_launch: float):
    """HBM traffic per launch from the committed counter summary, if it was taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "gemv_decode_sweep_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except OSError:
        return None
    if d.get("source_hash") != source_hash("gemv.hip", "common.h"):
        return None
    return d.get("traffic_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=60, help="untimed steps run right before the timed ones")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the GEMM and quantize blocks")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--details", default=None, help="write per-point results (JSON) to this path")
    ap.add_argument("--sweep-only", action="store_true",
                    help="time the sweep alone (no per-shape batches or after-idle figure): every point is then "
                         "launched equally often, as counter passes need")
    ap.add_argument("--gemm-only", action="store_true",
                    help="run only the QLoRA GEMM block and print its figures (for counter passes over the GEMM kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy (a known-size reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the W4A16 kernels run on a single GPU and this build has no "
              "multi-GPU path (--gpus must be 1)", file=sys.stderr)
        return 2

    import torch
    import gemv_int4_quantize_amd as w4
    import synth

    w4.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 268435456 bytes read and written once")

    if args.gemm_only:
        gm = bench_gemm(torch, w4, synth, reps=10)
        print(json.dumps({k: v for k, v in gm.items() if k not in ("points", "layer_points")}), flush=True)
        return 0
    g = bench_gemv(torch, w4, synth, args)
    log(f"GEMV sweep: {g['value']:.1f} GB/s per step" + ("" if args.sweep_only else
        f"; per-shape batches {g['per_point_gbs']:.1f} GB/s; first {args.steps} steps after idle "
        f"{g['after_idle_gbs']:.1f} GB/s"))
    per_launch_bytes = g["step_bytes"] / g["launches_per_step"]
    traffic = load_traffic(per_launch_bytes)
    result = {
        "metric": "W4A16 GEMV GB/s + GEMM TFLOP/s at Llama-7B shapes, % of MI355X roofline",
        "value": round(g["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode batched GEMV sweep, Llama-2-7B-like layers, groupwise g=128, M=1..4",
                   "shapes_NxK": [f"{n}x{k}" for n, k in DECODE_SHAPES], "M": [1, 2, 3, 4], "group": DECODE_G,
                   "launches_per_step": g["launches_per_step"], "bytes_per_step": g["step_bytes"],
                   "weight_pool_copies": g["pool_copies"]},
        # achieved: algorithmic bytes per launch / mean launch duration, both over the timed
        # region (every launch of the step is the GEMV kernel, so this equals the step rate)
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel (28 launches per step)",
                     "achieved": round(per_launch_bytes / (g["mean_launch_us"] * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(per_launch_bytes / (g["mean_launch_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "mean_launch_us": round(g["mean_launch_us"], 3),
                     "algorithmic_bytes_per_launch": round(per_launch_bytes, 1),
                     "per_shape_batches_gbs": None if args.sweep_only else round(g["per_point_gbs"], 1),
                     "sweep_after_idle_gbs": None if args.sweep_only else round(g["after_idle_gbs"], 1)},
    }
    # every untimed lead-in ahead of a timed region, stated: the sweep honours --warmup alone
    result["timing"] = {"sweep_lead_in_steps": args.warmup, "sweep_timed_steps": args.steps,
                        "other_blocks_lead_in_ms": WARM_MS,
                        "weights": "rotating through >= 1 GiB of copies wherever one copy fits the 256 MB "
                                   "last-level cache (the quantize input, 525 MB, never fits)"}
    details = {"gemv": g["points"]}
    if not args.sweep_only:
        sm = bench_single(torch, w4, synth)
        result["single_matmul"] = sm
        log(f"single matmul: {sm['us']} us per call ({sm['kernel']}), host enqueue {sm['host_enqueue_us_per_call']} us")
    if not args.no_extras:
        gm = bench_gemm(torch, w4, synth, reps=10)
        result["gemm"] = {k: v for k, v in gm.items() if k not in ("points", "layer_points")}
        result["gemm"]["roofline"] = {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "achieved_nt": gm["nt_tflops"], "achieved_t": gm["t_tflops"],
                                      "frac_nt": gm["nt_frac_of_peak"], "frac_t": gm["t_frac_of_peak"]}
        details["gemm"] = gm["points"]
        details["qlora_layer"] = gm["layer_points"]
        log(f"GEMM: NT {gm['nt_tflops']} TFLOP/s, T {gm['t_tflops']} TFLOP/s, T/NT {gm['t_over_nt_total']}")
        ls = gm["qlora_layer_step"]
        log(f"QLoRA layer step (bf16 out): fused {ls['fused_ms']} ms, dequantize + hipBLASLt {ls['dequant_ref_ms']} ms "
            f"({ls['speedup_vs_dequant_ref']}x), dense bf16 {ls['dense_bf16_ms']} ms; fp32 out {ls['fused_f32_out_ms']} ms")
        pf = bench_prefill(torch, w4, synth, reps=10)
        result["prefill"] = {k: v for k, v in pf.items() if k != "points"}
        details["prefill"] = pf["points"]
        log(f"prefill GEMM: {pf['tflops']} TFLOP/s over the 45 points, by M {pf['tflops_by_M']}, "
            f"M >= 512 minimum {pf['min_tflops_m_ge_512']}")
        mm_ = bench_midm(torch, w4, synth, reps=10)
        result["midm"] = {k: v for k, v in mm_.items() if k != "points"}
        details["midm"] = mm_["points"]
        log(f"mid-M GEMM: NT {mm_['nt_tflops']} TFLOP/s, T {mm_['t_tflops']} TFLOP/s; "
            f"NT at M <= 32 {mm_['nt_m_le_32']['GBps']} GB/s")
        qz = bench_quantize(torch, w4, synth, reps=10)
        result["quantize"] = {"workload": qz["workload"],
                              "GBps": {p["mode"]: p["GBps"] for p in qz["points"]},
                              "mae": {p["mode"]: p["mae"] for p in qz["points"]},
                              "compression": {p["mode"]: p["compression"] for p in qz["points"]}}
        details["quantize"] = qz["points"]
        log("quantize: " + ", ".join(f"{p['mode']} {p['GBps']} GB/s" for p in qz["points"]))
    if not args.no_cpu:
        cb = cpu_baseline(synth, args.cpu_budget)
        result["cpu_baseline"] = cb
        log(f"cpu baseline: {cb['value']} GB/s on {cb['cores']} threads ({cb['cpu_model']}); quantize "
            f"{cb['quantize']['GBps']} GB/s on 1 thread")
    else:
        result["cpu_baseline"] = None
    if args.details:
        os.makedirs(os.path.dirname(os.path.abspath(args.details)), exist_ok=True)
        with open(args.details, "w") as f:
            json.dump({"result": result, "details": details}, f, indent=1)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
