#!/usr/bin/env python3
"""Benchmark of the MI355X exact-attention library.

One step = the headline workload's whole training pass: bf16 causal forward
plus backward at B=2, H=16, N=8192, d=128 (fa_fwd, then fa_bwd's two
stages: the dQ kernel, which also forms delta = dO . O, and the dK/dV
kernel), inputs resident in HBM.  The value is its aggregate throughput in
TFLOP/s, counting 4*B*H*N*N*d/2 for the causal forward and 2.5x that for the
backward.  The remaining rows of the path are timed after the steps, each on
its own workload, and reported under "parts": the non-causal forward at the
same shape, the d=64 prefill forward, the split-KV decode (GB/s of the
algorithmic bytes K+V+Q+O+LSE) and the fp8 forward.

The device's clock climbs back over some tens of milliseconds after any pause
of the host (a part timed right after its inputs were made ran up to 15%
slower in its first 20 calls than from the fourth batch of 20 on).  The
headline steps are timed exactly as asked (W warmup steps, then K timed
ones); each part is timed after --settle-ms of its own calls, and the step
is timed once more the same way and reported as "step_steady", beside the
headline value, not in place of it.

Prints ONE JSON line.  --gpus above 1 is not supported (one-GPU build).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(fn, stream, min_ms):
    """Call fn() until at least min_ms of device time has passed on stream,
    so that a rate timed next is the sustained one."""
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    done, n = 0.0, 1
    while done < min_ms:
        s.record(stream)
        for _ in range(n):
            fn()
        e.record(stream)
        e.synchronize()
        done += s.elapsed_time(e)
        n = min(2 * n, 64)


def timed(fn, iters, stream, settle_ms=0.0):
    """Average ms of fn() over iters calls, measured with HIP events on stream
    (after settle_ms of untimed calls)."""
    import torch
    if settle_ms > 0:
        settle(fn, stream, settle_ms)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / iters


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "bwd_dkdv_kernel_causal_bf16_traffic.md")


def measured_traffic(path=TRAFFIC_PROFILE):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE/WRITE_SIZE, calibrated), or None when that summary is
    missing or the kernel sources have changed since the counters were taken."""
    import hashlib
    try:
        text = open(path).read()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines()
                if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    files = ["exact_attention_83_amd/csrc/fa_bwd.hip", "exact_attention_83_amd/csrc/fa_device.h",
             "exact_attention_83_amd/csrc/fa_launch.h", "exact_attention_83_amd/build.py"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256", "").strip() != h.hexdigest():
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def _host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(fp8_sample=None, c3_seconds=8.0, max_heads=8):
    """The fp64 oracle on the host cores, timed on a bounded sample of every
    workload (whole heads at full length; decode: whole (b, KV head) slabs),
    so the default run stays within minutes.  The headline value is the
    causal workload's forward + backward rate.  With `fp8_sample` (two heads
    of the fp8 workload's bf16 inputs and the GPU's fp8 output for them) the
    fp8 output's relative L2 error against exact attention on the
    unquantised inputs is measured here too, beside the oracle's own fp8
    pipeline's error (the e4m3 floor)."""
    import numpy as np
    import torch
    from oracle import attention as A
    from oracle import fp8 as F8
    from workloads import WORKLOADS, to_f64

    per = {}
    mk = lambda g, n, d: to_f64(torch.randn(n, d, generator=g).to(torch.bfloat16))

    def run(name, w, heads_max, seconds, fn, flops_per_unit, unit_name):
        g = torch.Generator("cpu").manual_seed(w.seed)
        n, dt = 0, 0.0
        while n < heads_max and (n == 0 or dt < seconds):
            dt += fn(g)
            n += 1
        per[name] = {"seconds": round(dt, 3), "units": n, "unit": unit_name,
                     "tflops": round(n * flops_per_unit / dt / 1e12, 6)}
        return n, dt

    # tiny fp32 B1 H1 N256 d64: forward + backward, best of 3
    wt = WORKLOADS["tiny_f32"]

    def tiny(g):
        q, k, v, do = (torch.randn(wt.Nq, wt.d, generator=g).double().numpy() for _ in range(4))
        best = 1e9
        for _ in range(3):
            t0 = time.perf_counter()
            A.head_forward(q, k, v, wt.scale, wt.causal)
            A.head_backward(q, k, v, do, wt.scale, wt.causal)
            best = min(best, time.perf_counter() - t0)
        return best
    run("tiny_f32 fwd+bwd", wt, 1, 0, tiny, wt.fwd_flops() + wt.bwd_flops(), "whole problem")

    # prefill d=64: forward of whole heads
    wp = WORKLOADS["prefill_bf16"]

    def prefill(g):
        q, k, v = (mk(g, wp.Nq, wp.d) for _ in range(3))
        t0 = time.perf_counter()
        A.head_forward(q, k, v, wp.scale, False)
        return time.perf_counter() - t0
    one_p = wp.scaled(B=1, Hq=1, Hkv=1)
    run("prefill_bf16 fwd", wp, 8, 1.0, prefill, one_p.fwd_flops(), "head")

    # headline causal B2 H16 N8192 d128: forward + backward of whole heads
    w = WORKLOADS["causal_bf16"]

    def causal(g):
        q, k, v, do = (mk(g, w.Nq, w.d) for _ in range(4))
        t0 = time.perf_counter()
        A.head_forward(q, k, v, w.scale, w.causal)
        A.head_backward(q, k, v, do, w.scale, w.causal)
        return time.perf_counter() - t0
    one = w.scaled(B=1, Hq=1, Hkv=1)
    heads, dt = run("causal_bf16 fwd+bwd", w, max_heads, c3_seconds, causal,
                    one.fwd_flops() + one.bwd_flops(), "head")

    # split-KV decode: one (b, KV head) slab (its 4 query heads, 131072 keys)
    wd = WORKLOADS["decode_gqa"]
    G = wd.Hq // wd.Hkv

    def decode(g):
        q = to_f64(torch.randn(1, G, 1, wd.d, generator=g).to(torch.bfloat16))
        kk = to_f64(torch.randn(1, 1, wd.Nk, wd.d, generator=g).to(torch.bfloat16))
        vv = to_f64(torch.randn(1, 1, wd.Nk, wd.d, generator=g).to(torch.bfloat16))
        t0 = time.perf_counter()
        A.decode_split(q, kk, vv, wd.scale, wd.num_splits)
        return time.perf_counter() - t0
    run("decode_gqa split+combine", wd, 2, 1.0, decode, 4.0 * G * wd.Nk * wd.d, "(b, KV head)")

    # fp8 forward: the oracle's fp8 pipeline (rotate, quantise, dequantise,
    # forward) on whole heads
    wf = WORKLOADS["fp8_fwd"]

    def fp8(g):
        q, k, v = (torch.randn(1, 1, wf.Nq, wf.d, generator=g).to(torch.bfloat16).float().numpy()
                   for _ in range(3))
        signs = np.where(np.arange(wf.d) % 3 == 0, -1.0, 1.0)
        t0 = time.perf_counter()
        deq = [F8.dequantize(*F8.quantize(F8.rotate(q, signs).astype(np.float32))),
               F8.dequantize(*F8.quantize(F8.rotate(k, signs).astype(np.float32))),
               F8.dequantize(*F8.quantize(v))]
        A.forward(*deq, wf.scale, False)
        return time.perf_counter() - t0
    one_f = wf.scaled(B=1, Hq=1, Hkv=1)
    run("fp8_fwd (emulated)", wf, 1, 0, fp8, one_f.fwd_flops(), "head")

    fp8_err = None
    if fp8_sample is not None:
        rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
        signs = fp8_sample["signs"].double().numpy()
        e_gpu, e_floor = [], []
        for h in range(fp8_sample["q"].shape[0]):
            q, k, v = (fp8_sample[n][h].float().numpy()[None, None] for n in ("q", "k", "v"))
            exact, _ = A.forward(q, k, v, wf.scale, False)
            deq = [F8.dequantize(*F8.quantize(F8.rotate(q, signs).astype(np.float32))),
                   F8.dequantize(*F8.quantize(F8.rotate(k, signs).astype(np.float32))),
                   F8.dequantize(*F8.quantize(v))]
            emul, _ = A.forward(*deq, wf.scale, False)
            e_gpu.append(rel(fp8_sample["o"][h].double().numpy(), exact[0, 0]))
            e_floor.append(rel(emul[0, 0], exact[0, 0]))
        fp8_err = {"rel_l2_vs_exact": round(max(e_gpu), 4),
                   "oracle_fp8_rel_l2_vs_exact": round(max(e_floor), 4),
                   "heads": fp8_sample["heads"]}

    flops = heads * (one.fwd_flops() + one.bwd_flops())
    out = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(_blas_threads()),
           "kind": "oracle", "seconds": round(dt, 3),
           "sample": f"forward+backward of {heads} of the {w.B * w.Hq} heads "
                     f"(N={w.Nq}, d={w.d}, causal), numpy fp64; per_config: a bounded sample "
                     "of every workload",
           "per_config": per, "host": _host_info()}
    return out, fp8_err


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed device time of its own calls before each part is timed")
    ap.add_argument("--only", default="", help="comma list of parts to time (default all)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain 256 MiB fp32 read+write kernel first (a known-size "
                         "reference for hardware byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py: --gpus {a.gpus} is not supported; this library and its benchmark "
              "run on one GPU (the multi-GPU design is described, not built).", file=sys.stderr)
        return 2

    import torch
    import exact_attention_83_amd as fa
    from workloads import WORKLOADS, make_inputs

    fa.load()
    fp8_sample = None
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    parts = {}
    only = set(x for x in a.only.split(",") if x)
    if a.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)   # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    # ------------------------------------------------ headline: causal fwd+bwd
    w = WORKLOADS["causal_bf16"]
    log(f"inputs {w.name}")
    x = make_inputs(w, device="cuda")
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Nq, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    args = (w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    sh = stream.cuda_stream

    def fwd(causal=True):
        fa.fa_fwd(q, k, v, o, lse, *args, w.scale, causal, sh)

    # fa_bwd's two stages: dQ (which also writes delta = dO . O), then dK/dV
    def bwd_dq():
        fa.fa_bwd_dq_delta(q, k, v, o, do, lse, dq, ws, ws_bytes, *args, w.scale, True, sh)

    def bwd_dkdv():
        fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, ws, ws_bytes, *args, w.scale, True, sh)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    log("warmup")
    for _ in range(a.warmup):
        fwd(); bwd_dq(); bwd_dkdv()
    torch.cuda.synchronize()
    marks = [tuple(ev() for _ in range(6)) for _ in range(a.steps)]
    t_start, t_end = ev(), ev()
    log(f"timing {a.steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for f0, f1, q0_, q1_, k0, k1 in marks:
        f0.record(stream)
        fwd()
        f1.record(stream)
        q0_.record(stream)
        bwd_dq()
        q1_.record(stream)
        k0.record(stream)
        bwd_dkdv()
        k1.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / a.steps
    avg = lambda i, j: sum(m[i].elapsed_time(m[j]) for m in marks) / a.steps
    fwd_ms, dq_ms, dkdv_ms = avg(0, 1), avg(2, 3), avg(4, 5)
    # per-step spread: median and minimum of each step (forward start to
    # dK/dV end) and of each dK/dV launch
    per_step = sorted(m[0].elapsed_time(m[5]) for m in marks)
    per_dkdv = sorted(m[4].elapsed_time(m[5]) for m in marks)
    median = lambda xs: xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] + xs[len(xs) // 2])
    step_flops = w.fwd_flops() + w.bwd_flops()
    value = step_flops / (ms_step * 1e-3) / 1e12
    rate = lambda flops, ms: flops / (ms * 1e-3) / 1e12
    # executed products: the forward is 2 GEMM units (QK^T, PV); the dK/dV
    # kernel 4 (S, dP, dV, dK); the dQ kernel 3 (S, dP, dQ)
    unit = w.fwd_flops() / 2
    kern = {"fwd_bf16_kernel<128,causal> (fa_fwd)": (w.fwd_flops(), fwd_ms),
            "bwd_dkdv_kernel<128,causal> (fa_bwd_dkdv)": (4 * unit, dkdv_ms),
            "bwd_dq_kernel<128,causal,delta> (fa_bwd_dq_delta)": (3 * unit, dq_ms)}
    dom = max(kern, key=lambda n: kern[n][1])
    bwd_ms = ms_step - fwd_ms
    parts["fwd_causal"] = {"ms": round(fwd_ms, 4), "tflops": round(rate(w.fwd_flops(), fwd_ms), 1),
                           "frac_peak": round(rate(w.fwd_flops(), fwd_ms) / PEAK_BF16_TFLOPS, 4)}
    parts["bwd_causal"] = {"ms": round(bwd_ms, 4), "dkdv_ms": round(dkdv_ms, 4),
                           "dq_ms": round(dq_ms, 4),
                           "tflops": round(rate(w.bwd_flops(), bwd_ms), 1),
                           "frac_peak": round(rate(w.bwd_flops(), bwd_ms) / PEAK_BF16_TFLOPS, 4),
                           "dkdv_executed_tflops": round(rate(4 * unit, dkdv_ms), 1),
                           "dq_executed_tflops": round(rate(3 * unit, dq_ms), 1),
                           "dkdv_ms_median": round(median(per_dkdv), 4),
                           "dkdv_ms_min": round(per_dkdv[0], 4)}
    parts["step_spread"] = {"ms_median": round(median(per_step), 4),
                            "ms_min": round(per_step[0], 4),
                            "ms_max": round(per_step[-1], 4)}
    log(f"step {ms_step:.3f} ms: fwd {fwd_ms:.3f} ms ({rate(w.fwd_flops(), fwd_ms):.0f} TF), "
        f"dkdv {dkdv_ms:.3f} ms, dq {dq_ms:.3f} ms, bwd {rate(w.bwd_flops(), bwd_ms):.0f} TF")

    # the same K steps again after --settle-ms of steps: the sustained rate,
    # reported beside the headline value (which is timed exactly after the W
    # warmup steps), never in its place
    if a.settle_ms > 0:
        settle(lambda: (fwd(), bwd_dq(), bwd_dkdv()), stream, a.settle_ms)
        sm = [tuple(ev() for _ in range(4)) for _ in range(a.steps)]
        for e0, e1, e2, e3 in sm:
            e0.record(stream)
            fwd()
            e1.record(stream)
            bwd_dq()
            e2.record(stream)
            bwd_dkdv()
            e3.record(stream)
        torch.cuda.synchronize()
        s_avg = lambda i, j: sum(m[i].elapsed_time(m[j]) for m in sm) / a.steps
        s_step, s_fwd, s_dq, s_dkdv = s_avg(0, 3), s_avg(0, 1), s_avg(1, 2), s_avg(2, 3)
        s_bwd = s_step - s_fwd
        parts["step_steady"] = {
            "settle_ms": a.settle_ms, "ms": round(s_step, 4),
            "tflops": round(rate(step_flops, s_step), 1),
            "frac_peak": round(rate(step_flops, s_step) / PEAK_BF16_TFLOPS, 4),
            "fwd_ms": round(s_fwd, 4),
            "fwd_frac_peak": round(rate(w.fwd_flops(), s_fwd) / PEAK_BF16_TFLOPS, 4),
            "bwd_ms": round(s_bwd, 4), "dq_ms": round(s_dq, 4), "dkdv_ms": round(s_dkdv, 4),
            "bwd_frac_peak": round(rate(w.bwd_flops(), s_bwd) / PEAK_BF16_TFLOPS, 4)}
        log(f"steady step {s_step:.3f} ms ({rate(step_flops, s_step):.0f} TF): fwd {s_fwd:.3f} ms, "
            f"dq {s_dq:.3f} ms, dkdv {s_dkdv:.3f} ms, bwd {rate(w.bwd_flops(), s_bwd):.0f} TF")

    iters = max(5, a.steps)
    if not only or "fp8_bwd" in only:
        # the same causal step's backward with the fp8 dS products (K and Q
        # quantisers, fp8-dQ kernel, fp8-dK dK/dV kernel)
        ws8_bytes = fa.fa_bwd_fp8_workspace_size(*args)
        ws8 = torch.empty(ws8_bytes, dtype=torch.uint8, device="cuda")
        k8 = torch.empty(k.shape, dtype=torch.uint8, device="cuda")
        ke = torch.empty((w.B, w.Hkv, (w.Nk + 31) // 32), dtype=torch.uint8, device="cuda")

        def b8():
            fa.fa_bwd_fp8(q, k, v, o, do, lse, dq, dk, dv, ws8, ws8_bytes, *args, w.scale, True,
                          sh)

        def kq():
            # (the quantiser of K; Q's has the same shape here)
            fa.fa_quantize_pow2_e4m3(k, k8, ke, w.B, w.Hkv, w.Nk, w.d, sh)

        b8()
        t8 = timed(b8, iters, stream, a.settle_ms)
        tq = timed(kq, iters, stream, a.settle_ms)
        parts["fp8_bwd_causal"] = {
            "ms": round(t8, 4), "tflops": round(rate(w.bwd_flops(), t8), 1),
            "vs_bf16_bwd": round(bwd_ms / t8, 4), "quant_ms_each": round(tq, 4),
            "kernels_ms_est": round(t8 - 2 * tq, 4)}
        log(f"fp8 bwd {t8:.3f} ms (bf16 {bwd_ms:.3f}), quantiser {tq:.3f} ms each (K, Q)")
        del ws8, k8, ke
    if not only or "fwd" in only:
        t = timed(lambda: fwd(False), iters, stream, a.settle_ms)
        tf = 2 * w.fwd_flops() / (t * 1e-3) / 1e12
        parts["fwd_noncausal"] = {"ms": round(t, 4), "tflops": round(tf, 1),
                                  "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"fwd non-causal {t:.3f} ms {tf:.0f} TF")
    del x, q, k, v, do, o, dq, dk, dv, ws
    torch.cuda.empty_cache()

    if not only or "prefill" in only:
        wp = WORKLOADS["prefill_bf16"]
        xp = make_inputs(wp, device="cuda")
        op = torch.empty_like(xp["q"])
        lp = torch.empty(wp.B, wp.Hq, wp.Nq, dtype=torch.float32, device="cuda")
        f = lambda: fa.fa_fwd(xp["q"], xp["k"], xp["v"], op, lp, wp.B, wp.Hq, wp.Hkv, wp.Nq,
                              wp.Nk, wp.d, wp.scale, False, sh)
        f()
        t = timed(f, iters, stream, a.settle_ms)
        tf = wp.fwd_flops() / (t * 1e-3) / 1e12
        parts["fwd_prefill_d64"] = {"ms": round(t, 4), "tflops": round(tf, 1),
                                    "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"prefill d=64 {t:.3f} ms {tf:.0f} TF")
        del xp, op, lp

    if not only or "decode" in only:
        wd = WORKLOADS["decode_gqa"]
        log("decode inputs")
        xd = make_inputs(wd, device="cuda")
        S = wd.num_splits
        od = torch.empty_like(xd["q"])
        ld = torch.empty(wd.B, wd.Hq, 1, dtype=torch.float32, device="cuda")
        opart = torch.empty(wd.B, wd.Hq, S, wd.d, dtype=torch.float32, device="cuda")
        lpart = torch.empty(wd.B, wd.Hq, S, dtype=torch.float32, device="cuda")

        def split():
            fa.fa_decode_splitkv(xd["q"], xd["k"], xd["v"], opart, lpart, wd.B, wd.Hq, wd.Hkv,
                                 wd.Nk, wd.d, wd.scale, S, sh)

        def combine():
            fa.fa_decode_combine(opart, lpart, od, ld, wd.B, wd.Hq, wd.d, S, sh)

        split(); combine()
        t_all = timed(lambda: (split(), combine()), iters, stream, a.settle_ms)
        t_split = timed(split, iters, stream, a.settle_ms)
        t_comb = timed(combine, iters, stream, a.settle_ms)
        nbytes = 2 * wd.B * wd.Hkv * wd.Nk * wd.d * 2 + 2 * wd.B * wd.Hq * wd.d * 2 + wd.B * wd.Hq * 4
        gbs = nbytes / (t_all * 1e-3) / 1e9
        parts["decode"] = {"ms": round(t_all, 4), "split_ms": round(t_split, 4),
                           "combine_ms": round(t_comb, 4), "algorithmic_bytes": nbytes,
                           "GB/s": round(gbs, 1), "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
                           "split_GB/s": round(nbytes / (t_split * 1e-3) / 1e9, 1)}
        log(f"decode {t_all:.3f} ms {gbs:.0f} GB/s (split {t_split:.3f} ms)")
        # the same KV with 4 query tokens per head (causal, end-aligned): 16
        # columns of each tile instead of 4, the same K/V bytes
        NQ = 4
        qt = torch.randn(wd.B, wd.Hq, NQ, wd.d, device="cuda").to(torch.bfloat16)
        ot = torch.empty_like(qt)
        lt = torch.empty(wd.B, wd.Hq, NQ, dtype=torch.float32, device="cuda")
        opt = torch.empty(wd.B, wd.Hq, NQ, S, wd.d, dtype=torch.float32, device="cuda")
        lpt = torch.empty(wd.B, wd.Hq, NQ, S, dtype=torch.float32, device="cuda")

        def tokens():
            fa.fa_decode_splitkv_q(qt, xd["k"], xd["v"], opt, lpt, wd.B, wd.Hq, wd.Hkv, NQ, wd.Nk,
                                   wd.d, wd.scale, True, S, sh)
            fa.fa_decode_combine(opt, lpt, ot, lt, wd.B, wd.Hq * NQ, wd.d, S, sh)

        tokens()
        t_tok = timed(tokens, iters, stream, a.settle_ms)
        nb_tok = (2 * wd.B * wd.Hkv * wd.Nk * wd.d * 2 + 2 * wd.B * wd.Hq * NQ * wd.d * 2
                  + wd.B * wd.Hq * NQ * 4)
        gbs_tok = nb_tok / (t_tok * 1e-3) / 1e9
        parts["decode_tokens"] = {"ms": round(t_tok, 4), "tokens": NQ, "causal": True,
                                  "algorithmic_bytes": nb_tok, "GB/s": round(gbs_tok, 1),
                                  "frac_peak": round(gbs_tok / PEAK_HBM_GBS, 4)}
        log(f"decode {NQ} tokens {t_tok:.3f} ms {gbs_tok:.0f} GB/s")
        del xd, od, ld, opart, lpart, qt, ot, lt, opt, lpt

    if not only or "window" in only:
        from workloads import WINDOWED
        ww = WINDOWED["window_bf16"]
        log("window inputs")
        xw = make_inputs(ww, device="cuda")
        ow = torch.empty_like(xw["q"])
        lw = torch.empty(ww.B, ww.Hq, ww.Nq, dtype=torch.float32, device="cuda")
        dqw, dkw, dvw = (torch.empty_like(xw[n]) for n in ("q", "k", "v"))
        wsb = fa.fa_bwd_workspace_size(ww.B, ww.Hq, ww.Nq, ww.d)
        wsw = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        wa = (ww.B, ww.Hq, ww.Hkv, ww.Nq, ww.Nk, ww.d, ww.scale, ww.causal, ww.window_left,
              ww.window_right, sh)

        def wf():
            fa.fa_fwd_window(xw["q"], xw["k"], xw["v"], ow, lw, *wa)

        def wb():
            fa.fa_bwd_window(xw["q"], xw["k"], xw["v"], ow, xw["do"], lw, dqw, dkw, dvw, wsw, wsb,
                             *wa)

        wf(); wb()
        tfw = timed(wf, iters, stream, a.settle_ms)
        tbw = timed(wb, iters, stream, a.settle_ms)
        fl = ww.fwd_flops()
        parts["window_causal"] = {"window": [ww.window_left, ww.window_right],
                                  "fwd_ms": round(tfw, 4),
                                  "fwd_tflops": round(fl / (tfw * 1e-3) / 1e12, 1),
                                  "bwd_ms": round(tbw, 4),
                                  "bwd_tflops": round(2.5 * fl / (tbw * 1e-3) / 1e12, 1),
                                  "fwd_frac_peak": round(fl / (tfw * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "bwd_frac_peak": round(2.5 * fl / (tbw * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"window fwd {tfw:.3f} ms, bwd {tbw:.3f} ms")
        del xw, ow, lw, dqw, dkw, dvw, wsw

    if not only or "sparse" in only:
        from workloads import SPARSE
        wsp = SPARSE["sparse_bf16"]
        log("block-sparse inputs")
        xs = make_inputs(wsp, device="cuda")
        ptr, idx = wsp.pattern()
        pd = torch.tensor(ptr, dtype=torch.int32, device="cuda")
        idd = torch.tensor(idx, dtype=torch.int32, device="cuda")
        mb = max(ptr[i + 1] - ptr[i] for i in range(len(ptr) - 1))
        osp = torch.empty_like(xs["q"])
        lsp = torch.empty(wsp.B, wsp.Hq, wsp.Nq, dtype=torch.float32, device="cuda")

        def spf():
            fa.fa_fwd_block_sparse(xs["q"], xs["k"], xs["v"], osp, lsp, wsp.B, wsp.Hq, wsp.Hkv,
                                   wsp.Nq, wsp.Nk, wsp.d, wsp.scale, wsp.causal, pd, idd, mb, sh)

        spf()
        t = timed(spf, iters, stream, a.settle_ms)
        tf = wsp.fwd_flops() / (t * 1e-3) / 1e12
        parts["fwd_block_sparse"] = {"ms": round(t, 4), "tflops": round(tf, 1),
                                     "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                     "density": round(wsp.visible_pairs() / (wsp.Nq * wsp.Nk), 4)}
        log(f"block-sparse fwd {t:.3f} ms {tf:.0f} TF")
        dqs, dks, dvs = (torch.empty_like(xs[n]) for n in ("q", "k", "v"))
        wss_bytes = fa.fa_bwd_block_sparse_workspace_size(wsp.B, wsp.Hq, wsp.Nq, wsp.Nk, wsp.d)
        wss = torch.empty(wss_bytes, dtype=torch.uint8, device="cuda")

        def spb():
            fa.fa_bwd_block_sparse(xs["q"], xs["k"], xs["v"], osp, xs["do"], lsp, dqs, dks, dvs,
                                   wss, wss_bytes, wsp.B, wsp.Hq, wsp.Hkv, wsp.Nq, wsp.Nk, wsp.d,
                                   wsp.scale, wsp.causal, pd, idd, mb, sh)

        spb()
        tb = timed(spb, iters, stream, a.settle_ms)
        tfb = wsp.bwd_flops() / (tb * 1e-3) / 1e12
        parts["fwd_block_sparse"].update({"bwd_ms": round(tb, 4), "bwd_tflops": round(tfb, 1),
                                          "bwd_frac_peak": round(tfb / PEAK_BF16_TFLOPS, 4)})
        log(f"block-sparse bwd {tb:.3f} ms {tfb:.0f} TF")
        del xs, osp, lsp, dqs, dks, dvs, wss

    if not only or "decode_paged" in only:
        from workloads import PAGED, make_paged_inputs
        wg = PAGED["decode_paged"]
        log("paged decode inputs")
        xg = make_paged_inputs(wg, device="cuda")
        S = wg.num_splits
        og = torch.empty_like(xg["q"])
        lg = torch.empty(wg.B, wg.Hq, 1, dtype=torch.float32, device="cuda")
        opg = torch.empty(wg.B, wg.Hq, S, wg.d, dtype=torch.float32, device="cuda")
        lpg = torch.empty(wg.B, wg.Hq, S, dtype=torch.float32, device="cuda")
        mx = max(wg.seqlens)

        def paged():
            fa.fa_decode_splitkv_paged(xg["q"], xg["k_cache"], xg["v_cache"], xg["block_table"],
                                       xg["seqlens"], opg, lpg, wg.B, wg.Hq, wg.Hkv,
                                       wg.num_pages, wg.page_size, wg.max_pages, mx, wg.d,
                                       wg.scale, S, sh)
            fa.fa_decode_combine(opg, lpg, og, lg, wg.B, wg.Hq, wg.d, S, sh)

        paged()
        t = timed(paged, iters, stream, a.settle_ms)
        keys = sum(wg.seqlens)
        nbytes = 2 * keys * wg.Hkv * wg.d * 2 + 2 * wg.B * wg.Hq * wg.d * 2 + wg.B * wg.Hq * 4
        gbs = nbytes / (t * 1e-3) / 1e9
        parts["decode_paged"] = {"ms": round(t, 4), "page_size": wg.page_size,
                                 "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
                                 "frac_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"paged decode {t:.3f} ms {gbs:.0f} GB/s")
        del xg, og, lg, opg, lpg

    if not only or "varlen" in only:
        from workloads import VARLEN, make_varlen_inputs
        wv = VARLEN["varlen_bf16"]
        log("varlen inputs")
        xv = make_varlen_inputs(wv, device="cuda")
        ov = torch.empty_like(xv["q"])
        lv = torch.empty(wv.Hq, wv.total, dtype=torch.float32, device="cuda")
        mx = max(wv.seqlens)

        def vfwd():
            fa.fa_fwd_varlen(xv["q"], xv["k"], xv["v"], ov, lv, xv["cu"], xv["cu"],
                             len(wv.seqlens), wv.Hq, wv.Hkv, wv.total, wv.total, mx, mx, wv.d,
                             wv.scale, wv.causal, sh)

        vfwd()
        t = timed(vfwd, iters, stream, a.settle_ms)
        tf = wv.fwd_flops() / (t * 1e-3) / 1e12
        parts["fwd_varlen"] = {"ms": round(t, 4), "tflops": round(tf, 1),
                               "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                               "sequences": len(wv.seqlens), "tokens": wv.total}
        log(f"varlen fwd {t:.3f} ms {tf:.0f} TF")
        dqv, dkv, dvv = (torch.empty_like(xv[n]) for n in ("q", "k", "v"))
        wsv_bytes = fa.fa_bwd_workspace_size(1, wv.Hq, wv.total, wv.d)
        wsv = torch.empty(wsv_bytes, dtype=torch.uint8, device="cuda")

        def vbwd():
            fa.fa_bwd_varlen(xv["q"], xv["k"], xv["v"], ov, xv["do"], lv, dqv, dkv, dvv, wsv,
                             wsv_bytes, xv["cu"], xv["cu"], len(wv.seqlens), wv.Hq, wv.Hkv,
                             wv.total, wv.total, mx, mx, wv.d, wv.scale, wv.causal, sh)

        vbwd()
        tb = timed(vbwd, iters, stream, a.settle_ms)
        tfb = wv.bwd_flops() / (tb * 1e-3) / 1e12
        parts["fwd_varlen"].update({"bwd_ms": round(tb, 4), "bwd_tflops": round(tfb, 1),
                                    "bwd_frac_peak": round(tfb / PEAK_BF16_TFLOPS, 4)})
        log(f"varlen bwd {tb:.3f} ms {tfb:.0f} TF")
        del xv, ov, lv, dqv, dkv, dvv, wsv

    if not only or "fp8" in only:
        wf = WORKLOADS["fp8_fwd"]
        log("fp8 inputs")
        xf = make_inputs(wf, device="cuda")
        q8, qs = fa.quantize_fp8(xf["q"], xf["signs"])
        k8, ks = fa.quantize_fp8(xf["k"], xf["signs"])
        v8, vs = fa.quantize_fp8(xf["v"], None)
        of = torch.empty_like(xf["q"])
        lf = torch.empty(wf.B, wf.Hq, wf.Nq, dtype=torch.float32, device="cuda")

        def quant():
            fa.fa_quantize_fp8(xf["q"], xf["signs"], q8, qs, wf.B, wf.Hq, wf.Nq, wf.d, sh)
            fa.fa_quantize_fp8(xf["k"], xf["signs"], k8, ks, wf.B, wf.Hkv, wf.Nk, wf.d, sh)
            fa.fa_quantize_fp8(xf["v"], None, v8, vs, wf.B, wf.Hkv, wf.Nk, wf.d, sh)

        def f8():
            fa.fa_fwd_fp8(q8, k8, v8, qs, ks, vs, of, lf, wf.B, wf.Hq, wf.Hkv, wf.Nq, wf.Nk,
                          wf.d, wf.scale, False, sh)

        f8()
        t = timed(f8, iters, stream, a.settle_ms)
        tq = timed(quant, iters, stream, a.settle_ms)
        tf = wf.fwd_flops() / (t * 1e-3) / 1e12
        qbytes = 3 * wf.B * wf.Hq * wf.Nq * wf.d * (2 + 1)
        parts["fp8_fwd"] = {"ms": round(t, 4), "tflops": round(tf, 1),
                            "frac_peak_fp8": round(tf / PEAK_FP8_TFLOPS, 4),
                            "quant_ms": round(tq, 4),
                            "quant_GB/s": round(qbytes / (tq * 1e-3) / 1e9, 1),
                            "tflops_incl_quant": round(wf.fwd_flops() / ((t + tq) * 1e-3) / 1e12, 1)}
        log(f"fp8 fwd {t:.3f} ms {tf:.0f} TF, quant {tq:.3f} ms")
        # two heads of inputs and output, for the error against exact
        # attention measured in the CPU leg
        fp8_sample = {"q": xf["q"][0, :2].cpu(), "k": xf["k"][0, :2].cpu(),
                      "v": xf["v"][0, :2].cpu(), "o": of[0, :2].cpu(),
                      "signs": xf["signs"].cpu(), "heads": [[0, 0], [0, 1]]}
        del xf

    result = {
        "metric": "attention TFLOPS (fwd, bwd) bf16 N=8K d=128 as % MFMA peak; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal_bf16 forward+backward", "B": w.B, "H": w.Hq,
                   "seq_len": w.Nq, "head_dim": w.d, "causal": True,
                   "flops_per_step": step_flops, "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
                   "wall_s": round(wall, 3)},
        "roofline": {"kernel": dom, "bound": "mfma",
                     "achieved": round(rate(*kern[dom]), 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(rate(*kern[dom]) / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if dom.startswith("bwd_dkdv") else None,
                     "algorithmic_flops_per_launch": kern[dom][0],
                     "avg_launch_ms": round(kern[dom][1], 4)},
        "parts": parts,
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"], fp8_err = cpu_baseline(fp8_sample)
        if fp8_err is not None:
            parts["fp8_fwd"].update(fp8_err)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
