"""Full-size parity: every row of every head of the benchmark's workloads, in
the launch configuration the benchmark times, against the fp64 oracle.

The GPU runs each workload once per module (a module-scoped fixture keeps its
outputs on the host as bf16/fp32 tensors); the oracle then checks the heads in
groups, so each test stays well inside the per-test time limit.  Every call
goes through the C ABI.

Tolerances as in the small-shape parity tests: bf16 O max-abs 1e-2, LSE
max-abs 1e-3, gradients relative L2 1e-2 (here per head, stricter than over
the whole tensor); the fp8 forward relative L2 5e-2 per head against the
oracle's own fp8 pipeline run from the same bf16 inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from tests.conftest import say
from workloads import SPARSE, VARLEN, WINDOWED, WORKLOADS, make_inputs, make_varlen_inputs

pytestmark = pytest.mark.gpu

BF16_O, BF16_LSE, BF16_GRAD = 1e-2, 1e-3, 1e-2
FP8_REL = 5e-2
GROUPS = 4


def f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def maxabs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def group_heads(B, H, g):
    """(b, h) pairs of head group g out of GROUPS (flat index b*H + h)."""
    n = B * H
    per = -(-n // GROUPS)
    return [divmod(i, H) for i in range(g * per, min(n, (g + 1) * per))]


def host(ts):
    return {n: t.cpu() for n, t in ts.items()}


def check_head(label, got, want):
    """got/want: (o, lse, dq, dk, dv) of one head (got from the GPU)."""
    eo, el = maxabs(got[0], want[0]), maxabs(got[1], want[1])
    assert eo <= BF16_O and el <= BF16_LSE, (label, eo, el)
    for name, a, b in zip(("dq", "dk", "dv"), got[2:], want[2:]):
        e = rel_l2(a, b)
        assert e <= BF16_GRAD, (label, name, e)


# ------------------------------------------------- causal B2 H16 N8192 d128

@pytest.fixture(scope="module")
def causal_run(fa_gpu):
    w = WORKLOADS["causal_bf16"]
    x = make_inputs(w)
    xc = {n: t.cuda() for n, t in x.items()}
    say("causal_bf16 full size: forward + backward on the GPU")
    o, lse = fa_gpu.forward(xc["q"], xc["k"], xc["v"], causal=True)
    dq, dk, dv = fa_gpu.backward(xc["q"], xc["k"], xc["v"], o, lse, xc["do"], causal=True)
    torch.cuda.synchronize()
    return w, x, host(dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))


@pytest.mark.parametrize("g", range(GROUPS))
def test_causal_config_all_heads(causal_run, g):
    """B=2 H=16 N=8192 d=128 causal: every O/LSE row and the complete
    dQ/dK/dV of each head in this group."""
    w, x, r = causal_run
    for b, h in group_heads(w.B, w.Hq, g):
        say(f"causal_bf16 oracle head ({b},{h})")
        want = A.head_forward_backward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                                       f64(x["do"][b, h]), w.scale, True)
        got = [f64(r[n][b, h]) for n in ("o", "lse", "dq", "dk", "dv")]
        check_head((b, h), got, want)


# ------------------------------------------ sliding window (4096, 0), causal

@pytest.fixture(scope="module")
def window_run(fa_gpu):
    w = WINDOWED["window_bf16"]
    x = make_inputs(w)
    xc = {n: t.cuda() for n, t in x.items()}
    win = (w.window_left, w.window_right)
    say("window_bf16 full size: forward + backward on the GPU")
    o, lse = fa_gpu.forward(xc["q"], xc["k"], xc["v"], causal=w.causal, window=win)
    dq, dk, dv = fa_gpu.backward(xc["q"], xc["k"], xc["v"], o, lse, xc["do"], causal=w.causal,
                                 window=win)
    torch.cuda.synchronize()
    return w, x, host(dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))


@pytest.mark.parametrize("g", range(GROUPS))
def test_window_config_all_heads(window_run, g):
    """B=2 H=16 N=8192 d=128, causal with a 4096-key left window: every
    O/LSE row and the complete gradients of each head in this group."""
    w, x, r = window_run
    win = (w.window_left, w.window_right)
    for b, h in group_heads(w.B, w.Hq, g):
        say(f"window_bf16 oracle head ({b},{h})")
        want = A.head_forward_backward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                                       f64(x["do"][b, h]), w.scale, w.causal, window=win)
        got = [f64(r[n][b, h]) for n in ("o", "lse", "dq", "dk", "dv")]
        check_head((b, h), got, want)


# ------------------------------------------- block-sparse local + global

@pytest.fixture(scope="module")
def sparse_run(fa_gpu):
    w = SPARSE["sparse_bf16"]
    x = make_inputs(w)
    xc = {n: t.cuda() for n, t in x.items()}
    ptr, idx = w.pattern()
    pd = torch.tensor(ptr, dtype=torch.int32, device="cuda")
    idd = torch.tensor(idx, dtype=torch.int32, device="cuda")
    say("sparse_bf16 full size: forward + backward on the GPU")
    o, lse = fa_gpu.forward_block_sparse(xc["q"], xc["k"], xc["v"], pd, idd)
    dq, dk, dv = fa_gpu.backward_block_sparse(xc["q"], xc["k"], xc["v"], o, lse, xc["do"], pd,
                                              idd)
    torch.cuda.synchronize()
    return w, x, (ptr, idx), host(dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))


@pytest.mark.parametrize("g", range(GROUPS))
def test_block_sparse_config_all_heads(sparse_run, g):
    """B=2 H=16 N=8192 d=128 with the local (+-1024 keys) + global (first 256
    keys) pattern: every O/LSE row and the complete gradients of each head
    in this group, against the oracle restricted to that head."""
    w, x, (ptr, idx), r = sparse_run
    for b, h in group_heads(w.B, w.Hq, g):
        say(f"sparse_bf16 oracle head ({b},{h})")
        one = [f64(x[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v", "do")]
        ro, rl = A.forward_block_sparse(*one[:3], w.scale, ptr, idx, w.block_q, w.block_k)
        rq, rk, rv = A.backward_block_sparse(*one, w.scale, ptr, idx, w.block_q, w.block_k)
        want = (ro[0, 0], rl[0, 0], rq[0, 0], rk[0, 0], rv[0, 0])
        got = [f64(r[n][b, h]) for n in ("o", "lse", "dq", "dk", "dv")]
        check_head((b, h), got, want)


# ------------------------------------------------ packed variable length

@pytest.fixture(scope="module")
def varlen_run(fa_gpu):
    w = VARLEN["varlen_bf16"]
    x = make_varlen_inputs(w, device="cuda")
    mx = max(w.seqlens)
    say("varlen_bf16 full size: forward + backward on the GPU")
    o, lse = fa_gpu.forward_varlen(x["q"], x["k"], x["v"], x["cu"], x["cu"], mx, mx,
                                   causal=w.causal)
    dq, dk, dv = fa_gpu.backward_varlen(x["q"], x["k"], x["v"], o, lse, x["do"], x["cu"],
                                        x["cu"], mx, mx, causal=w.causal)
    torch.cuda.synchronize()
    return w, host(x), host(dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))


@pytest.mark.parametrize("g", range(GROUPS))
def test_varlen_config_all_heads(varlen_run, g):
    """The packed workload (10 sequences, 31706 tokens, H=16, d=128, causal):
    every row of every sequence for the heads of this group, forward and
    backward, against the oracle on each sequence's own slice."""
    w, x, r = varlen_run
    cu = x["cu"].tolist()
    heads = [h for _, h in group_heads(1, w.Hq, g)]
    for h in heads:
        for b in range(len(w.seqlens)):
            sl = slice(cu[b], cu[b + 1])
            say(f"varlen_bf16 oracle head {h} sequence {b} ({cu[b + 1] - cu[b]} tokens)")
            want = A.head_forward_backward(*(f64(x[n][sl, h]) for n in ("q", "k", "v", "do")),
                                           w.scale, w.causal)
            got = [f64(r["o"][sl, h]), f64(r["lse"][h, sl]), f64(r["dq"][sl, h]),
                   f64(r["dk"][sl, h]), f64(r["dv"][sl, h])]
            check_head((b, h), got, want)


# ------------------------------------------------------ fp8 forward (C5)

@pytest.fixture(scope="module")
def fp8_run(fa_gpu):
    w = WORKLOADS["fp8_fwd"]
    x = make_inputs(w)
    xc = {n: t.cuda() for n, t in x.items()}
    say("fp8_fwd full size: quantiser (rotated Q, K) + fp8 forward on the GPU")
    q8, qs = fa_gpu.quantize_fp8(xc["q"], xc["signs"])
    k8, ks = fa_gpu.quantize_fp8(xc["k"], xc["signs"])
    v8, vs = fa_gpu.quantize_fp8(xc["v"], None)
    o, lse = fa_gpu.forward_fp8(q8, k8, v8, qs, ks, vs)
    torch.cuda.synchronize()
    return w, x, host(dict(o=o, lse=lse))


def oracle_fp8_head(x, b, h, scale):
    """The oracle's own fp8 pipeline for one head, from the bf16 inputs:
    rotate Q and K (fp32 result), per-128-row-block e4m3 quantisation of Q, K
    and V, dequantise, exact forward on the dequantised operands."""
    signs = x["signs"].double().numpy()
    qr = F8.rotate(f64(x["q"][b:b + 1, h:h + 1]), signs).astype(np.float32)
    kr = F8.rotate(f64(x["k"][b:b + 1, h:h + 1]), signs).astype(np.float32)
    vv = x["v"][b:b + 1, h:h + 1].float().numpy()
    deq = [F8.dequantize(*F8.quantize(t)) for t in (qr, kr, vv)]
    o, lse = A.forward(*deq, scale, False)
    return o[0, 0], lse[0, 0]


@pytest.mark.parametrize("g", range(GROUPS))
def test_fp8_config_all_heads(fp8_run, g):
    """B=2 H=16 N=8192 d=128 with 0.1% outliers of magnitude 50 in Q and K,
    rotated: for every head of this group, all 8192 rows of O against the
    oracle's fp8 pipeline run from the same bf16 inputs (relative L2 per
    head <= 5e-2), and against exact attention on the unquantised inputs no
    worse than that pipeline's own error (the e4m3 floor) plus the P
    rounding of the fp8 PV product."""
    w, x, r = fp8_run
    for b, h in group_heads(w.B, w.Hq, g):
        say(f"fp8_fwd oracle head ({b},{h})")
        ro, rl = oracle_fp8_head(x, b, h, w.scale)
        og = f64(r["o"][b, h])
        e = rel_l2(og, ro)
        row = np.linalg.norm(og - ro, axis=1) / np.linalg.norm(ro, axis=1)
        exact, _ = A.head_forward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                                  w.scale, False)
        e_hip, e_floor = rel_l2(og, exact), rel_l2(ro, exact)
        print(f"head ({b},{h}): vs fp8 oracle {e:.4f} (rows: p99 {np.quantile(row, 0.99):.4f} "
              f"max {row.max():.4f}); vs exact {e_hip:.4f}, oracle fp8 vs exact {e_floor:.4f}")
        assert e <= FP8_REL, (b, h, e)
        assert e_hip <= 1.15 * e_floor, (b, h, e_hip, e_floor)


@pytest.mark.xfail(strict=True, reason="e4m3 Q/K on the outlier workload: measured relative L2 "
                   "about 0.11 against exact attention (the format's floor at any block size; "
                   "0.045 without outliers), above the 5e-2 bar")
def test_fp8_config_against_exact_attention(fp8_run):
    """The 5e-2 bar read against exact attention on the unquantised inputs
    (two heads, one of each batch entry)."""
    w, x, r = fp8_run
    for b, h in ((0, 5), (1, 10)):
        say(f"fp8_fwd exact attention head ({b},{h})")
        exact, _ = A.head_forward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                                  w.scale, False)
        e = rel_l2(f64(r["o"][b, h]), exact)
        assert e <= FP8_REL, (b, h, e)
