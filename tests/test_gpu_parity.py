"""Parity of the HIP path against the fp64 oracle, element by element, on the
same seeded inputs.  Every call goes through the C ABI (ctypes binding).

Tolerances (the accuracy bars the library is held to):
  bf16, fp32 accumulation: O max-abs <= 1e-2, LSE max-abs <= 1e-3,
                           dQ/dK/dV relative L2 <= 1e-2
  fp32 tiny configuration: all of the above <= 1e-5
  fp8 forward:             relative L2 of O <= 5e-2 against the oracle fed the
                           dequantised operands the kernel receives (the
                           full-size fp8 check runs the oracle's own pipeline
                           from the bf16 inputs)
The full-size checks of every head of the benchmark's workloads are in
test_gpu_full_size.py.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from tests.conftest import say
from workloads import WORKLOADS, make_inputs, to_f64

pytestmark = pytest.mark.gpu

BF16_O, BF16_LSE, BF16_GRAD = 1e-2, 1e-3, 1e-2
F32_TOL = 1e-5
FP8_REL = 5e-2


def maxabs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def rel_l2(a, b):
    """Relative L2 error of a against b.  Where b is exactly zero (a single key:
    P = 1, so dS = dP - delta = 0 and dQ = dK = 0) the relative error is
    undefined and the absolute L2 error is returned instead."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def gen(B, Hq, Hkv, Nq, Nk, d, dtype, seed, grad=False):
    g = torch.Generator("cpu").manual_seed(seed)
    t = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn(B, Hq, Nq, d, generator=g).to(t)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(t)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(t)
    out = {"q": q.cuda(), "k": k.cuda(), "v": v.cuda()}
    if grad:
        out["do"] = torch.randn(B, Hq, Nq, d, generator=g).to(t).cuda()
    return out


# ------------------------------------------------------------------ forward

def check_forward(fa, x, causal, o_tol, lse_tol, label):
    q, k, v = x["q"], x["k"], x["v"]
    d = q.shape[-1]
    say(f"forward {label} shape={tuple(q.shape)} kv={tuple(k.shape)} causal={causal}")
    o, lse = fa.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(d), causal)
    eo, el = maxabs(to_f64(o), o_ref), maxabs(to_f64(lse), lse_ref)
    assert eo <= o_tol and el <= lse_tol, (label, eo, el)
    return o, lse


def test_tiny_f32_config(fa_gpu):
    """fp32 B=1 H=1 N=256 d=64: 64-row tiles, four KV blocks of rescaling."""
    w = WORKLOADS["tiny_f32"]
    x = make_inputs(w)
    x = {n: t.cuda() for n, t in x.items()}
    o, lse = check_forward(fa_gpu, x, False, F32_TOL, F32_TOL, "tiny_f32")
    say("backward tiny_f32")
    dq, dk, dv = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=False)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), w.scale, False)
    for got, want in zip((dq, dk, dv), ref):
        assert rel_l2(to_f64(got), want) <= F32_TOL


@pytest.mark.parametrize("shape,causal", [
    ((1, 2, 1, 200, 200), True), ((2, 4, 2, 130, 70), False), ((1, 1, 1, 64, 64), True)])
def test_f32_variants(fa_gpu, shape, causal):
    B, Hq, Hkv, Nq, Nk = shape
    x = gen(B, Hq, Hkv, Nq, Nk, 64, "f32", 11, grad=True)
    o, lse = check_forward(fa_gpu, x, causal, F32_TOL, F32_TOL, f"f32 {shape}")
    say(f"backward f32 {shape} causal={causal}")
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), 1 / 8, causal)
    for got, want in zip(grads, ref):
        assert rel_l2(to_f64(got), want) <= F32_TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 333, 333), (2, 2, 2, 256, 256), (1, 3, 1, 129, 129),
                                   (1, 2, 2, 40, 40), (2, 2, 1, 100, 100), (1, 1, 1, 1, 1)])
def test_bf16_forward_small(fa_gpu, d, causal, shape):
    B, Hq, Hkv, Nq, Nk = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 21)
    check_forward(fa_gpu, x, causal, BF16_O, BF16_LSE, f"bf16 d={d}")


def test_bf16_forward_cross_lengths(fa_gpu):
    """Non-causal with Nq != Nk and ragged tails on both sides."""
    x = gen(1, 2, 1, 77, 1000, 128, "bf16", 22)
    check_forward(fa_gpu, x, False, BF16_O, BF16_LSE, "Nq=77 Nk=1000")


def test_prefill_config(fa_gpu):
    """bf16 B=4 H=16 N=2048 d=64 non-causal, every output compared."""
    w = WORKLOADS["prefill_bf16"]
    x = {n: t.cuda() for n, t in make_inputs(w).items()}
    check_forward(fa_gpu, x, False, BF16_O, BF16_LSE, "prefill_bf16")


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 256, 256), (1, 4, 2, 300, 300), (2, 1, 1, 129, 129),
                                   (1, 2, 2, 40, 40), (1, 1, 1, 1, 1)])
def test_bf16_backward_small(fa_gpu, d, causal, shape):
    B, Hq, Hkv, Nq, Nk = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 31, grad=True)
    o, lse = check_forward(fa_gpu, x, causal, BF16_O, BF16_LSE, f"bwd-prep d={d}")
    say(f"backward bf16 d={d} shape={shape} causal={causal}")
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), 1 / math.sqrt(d), causal)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= BF16_GRAD, (name, e)


@pytest.mark.parametrize("shape", [(1, 2, 1, 300, 700, 128), (2, 4, 2, 777, 129, 64),
                                   (1, 2, 2, 64, 4000, 128), (1, 1, 1, 1000, 33, 128)])
def test_bf16_backward_unequal_lengths(fa_gpu, shape):
    """Non-causal backward with Nq != Nk (more keys than queries and the
    reverse, ragged on both sides, GQA), against the oracle."""
    B, Hq, Hkv, Nq, Nk, d = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 32, grad=True)
    o, lse = check_forward(fa_gpu, x, False, BF16_O, BF16_LSE, f"bwd-prep Nq={Nq} Nk={Nk}")
    say(f"backward bf16 unequal lengths shape={shape}")
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=False)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), 1 / math.sqrt(d), False)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= BF16_GRAD, (name, e)


def _random_shapes(n, seed):
    rs = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rs.choice([1, 2, 3]))
        g = int(rs.choice([1, 2, 4]))
        causal = bool(rs.integers(0, 2))
        nq = int(rs.integers(1, 700))
        nk = nq if causal else int(rs.integers(1, 700))
        out.append((int(rs.integers(1, 3)), hkv * g, hkv, nq, nk, int(rs.choice([64, 128])), causal))
    return out


@pytest.mark.parametrize("shape", _random_shapes(12, 2026))
def test_random_shapes_forward_backward(fa_gpu, shape):
    """Seeded random shapes (batch, group size, lengths from 1 to 699, both
    head dims, causal or not): forward and backward against the oracle."""
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 96, grad=True)
    o, lse = check_forward(fa_gpu, x, causal, BF16_O, BF16_LSE, f"random {shape}")
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), 1 / math.sqrt(d), causal)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= BF16_GRAD, (name, e)


def test_long_sequence_causal(fa_gpu):
    """N = 65536 (eight times the benchmark length; GQA 2:1, d = 128, causal):
    sampled forward rows and dQ rows against the oracle row by row, and two
    identities that hold at any size and test every dK and dV: the keys' dK
    sum to zero (each row of dS sums to zero) and the keys' dV sum to the
    sum of dO over the query rows and heads (each row of P sums to one)."""
    N, d = 65536, 128
    x = gen(1, 2, 1, N, N, d, "bf16", 95, grad=True)
    say("long sequence N=65536 forward")
    o, lse = fa_gpu.forward(x["q"], x["k"], x["v"], causal=True)
    say("long sequence N=65536 backward")
    dq, dk, dv = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    rows = np.array([0, 1, 255, 256, 12345, 32767, 40000, 65535])
    ro, rl = A.forward(q, k, v, scale, True, rows=rows)
    assert maxabs(to_f64(o)[:, :, rows], ro) <= BF16_O
    assert maxabs(to_f64(lse)[:, :, rows], rl) <= BF16_LSE
    dq = to_f64(dq)
    for h in range(2):
        want = A.head_dq_rows(q[0, h], k[0, 0], v[0, 0], do[0, h], scale, True, rows)
        assert rel_l2(dq[0, h, rows], want) <= BF16_GRAD, h
    dk, dv = to_f64(dk)[0, 0], to_f64(dv)[0, 0]
    assert rel_l2(dv.sum(axis=0), do[0].sum(axis=(0, 1))) <= BF16_GRAD
    assert np.linalg.norm(dk.sum(axis=0)) <= 2e-2 * np.linalg.norm(dk)


def test_hip_graph_replays_match_eager(fa_gpu):
    """The forward, the backward and the split decode + combine captured in
    one HIP graph (no allocation or memset inside the library calls): three
    replays, with new inputs copied in eagerly and a synchronisation between
    them, each bit-identical to the eager calls on the same inputs."""
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    x = gen(B, Hq, Hkv, N, N, d, "bf16", 97, grad=True)
    xd = gen(2, 8, 2, 1, 4096, d, "bf16", 98)
    S = 8
    o = torch.empty_like(x["q"])
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x[n]) for n in ("q", "k", "v"))
    wsb = fa_gpu.fa_bwd_workspace_size(B, Hq, N, d)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    op = torch.empty(2, 8, S, d, dtype=torch.float32, device="cuda")
    lp = torch.empty(2, 8, S, dtype=torch.float32, device="cuda")
    od = torch.empty_like(xd["q"])
    ld = torch.empty(2, 8, 1, dtype=torch.float32, device="cuda")
    sc = 1 / math.sqrt(d)

    def work():
        fa_gpu.fa_fwd(x["q"], x["k"], x["v"], o, lse, B, Hq, Hkv, N, N, d, sc, True)
        fa_gpu.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, ws, wsb, B, Hq, Hkv,
                      N, N, d, sc, True)
        fa_gpu.fa_decode_splitkv(xd["q"], xd["k"], xd["v"], op, lp, 2, 8, 2, 4096, d, sc, S)
        fa_gpu.fa_decode_combine(op, lp, od, ld, 2, 8, d, S)

    say("hip graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()  # warm the launch path outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    g = torch.Generator("cpu").manual_seed(99)
    for rep in range(3):
        for t in (x["q"], x["k"], x["v"], x["do"], xd["q"], xd["k"], xd["v"]):
            t.copy_(torch.randn(t.shape, generator=g).to(t.dtype).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv, od, ld)]
        work()
        torch.cuda.synchronize()
        for a_, b_ in zip(got, (o, lse, dq, dk, dv, od, ld)):
            assert torch.equal(a_, b_), rep


def test_backward_is_deterministic(fa_gpu):
    """No atomics and a fixed accumulation order: repeated backward passes
    (plain and windowed, GQA, causal) give bit-identical gradients."""
    x = gen(2, 8, 2, 1500, 1500, 128, "bf16", 93, grad=True)
    say("backward determinism")
    o, lse = fa_gpu.forward(x["q"], x["k"], x["v"], causal=True)
    runs = [fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=True)
            for _ in range(3)]
    ow, lw = fa_gpu.forward(x["q"], x["k"], x["v"], causal=True, window=(300, 0))
    runs_w = [fa_gpu.backward(x["q"], x["k"], x["v"], ow, lw, x["do"], causal=True,
                              window=(300, 0)) for _ in range(3)]
    torch.cuda.synchronize()
    for rr in (runs, runs_w):
        for r in rr[1:]:
            for a, b in zip(r, rr[0]):
                assert torch.equal(a, b)


# ----------------------------------------------------------- sliding window

WINDOWS = [(37, 5), (0, 0), (200, -1), (-1, 100), (300, 300), (1000, 0), (64, 63)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,shape", [(128, (1, 4, 2, 700)), (64, (2, 2, 1, 1111))])
def test_window_forward_backward_small(fa_gpu, window, causal, d, shape):
    B, Hq, Hkv, N = shape
    x = gen(B, Hq, Hkv, N, N, d, "bf16", 91, grad=True)
    say(f"window fwd+bwd window={window} causal={causal} d={d} shape={shape}")
    o, lse = fa_gpu.forward(x["q"], x["k"], x["v"], causal=causal, window=window)
    torch.cuda.synchronize()
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ro, rl = A.forward(q, k, v, 1 / math.sqrt(d), causal, window=window)
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(to_f64(lse), rl) <= BF16_LSE
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal,
                            window=window)
    torch.cuda.synchronize()
    ref = A.backward(q, k, v, do, 1 / math.sqrt(d), causal, window=window)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= BF16_GRAD, (name, e)


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_everything_equals_dense(fa_gpu, causal):
    """A window wider than the sequence runs the windowed kernels with every
    mask test false: outputs and gradients equal the plain kernels' bit for
    bit."""
    N = 1000
    x = gen(2, 4, 2, N, N, 128, "bf16", 92, grad=True)
    say(f"window covering everything causal={causal}")
    o, lse = fa_gpu.forward(x["q"], x["k"], x["v"], causal=causal)
    ow, lw = fa_gpu.forward(x["q"], x["k"], x["v"], causal=causal, window=(N, N))
    g = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
    gw = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal, window=(N, N))
    torch.cuda.synchronize()
    assert torch.equal(o, ow) and torch.equal(lse, lw)
    for a, b in zip(g, gw):
        assert torch.equal(a, b)


# ------------------------------------------------------------- block-sparse

def random_pattern(nq, nk, seed, p=0.4):
    """Random CSR lists (shuffled, some empty) over nq query tiles, nk key blocks."""
    rs = np.random.default_rng(seed)
    ptr, idx = [0], []
    for t in range(nq):
        blocks = [c for c in range(nk) if rs.random() < p] if t % 3 != 1 else []
        rs.shuffle(blocks)
        idx += blocks
        ptr.append(len(idx))
    return ptr, idx


@pytest.mark.parametrize("shape,causal", [((1, 4, 2, 700, 700, 128), False),
                                          ((1, 4, 2, 700, 700, 128), True),
                                          ((2, 2, 1, 513, 600, 64), False),
                                          ((1, 2, 2, 1100, 1100, 128), True)])
def test_block_sparse_small(fa_gpu, shape, causal):
    """Random shuffled lists with empty query tiles (their rows: O = 0,
    LSE = -inf) and ragged ends, against the oracle."""
    B, Hq, Hkv, Nq, Nk, d = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 101)
    nq, nk = -(-Nq // fa_gpu.SPARSE_BLOCK_Q), -(-Nk // fa_gpu.SPARSE_BLOCK_K)
    ptr, idx = random_pattern(nq, nk, 7 + Nq)
    say(f"block-sparse fwd shape={shape} causal={causal} nnz={len(idx)}")
    pd = torch.tensor(ptr, dtype=torch.int32, device="cuda")
    idd = torch.tensor(idx if idx else [0], dtype=torch.int32, device="cuda")
    o, lse = fa_gpu.forward_block_sparse(x["q"], x["k"], x["v"], pd, idd, causal=causal)
    torch.cuda.synchronize()
    ro, rl = A.forward_block_sparse(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]),
                                    1 / math.sqrt(d), ptr, idx, fa_gpu.SPARSE_BLOCK_Q,
                                    fa_gpu.SPARSE_BLOCK_K, causal)
    got_o, got_l = to_f64(o), to_f64(lse)
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(got_l), dead)
    assert not np.any(got_o[dead])
    assert maxabs(got_o, ro) <= BF16_O
    assert maxabs(got_l[~dead], rl[~dead]) <= BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_all_blocks_equals_dense(fa_gpu, causal):
    """Every key block listed in ascending order: the same tiles in the same
    order as the dense kernel, so outputs agree bit for bit."""
    N = 1000
    x = gen(2, 4, 2, N, N, 128, "bf16", 102)
    nq, nk = -(-N // fa_gpu.SPARSE_BLOCK_Q), -(-N // fa_gpu.SPARSE_BLOCK_K)
    ptr = [t * nk for t in range(nq + 1)]
    idx = list(range(nk)) * nq
    say(f"block-sparse all blocks causal={causal}")
    o, lse = fa_gpu.forward_block_sparse(x["q"], x["k"], x["v"],
                                         torch.tensor(ptr, dtype=torch.int32, device="cuda"),
                                         torch.tensor(idx, dtype=torch.int32, device="cuda"),
                                         causal=causal)
    od, ld = fa_gpu.forward(x["q"], x["k"], x["v"], causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(lse, ld)


@pytest.mark.parametrize("shape,causal", [((1, 4, 2, 700, 700, 128), False),
                                          ((1, 4, 2, 700, 700, 128), True),
                                          ((2, 2, 1, 513, 600, 64), False),
                                          ((1, 2, 2, 1100, 1100, 128), True)])
def test_block_sparse_backward_small(fa_gpu, shape, causal):
    """Random shuffled lists with empty query tiles and ragged ends (rows that
    see no key: dQ = 0; keys no row sees: dK = dV = 0), against the oracle."""
    B, Hq, Hkv, Nq, Nk, d = shape
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 103, grad=True)
    nq, nk = -(-Nq // fa_gpu.SPARSE_BLOCK_Q), -(-Nk // fa_gpu.SPARSE_BLOCK_K)
    ptr, idx = random_pattern(nq, nk, 11 + Nq)
    say(f"block-sparse bwd shape={shape} causal={causal} nnz={len(idx)}")
    pd = torch.tensor(ptr, dtype=torch.int32, device="cuda")
    idd = torch.tensor(idx if idx else [0], dtype=torch.int32, device="cuda")
    o, lse = fa_gpu.forward_block_sparse(x["q"], x["k"], x["v"], pd, idd, causal=causal)
    grads = fa_gpu.backward_block_sparse(x["q"], x["k"], x["v"], o, lse, x["do"], pd, idd,
                                         causal=causal)
    torch.cuda.synchronize()
    ref = A.backward_block_sparse(*(to_f64(x[n]) for n in ("q", "k", "v", "do")),
                                  1 / math.sqrt(d), ptr, idx, fa_gpu.SPARSE_BLOCK_Q,
                                  fa_gpu.SPARSE_BLOCK_K, causal)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        g = to_f64(got)
        assert np.all(np.isfinite(g)), name
        e = rel_l2(g, want)
        assert e <= BF16_GRAD, (name, e)
    ok = A.block_sparse_allowed(Nq, Nk, ptr, idx, fa_gpu.SPARSE_BLOCK_Q, fa_gpu.SPARSE_BLOCK_K,
                                causal)
    dq, dk, dv = (to_f64(t) for t in grads)
    assert not dq[:, :, ~ok.any(axis=1)].any()
    assert not dk[:, :, ~ok.any(axis=0)].any() and not dv[:, :, ~ok.any(axis=0)].any()


def test_block_sparse_backward_rows_without_keys(fa_gpu):
    """Causal pattern whose first query tile lists only a later key block:
    rows before that block see nothing (LSE = -inf) and must get dQ = 0 with
    no NaN, while the block's keys still get gradients from later rows."""
    N, d = 700, 128
    x = gen(1, 2, 2, N, N, d, "bf16", 104, grad=True)
    ptr, idx = [0, 1, 3, 5], [2, 0, 5, 8, 10]     # tile 0 -> keys 128..191 only
    pd = torch.tensor(ptr, dtype=torch.int32, device="cuda")
    idd = torch.tensor(idx, dtype=torch.int32, device="cuda")
    say("block-sparse bwd rows without keys")
    o, lse = fa_gpu.forward_block_sparse(x["q"], x["k"], x["v"], pd, idd, causal=True)
    grads = fa_gpu.backward_block_sparse(x["q"], x["k"], x["v"], o, lse, x["do"], pd, idd,
                                         causal=True)
    torch.cuda.synchronize()
    assert np.isneginf(to_f64(lse)[0, 0, 0])
    ref = A.backward_block_sparse(*(to_f64(x[n]) for n in ("q", "k", "v", "do")),
                                  1 / math.sqrt(d), ptr, idx, 256, 64, True)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        g = to_f64(got)
        assert np.all(np.isfinite(g)), name
        assert rel_l2(g, want) <= BF16_GRAD, name
    assert not to_f64(grads[0])[:, :, :128].any()


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_all_blocks_equals_dense(fa_gpu, causal):
    """Every key block listed in ascending order: dQ visits the same tiles in
    the same order as the dense kernel, and every dK/dV unit the same query
    tiles, so the gradients agree bit for bit."""
    N = 1000
    x = gen(2, 4, 2, N, N, 128, "bf16", 105, grad=True)
    nq, nk = -(-N // fa_gpu.SPARSE_BLOCK_Q), -(-N // fa_gpu.SPARSE_BLOCK_K)
    pd = torch.tensor([t * nk for t in range(nq + 1)], dtype=torch.int32, device="cuda")
    idd = torch.tensor(list(range(nk)) * nq, dtype=torch.int32, device="cuda")
    say(f"block-sparse bwd all blocks causal={causal}")
    o, lse = fa_gpu.forward(x["q"], x["k"], x["v"], causal=causal)
    gs = fa_gpu.backward_block_sparse(x["q"], x["k"], x["v"], o, lse, x["do"], pd, idd,
                                      causal=causal)
    gd = fa_gpu.backward(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(gs, gd):
        assert torch.equal(a, b)


# ------------------------------------------------------------------- decode

def check_decode(fa, B, Hq, Hkv, Nk, d, splits, seed):
    x = gen(B, Hq, Hkv, 1, Nk, d, "bf16", seed)
    say(f"decode B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} d={d} splits={splits}")
    o, lse, op, lp = fa.decode(x["q"], x["k"], x["v"], splits, return_partials=True)
    torch.cuda.synchronize()
    ref = A.decode_split(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), 1 / math.sqrt(d), splits)
    assert maxabs(to_f64(o), ref[0]) <= BF16_O
    assert maxabs(to_f64(lse), ref[1]) <= BF16_LSE
    assert maxabs(to_f64(op), ref[2]) <= BF16_O
    assert maxabs(to_f64(lp), ref[3]) <= BF16_LSE
    return x, o, lse


@pytest.mark.parametrize("cfg", [
    (2, 8, 2, 4096, 128, 8), (1, 4, 4, 1000, 128, 8), (2, 16, 2, 2048, 64, 4),
    (1, 32, 1, 640, 128, 5), (3, 6, 2, 96, 128, 3)])
def test_decode_small(fa_gpu, cfg):
    check_decode(fa_gpu, *cfg, seed=41)


@pytest.mark.parametrize("cfg", [
    # B, Hq, Hkv, Nq, Nk, d, splits
    (2, 8, 2, 4, 4096, 128, 8),     # 4 heads x 4 tokens
    (1, 32, 4, 4, 2000, 128, 10),   # 8 heads x 4 tokens = 32 columns, ragged chunks of 200
    (2, 4, 4, 32, 640, 64, 5),      # one head x 32 tokens, d = 64
    (1, 6, 2, 7, 96, 128, 3),       # 3 heads x 7 tokens, the mask crosses chunks
])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_tokens(fa_gpu, cfg, causal):
    """A few query tokens per head (the newest positions) against the keys,
    with and without the end-aligned causal mask, against the oracle."""
    B, Hq, Hkv, Nq, Nk, d, splits = cfg
    x = gen(B, Hq, Hkv, Nq, Nk, d, "bf16", 43)
    say(f"decode tokens B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} splits={splits} "
        f"causal={causal}")
    o, lse = fa_gpu.decode_tokens(x["q"], x["k"], x["v"], splits, causal=causal)
    torch.cuda.synchronize()
    ro, rl = A.decode_multi(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), 1 / math.sqrt(d),
                            causal)
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(to_f64(lse), rl) <= BF16_LSE


def test_decode_tokens_one_token_is_decode(fa_gpu):
    """Nq = 1 runs the single-token decode's arithmetic: bit-identical."""
    x = gen(2, 8, 2, 1, 4096, 128, "bf16", 44)
    say("decode tokens Nq=1 vs decode")
    a = fa_gpu.decode_tokens(x["q"], x["k"], x["v"], 8, causal=True)
    b = fa_gpu.decode(x["q"], x["k"], x["v"], 8)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_tokens_config_sampled(fa_gpu):
    """The decode workload's KV (B=8 Hkv=8, 131072 keys, d=128, 64 splits)
    with 4 causal query tokens per head (Hq=32: 16 columns per tile): every
    output against the oracle."""
    w = WORKLOADS["decode_gqa"]
    g = torch.Generator("cuda").manual_seed(45)
    k = torch.randn(w.B, w.Hkv, w.Nk, w.d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(w.B, w.Hkv, w.Nk, w.d, device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn(w.B, w.Hq, 4, w.d, device="cuda", generator=g).to(torch.bfloat16)
    say("decode tokens full size")
    o, lse = fa_gpu.decode_tokens(q, k, v, 64, causal=True)
    torch.cuda.synchronize()
    o, lse, qh = to_f64(o), to_f64(lse), to_f64(q)
    G = w.Hq // w.Hkv
    for b in range(w.B):   # the oracle widens one (b, KV head) slab at a time
        for hk in range(w.Hkv):
            kk = k[b:b + 1, hk:hk + 1].float().cpu().numpy()
            vv = v[b:b + 1, hk:hk + 1].float().cpu().numpy()
            hs = slice(hk * G, (hk + 1) * G)
            ro, rl = A.decode_multi(qh[b:b + 1, hs], kk, vv, w.scale, True)
            assert maxabs(o[b:b + 1, hs], ro) <= BF16_O, (b, hk)
            assert maxabs(lse[b:b + 1, hs], rl) <= BF16_LSE, (b, hk)


def test_decode_split_count_invariance(fa_gpu):
    x = gen(2, 8, 2, 1, 8192, 128, "bf16", 42)
    outs = []
    for s in (1, 2, 64, 128):
        say(f"decode invariance splits={s}")
        o, lse = fa_gpu.decode(x["q"], x["k"], x["v"], s)
        torch.cuda.synchronize()
        outs.append((to_f64(o), to_f64(lse)))
    ref = A.forward(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), 1 / math.sqrt(128))
    for o, lse in outs:
        assert maxabs(o, ref[0]) <= BF16_O and maxabs(lse, ref[1]) <= BF16_LSE


@pytest.mark.parametrize("B,Hq,S,d", [(2, 3, 7, 100), (1, 2, 300, 30), (1, 5, 64, 256),
                                        (3, 1, 1, 128), (2, 4, 513, 64)])
def test_decode_combine_direct(fa_gpu, B, Hq, S, d):
    """The merge alone on arbitrary partials: odd d (vector and scalar paths),
    more splits than threads, one split, and chunks whose lse is -inf (empty
    chunks weigh nothing)."""
    say(f"decode combine direct B={B} Hq={Hq} S={S} d={d}")
    g = torch.Generator("cpu").manual_seed(1000 + S + d)
    op = torch.randn(B, Hq, S, d, generator=g, dtype=torch.float32)
    lp = 3 * torch.randn(B, Hq, S, generator=g, dtype=torch.float32)
    if S > 1:
        lp[..., 1] = -math.inf
    o = torch.empty(B, Hq, 1, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, 1, dtype=torch.float32, device="cuda")
    opc, lpc = op.cuda(), lp.cuda()
    fa_gpu.fa_decode_combine(opc, lpc, o, lse, B, Hq, d, S)
    torch.cuda.synchronize()
    ro, rl = A.combine(op.double().numpy(), lp.double().numpy())
    assert maxabs(to_f64(o)[:, :, 0], ro) <= BF16_O
    assert maxabs(to_f64(lse)[:, :, 0], rl) <= 1e-5


def test_decode_combine_rows_without_keys(fa_gpu):
    """A row whose splits all have lse = -inf saw no key: the merge writes
    O = 0 and LSE = -inf (never NaN); the other rows are merged as usual."""
    B, Hq, S, d = 2, 3, 9, 128
    say(f"decode combine rows without keys B={B} Hq={Hq} S={S} d={d}")
    g = torch.Generator("cpu").manual_seed(1234)
    op = torch.randn(B, Hq, S, d, generator=g, dtype=torch.float32)
    lp = 3 * torch.randn(B, Hq, S, generator=g, dtype=torch.float32)
    lp[0, 1, :] = -math.inf
    lp[1, 2, :] = -math.inf
    lp[1, 0, ::2] = -math.inf
    o = torch.empty(B, Hq, 1, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, 1, dtype=torch.float32, device="cuda")
    fa_gpu.fa_decode_combine(op.cuda(), lp.cuda(), o, lse, B, Hq, d, S)
    torch.cuda.synchronize()
    ro, rl = A.combine(op.double().numpy(), lp.double().numpy())
    on, ln = to_f64(o)[:, :, 0], to_f64(lse)[:, :, 0]
    assert not np.isnan(on).any() and not np.isnan(ln).any()
    dead = np.isneginf(rl)
    assert dead.sum() == 2 and np.array_equal(np.isneginf(ln), dead)
    assert not on[dead].any()
    assert maxabs(on[~dead], ro[~dead]) <= BF16_O
    assert maxabs(ln[~dead], rl[~dead]) <= 1e-5


def test_decode_config_full(fa_gpu):
    """B=8 Hq=32 Hkv=8 Nk=131072 d=128, 64 splits: every output and partial,
    the oracle widening one (b, KV head) slab at a time."""
    w = WORKLOADS["decode_gqa"]
    say("decode_gqa inputs")
    x = make_inputs(w, device="cuda")
    say("decode_gqa full size")
    o, lse, op, lp = fa_gpu.decode(x["q"], x["k"], x["v"], w.num_splits, return_partials=True)
    torch.cuda.synchronize()
    o, lse, op, lp = (to_f64(t) for t in (o, lse, op, lp))
    qh = to_f64(x["q"])
    G = w.Hq // w.Hkv
    for b in range(w.B):
        for hk in range(w.Hkv):
            kk = x["k"][b:b + 1, hk:hk + 1].float().cpu().numpy()
            vv = x["v"][b:b + 1, hk:hk + 1].float().cpu().numpy()
            qq = qh[b:b + 1, hk * G:(hk + 1) * G]
            ro, rl, rop, rlp = A.decode_split(qq, np.repeat(kk, 1, 1), vv, w.scale, w.num_splits)
            sl = slice(hk * G, (hk + 1) * G)
            assert maxabs(o[b, sl], ro[0]) <= BF16_O
            assert maxabs(lse[b, sl], rl[0]) <= BF16_LSE
            assert maxabs(op[b, sl], rop[0]) <= BF16_O
            assert maxabs(lp[b, sl], rlp[0]) <= BF16_LSE


# ---------------------------------------------------------- varlen forward

def varlen_case(lens_q, Hq, Hkv, d, seed, lens_k=None):
    lens_k = lens_q if lens_k is None else lens_k
    g = torch.Generator("cpu").manual_seed(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = torch.randn(tq, Hq, d, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(tk, Hkv, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(tk, Hkv, d, generator=g).to(torch.bfloat16).cuda()
    cq, ck = [0], [0]
    for a, b in zip(lens_q, lens_k):
        cq.append(cq[-1] + a)
        ck.append(ck[-1] + b)
    return q, k, v, cq, ck


@pytest.mark.parametrize("lens,Hq,Hkv,d", [
    ((5, 300, 1, 257), 4, 2, 128),       # ragged tails, a single-token sequence
    ((1000,), 2, 2, 64),
    ((40, 0, 77, 513), 8, 1, 128),       # an empty sequence; G = 8
    ((256, 255, 257), 2, 2, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_forward_small(fa_gpu, lens, Hq, Hkv, d, causal):
    q, k, v, cq, ck = varlen_case(lens, Hq, Hkv, d, seed=71)
    say(f"varlen forward lens={lens} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    o, lse = fa_gpu.forward_varlen(q, k, v, cqd, cqd, max(lens), max(lens), causal=causal)
    torch.cuda.synchronize()
    ro, rl = A.forward_varlen(to_f64(q), to_f64(k), to_f64(v), cq, ck, 1 / math.sqrt(d), causal)
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(to_f64(lse), rl) <= BF16_LSE


def test_varlen_queries_without_keys(fa_gpu):
    """Non-causal pack where one sequence has queries but no keys: its rows
    get O = 0 and LSE = -inf; the others are unaffected."""
    q, k, v, cq, ck = varlen_case((5, 9, 70), 2, 2, 128, seed=72, lens_k=(0, 33, 100))
    say("varlen forward, a sequence without keys")
    o, lse = fa_gpu.forward_varlen(q, k, v, torch.tensor(cq, dtype=torch.int32, device="cuda"),
                                   torch.tensor(ck, dtype=torch.int32, device="cuda"), 70, 100)
    torch.cuda.synchronize()
    ro, rl = A.forward_varlen(to_f64(q), to_f64(k), to_f64(v), cq, ck, 1 / math.sqrt(128))
    lo = to_f64(lse)
    assert np.all(np.isneginf(lo[:, :5])) and not np.any(to_f64(o)[:5])
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(lo[:, 5:], rl[:, 5:]) <= BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_dense(fa_gpu, causal):
    """Sequences of equal length packed token-major run the same arithmetic as
    the [B][H][N][d] forward: outputs agree bit for bit."""
    B, N, Hq, Hkv, d = 3, 1000, 4, 2, 128
    q, k, v, cq, _ = varlen_case((N,) * B, Hq, Hkv, d, seed=73)
    say(f"varlen vs dense causal={causal}")
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    o, lse = fa_gpu.forward_varlen(q, k, v, cqd, cqd, N, N, causal=causal)
    qd = q.view(B, N, Hq, d).permute(0, 2, 1, 3).contiguous()
    kd = k.view(B, N, Hkv, d).permute(0, 2, 1, 3).contiguous()
    vd = v.view(B, N, Hkv, d).permute(0, 2, 1, 3).contiguous()
    od, lsed = fa_gpu.forward(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(B, N, Hq, d).permute(0, 2, 1, 3), od)
    assert torch.equal(lse.view(Hq, B, N).permute(1, 0, 2), lsed)


# --------------------------------------------------------- varlen backward

def varlen_grad_case(lens_q, Hq, Hkv, d, seed, lens_k=None):
    q, k, v, cq, ck = varlen_case(lens_q, Hq, Hkv, d, seed, lens_k)
    g = torch.Generator("cpu").manual_seed(seed + 1000)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    return q, k, v, do, cq, ck


_VARLEN_EQUAL = [
    ((5, 300, 1, 257), None, 4, 2, 128),     # ragged tails, a single-token sequence
    ((40, 0, 77, 513), None, 8, 1, 128),     # an empty sequence; G = 8
    ((256, 255, 257), None, 2, 2, 64),
    ((1000,), None, 2, 1, 64),
]
# unequal query and key lengths: non-causal only (causal packs are square)
_VARLEN_UNEQUAL = [
    ((5, 9, 70), (0, 33, 100), 2, 2, 128),   # queries without keys
    ((0, 50, 64), (30, 50, 300), 4, 4, 128),  # keys without queries
]


@pytest.mark.parametrize("lens_q,lens_k,Hq,Hkv,d,causal",
                         [c + (cz,) for c in _VARLEN_EQUAL for cz in (False, True)] +
                         [c + (False,) for c in _VARLEN_UNEQUAL])
def test_varlen_backward_small(fa_gpu, lens_q, lens_k, Hq, Hkv, d, causal):
    q, k, v, do, cq, ck = varlen_grad_case(lens_q, Hq, Hkv, d, seed=74, lens_k=lens_k)
    lk = lens_q if lens_k is None else lens_k
    say(f"varlen backward lens_q={lens_q} lens_k={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    ckd = torch.tensor(ck, dtype=torch.int32, device="cuda")
    mq, mk = max(max(lens_q), 1), max(max(lk), 1)
    o, lse = fa_gpu.forward_varlen(q, k, v, cqd, ckd, mq, mk, causal=causal)
    grads = fa_gpu.backward_varlen(q, k, v, o, lse, do, cqd, ckd, mq, mk, causal=causal)
    torch.cuda.synchronize()
    ref = A.backward_varlen(to_f64(q), to_f64(k), to_f64(v), to_f64(do), cq, ck,
                            1 / math.sqrt(d), causal)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= BF16_GRAD, (name, e)
    dq, dk, dv = (to_f64(t) for t in grads)
    for b in range(len(lens_q)):
        if lk[b] == 0:
            assert not dq[cq[b]:cq[b + 1]].any()
        if lens_q[b] == 0:
            assert not dk[ck[b]:ck[b + 1]].any() and not dv[ck[b]:ck[b + 1]].any()


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_equals_dense(fa_gpu, causal):
    """Equal-length sequences packed token-major run the same arithmetic as
    the [B][H][N][d] backward: gradients agree bit for bit."""
    B, N, Hq, Hkv, d = 3, 1000, 4, 2, 128
    q, k, v, do, cq, _ = varlen_grad_case((N,) * B, Hq, Hkv, d, seed=75)
    say(f"varlen backward vs dense causal={causal}")
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    o, lse = fa_gpu.forward_varlen(q, k, v, cqd, cqd, N, N, causal=causal)
    dq, dk, dv = fa_gpu.backward_varlen(q, k, v, o, lse, do, cqd, cqd, N, N, causal=causal)

    def dense(t, H):
        return t.view(B, N, H, d).permute(0, 2, 1, 3).contiguous()

    od = dense(o, Hq)
    lsed = lse.view(Hq, B, N).permute(1, 0, 2).contiguous()
    gd = fa_gpu.backward(dense(q, Hq), dense(k, Hkv), dense(v, Hkv), od, lsed, dense(do, Hq),
                         causal=causal)
    torch.cuda.synchronize()
    for got, want, H in zip((dq, dk, dv), gd, (Hq, Hkv, Hkv)):
        assert torch.equal(dense(got, H), want)


# ------------------------------------------------------------- paged decode

def paged_case(B, Hq, Hkv, seqlens, page, d, splits, seed, spare=3):
    import dataclasses
    from workloads import PAGED, make_paged_inputs
    w = dataclasses.replace(PAGED["decode_paged"], B=B, Hq=Hq, Hkv=Hkv, seqlens=tuple(seqlens),
                            page_size=page, d=d, num_splits=splits, seed=seed,
                            spare_pages=spare)
    return w, make_paged_inputs(w, device="cuda")


@pytest.mark.parametrize("cfg", [
    (2, 8, 2, (1000, 77), 16, 128, 8),       # ragged lengths, 16-key pages
    (3, 4, 4, (1, 33, 512), 32, 128, 4),     # a single key; chunks past the end
    (1, 32, 4, (4096,), 64, 128, 16),        # G = 8
    (2, 16, 2, (3000, 2048), 256, 64, 5),    # d = 64, large pages
    (2, 6, 2, (95, 200), 16, 64, 7)])
def test_decode_paged_small(fa_gpu, cfg):
    B, Hq, Hkv, seqlens, page, d, splits = cfg
    w, x = paged_case(*cfg, seed=61)
    say(f"decode paged B={B} Hq={Hq} Hkv={Hkv} seqlens={seqlens} page={page} d={d} splits={splits}")
    o, lse, op, lp = fa_gpu.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"],
                                         x["seqlens"], splits, max_seqlen=max(seqlens),
                                         return_partials=True)
    torch.cuda.synchronize()
    ro, rl = A.decode_paged(to_f64(x["q"]), to_f64(x["k_cache"]), to_f64(x["v_cache"]),
                            x["block_table"].cpu().numpy(), seqlens, w.scale)
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(to_f64(lse), rl) <= BF16_LSE
    # chunks that start past a sequence's end hold exactly O = 0, lse = -inf
    per = -(-max(seqlens) // splits)
    L = -(-per // 32) * 32
    lpn, opn = lp.cpu().numpy(), op.cpu().numpy()
    for b, n in enumerate(seqlens):
        for c in range(splits):
            if c * L >= n:
                assert np.all(np.isneginf(lpn[b, :, c])) and not np.any(opn[b, :, c])
            else:
                assert np.all(np.isfinite(lpn[b, :, c]))


@pytest.mark.parametrize("cfg", [
    # B, Hq, Hkv, seqlens, page, d, splits, Nq
    (2, 8, 2, (1000, 77), 16, 128, 8, 4),    # ragged lengths, 4 heads x 4 tokens
    (3, 4, 4, (5, 33, 512), 32, 128, 4, 5),  # a sequence barely longer than the tokens
    (1, 32, 8, (4096,), 64, 64, 16, 8),      # 4 heads x 8 tokens = 32 columns, d = 64
])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged_tokens(fa_gpu, cfg, causal):
    """A few query tokens over a paged cache, with and without the end-aligned
    causal mask, against the oracle (gather through the table, then the
    few-token decode)."""
    B, Hq, Hkv, seqlens, page, d, splits, Nq = cfg
    w, x = paged_case(B, Hq, Hkv, seqlens, page, d, splits, seed=62)
    g = torch.Generator("cpu").manual_seed(63)
    q = torch.randn(B, Hq, Nq, d, generator=g).to(torch.bfloat16).cuda()
    say(f"decode paged tokens B={B} Hq={Hq} Hkv={Hkv} seqlens={seqlens} page={page} d={d} "
        f"splits={splits} Nq={Nq} causal={causal}")
    o, lse = fa_gpu.decode_paged_tokens(q, x["k_cache"], x["v_cache"], x["block_table"],
                                        x["seqlens"], splits, causal=causal,
                                        max_seqlen=max(seqlens))
    torch.cuda.synchronize()
    ro, rl = A.decode_paged_multi(to_f64(q), to_f64(x["k_cache"]), to_f64(x["v_cache"]),
                                  x["block_table"].cpu().numpy(), seqlens, w.scale, causal)
    assert maxabs(to_f64(o), ro) <= BF16_O
    assert maxabs(to_f64(lse), rl) <= BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged_tokens_fewer_keys_than_tokens(fa_gpu, causal):
    """An entry with fewer keys than query tokens: under the end-aligned causal
    mask its first tokens see no key, so every split is empty and the merge
    must write O = 0 and LSE = -inf for them (not NaN); the other tokens and
    entries match the oracle."""
    B, Hq, Hkv, seqlens, page, d, splits, Nq = 3, 4, 2, (2, 300, 4), 16, 128, 4, 5
    w, x = paged_case(B, Hq, Hkv, seqlens, page, d, splits, seed=65)
    g = torch.Generator("cpu").manual_seed(66)
    q = torch.randn(B, Hq, Nq, d, generator=g).to(torch.bfloat16).cuda()
    say(f"decode paged tokens seqlens={seqlens} Nq={Nq} causal={causal}")
    o, lse = fa_gpu.decode_paged_tokens(q, x["k_cache"], x["v_cache"], x["block_table"],
                                        x["seqlens"], splits, causal=causal,
                                        max_seqlen=max(seqlens))
    torch.cuda.synchronize()
    ro, rl = A.decode_paged_multi(to_f64(q), to_f64(x["k_cache"]), to_f64(x["v_cache"]),
                                  x["block_table"].cpu().numpy(), seqlens, w.scale, causal)
    on, ln = to_f64(o), to_f64(lse)
    assert not np.isnan(on).any() and not np.isnan(ln).any()
    dead = np.isneginf(rl)
    assert dead.sum() == (Hq * (3 + 1) if causal else 0)   # 3 tokens of entry 0, 1 of entry 2
    assert np.array_equal(np.isneginf(ln), dead) and not on[dead].any()
    assert maxabs(on[~dead], ro[~dead]) <= BF16_O
    assert maxabs(ln[~dead], rl[~dead]) <= BF16_LSE


def test_decode_paged_tokens_one_token_is_paged_decode(fa_gpu):
    """Nq = 1 runs the paged single-token decode's arithmetic: bit-identical."""
    w, x = paged_case(2, 8, 2, (1000, 77), 16, 128, 8, seed=64)
    say("decode paged tokens Nq=1 vs paged decode")
    a = fa_gpu.decode_paged_tokens(x["q"], x["k_cache"], x["v_cache"], x["block_table"],
                                   x["seqlens"], 8, causal=True, max_seqlen=1000)
    b = fa_gpu.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["seqlens"],
                            8, max_seqlen=1000)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_paged_equals_dense(fa_gpu):
    """The same K/V rows laid out densely and scattered over 16-key pages,
    with the same 512-key chunks: the two kernels run the same arithmetic, so
    partials and outputs agree bit for bit."""
    B, Hq, Hkv, N, d, splits, page = 2, 8, 2, 4096, 128, 8, 16
    w, x = paged_case(B, Hq, Hkv, (N, N), page, d, splits, seed=62)
    say("decode paged vs dense")
    op = fa_gpu.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"],
                             x["seqlens"], splits, return_partials=True)
    t = torch.arange(N, device="cuda")
    kd = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    for b in range(B):
        rows = x["block_table"][b].long()[t // page]
        kd[b] = x["k_cache"][rows, t % page].permute(1, 0, 2)
        vd[b] = x["v_cache"][rows, t % page].permute(1, 0, 2)
    od = fa_gpu.decode(x["q"], kd.contiguous(), vd.contiguous(), splits, return_partials=True)
    torch.cuda.synchronize()
    for a, b_ in zip(op, od):
        assert torch.equal(a, b_)


def test_decode_paged_config(fa_gpu):
    """B=8 Hq=32 Hkv=8, 131072 keys each in 16-key pages scattered over the
    cache, 64 splits: equal bit for bit to the dense kernel on the gathered
    rows (itself checked against the oracle at full size), and two (b, KV
    head) groups against the oracle directly."""
    from workloads import PAGED, make_paged_inputs
    w = PAGED["decode_paged"]
    say("decode_paged inputs")
    x = make_paged_inputs(w, device="cuda")
    say("decode_paged full size")
    o, lse = fa_gpu.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"],
                                 x["seqlens"], w.num_splits)
    N, page = w.seqlens[0], w.page_size
    t = torch.arange(N, device="cuda")
    kd = torch.empty(w.B, w.Hkv, N, w.d, dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    for b in range(w.B):
        rows = x["block_table"][b].long()[t // page]
        kd[b] = x["k_cache"][rows, t % page].permute(1, 0, 2)
        vd[b] = x["v_cache"][rows, t % page].permute(1, 0, 2)
    od, lsed = fa_gpu.decode(x["q"], kd, vd, w.num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(lse, lsed)
    G = w.Hq // w.Hkv
    for b, hk in ((0, 0), (w.B - 1, w.Hkv - 1)):
        qq = to_f64(x["q"][b:b + 1, hk * G:(hk + 1) * G])
        ro, rl = A.forward(qq, to_f64(kd[b:b + 1, hk:hk + 1]), to_f64(vd[b:b + 1, hk:hk + 1]),
                           w.scale)
        assert maxabs(to_f64(o[b:b + 1, hk * G:(hk + 1) * G]), ro) <= BF16_O
        assert maxabs(to_f64(lse[b:b + 1, hk * G:(hk + 1) * G]), rl) <= BF16_LSE
    del kd, vd


# ---------------------------------------------------------------------- fp8

def test_quantizer_codes_match_oracle_bytes(fa_gpu):
    """Without rotation the codes are a pure function of the fp32 inputs: they
    must equal the oracle's e4m3 codes byte for byte, scales exactly."""
    x = gen(2, 3, 3, 300, 300, 128, "bf16", 51)["q"]
    x[0, 0, 5, 7] = 50.0
    x[1, 2, 299, :] = 0.0
    say("quantize_fp8 no rotation")
    codes, scales = fa_gpu.quantize_fp8(x)
    torch.cuda.synchronize()
    ref_c, ref_s = F8.quantize(x.float().cpu().numpy())
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantizer_all_zero_block(fa_gpu):
    x = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    say("quantize_fp8 zero block")
    codes, scales = fa_gpu.quantize_fp8(x)
    torch.cuda.synchronize()
    assert float(scales[0, 0, 0]) == 1.0 and int(codes.abs().max() if False else codes.max()) == 0


def test_quantizer_rotation(fa_gpu):
    """With the Hadamard rotation the fp32 pre-quantisation values differ from
    the oracle's fp64 rotation by rounding only, so a code may move by one
    e4m3 step where the value sits on a rounding boundary."""
    x = gen(1, 2, 2, 256, 256, 128, "bf16", 52)["q"]
    signs = (torch.randint(0, 2, (128,), generator=torch.Generator().manual_seed(5)) * 2 - 1).to(torch.int8)
    say("quantize_fp8 rotation")
    codes, scales = fa_gpu.quantize_fp8(x, signs.cuda())
    torch.cuda.synchronize()
    rot = F8.rotate(x.float().cpu().numpy(), signs.numpy()).astype(np.float32)
    ref_c, ref_s = F8.quantize(rot)
    assert np.allclose(scales.cpu().numpy(), ref_s, rtol=1e-6)
    got = F8.dequantize(codes.cpu().numpy(), scales.cpu().numpy())
    want = F8.dequantize(ref_c, ref_s)
    mismatch = (codes.cpu().numpy() != ref_c)
    assert mismatch.mean() < 1e-3
    step = np.abs(want) * 2.0 ** -3 + ref_s.max() * 2.0 ** -9
    assert np.all(np.abs(got - want) <= step + 1e-12)


def fp8_pipeline(fa, x, signs, causal=False):
    q8, qs = fa.quantize_fp8(x["q"], signs)
    k8, ks = fa.quantize_fp8(x["k"], signs)
    v8, vs = fa.quantize_fp8(x["v"], None)
    o, lse = fa.forward_fp8(q8, k8, v8, qs, ks, vs, causal=causal)
    return o, lse, (q8, qs, k8, ks, v8, vs)


def oracle_fp8_inputs(x, signs):
    """The oracle's own quantised operands, from the bf16 inputs (never from
    the library's codes): Q and K rotated by J when signs are given (fp64
    product rounded to fp32, as the quantiser's input), then per-128-row-block
    e4m3 quantisation of Q, K and V, dequantised to float64.  With a rotation
    a code can sit one e4m3 step from the library's where the fp32 rotation
    lands on a rounding boundary (under 0.1% of them, bounded in
    test_quantizer_rotation); the forward's tolerance covers that."""
    q, k, v = (x[n].float().cpu().numpy() for n in ("q", "k", "v"))
    if signs is not None:
        sg = signs.cpu().numpy().astype(np.float64)
        q, k = (F8.rotate(t, sg).astype(np.float32) for t in (q, k))
    return tuple(F8.dequantize(*F8.quantize(t)) for t in (q, k, v))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_small(fa_gpu, causal):
    x = gen(1, 4, 2, 384, 384, 128, "bf16", 61)
    signs = (torch.randint(0, 2, (128,), generator=torch.Generator().manual_seed(6)) * 2 - 1).to(torch.int8).cuda()
    say(f"fp8 forward small causal={causal}")
    o, lse, _ = fp8_pipeline(fa_gpu, x, signs, causal)
    torch.cuda.synchronize()
    dq, dk, dv = oracle_fp8_inputs(x, signs)
    ro, rl = A.forward(dq, dk, dv, 1 / math.sqrt(128), causal)
    assert rel_l2(to_f64(o), ro) <= FP8_REL
    assert maxabs(to_f64(lse), rl) <= 5e-2


@pytest.mark.parametrize("case", ["ragged_gqa", "v_scales", "rising_scores", "tiles_1", "tiles_3",
                                  "tiles_7"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_edge_cases(fa_gpu, case, causal):
    """Ragged key tail with GQA; V blocks whose scales differ 50x (the fold
    of s_v relative to the largest V scale); scores that grow along the keys,
    so the reference max must move up many times (the rescale path); key
    counts of 1, 3 and 7 tiles of 64 (every remainder of the four-slot load
    rotation, and units shorter than one round of it)."""
    N = {"ragged_gqa": 300, "tiles_1": 40, "tiles_3": 190, "tiles_7": 448}.get(case, 640)
    Hq, Hkv = (4, 2) if case == "ragged_gqa" else (2, 2)
    x = gen(1, Hq, Hkv, N, N, 128, "bf16", 63)
    if case == "v_scales":
        f = torch.ones(N, device="cuda")
        f[128:256] = 50.0
        f[384:512] = 0.05
        x["v"] = (x["v"].float() * f[None, None, :, None]).to(torch.bfloat16)
    if case == "rising_scores":
        ramp = torch.linspace(0.2, 3.0, N, device="cuda")
        x["k"] = (x["k"].float() * ramp[None, None, :, None]).to(torch.bfloat16)
        x["q"] = (x["q"].float().abs() + 0.5).to(torch.bfloat16)
        x["k"] = x["k"].float().abs().to(torch.bfloat16)
    say(f"fp8 forward edge case={case} causal={causal}")
    o, lse, _ = fp8_pipeline(fa_gpu, x, None, causal)
    torch.cuda.synchronize()
    dq, dk, dv = oracle_fp8_inputs(x, None)
    ro, rl = A.forward(dq, dk, dv, 1 / math.sqrt(128), causal)
    assert rel_l2(to_f64(o), ro) <= FP8_REL, rel_l2(to_f64(o), ro)
    assert maxabs(to_f64(lse), rl) <= 5e-2


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_bf16_backward(fa_gpu, causal):
    """The mixed mode the pages name as the fp8 fallback: fp8 forward (rotated,
    per-block e4m3) for O and LSE, then the bf16 backward on the unquantised
    inputs with those O and LSE.  On N(0,1) inputs the gradients stay within
    the fp8 tolerance of the exact ones."""
    x = gen(1, 2, 2, 1024, 1024, 128, "bf16", 65, grad=True)
    signs = (torch.randint(0, 2, (128,), generator=torch.Generator().manual_seed(8)) * 2 - 1).to(torch.int8).cuda()
    say(f"fp8 forward + bf16 backward causal={causal}")
    o8, l8, _ = fp8_pipeline(fa_gpu, x, signs, causal)
    grads = fa_gpu.backward(x["q"], x["k"], x["v"], o8, l8, x["do"], causal=causal)
    torch.cuda.synchronize()
    ref = A.backward(*(to_f64(x[n]) for n in ("q", "k", "v", "do")), 1 / math.sqrt(128), causal)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        e = rel_l2(to_f64(got), want)
        assert e <= FP8_REL, (name, e)

