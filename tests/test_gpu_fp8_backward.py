"""Parity of the fp8-dS backward (fa_bwd_fp8) and of its power-of-two e4m3
quantiser (fa_quantize_pow2_e4m3) against the oracle's emulation
(oracle/fp8_backward.py, oracle/fp8.py), through the C ABI.

The backward's inputs O and LSE come from the oracle's forward (O rounded to
bf16, the interface's precision), and the emulation forms delta = rowsum(dO *
O) from that same O.  Both sides must see one O: an e5m2 step is up to a
quarter of a dS element, so the few-ulp difference between the GPU forward's
O and the exact one moves a dS element of a row that sees few keys across a
rounding boundary now and then, and with it that whole row of dQ.  The GPU
forward followed by the fp8 backward is checked end to end against the exact
gradient instead.

Tolerances:
  quantiser: bit-exact (codes and scale bytes; both sides scale by an exact
             power of two and round to nearest even);
  dQ, dK:    relative L2 <= 1e-2 against the emulation (what remains is fp32
             summation order, the bf16 rounding of the output and rare e5m2
             codes that flip where the kernel's fp32 dS and the oracle's differ
             in the last bits), and at most a quarter of its distance to the
             exact gradient, so an unquantised or wrongly scaled product fails;
             end to end: within 1.15 x the emulation's own error against the
             exact gradient;
  dV:        the bf16 path's: relative L2 <= 1e-2 against the exact backward.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from oracle import fp8_backward as FB
from tests.conftest import say
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2


def f64(t):
    return t.double().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def gen(B, Hq, Hkv, Nq, Nk, seed, d=128):
    g = torch.Generator("cpu").manual_seed(seed)
    x = {"q": torch.randn(B, Hq, Nq, d, generator=g), "k": torch.randn(B, Hkv, Nk, d, generator=g),
         "v": torch.randn(B, Hkv, Nk, d, generator=g), "do": torch.randn(B, Hq, Nq, d, generator=g)}
    return {n: t.to(torch.bfloat16) for n, t in x.items()}


# ----------------------------------------------------------------- quantiser

@pytest.mark.parametrize("N", [300, 32, 7])
def test_quantize_pow2_e4m3_bit_exact(fa_gpu, N):
    """Rows spread over 40 binades (so blocks differ widely and small values
    go subnormal), an all-zero block, a ragged last block."""
    g = torch.Generator("cpu").manual_seed(71 + N)
    x = torch.randn(2, 3, N, 128, generator=g)
    x *= torch.exp2(torch.randint(-20, 20, (2, 3, N, 1), generator=g).float())
    x[0, 1, :min(N, 32)] = 0.0
    x = x.to(torch.bfloat16)
    say(f"quantize_pow2_e4m3 N={N}")
    x8, xe = fa_gpu.quantize_pow2_e4m3(x.cuda())
    torch.cuda.synchronize()
    x8, xe = x8.cpu().numpy(), xe.cpu().numpy().astype(np.int64)
    for b in range(2):
        for h in range(3):
            deq, exps = F8.quantize_pow2(x[b, h].float().numpy(), "e4m3", (32, 128))
            assert np.array_equal(xe[b, h] - 127, exps[:, 0]), (b, h)
            got = F8.e4m3_decode(x8[b, h]) * np.exp2(np.repeat(exps[:, 0], 32)[:N, None].astype(np.float64))
            assert np.array_equal(got, deq), (b, h)


# ------------------------------------------------------------------ backward

def oracle_o_lse(q, k, v, sc, causal):
    """The oracle's forward: O rounded to bf16 and LSE as float32 tensors."""
    o, lse = A.forward(q, k, v, sc, causal)
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse).to(torch.float32)


def run(fa, x, causal, o, lse):
    xc = {n: t.cuda() for n, t in x.items()}
    grads = fa.backward_fp8(xc["q"], xc["k"], xc["v"], o.cuda(), lse.cuda(), xc["do"],
                            causal=causal)
    torch.cuda.synchronize()
    return [t.cpu() for t in grads]


def check(fa, x, causal):
    q, k, v, do = (x[n].float().numpy() for n in ("q", "k", "v", "do"))
    sc = 1 / math.sqrt(q.shape[-1])
    o, lse = oracle_o_lse(q, k, v, sc, causal)
    grads = run(fa, x, causal, o, lse)
    emul = FB.backward_fp8(q, k, v, do, sc, causal, o=o.double().numpy())
    exact = A.backward(q, k, v, do, sc, causal)
    for i, name in enumerate(("dq", "dk")):
        g = f64(grads[i])
        e_emul, e_exact = rel_l2(g, emul[i]), rel_l2(g, exact[i])
        print(f"{name} rel-L2: vs emulated fp8 {e_emul:.2e}, vs exact {e_exact:.2e}, "
              f"emulated vs exact {rel_l2(emul[i], exact[i]):.2e}")
        assert e_emul <= GRAD_TOL and e_emul <= 0.25 * e_exact, (name, e_emul, e_exact)
    e = rel_l2(f64(grads[2]), exact[2])
    assert e <= GRAD_TOL, ("dv", e)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 300), (2, 2, 2, 280, 280), (1, 2, 1, 40, 40),
                                   (1, 3, 3, 520, 520)])
def test_fp8_backward_against_emulation(fa_gpu, shape, causal):
    """GQA; ragged key tails with more (300 = 4*64 + 44) and fewer (280 = 4*64
    + 24: the tile's second 32-key block lies past the end) than 32 keys in
    the last tile; a single partial tile; three query tiles with a tail."""
    B, Hq, Hkv, Nq, Nk = shape
    x = gen(B, Hq, Hkv, Nq, Nk, 91 + Nq)
    say(f"fp8 backward shape={shape} causal={causal}")
    check(fa_gpu, x, causal)


def test_fp8_backward_unequal_lengths(fa_gpu):
    x = gen(1, 2, 2, 200, 600, 95)
    say("fp8 backward Nq=200 Nk=600")
    check(fa_gpu, x, False)


def test_fp8_backward_wide_range_rows_and_zero_key_block(fa_gpu):
    """dO rows scaled by powers of two from 2^-12 to 2^12 (dS rows follow, so
    the per-(query, 32-key) dS scales spread widely) and a block of 32 keys
    that is all zero (its K scale is 2^0 and its codes zero)."""
    x = gen(1, 2, 2, 384, 384, 97)
    g = torch.Generator("cpu").manual_seed(5)
    x["do"] = (x["do"].float() * torch.exp2(torch.randint(-12, 13, (1, 2, 384, 1), generator=g).float())
               ).to(torch.bfloat16)
    x["k"][:, :, 64:96] = 0
    say("fp8 backward wide-range dO rows, zero key block")
    check(fa_gpu, x, True)


def test_fp8_backward_is_deterministic(fa_gpu):
    x = gen(1, 4, 2, 520, 520, 99)
    o, lse = oracle_o_lse(*(x[n].float().numpy() for n in ("q", "k", "v")), 1 / math.sqrt(128),
                          True)
    say("fp8 backward determinism")
    a = run(fa_gpu, x, True, o, lse)
    b = run(fa_gpu, x, True, o, lse)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


# ------------------------------------------- full size: B2 H16 N8192 d128

HEADS = [(0, 0), (1, 15)]


@pytest.fixture(scope="module")
def full_run(fa_gpu):
    """The benchmark's causal workload, twice: end to end (the GPU forward's O
    and LSE), and with the checked heads' O and LSE taken from the oracle."""
    w = WORKLOADS["causal_bf16"]
    x = make_inputs(w)
    xc = {n: t.cuda() for n, t in x.items()}
    say("fp8 backward full size B2 H16 N8192 d128 causal: end to end")
    o, lse = fa_gpu.forward(xc["q"], xc["k"], xc["v"], causal=True)
    dq_e2e, dk_e2e, _ = fa_gpu.backward_fp8(xc["q"], xc["k"], xc["v"], o, lse, xc["do"],
                                            causal=True)
    torch.cuda.synchronize()
    e2e = (dq_e2e.cpu(), dk_e2e.cpu())
    sc = 1 / math.sqrt(w.d)
    oref = {}
    for b, h in HEADS:
        q, k, v = (x[n][b, h].float().numpy() for n in ("q", "k", "v"))
        ob, lb = A.head_forward(q, k, v, sc, True)
        oref[(b, h)] = torch.from_numpy(ob).to(torch.bfloat16)
        o[b, h] = oref[(b, h)].cuda()
        lse[b, h] = torch.from_numpy(lb).to(torch.float32).cuda()
    say("fp8 backward full size with the oracle's O and LSE on the checked heads")
    dq, dk, dv = fa_gpu.backward_fp8(xc["q"], xc["k"], xc["v"], o, lse, xc["do"], causal=True)
    torch.cuda.synchronize()
    return x, oref, e2e, dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("bh", HEADS)
def test_fp8_backward_full_size_heads(full_run, bh):
    """Two heads of the benchmark's causal workload, every row: dQ and dK
    against the emulated fp8 backward of that head (one query head per KV
    head here), dV against the exact backward, and the end-to-end dQ and dK
    against the exact ones."""
    x, oref, e2e, dq, dk, dv = full_run
    b, h = bh
    q, k, v, do = (x[n][b, h].float().numpy() for n in ("q", "k", "v", "do"))
    sc = 1 / math.sqrt(q.shape[-1])
    emul = FB.head_backward_fp8(q, k, v, do, sc, True, o=oref[bh].double().numpy())
    _, _, rq, rk, rv = A.head_forward_backward(q, k, v, do, sc, True)
    for name, got, em, ex, end in (("dq", dq, emul[0], rq, e2e[0]), ("dk", dk, emul[1], rk, e2e[1])):
        g = f64(got[b, h])
        e_emul, e_exact, floor = rel_l2(g, em), rel_l2(g, ex), rel_l2(em, ex)
        e_end = rel_l2(f64(end[b, h]), ex)
        print(f"head {bh} {name}: vs emulated {e_emul:.2e}, vs exact {e_exact:.2e}; emulated vs "
              f"exact {floor:.2e}; end to end vs exact {e_end:.2e}")
        assert e_emul <= GRAD_TOL and e_emul <= 0.25 * e_exact, (name, e_emul, e_exact)
        assert e_end <= 1.15 * floor, (name, e_end, floor)
    assert rel_l2(f64(dv[b, h]), rv) <= GRAD_TOL
