"""Emulated FP8 backward of exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the benchmark's CPU-baseline leg may use this module;
it shares no code with the HIP library.

[CH18] "第 18 章 FlashAttention" §18.6.2 (3) (FP8 backward): P and dS are
formed in high precision; dS is quantised blockwise to E5M2 and the two dS
products, dQ = dS K and dK = dS^T Q, run on fp8 with fp32 accumulation.
dV = P^T dO keeps the high-precision path.

Readings where the page is silent or garbled (each listed in the design notes):
  * Q and K enter those two products as E4M3 (the forward's operand format),
    dS as E5M2 (the page's gradient format);
  * every block scale is a power of two, 2^e with e the smallest integer that
    brings the block's largest magnitude within the format's range
    (oracle.fp8.pow2_exponent), so scaling is exact and only the rounding to
    the 8-bit format loses information;
  * blocks follow the contraction each product performs: for dQ = dS K, dS in
    blocks of one query row x 32 keys and K in blocks of 32 key rows; for
    dK = dS^T Q, dS in blocks of one key x 32 query rows and Q in blocks of 32
    query rows (all blocks aligned at multiples of 32 from the first row);
  * rounding is to nearest, ties to even; no value exceeds the format's
    largest finite value, by the choice of scale;
  * delta_i = rowsum(dO_i * O_i) ([CH18] §18.4.4) is formed from O as the
    backward receives it, the forward's output in the interface's precision
    (bf16) -- the caller passes it as ``o``; without ``o`` the exact
    rowsum(P * dP) is used.  With e5m2's coarse steps the difference matters:
    a change of delta in its ninth bit can move an element of dS across a
    rounding boundary, one step being up to a quarter of its value, which in
    a row that sees few keys shifts the whole row of dQ.

With power-of-two scales a normal value rounds to the same relative grid
whatever its block's exponent; the exponent decides only which small values
become subnormal or round to zero (those more than about 30 binades below the
block maximum for e5m2, 15 for e4m3).
"""
from __future__ import annotations

import numpy as np

from oracle import attention as A
from oracle import fp8 as F8


def head_backward_fp8(q, k, v, do, scale, causal, quantize=True, o=None):
    """One head's (dq, dk, dv) with fp8 dS products (see the module notes).
    q, do [Nq][d]; k, v [Nk][d] (float32 values, e.g. widened bf16); o [Nq][d]
    the forward's output as the backward receives it (delta = rowsum(dO * O)),
    or None for the exact delta.  With quantize=False every quantisation step
    is the identity, which must give the exact backward
    (oracle.attention.head_backward) when o is exact."""
    q32, k32 = np.asarray(q, np.float32), np.asarray(k, np.float32)
    qd, kd, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
    p, _, _ = A.softmax_rows(A.scores(qd, kd, scale, causal))
    dv = p.T @ do
    dp = do @ v.T
    if o is None:
        ds = A.softmax_backward(p, dp)
    else:
        delta = (do * np.asarray(o, np.float64)).sum(axis=1)
        ds = p * (dp - delta[:, None])
    nq, nk = ds.shape
    if not quantize:
        return scale * (ds @ kd), scale * (ds.T @ qd), dv
    ds32 = ds.astype(np.float32)
    # dQ = dS K: dS per (query row, 32-key block), K per 32 key rows
    ds_q, _ = F8.quantize_pow2(ds32, "e5m2", (1, 32))
    k8, _ = F8.quantize_pow2(k32, "e4m3", (32, k32.shape[1]))
    dq = scale * (ds_q @ k8)
    # dK = dS^T Q: dS per (32-query block, key), Q per 32 query rows
    ds_k, _ = F8.quantize_pow2(ds32, "e5m2", (32, 1))
    q8, _ = F8.quantize_pow2(q32, "e4m3", (32, q32.shape[1]))
    dk = scale * (ds_k.T @ q8)
    return dq, dk, dv


def backward_fp8(q, k, v, do, scale, causal=False, quantize=True, o=None):
    """Batched fp8-dS backward: q, do (and o, if given) [B][Hq][Nq][d], k, v
    [B][Hkv][Nk][d] -> (dQ, dK, dV) float64; a KV head's gradients sum over
    its query heads."""
    q, k, v, do = (np.asarray(t, np.float32) for t in (q, k, v, do))
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            hk = A.kv_head(h, Hq, Hkv)
            a, bk, bv = head_backward_fp8(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal,
                                          quantize, None if o is None else o[b, h])
            dq[b, h] = a
            dk[b, hk] += bk
            dv[b, hk] += bv
    return dq, dk, dv
