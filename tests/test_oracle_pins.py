"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

None of these tests call the HIP library.  Each check is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong mask edge) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from oracle import schedule as SCH

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rnd(*shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("gqa", [(2, 2), (4, 2), (4, 1)])
def test_forward_matches_torch_sdpa_fp64(causal, gqa):
    """Library routine: torch's math SDPA in float64 on the CPU."""
    Hq, Hkv = gqa
    B, N, d = 2, 37, 16
    q, k, v = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d)
    scale = 0.3
    o, lse = A.forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv)).numpy()
    assert np.abs(o - ref).max() < 1e-12
    # LSE against torch.logsumexp of the masked score matrix
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", q, kk)
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    assert np.abs(lse - ref_lse).max() < 1e-12


def test_forward_brute_force_loops():
    """Brute force with scalar loops and math.exp on a tiny causal GQA case."""
    B, Hq, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d)
    scale = 0.7
    o, lse = A.forward(q, k, v, scale, causal=True)
    for h in range(Hq):
        for i in range(N):
            s = [scale * sum(q[0, h, i, c] * k[0, 0, j, c] for c in range(d))
                 for j in range(i + 1)]
            z = sum(math.exp(x) for x in s)
            for c in range(d):
                ref = sum(math.exp(s[j]) * v[0, 0, j, c] for j in range(i + 1)) / z
                assert abs(o[0, h, i, c] - ref) < 1e-12
            assert abs(lse[0, h, i] - math.log(z)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean_of_v(causal):
    """Q = 0 makes every allowed score equal: O_i is the mean of the allowed V
    rows and LSE_i = ln(#allowed)."""
    N, d = 40, 8
    q = np.zeros((1, 1, N, d))
    k, v = rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = A.forward(q, k, v, 0.125, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.abs(o[0, 0, i] - v[0, 0, :n].mean(axis=0)).max() < 1e-14
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-14


def test_one_hot_scores_pick_a_row_of_v():
    """K rows c*e_j and q_i = e_pi(i) with scale*c = 50: O_i = v_pi(i) up to
    (Nk-1) e^-50."""
    Nk = d = 12
    perm = rng.permutation(Nk)
    c, scale = 500.0, 0.1
    k = (c * np.eye(Nk))[None, None]
    q = np.eye(Nk)[perm][None, None]
    v = rnd(1, 1, Nk, d)
    o, lse = A.forward(q, k, v, scale, False)
    assert np.abs(o[0, 0] - v[0, 0, perm]).max() < Nk * math.exp(-50) * 10
    assert np.abs(lse[0, 0] - 50.0).max() < 1e-12


def test_probability_rows_sum_to_one():
    for causal in (False, True):
        p = A.probabilities(rnd(30, 8), rnd(30, 8), 0.5, causal)
        assert np.abs(p.sum(axis=1) - 1).max() < 1e-15
        if causal:
            assert np.all(p[np.triu_indices(30, 1)] == 0)


def test_row_constant_shift_leaves_p_unchanged():
    """Adding c_i to row i of the scores (via an extra head-dim column: Q gains
    c_i/scale, K gains 1) leaves O unchanged and shifts LSE_i by c_i."""
    N, d, scale = 25, 6, 0.4
    q, k, v = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    cvec = rnd(N) * 30
    q2 = np.concatenate([q, (cvec / scale)[None, None, :, None]], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, N, 1))], axis=-1)
    for causal in (False, True):
        o1, l1 = A.forward(q, k, v, scale, causal)
        o2, l2 = A.forward(q2, k2, v, scale, causal)
        assert np.abs(o1 - o2).max() < 1e-12
        assert np.abs((l2 - l1)[0, 0] - cvec).max() < 1e-11


def _online_softmax_emulation(q, k, v, scale, bc):
    """The tiled forward of the pages, written in their notation: stream K/V
    blocks, keep running (m, l) and an unnormalised output, rescale by
    exp(m_old - m_new), divide by l once at the end ([CH18] §18.4.2 (3),
    §18.4.3; [L21] slide 12)."""
    n = k.shape[0]
    m = np.full(q.shape[0], -np.inf)
    l = np.zeros(q.shape[0])
    o = np.zeros((q.shape[0], v.shape[1]))
    for j0 in range(0, n, bc):
        s = scale * q @ k[j0:j0 + bc].T
        m_t = s.max(axis=1)
        p_t = np.exp(s - m_t[:, None])
        l_t = p_t.sum(axis=1)
        m_new = np.maximum(m, m_t)
        a = np.exp(m - m_new)
        b = np.exp(m_t - m_new)
        l = a * l + b * l_t
        o = a[:, None] * o + b[:, None] * (p_t @ v[j0:j0 + bc])
        m = m_new
    return o / l[:, None], m + np.log(l)


@pytest.mark.parametrize("bc", [1, 7, 64, 100])
def test_online_softmax_blocks_equal_naive(bc):
    N, d, scale = 100, 16, 0.25
    q, k, v = rnd(N, d) * 3, rnd(N, d), rnd(N, d)
    o_ref, l_ref = A.head_forward(q, k, v, scale, False)
    o, l = _online_softmax_emulation(q, k, v, scale, bc)
    assert np.abs(o - o_ref).max() < 1e-13
    assert np.abs(l - l_ref).max() < 1e-13


def test_two_block_rescaling_identity():
    """[L21] slide 12: O^(2) = (l1/l2) O^(1) + A2 V2 / l2 with l2 the total
    denominator; O^(1) is the block-1 output normalised by its own l1."""
    N, d, scale = 50, 8, 0.5
    q, k, v = rnd(N, d), rnd(N, d), rnd(N, d)
    h = 23
    o1, lse1 = A.head_forward(q, k[:h], v[:h], scale, False)
    l1 = np.exp(lse1)
    a2 = np.exp(scale * q @ k[h:].T)
    l2 = l1 + a2.sum(axis=1)
    o2 = (l1 / l2)[:, None] * o1 + (a2 @ v[h:]) / l2[:, None]
    o, lse = A.head_forward(q, k, v, scale, False)
    assert np.abs(o2 - o).max() < 1e-13
    assert np.abs(np.log(l2) - lse).max() < 1e-13


# --------------------------------------------------------------- backward pins

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [5, 8])
def test_backward_finite_differences(causal, N):
    """Central differences of L = sum(O * G) match the analytic gradients,
    including the GQA sum over the two query heads sharing a KV head."""
    B, Hq, Hkv, d, scale, h = 1, 2, 1, 4, 0.6, 1e-6
    q, k, v, g = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d), rnd(B, Hq, N, d)

    def loss(q_, k_, v_):
        return float((A.forward(q_, k_, v_, scale, causal)[0] * g).sum())

    dq, dk, dv = A.backward(q, k, v, g, scale, causal)
    for x, dx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        rel = np.linalg.norm(num - dx) / np.linalg.norm(dx)
        assert rel < 1e-7, (which, rel)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_finite_differences(causal):
    """The row-by-row dQ (for sizes where whole matrices do not fit) against
    central differences of L = sum(O * G) with respect to the listed rows of Q."""
    N, d, scale, h = 7, 3, 0.8, 1e-6
    q, k, v, g = rnd(N, d), rnd(N, d), rnd(N, d), rnd(N, d)
    rows = [0, 3, 6]
    got = A.head_dq_rows(q, k, v, g, scale, causal, rows)

    def loss(q_):
        return float((A.head_forward(q_, k, v, scale, causal)[0] * g).sum())

    for a, i in enumerate(rows):
        for c in range(d):
            qp, qm = q.copy(), q.copy()
            qp[i, c] += h
            qm[i, c] -= h
            num = (loss(qp) - loss(qm)) / (2 * h)
            assert abs(num - got[a, c]) <= 1e-7 * max(1.0, abs(num))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    B, Hq, Hkv, N, d, scale = 2, 4, 2, 33, 16, 0.25
    q, k, v, g = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d), rnd(B, Hq, N, d)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    out.backward(torch.from_numpy(g))
    dq, dk, dv = A.backward(q, k, v, g, scale, causal)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, (5, 0)),
                                           (False, (3, 2))])
def test_head_forward_backward_equals_separate_calls(causal, window):
    """The one-pass helper used by the full-size parity checks returns exactly
    what head_forward and head_backward return (bit for bit)."""
    N, d = 23, 8
    q, k, v, do = rnd(N, d), rnd(N, d), rnd(N, d), rnd(N, d)
    o, lse, dq, dk, dv = A.head_forward_backward(q, k, v, do, 0.4, causal, window)
    ro, rl = A.head_forward(q, k, v, 0.4, causal, window=window)
    rq, rk, rv, _ = A.head_backward(q, k, v, do, 0.4, causal, window)
    for a, b in ((o, ro), (lse, rl), (dq, rq), (dk, rk), (dv, rv)):
        assert np.array_equal(a, b)


def test_delta_equals_rowwise_do_dot_o():
    """delta_i = sum_j P_ij dP_ij equals dO_i . O_i (the identity that lets a
    pre-pass compute it from O and dO)."""
    N, d, scale = 31, 8, 0.3
    q, k, v, do = rnd(N, d), rnd(N, d), rnd(N, d), rnd(N, d)
    for causal in (False, True):
        _, _, _, delta = A.head_backward(q, k, v, do, scale, causal)
        o, _ = A.head_forward(q, k, v, scale, causal)
        assert np.abs(delta - (do * o).sum(axis=1)).max() < 1e-12


def test_key_shift_invariance_of_gradients():
    """Each row of dS sums to zero, hence sum_j dK_j = 0 per KV head (a shift
    of every key by the same vector leaves the softmax unchanged)."""
    B, Hq, Hkv, N, d, scale = 1, 2, 1, 20, 6, 0.4
    q, k, v, do = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d), rnd(B, Hq, N, d)
    for causal in (False, True):
        p = A.probabilities(q[0, 0], k[0, 0], scale, causal)
        ds = A.softmax_backward(p, do[0, 0] @ v[0, 0].T)
        assert np.abs(ds.sum(axis=1)).max() < 1e-13
        _, dk, _ = A.backward(q, k, v, do, scale, causal)
        assert np.abs(dk.sum(axis=2)).max() < 1e-12


def test_backward_closed_forms():
    """Q = 0 (uniform P, non-causal): dV_j = (1/Nk) sum_i dO_i for every j.
    Identical V rows: dP is constant along each row, so dS = 0 and dQ = dK = 0."""
    Nq, Nk, d = 9, 13, 5
    q = np.zeros((1, 1, Nq, d))
    k, v, do = rnd(1, 1, Nk, d), rnd(1, 1, Nk, d), rnd(1, 1, Nq, d)
    _, _, dv = A.backward(q, k, v, do, 0.5, False)
    assert np.abs(dv[0, 0] - do[0, 0].sum(axis=0) / Nk).max() < 1e-14
    q = rnd(1, 1, Nq, d)
    v = np.repeat(rnd(1, 1, 1, d), Nk, axis=2)
    dq, dk, _ = A.backward(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


# ----------------------------------------------------------------- decode pins

@pytest.mark.parametrize("splits", [1, 2, 64, 128])
def test_split_combine_equals_unsplit(splits):
    B, Hq, Hkv, Nk, d, scale = 2, 4, 2, 128, 8, 0.35
    q, k, v = rnd(B, Hq, 1, d) * 2, rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    o, lse, op, lp = A.decode_split(q, k, v, scale, splits)
    o_ref, lse_ref = A.forward(q, k, v, scale, False)
    assert np.abs(o - o_ref).max() < 1e-13
    assert np.abs(lse - lse_ref).max() < 1e-13
    assert op.shape == (B, Hq, splits, d) and lp.shape == (B, Hq, splits)


def test_combine_matches_page_formula_with_unnormalised_partials():
    """[CH18] §18.8.2 (2) merges (m_t, l_t, unnormalised O_t) with weights
    e^{m_t - m}; the (normalised O_t, lse_t) form used here is the same."""
    S, d = 7, 5
    m_t, l_t = rnd(S) * 3, np.exp(rnd(S))
    ou = rnd(S, d)
    mg = m_t.max()
    ref = (ou * np.exp(m_t - mg)[:, None]).sum(0) / (l_t * np.exp(m_t - mg)).sum()
    o, lse = A.combine(ou / l_t[:, None], m_t + np.log(l_t))
    assert np.abs(o - ref).max() < 1e-14
    assert abs(lse - (mg + math.log((l_t * np.exp(m_t - mg)).sum()))) < 1e-14


def test_combine_weighs_empty_chunks_zero_and_empty_rows_give_zero():
    """A chunk with no visible key has lse_c = -inf: it must weigh nothing,
    so merging with it equals merging the other chunks alone.  A row whose
    chunks are all empty saw no key at all: O = 0 and lse = -inf (the
    log-sum over an empty set), never NaN."""
    S, d = 6, 4
    op, lp = rnd(2, S, d), rnd(2, S) * 2
    lp[0, [1, 4]] = -np.inf
    lp[1, :] = -np.inf
    o, lse = A.combine(op, lp)
    keep = [0, 2, 3, 5]
    o_ref, lse_ref = A.combine(op[0, keep], lp[0, keep])
    assert np.abs(o[0] - o_ref).max() < 1e-14 and abs(lse[0] - lse_ref) < 1e-14
    assert np.array_equal(o[1], np.zeros(d)) and lse[1] == -np.inf
    assert not np.isnan(o).any()


# -------------------------------------------------------------------- fp8 pins

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F8.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_matches_torch_in_range():
    """torch's float -> float8_e4m3fn cast is round-to-nearest-even; within the
    finite range it must agree byte for byte (including exact ties)."""
    vals = torch.from_numpy(F8.e4m3_decode(np.arange(256, dtype=np.uint8)))
    fin = vals[~torch.isnan(vals)].to(torch.float32)
    mids = []
    s = torch.sort(fin.unique())[0]
    mids = ((s[1:].double() + s[:-1].double()) / 2).float()  # exact ties
    x = torch.cat([fin, mids, torch.from_numpy(rng.standard_normal(20000).astype(np.float32)) * 60,
                   torch.from_numpy(rng.standard_normal(20000).astype(np.float32)) * 0.01])
    x = x[x.abs() <= 448]
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F8.e4m3_encode(x.numpy())
    assert np.array_equal(ref, ours)


def test_e4m3_encode_saturates_and_ties_to_even():
    assert F8.e4m3_encode(np.float32(1e6)) == 0x7E          # +448
    assert F8.e4m3_encode(np.float32(-470.0)) == 0xFE       # -448
    assert F8.e4m3_encode(np.float32(464.0)) == 0x7E
    # 1 + 1/16 lies halfway between 1 (mantissa 0, even) and 1.125 (mantissa 1)
    assert F8.e4m3_encode(np.float32(1.0625)) == 0x38
    # 1.1875 lies halfway between 1.125 (odd) and 1.25 (even)
    assert F8.e4m3_encode(np.float32(1.1875)) == 0x3A
    # smallest subnormal 2^-9; half of it ties to zero (even)
    assert F8.e4m3_encode(np.float32(2.0 ** -9)) == 0x01
    assert F8.e4m3_encode(np.float32(2.0 ** -10)) == 0x00


def test_quantize_block_roundtrip_error_bound():
    """Dequantised values lie within half an e4m3 step of the input, and the
    block maximum maps exactly to code 448."""
    x = rng.standard_normal((128, 128)).astype(np.float32)
    codes, s = F8.quantize_block(x)
    deq = F8.e4m3_decode(codes) * s
    a = np.abs(x).max()
    assert np.abs(F8.e4m3_decode(codes)).max() == 448.0
    # relative step of e4m3 is 2^-3, so half a step is 2^-4 of the binade
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, a / 448 * 2.0 ** -10) * 1.0001)
    zc, zs = F8.quantize_block(np.zeros((4, 4), np.float32))
    assert zs == 1.0 and not zc.any()


@pytest.mark.parametrize("block_rows", [128, 32])
def test_quantize_multi_block_scales_and_partial_tail(block_rows):
    """Per-block quantisation over several (b, h, row-block) slabs whose
    maxima differ by four orders of magnitude, with a partial last block
    ([CH18] §18.6.2 (1)(2): one scale s = amax / 448 per block).  For every
    block: its stored scale is its own amax / 448, its largest element maps
    to code +-448, and dequantising with that scale returns every element
    within half an e4m3 step of the input.  A scale index shifted by one
    block, a block sliced at the wrong rows, or a tail taken from the wrong
    slab breaks these bounds by orders of magnitude."""
    B, H, d = 2, 3, 16
    nb_full = 3
    N = nb_full * block_rows + block_rows // 4 + 3           # partial last block
    nb = (N + block_rows - 1) // block_rows
    x = rng.standard_normal((B, H, N, d)).astype(np.float32)
    mags = np.array([0.01, 1.0, 300.0, 7.0])
    amax_ref = np.empty((B, H, nb))
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                r0, r1 = i * block_rows, min(N, (i + 1) * block_rows)
                m = mags[(i + b + 2 * h) % len(mags)]
                blk = x[b, h, r0:r1]
                blk *= np.float32(m / np.abs(blk).max())   # amax of the block is exactly m
                amax_ref[b, h, i] = np.abs(blk).max()
    codes, scales = F8.quantize(x, block_rows)
    assert scales.shape == (B, H, nb) and codes.shape == x.shape
    deq = F8.dequantize(codes, scales, block_rows)
    mag = F8.e4m3_decode(codes)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                r0, r1 = i * block_rows, min(N, (i + 1) * block_rows)
                a = amax_ref[b, h, i]
                assert scales[b, h, i] == np.float32(np.float32(a) / np.float32(448.0))
                assert np.abs(mag[b, h, r0:r1]).max() == 448.0
                xb = x[b, h, r0:r1].astype(np.float64)
                err = np.abs(deq[b, h, r0:r1] - xb)
                # half a step: 2^-4 relative for normals, 2^-10 * s for subnormals
                bound = np.maximum(np.abs(xb) * 2.0 ** -4, a / 448 * 2.0 ** -10) * 1.0001
                assert np.all(err <= bound), (b, h, i)


def test_hadamard_rotation_properties():
    import scipy.linalg
    n = 128
    assert np.array_equal(F8.sylvester(n), scipy.linalg.hadamard(n))
    signs = rng.choice([-1.0, 1.0], n)
    J = F8.rotation(signs)
    assert np.abs(J @ J.T - np.eye(n)).max() < 1e-15
    q, k = rnd(20, n), rnd(30, n)
    assert np.abs(F8.rotate(q, signs) @ F8.rotate(k, signs).T - q @ k.T).max() < 1e-12


def test_incoherent_processing_error_is_reported():
    """[L21] slide 24 reports 2.6x lower FP8 error on the authors' simulated
    outlier data.  Here the ratio is only reported: with e4m3 (a floating-point
    format) and 128-row block scales, the relative rounding error does not
    depend on the block maximum, so on 0.1% outliers of magnitude 50 the
    rotation does not lower the error of the quantised Q K^T.  What is pinned
    is that both quantised products stay within e4m3's rounding bound of the
    exact one (the rotation itself is exact: see the Hadamard test)."""
    n = 128
    q = rng.standard_normal((1, 1, 1024, n)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1024, n)).astype(np.float32)
    for t in (q, k):
        flat = t.reshape(-1)
        pos = rng.choice(flat.size, int(round(1e-3 * flat.size)), replace=False)
        flat[pos] = rng.choice([-50.0, 50.0], pos.size)
    signs = rng.choice([-1.0, 1.0], n)
    exact = q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T

    def err(qq, kk):
        cq, sq = F8.quantize(qq)
        ck, sk = F8.quantize(kk)
        s = F8.dequantize(cq, sq)[0, 0] @ F8.dequantize(ck, sk)[0, 0].T
        return np.linalg.norm(s - exact) / np.linalg.norm(exact)

    plain = err(q, k)
    rot = err(F8.rotate(q, signs).astype(np.float32), F8.rotate(k, signs).astype(np.float32))
    print(f"quantised QK^T rel-L2: plain {plain:.4f}, rotated {rot:.4f}, ratio {plain / rot:.3f}")
    # two operands each rounded with relative error <= 2^-4
    assert plain < 2 * 2.0 ** -4 and rot < 2 * 2.0 ** -4


def _outlier_inputs(n, d, seed, outliers=True):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((1, 1, n, d)).astype(np.float32) for _ in range(3))
    if outliers:
        for t in (q, k):
            flat = t.reshape(-1)
            pos = r.choice(flat.size, int(round(1e-3 * flat.size)), replace=False)
            flat[pos] = r.choice([-50.0, 50.0], pos.size)
    return q, k, v, r.choice([-1.0, 1.0], d)


def test_fp8_error_floor_against_exact_attention():
    """The fp8 workload's 5e-2 bar measured against exact attention on the
    unquantised inputs is out of reach of e4m3 operands on outlier data, at
    any scale granularity: e4m3 keeps 3 mantissa bits, so every operand
    carries a relative rounding error of up to 2^-4 whatever its block scale,
    and a key with a magnitude-50 outlier gives scores of spread 50 * scale
    ~ 4.4 whose rounding error (~0.1) moves the softmax weights by ~10%.
    Pinned here with the oracle alone: per-block (128 rows) and per-row
    scales, with and without the rotation, all stay above 5e-2; the same
    pipeline on N(0,1) inputs without outliers stays below it."""
    n, d = 1024, 128
    sc = 1 / math.sqrt(d)

    def e2e(q, k, v, signs, rot, rows):
        qq = F8.rotate(q, signs).astype(np.float32) if rot else q
        kk = F8.rotate(k, signs).astype(np.float32) if rot else k
        deq = [F8.dequantize(*F8.quantize(t, rows), rows) for t in (qq, kk, v)]
        o, _ = A.forward(*deq, sc, False)
        ex, _ = A.forward(q, k, v, sc, False)
        return np.linalg.norm(o - ex) / np.linalg.norm(ex)

    q, k, v, signs = _outlier_inputs(n, d, 8305)
    errs = {(rot, rows): e2e(q, k, v, signs, rot, rows) for rot in (False, True)
            for rows in (128, 1)}
    print("fp8 end-to-end rel-L2 vs exact on outlier data:", errs)
    assert min(errs.values()) > 5e-2
    q0, k0, v0, s0 = _outlier_inputs(n, d, 8305, outliers=False)
    clean = e2e(q0, k0, v0, s0, False, 128)
    print("without outliers:", clean)
    assert clean < 5e-2


# -------------------------------------------------------------- schedule pins

def test_lpt_worked_example_from_the_lecture():
    g = json.load(open(os.path.join(GOLD, "lpt_worked_example.json")))
    costs, W = g["costs_in_order"], g["workers"]
    loads, _ = SCH.list_schedule(costs, W)
    assert loads == g["loads_in_order"]
    order = SCH.lpt_order(costs)
    loads, _ = SCH.list_schedule([costs[i] for i in order], W)
    assert loads == g["loads_longest_first"]


def test_causal_tile_costs():
    # 128-row query tiles, 64-key KV tiles: tile i visits 2(i+1) KV tiles
    c = SCH.causal_tile_costs(2, 4, 128, 64)
    assert c == [2, 4, 6, 8] * 2
    c = SCH.causal_tile_costs(1, 3, 64, 128)
    assert c == [1, 1, 2]


# --------------------------------------------------------- flop-count pin

def test_flop_formula_against_table_18_5():
    """The benchmark counts 4*B*H*Nq*Nk*d forward FLOPs: two GEMMs of 2 n^2 d,
    whose Q K^T half is printed per head in Table 18-5."""
    from workloads import Workload
    g = json.load(open(os.path.join(GOLD, "qk_flops_table_18_5.json")))
    for row in g["rows"]:
        w = Workload("t", 1, 1, 1, row["n"], row["n"], g["d"], "bf16")
        assert abs(w.fwd_flops() / 2 - row["qk_flops"]) <= row["rel_tol"] * row["qk_flops"]
        wc = w.scaled(causal=True)
        assert wc.fwd_flops() == w.fwd_flops() / 2
        assert w.bwd_flops() == 2.5 * w.fwd_flops()


# ------------------------------------------------------- multi-token decode

@pytest.mark.parametrize("causal", [False, True])
def test_decode_multi_uniform_scores(causal):
    """Closed form: Q = 0 makes token t the mean of the V rows it sees, rows
    0 .. Nk-Nq+t when causal (all Nk otherwise), with LSE = ln(count)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 3, 11, 5
    q = np.zeros((B, Hq, Nq, d))
    k, v = rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    o, lse = A.decode_multi(q, k, v, 0.9, causal)
    for h in range(Hq):
        for t in range(Nq):
            cnt = Nk - Nq + t + 1 if causal else Nk
            assert np.allclose(o[0, h, t], v[0, h // 2, :cnt].mean(axis=0), atol=1e-13)
            assert abs(lse[0, h, t] - math.log(cnt)) < 1e-13


def test_decode_multi_special_cases():
    """One token: causal or not, it is the single-query decode (the forward
    with Nq = 1).  Nq = Nk: the end-aligned causal mask is the top-left one,
    so it is the causal forward.  Scalar loops for a general case."""
    B, Hq, Hkv, Nk, d, sc = 2, 2, 1, 9, 4, 0.5
    k, v = rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    q1 = rnd(B, Hq, 1, d)
    for causal in (False, True):
        o, l = A.decode_multi(q1, k, v, sc, causal)
        of, lf = A.forward(q1, k, v, sc, False)
        assert np.allclose(o, of, atol=1e-14) and np.allclose(l, lf, atol=1e-14)
    qn = rnd(B, Hq, Nk, d)
    o, l = A.decode_multi(qn, k, v, sc, True)
    of, lf = A.forward(qn, k, v, sc, True)
    assert np.allclose(o, of, atol=1e-14) and np.allclose(l, lf, atol=1e-14)
    Nq = 3
    q = rnd(B, Hq, Nq, d)
    o, l = A.decode_multi(q, k, v, sc, True)
    for b in range(B):
        for h in range(Hq):
            for t in range(Nq):
                w = [math.exp(sc * float(q[b, h, t] @ k[b, 0, j])) if j <= Nk - Nq + t else 0.0
                     for j in range(Nk)]
                w = np.array(w)
                assert np.allclose(o[b, h, t], (w[:, None] * v[b, 0]).sum(0) / w.sum(), atol=1e-12)
                assert abs(l[b, h, t] - math.log(w.sum())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged_multi_uniform_scores(causal):
    """Closed form through the page table: Q = 0 makes token t of entry b the
    mean of its logical V rows 0 .. seqlen-Nq+t (all seqlen rows when not
    causal), with LSE = ln(count); the pages are randomly permuted."""
    page, Hkv, Hq, d, Nq = 4, 2, 4, 3, 3
    lens = [9, 14]
    npages = 10
    cache_k, cache_v = rnd(npages, page, Hkv, d), rnd(npages, page, Hkv, d)
    perm = rng.permutation(npages)
    table = np.stack([perm[:4], perm[4:8]])
    q = np.zeros((2, Hq, Nq, d))
    o, lse = A.decode_paged_multi(q, cache_k, cache_v, table, lens, 0.7, causal)
    for b, n in enumerate(lens):
        for h in range(Hq):
            hk = h // 2
            rows = np.stack([cache_v[table[b][j // page], j % page, hk] for j in range(n)])
            for t in range(Nq):
                cnt = n - Nq + t + 1 if causal else n
                assert np.allclose(o[b, h, t], rows[:cnt].mean(axis=0), atol=1e-13)
                assert abs(lse[b, h, t] - math.log(cnt)) < 1e-13


def test_decode_paged_multi_fewer_keys_than_tokens():
    """An entry shorter than the Nq tokens: with the end-aligned causal mask
    token t sees logical keys 0 .. n-Nq+t, which is empty for the first
    Nq-n tokens (O = 0, LSE = -inf); the others are the mean of the rows they
    see under uniform scores.  Without the mask every token sees all n keys."""
    page, Hkv, Hq, d, Nq = 16, 1, 2, 3, 5
    lens = [2, 7]
    cache_k, cache_v = rnd(3, page, Hkv, d), rnd(3, page, Hkv, d)
    table = np.array([[2], [0]])
    q = np.zeros((2, Hq, Nq, d))
    for causal in (True, False):
        o, lse = A.decode_paged_multi(q, cache_k, cache_v, table, lens, 0.7, causal)
        for b, n in enumerate(lens):
            rows = cache_v[table[b][0], :n, 0]
            for h in range(Hq):
                for t in range(Nq):
                    cnt = min(n, n - Nq + t + 1) if causal else n
                    if cnt <= 0:
                        assert np.array_equal(o[b, h, t], np.zeros(d)) and lse[b, h, t] == -np.inf
                    else:
                        assert np.allclose(o[b, h, t], rows[:cnt].mean(axis=0), atol=1e-13)
                        assert abs(lse[b, h, t] - math.log(cnt)) < 1e-13


# ---------------------------------------------------------------- varlen pins

def _pack_lengths(lens):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    return cu


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_uniform_scores_mean_of_own_sequence(causal):
    """Closed form: Q = 0 makes every visible score equal, so row i of
    sequence b is the mean of the V rows it may see in its own sequence and
    LSE = ln(count); rows of other sequences never contribute."""
    lens = [5, 1, 7, 3]
    cu = _pack_lengths(lens)
    Hq, Hkv, d = 4, 2, 6
    q = np.zeros((cu[-1], Hq, d))
    k, v = rnd(cu[-1], Hkv, d), rnd(cu[-1], Hkv, d)
    o, lse = A.forward_varlen(q, k, v, cu, cu, 0.7, causal)
    for b, n in enumerate(lens):
        for i in range(n):
            row = cu[b] + i
            cnt = i + 1 if causal else n
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                ref = v[cu[b]:cu[b] + cnt, hk].mean(axis=0)
                assert np.allclose(o[row, h], ref, rtol=0, atol=1e-13)
                assert abs(lse[h, row] - math.log(cnt)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_block_diagonal_masked_attention(causal):
    """Brute force: attention over the whole packed token axis with a
    block-diagonal mask (same sequence, and j <= i within it when causal),
    written with explicit loops, independent of the per-sequence slicing."""
    lens = [4, 9, 2]
    cu = _pack_lengths(lens)
    T, Hq, Hkv, d = cu[-1], 2, 1, 5
    q, k, v = rnd(T, Hq, d), rnd(T, Hkv, d), rnd(T, Hkv, d)
    scale = 0.45
    o, lse = A.forward_varlen(q, k, v, cu, cu, scale, causal)
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(n) for n in lens])
    for h in range(Hq):
        for i in range(T):
            w = []
            for j in range(T):
                ok = seq[i] == seq[j] and (not causal or pos[j] <= pos[i])
                w.append(math.exp(scale * float(q[i, h] @ k[j, 0])) if ok else 0.0)
            w = np.array(w)
            assert np.allclose(o[i, h], (w[:, None] * v[:, 0]).sum(0) / w.sum(), atol=1e-12)
            assert abs(lse[h, i] - math.log(w.sum())) < 1e-12


def test_varlen_sequences_are_isolated():
    """Changing one sequence's K/V rows leaves every other sequence's output
    unchanged (no attention across the packing boundary)."""
    lens = [6, 3, 8]
    cu = _pack_lengths(lens)
    T, Hq, d = cu[-1], 2, 4
    q, k, v = rnd(T, Hq, d), rnd(T, Hq, d), rnd(T, Hq, d)
    o1, l1 = A.forward_varlen(q, k, v, cu, cu, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 3.0
    v2[cu[1]:cu[2]] -= 2.0
    o2, l2 = A.forward_varlen(q, k2, v2, cu, cu, 0.5, True)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    assert np.array_equal(o1[keep], o2[keep]) and np.array_equal(l1[:, keep], l2[:, keep])
    assert not np.allclose(o1[cu[1]:cu[2]], o2[cu[1]:cu[2]])


@pytest.mark.parametrize("causal,lens_q,lens_k", [
    (True, [4, 2, 5], [4, 2, 5]),
    (False, [3, 2, 0, 4], [2, 0, 3, 5]),   # queries without keys, keys without queries
])
def test_varlen_backward_finite_differences(causal, lens_q, lens_k):
    """Central differences of L = sum(O * G) over the packed forward match
    backward_varlen (GQA), including the zero gradients of rows with no
    visible key and of keys that no query sees."""
    cq, ck = _pack_lengths(lens_q), _pack_lengths(lens_k)
    Hq, Hkv, d, scale, h = 2, 1, 3, 0.6, 1e-6
    q, k, v = rnd(cq[-1], Hq, d), rnd(ck[-1], Hkv, d), rnd(ck[-1], Hkv, d)
    g = rnd(cq[-1], Hq, d)
    dq, dk, dv = A.backward_varlen(q, k, v, g, cq, ck, scale, causal)

    def loss(q_, k_, v_):
        return float((A.forward_varlen(q_, k_, v_, cq, ck, scale, causal)[0] * g).sum())

    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.linalg.norm(num - dx) <= 1e-7 * max(1.0, np.linalg.norm(dx))
    for b in range(len(lens_q)):
        if lens_k[b] == 0:
            assert not dq[cq[b]:cq[b + 1]].any()
        if lens_q[b] == 0:
            assert not dk[ck[b]:ck[b + 1]].any() and not dv[ck[b]:ck[b + 1]].any()


# ------------------------------------------------------------ paged KV pins

def test_paged_gather_reproduces_scattered_rows():
    """Rows scattered into randomly permuted physical pages come back in
    logical order through the page table, including a partial last page."""
    page, Hkv, d, n = 4, 3, 5, 18
    npages = 9
    contig = rnd(n, Hkv, d)
    perm = rng.permutation(npages)
    cache = rnd(npages, page, Hkv, d)          # unused slots hold noise
    table = perm[: (n + page - 1) // page]
    for t in range(n):
        cache[table[t // page], t % page] = contig[t]
    for hk in range(Hkv):
        assert np.array_equal(A.gather_pages(cache, table, n, hk), contig[:, hk])


def test_paged_decode_uniform_scores_mean_of_first_rows():
    """Closed form: Q = 0 gives O = mean of the sequence's first seqlen
    logical V rows and LSE = ln(seqlen); rows past seqlen (still inside the
    last page) must not count."""
    page, Hq, Hkv, d = 8, 4, 2, 6
    seqlens = [13, 1, 16]
    npages = 10
    kc, vc = rnd(npages, page, Hkv, d), rnd(npages, page, Hkv, d)
    table = np.stack([rng.permutation(npages)[:2] for _ in seqlens])
    q = np.zeros((len(seqlens), Hq, 1, d))
    o, lse = A.decode_paged(q, kc, vc, table, seqlens, 0.9)
    for b, n in enumerate(seqlens):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            rows = [vc[table[b][t // page], t % page, hk] for t in range(n)]
            assert np.allclose(o[b, h, 0], np.mean(rows, axis=0), atol=1e-13)
            assert abs(lse[b, h, 0] - math.log(n)) < 1e-13


# ------------------------------------------------------- sliding-window pins

@pytest.mark.parametrize("causal,window", [(False, (3, 2)), (True, (4, -1)), (True, (0, 0)),
                                           (False, (-1, 1)), (False, (0, 5))])
def test_window_uniform_scores_mean_of_window(causal, window):
    """Closed form: Q = 0 gives row i the mean of V over the keys
    max(0, i-left) .. min(N-1, i+right) (and <= i when causal), and
    LSE = ln(count)."""
    N, d = 11, 4
    q = np.zeros((1, 1, N, d))
    k, v = rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = A.forward(q, k, v, 0.8, causal, window=window)
    left, right = window
    for i in range(N):
        lo = 0 if left < 0 else max(0, i - left)
        hi = N - 1 if right < 0 else min(N - 1, i + right)
        if causal:
            hi = min(hi, i)
        assert np.allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(axis=0), atol=1e-13)
        assert abs(lse[0, 0, i] - math.log(hi - lo + 1)) < 1e-13


def test_window_brute_force_loops():
    """Scalar loops over (i, j) with the window written out."""
    N, d, left, right, scale = 9, 3, 2, 3, 0.6
    q, k, v = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = A.forward(q, k, v, scale, False, window=(left, right))
    for i in range(N):
        w = [math.exp(scale * float(q[0, 0, i] @ k[0, 0, j])) if i - left <= j <= i + right
             else 0.0 for j in range(N)]
        w = np.array(w)
        assert np.allclose(o[0, 0, i], (w[:, None] * v[0, 0]).sum(0) / w.sum(), atol=1e-12)
        assert abs(lse[0, 0, i] - math.log(w.sum())) < 1e-12


def test_window_degenerate_and_trivial_cases():
    """(0, 0): each row sees only its own key, so O = V and LSE = s_ii.
    (-1, -1) is global attention; causal with (-1, 0) or (N, 0) is causal."""
    N, d, scale = 7, 5, 0.9
    q, k, v = rnd(2, 2, N, d), rnd(2, 2, N, d), rnd(2, 2, N, d)
    o, lse = A.forward(q, k, v, scale, False, window=(0, 0))
    assert np.allclose(o, v, atol=1e-14)
    assert np.allclose(lse, scale * np.einsum("bhnd,bhnd->bhn", q, k), atol=1e-13)
    og, lg = A.forward(q, k, v, scale, False)
    ow, lw = A.forward(q, k, v, scale, False, window=(-1, -1))
    assert np.array_equal(og, ow) and np.array_equal(lg, lw)
    oc, lc = A.forward(q, k, v, scale, True)
    for win in ((-1, 0), (N, 0), (-1, -1)):
        ow, lw = A.forward(q, k, v, scale, True, window=win)
        assert np.array_equal(oc, ow) and np.array_equal(lc, lw)


@pytest.mark.parametrize("causal,window", [(True, (2, -1)), (False, (1, 2))])
def test_window_backward_finite_differences(causal, window):
    """Central differences of L = sum(O * G) under a sliding window (GQA)."""
    B, Hq, Hkv, N, d, scale = 1, 2, 1, 6, 3, 0.7
    q, k, v, g = rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d), rnd(B, Hq, N, d)
    dq, dk, dv = A.backward(q, k, v, g, scale, causal, window=window)

    def loss(q_, k_, v_):
        return float((A.forward(q_, k_, v_, scale, causal, window=window)[0] * g).sum())

    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.linalg.norm(num - dx) <= 1e-7 * max(1.0, np.linalg.norm(dx))


# -------------------------------------------------------- block-sparse pins

def _csr(rows):
    ptr, idx = [0], []
    for r in rows:
        idx += list(r)
        ptr.append(len(idx))
    return ptr, idx


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_uniform_scores_and_empty_rows(causal):
    """Closed form: Q = 0 gives each row the mean of V over its visible keys
    (the union of its listed blocks, intersected with j <= i when causal)
    and LSE = ln(count); a row with no listed block gets O = 0, LSE = -inf."""
    N, d, bq, bk = 12, 3, 4, 3
    ptr, idx = _csr([[0, 2], [], [3, 1]])       # query blocks 0, 1, 2
    q = np.zeros((1, 1, N, d))
    k, v = rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = A.forward_block_sparse(q, k, v, 0.5, ptr, idx, bq, bk, causal)
    vis = {0: set(range(0, 3)) | set(range(6, 9)), 1: set(), 2: set(range(9, 12)) | set(range(3, 6))}
    for i in range(N):
        keys = sorted(j for j in vis[i // bq] if not causal or j <= i)
        if not keys:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
        else:
            assert np.allclose(o[0, 0, i], v[0, 0, keys].mean(axis=0), atol=1e-13)
            assert abs(lse[0, 0, i] - math.log(len(keys))) < 1e-13


def test_block_sparse_brute_force_loops():
    """Scalar loops over (i, j) with the block test written out."""
    N, Nk, d, bq, bk, scale = 7, 10, 3, 3, 4, 0.7
    ptr, idx = _csr([[2], [0, 1], [1, 2]])
    q, k, v = rnd(1, 1, N, d), rnd(1, 1, Nk, d), rnd(1, 1, Nk, d)
    o, lse = A.forward_block_sparse(q, k, v, scale, ptr, idx, bq, bk)
    for i in range(N):
        blocks = idx[ptr[i // bq]:ptr[i // bq + 1]]
        w = np.array([math.exp(scale * float(q[0, 0, i] @ k[0, 0, j])) if j // bk in blocks else 0.0
                      for j in range(Nk)])
        assert np.allclose(o[0, 0, i], (w[:, None] * v[0, 0]).sum(0) / w.sum(), atol=1e-12)
        assert abs(lse[0, 0, i] - math.log(w.sum())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_all_blocks_is_dense(causal):
    """Listing every key block reproduces the dense (or causal) forward."""
    N, d, bq, bk = 20, 4, 8, 6
    q, k, v = rnd(2, 2, N, d), rnd(2, 2, N, d), rnd(2, 2, N, d)
    nb = -(-N // bk)
    ptr, idx = _csr([list(range(nb))] * (-(-N // bq)))
    o, lse = A.forward_block_sparse(q, k, v, 0.4, ptr, idx, bq, bk, causal)
    od, ld = A.forward(q, k, v, 0.4, causal)
    assert np.allclose(o, od, atol=1e-14) and np.allclose(lse, ld, atol=1e-14)


@pytest.mark.parametrize("causal,rows", [
    (False, [[0, 2], [], [1]]),         # an empty query block; key block 3 never listed
    (True, [[1], [0, 2], [3, 1, 0]]),   # causal: rows 0..3 list only block 1 (all after them)
])
def test_block_sparse_backward_finite_differences(causal, rows):
    """Central differences of L = sum(O * G) over the block-sparse forward
    match backward_block_sparse (GQA), including exactly-zero gradients for
    rows that see no key and for keys in no visible block."""
    N, d, bq, bk, scale, h = 12, 3, 4, 3, 0.6, 1e-6
    ptr, idx = _csr(rows)
    q, k, v, g = rnd(1, 2, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 2, N, d)
    dq, dk, dv = A.backward_block_sparse(q, k, v, g, scale, ptr, idx, bq, bk, causal)

    def loss(q_, k_, v_):
        return float((A.forward_block_sparse(q_, k_, v_, scale, ptr, idx, bq, bk, causal)[0]
                      * g).sum())

    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.linalg.norm(num - dx) <= 1e-7 * max(1.0, np.linalg.norm(dx))
    ok = A.block_sparse_allowed(N, N, ptr, idx, bq, bk, causal)
    assert not dq[:, :, ~ok.any(axis=1)].any()
    assert not dk[:, :, ~ok.any(axis=0)].any() and not dv[:, :, ~ok.any(axis=0)].any()
    assert (~ok.any(axis=1)).any() and (~ok.any(axis=0)).any()


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_all_blocks_is_dense(causal):
    """Listing every key block reproduces the dense (or causal) backward."""
    N, d, bq, bk = 20, 4, 8, 6
    q, k, v, g = rnd(2, 2, N, d), rnd(2, 1, N, d), rnd(2, 1, N, d), rnd(2, 2, N, d)
    nb = -(-N // bk)
    ptr, idx = _csr([list(range(nb))] * (-(-N // bq)))
    got = A.backward_block_sparse(q, k, v, g, 0.4, ptr, idx, bq, bk, causal)
    want = A.backward(q, k, v, g, 0.4, causal)
    for a, b in zip(got, want):
        assert np.allclose(a, b, atol=1e-13)
