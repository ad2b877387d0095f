"""Pins of the emulated FP8 backward oracle (oracle/fp8_backward.py) and of the
e5m2 codec and power-of-two block scales it uses (oracle/fp8.py), against
torch's float8 formats, exact rational arithmetic, brute force on tiny inputs
and central differences of the loss.  None of these tests call the HIP library.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from oracle import fp8_backward as FB

rng = np.random.default_rng(5150)


# ------------------------------------------------------------------ e5m2 codec

def test_e5m2_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = F8.e5m2_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 6
    assert np.array_equal(ref[~nan], ours[~nan])
    fin = ours[np.isfinite(ours)]
    assert fin.max() == F8.E5M2_MAX and fin[fin > 0].min() == 2.0 ** -16


def test_e5m2_encode_matches_torch_in_range():
    """torch's float -> float8_e5m2 cast rounds to nearest even: within the
    finite range it agrees byte for byte, exact ties included."""
    vals = F8.e5m2_decode(np.arange(256, dtype=np.uint8))
    fin = np.unique(vals[np.isfinite(vals)]).astype(np.float32)
    mids = ((fin[1:].astype(np.float64) + fin[:-1]) / 2).astype(np.float32)   # exact ties
    x = np.concatenate([fin, mids,
                        rng.standard_normal(20000).astype(np.float32) * 3000,
                        rng.standard_normal(20000).astype(np.float32) * 1e-3,
                        rng.standard_normal(20000).astype(np.float32) * 1e-5])
    x = x[np.abs(x) <= F8.E5M2_MAX]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(F8.e5m2_encode(x), ref)


def test_e5m2_encode_hand_picked_ties():
    # 1 + 1/8 lies halfway between 1 (mantissa 0, even) and 1.25 (mantissa 1)
    assert F8.e5m2_encode(np.float32(1.125)) == 0x3C
    # 1.375 lies halfway between 1.25 (odd) and 1.5 (even)
    assert F8.e5m2_encode(np.float32(1.375)) == 0x3E
    # 1.75 + 1/8 lies halfway between 1.75 (odd) and 2 (even, next binade)
    assert F8.e5m2_encode(np.float32(1.875)) == 0x40
    # smallest subnormal 2^-16; half of it ties to zero (even)
    assert F8.e5m2_encode(np.float32(2.0 ** -16)) == 0x01
    assert F8.e5m2_encode(np.float32(2.0 ** -17)) == 0x00
    assert F8.e5m2_encode(np.float32(-57344.0)) == 0xFB


# ----------------------------------------------------- power-of-two exponents

def _exact_exponent(amax, fmt_max):
    """Smallest integer e with amax <= fmt_max * 2^e, in exact rationals."""
    r = Fraction(float(amax)) / Fraction(fmt_max)
    e = 0
    while r > Fraction(2) ** e:
        e += 1
    while r <= Fraction(2) ** (e - 1):
        e -= 1
    return e


@pytest.mark.parametrize("fmt_max", [F8.E4M3_MAX, F8.E5M2_MAX])
def test_pow2_exponent_against_exact_rationals(fmt_max):
    edge = [fmt_max * 2.0 ** k for k in range(-30, 12)]          # exactly on a boundary
    near = [np.nextafter(np.float32(v), np.float32(np.inf)) for v in edge[:-1]]
    rand = np.exp(rng.uniform(-40, 20, 3000)).astype(np.float32)
    vals = np.array(edge + near + list(rand), np.float64)
    want = np.array([_exact_exponent(a, fmt_max) for a in vals])
    got1 = np.array([F8.pow2_exponent(a, fmt_max) for a in vals])
    got2 = F8.pow2_exponents(vals, fmt_max)
    assert np.array_equal(got1, want) and np.array_equal(got2, want)
    assert F8.pow2_exponent(0.0, fmt_max) == 0 and F8.pow2_exponents(np.zeros(3), fmt_max).tolist() == [0] * 3
    # on a boundary the block maximum lands on the format maximum itself
    assert F8.pow2_exponent(fmt_max * 8, fmt_max) == 3
    assert F8.pow2_exponent(F8.E4M3_MAX, F8.E4M3_MAX) == 0 and F8.pow2_exponent(1.0, F8.E4M3_MAX) == -8


# ------------------------------------------------------ blockwise quantiser

def _quantize_pow2_loops(x, fmt, block):
    """Brute force: every block by explicit loops, scalar exponent rule,
    element-by-element rounding."""
    enc, dec, mx = ((F8.e4m3_encode, F8.e4m3_decode, F8.E4M3_MAX) if fmt == "e4m3"
                    else (F8.e5m2_encode, F8.e5m2_decode, F8.E5M2_MAX))
    R, C = x.shape
    br, bc = block
    out = np.zeros((R, C))
    exps = np.zeros((-(-R // br), -(-C // bc)), np.int64)
    for bi in range(exps.shape[0]):
        for bj in range(exps.shape[1]):
            rows = range(bi * br, min(R, (bi + 1) * br))
            cols = range(bj * bc, min(C, (bj + 1) * bc))
            amax = max(abs(float(x[i, j])) for i in rows for j in cols)
            e = F8.pow2_exponent(amax, mx)
            exps[bi, bj] = e
            for i in rows:
                for j in cols:
                    y = np.float32(float(x[i, j]) * 2.0 ** -e)
                    out[i, j] = float(dec(enc(y))) * 2.0 ** e
    return out, exps


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("block", [(1, 32), (32, 1), (32, 16), (5, 7)])
def test_quantize_pow2_equals_brute_force(fmt, block):
    """Ragged on both axes, blocks of magnitudes twelve orders apart and an
    all-zero block."""
    R, C = 70, 45
    x = rng.standard_normal((R, C)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (R, 1))).astype(np.float32)
    x[:block[0], :block[1]] = 0.0
    got, ge = F8.quantize_pow2(x, fmt, block)
    want, we = _quantize_pow2_loops(x, fmt, block)
    assert np.array_equal(ge, we) and np.array_equal(got, want)


@pytest.mark.parametrize("fmt,half_step,sub_half", [("e4m3", 2.0 ** -4, 2.0 ** -10),
                                                    ("e5m2", 2.0 ** -3, 2.0 ** -17)])
def test_quantize_pow2_error_bound_and_block_maximum(fmt, half_step, sub_half):
    """Each value comes back within half a step of its format (relative for
    normals, absolute 2^e times half the smallest subnormal below), the
    scaled block maximum lies in (max/2, max], and the scaling is exact:
    multiplying one block by a power of two multiplies its output by the
    same power and leaves every other block unchanged."""
    mx = F8.E4M3_MAX if fmt == "e4m3" else F8.E5M2_MAX
    x = (rng.standard_normal((96, 64)) * np.exp2(rng.integers(-10, 10, (96, 1)))).astype(np.float32)
    deq, exps = F8.quantize_pow2(x, fmt, (32, 16))
    e_el = np.repeat(np.repeat(exps, 32, 0), 16, 1).astype(np.float64)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * half_step, sub_half * np.exp2(e_el)))
    amax = np.abs(x).reshape(3, 32, 4, 16).max(axis=(1, 3)) * np.exp2(-exps.astype(np.float64))
    assert np.all((amax > mx / 2) & (amax <= mx))
    y = x.copy()
    y[32:64, 16:32] *= np.float32(2.0 ** -37)
    deq2, exps2 = F8.quantize_pow2(y, fmt, (32, 16))
    assert exps2[1, 1] == exps[1, 1] - 37
    want = deq.copy()
    want[32:64, 16:32] *= 2.0 ** -37
    assert np.array_equal(deq2, want)


# ---------------------------------------------------------- FP8 backward

@pytest.mark.parametrize("causal", [False, True])
def test_unquantised_path_is_the_exact_backward(causal):
    B, Hq, Hkv, N, d, scale = 1, 4, 2, 45, 16, 0.3
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d),
                                                      (B, Hkv, N, d), (B, Hq, N, d)))
    q, k, v, do = (t.astype(np.float32) for t in (q, k, v, do))
    got = FB.backward_fp8(q, k, v, do, scale, causal, quantize=False)
    want = A.backward(q, k, v, do, scale, causal)
    for a, b in zip(got, want):
        assert np.abs(a - b).max() < 1e-13 * max(1.0, np.abs(b).max())


def test_delta_from_the_given_output():
    """With o = the exact O the delta rowsum(dO * O) equals rowsum(P * dP)
    ([CH18] §18.4.4), so the unquantised result is the exact backward; a
    perturbation E of o moves delta_i by rowsum(dO_i * E_i) and dQ_i by
    exactly -scale * delta_i' * (P K)_i (dK_j by -scale * sum_i delta_i' P_ij
    Q_i), the closed form of dS = P (dP - delta)."""
    N, d, scale = 37, 8, 0.45
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        o, _ = A.head_forward(q, k, v, scale, causal)
        base = FB.head_backward_fp8(q, k, v, do, scale, causal, quantize=False)
        with_o = FB.head_backward_fp8(q, k, v, do, scale, causal, quantize=False, o=o)
        for a, b in zip(base, with_o):
            assert np.abs(a - b).max() < 1e-12
        e = rng.standard_normal((N, d)) * 1e-3
        pert = FB.head_backward_fp8(q, k, v, do, scale, causal, quantize=False, o=o + e)
        dd = (do * e).sum(axis=1)
        p, _, _ = A.softmax_rows(A.scores(q, k, scale, causal))
        assert np.abs(pert[0] - (with_o[0] - scale * dd[:, None] * (p @ k))).max() < 1e-12
        assert np.abs(pert[1] - (with_o[1] - scale * (p * dd[:, None]).T @ q)).max() < 1e-12
        assert np.array_equal(pert[2], with_o[2])


def _bounds(ds, other, fmt_ds, blk_ds, blk_other, scale):
    """Elementwise bound on |scale * (ds^ other^ - ds other)| from the two
    operands' per-element rounding bounds:
    |x^y^ - xy| <= |x^ - x| |y^| + |x| |y^ - y|."""
    h_ds, s_ds = (2.0 ** -3, 2.0 ** -17) if fmt_ds == "e5m2" else (2.0 ** -4, 2.0 ** -10)
    ds32 = ds.astype(np.float32)
    ds_q, e_ds = F8.quantize_pow2(ds32, fmt_ds, blk_ds)
    o_q, e_o = F8.quantize_pow2(other.astype(np.float32), "e4m3", blk_other)

    def per_elem(x, exps, blk, h, s):
        e_el = np.repeat(np.repeat(exps, blk[0], 0), blk[1], 1)[:x.shape[0], :x.shape[1]]
        return np.maximum(np.abs(x) * h, s * np.exp2(e_el.astype(np.float64)))

    b_ds = per_elem(ds32.astype(np.float64), e_ds, blk_ds, h_ds, s_ds)
    b_o = per_elem(other, e_o, blk_other, 2.0 ** -4, 2.0 ** -10)
    # plus the rounding of dS to float32 before quantisation
    return abs(scale) * (b_ds @ np.abs(o_q) + np.abs(ds) @ b_o + np.abs(ds) * 2.0 ** -24 @ np.abs(o_q))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_gradients_against_central_differences(causal):
    """The fp8 gradients dQ and dK stand within the operands' rounding bound
    of central differences of L = sum(O * G), and dV (high precision) matches
    them; quantisation visibly happened (dQ, dK differ from the exact ones)."""
    N, d, scale, h = 40, 8, 0.5, 1e-6
    q, k, v, g = (rng.standard_normal((N, d)).astype(np.float32) for _ in range(4))
    q64, k64, v64, g64 = (t.astype(np.float64) for t in (q, k, v, g))

    def loss(q_, k_, v_):
        return float((A.head_forward(q_, k_, v_, scale, causal)[0] * g64).sum())

    def num_grad(which):
        base = [q64, k64, v64]
        out = np.zeros_like(base[which])
        for i in range(N):
            for c in range(d):
                p = [t.copy() for t in base]
                m = [t.copy() for t in base]
                p[which][i, c] += h
                m[which][i, c] -= h
                out[i, c] = (loss(*p) - loss(*m)) / (2 * h)
        return out

    dq, dk, dv = FB.head_backward_fp8(q, k, v, g, scale, causal)
    nq, nk, nv = num_grad(0), num_grad(1), num_grad(2)
    p, _, _ = A.softmax_rows(A.scores(q64, k64, scale, causal))
    ds = A.softmax_backward(p, g64 @ v64.T)
    bq = _bounds(ds, k64, "e5m2", (1, 32), (32, d), scale)
    bk = _bounds(ds.T, q64, "e5m2", (1, 32), (32, d), scale)
    fd = 1e-7
    assert np.all(np.abs(dq - nq) <= bq + fd)
    assert np.all(np.abs(dk - nk) <= bk + fd)
    assert np.abs(dv - nv).max() <= fd
    assert np.abs(dq - nq).max() > 1e-4 and np.abs(dk - nk).max() > 1e-4


def test_block_geometry_decides_what_flushes_to_zero():
    """With power-of-two scales a block's exponent does not change how a
    normal value rounds; it decides which values fall below the format's
    smallest subnormal.  Rows of dO (hence of dS, which is linear in each
    row of dO) scaled by 2^-40 sit 40 binades below their neighbours, more
    than e5m2 spans.  dK's dS blocks span 32 queries of one key, so those
    rows flush to zero there: dK equals dK with the rows zeroed, bit for
    bit.  dQ's blocks span 32 keys of one query, so such a row keeps its own
    exponent: its dQ row is exactly 2^-40 times the unscaled one and every
    other row is unchanged.  Blocks laid along the other axis fail both."""
    N, d, scale = 96, 16, 0.25
    q, k, v, g = (rng.standard_normal((N, d)).astype(np.float32) for _ in range(4))
    dq0, dk0, _ = FB.head_backward_fp8(q, k, v, g, scale, False)
    gs, gz = g.copy(), g.copy()
    gs[40:48] *= np.float32(2.0 ** -40)
    gz[40:48] = 0.0
    dqs, dks, _ = FB.head_backward_fp8(q, k, v, gs, scale, False)
    _, dkz, _ = FB.head_backward_fp8(q, k, v, gz, scale, False)
    assert np.array_equal(dks, dkz) and not np.array_equal(dk0, dkz)
    assert np.array_equal(np.delete(dqs, np.s_[40:48], 0), np.delete(dq0, np.s_[40:48], 0))
    assert np.array_equal(dqs[40:48], dq0[40:48] * 2.0 ** -40)
    assert np.abs(dqs[40:48]).min() > 0


def test_gqa_sums_query_heads():
    B, Hq, Hkv, N, d, scale = 1, 4, 2, 40, 8, 0.4
    q, do = (rng.standard_normal((B, Hq, N, d)).astype(np.float32) for _ in range(2))
    k, v = (rng.standard_normal((B, Hkv, N, d)).astype(np.float32) for _ in range(2))
    dq, dk, dv = FB.backward_fp8(q, k, v, do, scale, True)
    for h in range(Hq):
        a, bk, bv = FB.head_backward_fp8(q[0, h], k[0, h // 2], v[0, h // 2], do[0, h], scale, True)
        assert np.array_equal(dq[0, h], a)
    parts = [FB.head_backward_fp8(q[0, h], k[0, 1], v[0, 1], do[0, h], scale, True) for h in (2, 3)]
    assert np.abs(dk[0, 1] - (parts[0][1] + parts[1][1])).max() < 1e-13
    assert np.abs(dv[0, 1] - (parts[0][2] + parts[1][2])).max() < 1e-13
