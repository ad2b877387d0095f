"""FP8 (e4m3) reference for the quantised forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the benchmark's CPU-baseline leg may use this module;
it shares no code with the HIP library.

Pages cited:
  [L21]  "CMU 11-868 L21 FlashAttention" digest (quidproquo.cc), slide 24:
         incoherent processing -- multiply Q and K by the same random
         orthogonal (Hadamard) matrix J; (QJ)(KJ)^T = QK^T, outliers spread out.
  [CH18] "第 18 章 FlashAttention", §18.6.2 (1)(2): E4M3 with range +-448,
         per-block scale s = amax / 448, FP32 accumulation and softmax.

  [CH18] §18.6.2 (3): the backward quantises dS blockwise to E5M2 (range
         +-57344, 2 mantissa bits) and runs dQ = dS K and dK = dS^T Q on fp8
         products, with fp32 accumulation.

Readings where the pages are silent (each listed in the design notes):
  * the format is OCP e4m3fn: bias 7, no infinities, only S.1111.111 is NaN,
    largest finite 448;
  * rounding is to nearest, ties to even mantissa; values beyond 448 saturate
    to +-448 (no NaN is ever produced);
  * a block is one (b, h, 128-row) slab over the full head dimension, for Q, K
    and V alike; if the block is all zero its scale is 1;
  * the quantiser multiplies by the fp32 reciprocal r = fp32(448 / amax) and
    rounds fp32(x * r); the stored scale is fp32(amax / 448);
  * J = diag(sigma) H / sqrt(n) with H the Sylvester Hadamard matrix and sigma
    a seeded +-1 vector; it rotates the head dimension of Q and K only.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6     # 2^-6 is the smallest normal
_MANT_BITS = 3


def e4m3_decode(codes) -> np.ndarray:
    """Value (float64) of each e4m3fn byte; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS)
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(y) -> np.ndarray:
    """Round float32 values to e4m3fn codes: nearest, ties to even, saturating.

    Works on the exact value of each float32 (widened to float64, where every
    step below is exact: scaling by powers of two and rounding to an integer).
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # exponent of the binade holding a (frexp: a = f * 2^ex, 0.5 <= f < 1)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    quantum = np.exp2((e - _MANT_BITS).astype(np.float64))
    n = np.rint(a / quantum)            # round half to even
    val = n * quantum                   # rounded magnitude (<= 448 after clamp)
    _, ex2 = np.frexp(val)
    e2 = ex2.astype(np.int64) - 1
    normal = val >= 2.0 ** _MIN_NORMAL_EXP
    exp_field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, val / np.exp2((e2 - _MANT_BITS).astype(np.float64)) - 8,
                    val / 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS))
    code = (exp_field << 3) | mant.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def quantize_block(x32):
    """Quantise one block (any shape) of float32 values.

    Returns (codes uint8 same shape, scale float32).  amax = max |x|;
    r = fp32(448 / amax); codes = e4m3(fp32(x * r)); scale = fp32(amax / 448).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    a = np.float32(np.abs(x32).max()) if x32.size else np.float32(0)
    if a == 0:
        return np.zeros(x32.shape, np.uint8), np.float32(1.0)
    r = np.float32(E4M3_MAX) / a
    y = (x32 * r).astype(np.float32)
    return e4m3_encode(y), np.float32(a / np.float32(E4M3_MAX))


def quantize(x32, block_rows=128):
    """Per-(b, h, row-block) quantisation of x [B][H][N][d] (float32 values).

    Returns (codes [B][H][N][d] uint8, scales [B][H][ceil(N/block_rows)] fp32).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    B, H, N, d = x32.shape
    nb = (N + block_rows - 1) // block_rows
    codes = np.empty(x32.shape, np.uint8)
    scales = np.empty((B, H, nb), np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sl = slice(i * block_rows, min(N, (i + 1) * block_rows))
                codes[b, h, sl], scales[b, h, i] = quantize_block(x32[b, h, sl])
    return codes, scales


def dequantize(codes, scales, block_rows=128):
    """Values decode(code) * scale of the code's block, as float64."""
    vals = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, np.float64), block_rows, axis=-1)
    return vals * s[..., :vals.shape[2], None]


E5M2_MAX = 57344.0


def e5m2_decode(codes) -> np.ndarray:
    """Value (float64) of each e5m2 byte: bias 15, 2 mantissa bits, subnormals
    below 2^-14; exponent field 31 is inf (mantissa 0) or NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    sub = m * 2.0 ** (-14 - 2)
    nrm = (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def e5m2_encode(y) -> np.ndarray:
    """Round float32 values to e5m2 codes: nearest, ties to even mantissa.
    Only for |y| <= 57344 (the largest finite value), which the power-of-two
    block scales below guarantee; exact in float64 like e4m3_encode."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    assert np.all(np.abs(y) <= E5M2_MAX)
    neg = np.signbit(y)
    a = np.abs(y)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -14)
    quantum = np.exp2((e - 2).astype(np.float64))
    val = np.rint(a / quantum) * quantum
    _, ex2 = np.frexp(val)
    e2 = ex2.astype(np.int64) - 1
    normal = val >= 2.0 ** -14
    exp_field = np.where(normal, e2 + 15, 0)
    mant = np.where(normal, val / np.exp2((e2 - 2).astype(np.float64)) - 4, val / 2.0 ** -16)
    code = (exp_field << 2) | mant.astype(np.int64)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def pow2_exponent(amax, fmt_max):
    """Smallest integer e with amax <= fmt_max * 2^e (0 for an all-zero block):
    scaling a block by 2^-e then puts its largest magnitude in
    (fmt_max/2, fmt_max], and the scaling itself is exact."""
    a = float(amax)
    if a == 0.0:
        return 0
    e = int(np.ceil(np.log2(a / fmt_max)))
    while a > fmt_max * 2.0 ** e:
        e += 1
    while a <= fmt_max * 2.0 ** (e - 1):
        e -= 1
    return e


def pow2_exponents(amax, fmt_max):
    """pow2_exponent over an array of block maxima (same rule, vectorised:
    a first guess from log2, then the two corrections of the definition)."""
    a = np.asarray(amax, np.float64)
    safe = np.where(a > 0, a, fmt_max)
    e = np.ceil(np.log2(safe / fmt_max)).astype(np.int64)
    e = np.where(safe > fmt_max * np.exp2(e.astype(np.float64)), e + 1, e)
    e = np.where(safe <= fmt_max * np.exp2((e - 1).astype(np.float64)), e - 1, e)
    return np.where(a > 0, e, 0)


def quantize_pow2(x, fmt, block):
    """Blockwise quantisation of a 2-D array with power-of-two scales.
    ``x`` [R][C] (float32 values); ``block`` = (rows, cols) of one block,
    blocks aligned at (0, 0) (the last ones may be partial).  Each block gets
    e = pow2_exponent(max |x| over the block) and codes = fmt(x * 2^-e),
    rounded to nearest even (fmt "e4m3" or "e5m2").  Returns the dequantised
    values code * 2^e (float64) and the exponent of every block
    [ceil(R/rows)][ceil(C/cols)]."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    br, bc = block
    nbr, nbc = -(-R // br), -(-C // bc)
    enc, dec, mx = ((e4m3_encode, e4m3_decode, E4M3_MAX) if fmt == "e4m3"
                    else (e5m2_encode, e5m2_decode, E5M2_MAX))
    pad = np.zeros((nbr * br, nbc * bc), np.float64)
    pad[:R, :C] = np.abs(x)
    amax = pad.reshape(nbr, br, nbc, bc).max(axis=(1, 3))
    exps = pow2_exponents(amax, mx)
    e_el = np.repeat(np.repeat(exps, br, axis=0), bc, axis=1)[:R, :C].astype(np.float64)
    scaled = (x.astype(np.float64) * np.exp2(-e_el)).astype(np.float32)
    return dec(enc(scaled)) * np.exp2(e_el), exps


def sylvester(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    assert n >= 1 and (n & (n - 1)) == 0
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs) -> np.ndarray:
    """J = diag(sigma) H / sqrt(n), an orthogonal matrix ([L21] slide 24)."""
    s = np.asarray(signs, dtype=np.float64)
    n = s.shape[0]
    return (s[:, None] * sylvester(n)) / np.sqrt(n)


def rotate(x, signs) -> np.ndarray:
    """x J over the last (head) dimension, in float64."""
    return np.asarray(x, np.float64) @ rotation(signs)
