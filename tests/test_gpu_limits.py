"""The largest inputs the dense entry points accept, against the oracle.

One head of 2^23 - 40 keys: K and V hold 2^31 - 20480 bytes each, just under
the 2^31-byte bound on one head's rows that the C ABI enforces (the kernels
address a head's rows with 32-bit buffer offsets), and the last 64-key tile
is ragged (24 keys).  The forward and the split-KV decode are checked on
sampled query rows, the backward (one query tile of 32 rows) on every
gradient element.  The decode, whose splits must divide the key count,
takes the first 2^23 - 64 of those keys: 64 chunks of 131071 keys, each
ending in a ragged tile.  Inputs are seeded N(0, 1) draws on the device;
the oracle runs in fp64 on the host (about 40 GB for the backward).

Tolerances are the bf16 ones of the parity tests: O max-abs 1e-2, LSE max-abs
1e-3, gradients relative L2 1e-2; with millions of keys each row of O is a
mean of nearly uniform weights and its entries are small (about 1e-3 here),
so O is also held to relative L2 1e-2 per checked row.

The fp8 quantiser and forward are checked at their own limit, one head of
2^24 - 40 one-byte keys, in the last test.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8
from tests.conftest import say

pytestmark = pytest.mark.gpu

NK = (1 << 23) - 40          # keys in the head; NK * 128 * 2 < 2^31
NKD = (1 << 23) - 64         # the decode's keys: 64 splits of 131071
D = 128
BF16_O, BF16_LSE, BF16_GRAD = 1e-2, 1e-3, 1e-2


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.fixture(scope="module")
def long_kv(fa_gpu):
    """K and V of one KV head with NK keys (bf16, on the device)."""
    assert NK * D * 2 < 1 << 31
    g = torch.Generator(device="cuda").manual_seed(8401)
    k = torch.randn(1, 1, NK, D, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(1, 1, NK, D, generator=g, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    return k, v


def test_forward_longest_head(fa_gpu, long_kv):
    """GQA (two query heads on the KV head), 96 query rows (a partial query
    tile), non-causal; rows 0, 47 and 95 of both heads."""
    k, v = long_kv
    g = torch.Generator(device="cuda").manual_seed(8402)
    q = torch.randn(1, 2, 96, D, generator=g, device="cuda").to(torch.bfloat16)
    say(f"forward at the key-length limit: Nq=96 Nk={NK} Hq=2 Hkv=1")
    o, lse = fa_gpu.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    rows = [0, 47, 95]
    ro, rl = A.forward(f64(q), f64(k), f64(v), 1 / math.sqrt(D), False, rows=rows)
    got = f64(o)[:, :, rows]
    eo, el = np.abs(got - ro).max(), np.abs(f64(lse)[:, :, rows] - rl).max()
    er = max(rel_l2(got[0, h, i], ro[0, h, i]) for h in range(2) for i in range(len(rows)))
    print(f"O max-abs {eo:.2e}, worst row relative L2 {er:.2e}, LSE max-abs {el:.2e}")
    assert eo <= BF16_O and el <= BF16_LSE and er <= BF16_GRAD, (eo, el, er)


def test_decode_longest_head(fa_gpu, long_kv):
    """Four query heads packed on the KV head, 64 splits; output and LSE
    against the oracle's split-KV decode and against exact attention."""
    k, v = (t[:, :, :NKD] for t in long_kv)
    assert NKD % 64 == 0 and k.is_contiguous() and v.is_contiguous()
    g = torch.Generator(device="cuda").manual_seed(8403)
    q = torch.randn(1, 4, 1, D, generator=g, device="cuda").to(torch.bfloat16)
    say(f"decode at the key-length limit: Nk={NKD} Hq=4 Hkv=1 splits=64")
    o, lse = fa_gpu.decode(q, k, v, 64)
    torch.cuda.synchronize()
    qd, kd, vd = f64(q), f64(k), f64(v)
    ref = A.decode_split(qd, kd, vd, 1 / math.sqrt(D), 64)
    eo, el = np.abs(f64(o) - ref[0]).max(), np.abs(f64(lse) - ref[1]).max()
    er = max(rel_l2(f64(o)[0, h, 0], ref[0][0, h, 0]) for h in range(4))
    print(f"vs split-KV oracle: O max-abs {eo:.2e}, worst row relative L2 {er:.2e}, "
          f"LSE max-abs {el:.2e}")
    assert eo <= BF16_O and el <= BF16_LSE and er <= BF16_GRAD, (eo, el, er)
    xo, xl = A.forward(qd, kd, vd, 1 / math.sqrt(D), False)
    assert np.abs(f64(o) - xo).max() <= BF16_O and np.abs(f64(lse) - xl).max() <= BF16_LSE


def test_backward_longest_head(fa_gpu, long_kv):
    """One query tile of 32 rows against all NK keys: dQ, and dK, dV of every
    key (the dK/dV work units span the whole 2 GB of K and V)."""
    k, v = long_kv
    g = torch.Generator(device="cuda").manual_seed(8404)
    q = torch.randn(1, 1, 32, D, generator=g, device="cuda").to(torch.bfloat16)
    do = torch.randn(1, 1, 32, D, generator=g, device="cuda").to(torch.bfloat16)
    say(f"backward at the key-length limit: Nq=32 Nk={NK}")
    o, lse = fa_gpu.forward(q, k, v, causal=False)
    dq, dk, dv = fa_gpu.backward(q, k, v, o, lse, do, causal=False)
    torch.cuda.synchronize()
    rq, rk, rv = A.backward(f64(q), f64(k), f64(v), f64(do), 1 / math.sqrt(D), False)
    for name, got, want in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = rel_l2(f64(got), want)
        print(f"{name} relative L2 {e:.2e}")
        assert e <= BF16_GRAD, (name, e)


# fp8: one head of 2^24 - 40 keys.  The e4m3 K and V hold 2^31 - 5120 bytes
# each (the same 2^31-byte bound, now on one-byte elements); their bf16
# sources, 4 GiB each, go through the quantiser, whose per-block addresses
# are 64-bit.  The last 128-row block holds 88 rows, the last 64-key tile 24.
NK8 = (1 << 24) - 40
P8 = 128 * 1021          # key period: whole 128-row blocks, a prime count of them
FP8_REL = 5e-2


def test_fp8_longest_head(fa_gpu):
    """Quantiser and fp8 forward at the fp8 key-length limit, GQA (two query
    heads on the KV head), 96 query rows, non-causal, no rotation.

    K and V repeat a seeded pattern of P8 keys (128 whole periods and a
    partial one of 49112 keys), so the oracle quantises 179800 rows rather
    than 16.8 million: its quantisation works per 128-row block and the
    period is a whole number of blocks, so the blocks of the full head are
    the pattern's blocks repeated, then the partial period's own blocks
    (whose last one is the head's ragged 88-row block).  A read from the
    wrong key tile lands on other data, since 1021 blocks is prime to every
    power of two.  The forward itself runs in the oracle over all NK8 keys.
    Codes and scales of K and V are checked bit-exact over the whole head;
    O (rows 0, 47, 95 of both heads) to relative L2 5e-2 per row against the
    oracle's fp8 pipeline, LSE to 5e-2 absolute."""
    assert NK8 * D < 1 << 31
    m, rem = divmod(NK8, P8)
    g = torch.Generator(device="cuda").manual_seed(8405)
    kp = torch.randn(P8, D, generator=g, device="cuda").to(torch.bfloat16)
    vp = torch.randn(P8, D, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(1, 2, 96, D, generator=g, device="cuda").to(torch.bfloat16)
    k = kp.repeat(m + 1, 1)[:NK8].reshape(1, 1, NK8, D).contiguous()
    v = vp.repeat(m + 1, 1)[:NK8].reshape(1, 1, NK8, D).contiguous()
    say(f"fp8 quantiser + forward at the key-length limit: Nq=96 Nk={NK8} Hq=2 Hkv=1")
    q8, qs = fa_gpu.quantize_fp8(q, None)
    k8, ks = fa_gpu.quantize_fp8(k, None)
    v8, vs = fa_gpu.quantize_fp8(v, None)
    o, lse = fa_gpu.forward_fp8(q8, k8, v8, qs, ks, vs, causal=False)
    torch.cuda.synchronize()
    del k, v

    say("fp8 limit: oracle quantisation of the key pattern")
    qd = F8.dequantize(*F8.quantize(q.float().cpu().numpy()))
    deq = []
    for name, pat, got8, gots in (("k", kp, k8, ks), ("v", vp, v8, vs)):
        pat = pat.float().cpu().numpy()[None, None]
        cp, sp = F8.quantize(pat)
        cr, sr = F8.quantize(pat[:, :, :rem])
        got8, gots = got8.cpu().numpy(), gots.cpu().numpy()
        want_s = np.concatenate([np.tile(sp, (1, 1, m)), sr], axis=2)
        assert np.array_equal(gots, want_s), name
        for i in range(m):
            assert np.array_equal(got8[:, :, i * P8:(i + 1) * P8], cp), (name, i)
        assert np.array_equal(got8[:, :, m * P8:], cr), name
        del got8
        full = np.empty((1, 1, NK8, D))
        dp, dr = F8.dequantize(cp, sp), F8.dequantize(cr, sr)
        for i in range(m):
            full[:, :, i * P8:(i + 1) * P8] = dp
        full[:, :, m * P8:] = dr
        deq.append(full)
    print(f"codes and scales of K and V bit-exact ({NK8} keys)")

    say("fp8 limit: oracle forward over all keys")
    rows = [0, 47, 95]
    ro, rl = A.forward(qd, deq[0], deq[1], 1 / math.sqrt(D), False, rows=rows)
    got = f64(o)[:, :, rows]
    er = max(rel_l2(got[0, h, i], ro[0, h, i]) for h in range(2) for i in range(len(rows)))
    el = np.abs(f64(lse)[:, :, rows] - rl).max()
    print(f"O worst row relative L2 {er:.2e}, LSE max-abs {el:.2e}")
    assert er <= FP8_REL and el <= 5e-2, (er, el)
