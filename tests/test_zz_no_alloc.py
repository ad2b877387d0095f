"""The decode entry point that allocates nothing (fa_decode_splitkv_noalloc):
its output against fa_decode_splitkv + fa_decode_combine on the same inputs,
through the C ABI, on two calls in a row (the second smaller, so stale
scratch contents from the first would show), plus its size limit."""
import math

import pytest
import torch

from tests.conftest import say

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nk, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, 1, d, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16).cuda()
    return q, k, v


def test_noalloc_decode_matches_workspace_decode(fa_gpu):
    fa = fa_gpu
    # the decode workload's shape (8.4 MB of partials), then a smaller call
    cases = [(8, 32, 8, 131072, 128, 64, 71), (2, 6, 2, 4096, 64, 16, 72)]
    for B, Hq, Hkv, Nk, d, S, seed in cases:
        say(f"noalloc decode B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} d={d} splits={S}")
        q, k, v = _inputs(B, Hq, Hkv, Nk, d, seed)
        scale = 1 / math.sqrt(d)
        o = torch.full((B, Hq, 1, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq, 1), float("nan"), dtype=torch.float32, device="cuda")
        fa.fa_decode_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nk, d, scale, S)
        ref_o, ref_lse = fa.decode(q, k, v, S, scale=scale)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: bit-identical
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), (B, Hq, Nk, d, S)


def test_noalloc_decode_rejects_partials_beyond_scratch(fa_gpu):
    fa = fa_gpu
    lim = fa.load().fa_decode_workspace_size(8, 32, 128, 64)
    assert lim <= 16 << 20
    # 8 * 64 * 128 splits of 129 floats: 33.8 MB > 16 MiB
    B, Hq, Hkv, Nk, d, S = 8, 64, 8, 4096, 128, 128
    assert fa.load().fa_decode_workspace_size(B, Hq, d, S) > 16 << 20
    q, k, v = _inputs(1, 1, 1, 128, d, 73)   # never read: the call is refused first
    o = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAArgumentError) as e:
        fa.fa_decode_splitkv_noalloc(q, k, v, o, o, B, Hq, Hkv, Nk, d, 0.1, S)
    assert e.value.code == fa.FA_ERR_WORKSPACE
