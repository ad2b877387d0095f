"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and shapes them; it holds none of the
attention arithmetic.  Both the HIP path's callers (tests, bench, smoke) and the
fp64 oracle take their inputs from here, so the two sides always see the same
values.

Every tensor is contiguous [B][H][N][d] ("BHSD").  Values are drawn with
``torch.randn`` in float32 (the pages' checks and benchmarks all use
``torch.randn`` inputs) and then rounded to bf16 (round-to-nearest-even) where
the workload is bf16.  Draw order inside one workload: Q, K, V, dO, then the
FP8 extras (Q outlier positions, Q outlier signs, K outlier positions, K outlier
signs, the Hadamard sign vector).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str            # "f32", "bf16" or "fp8"
    causal: bool = False
    backward: bool = False
    num_splits: int = 0   # >0: split-KV decode
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_mag: float = 0.0
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self) -> float:
        # two GEMMs of 2*Nq*Nk*d each per (b, hq); causal keeps half.
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f * 0.5 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 1, 256, 256, 64, "f32", causal=False,
                         backward=True, seed=8301,
                         note="fp32, 64-row tiles => 4 KV blocks of online rescaling"),
    "prefill_bf16": Workload("prefill_bf16", 4, 16, 16, 2048, 2048, 64, "bf16",
                             causal=False, seed=8302),
    "causal_bf16": Workload("causal_bf16", 2, 16, 16, 8192, 8192, 128, "bf16",
                            causal=True, backward=True, seed=8303),
    "decode_gqa": Workload("decode_gqa", 8, 32, 8, 1, 131072, 128, "bf16",
                           num_splits=64, seed=8304),
    "fp8_fwd": Workload("fp8_fwd", 2, 16, 16, 8192, 8192, 128, "fp8", causal=False,
                        seed=8305, outlier_frac=1e-3, outlier_mag=50.0),
}


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device)


def make_inputs(w: Workload, device: str = "cpu", seed: int | None = None):
    """Draw Q, K, V (and dO for backward workloads) for workload ``w``.

    Returns a dict of tensors on ``device``: q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d],
    optionally do [B][Hq][Nq][d].  bf16 and fp8 workloads return bf16 tensors
    (the fp8 path quantises them itself); f32 returns float32.  fp8 workloads
    also get outliers planted in Q and K and a ``signs`` int8 vector of +-1 of
    length d for the Hadamard rotation.
    """
    gen = _gen(w.seed if seed is None else seed, device)
    qs = (w.B, w.Hq, w.Nq, w.d)
    ks = (w.B, w.Hkv, w.Nk, w.d)
    q = _randn(qs, gen, device)
    k = _randn(ks, gen, device)
    v = _randn(ks, gen, device)
    out = {}
    if w.backward:
        out["do"] = _randn(qs, gen, device)
    if w.outlier_frac > 0:
        for name, t in (("q", q), ("k", k)):
            n = t.numel()
            cnt = int(round(w.outlier_frac * n))
            pos = torch.randperm(n, generator=gen, device=device)[:cnt]
            sgn = torch.randint(0, 2, (cnt,), generator=gen, device=device).float() * 2 - 1
            t.view(-1)[pos] = sgn * w.outlier_mag
    if w.dtype == "fp8":
        out["signs"] = (torch.randint(0, 2, (w.d,), generator=gen, device=device)
                        .to(torch.int8) * 2 - 1)
    cast = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out["q"] = q.to(cast).contiguous()
    out["k"] = k.to(cast).contiguous()
    out["v"] = v.to(cast).contiguous()
    if "do" in out:
        out["do"] = out["do"].to(cast).contiguous()
    return out


def to_f64(t: torch.Tensor):
    """Exact widening of a bf16 / fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


# ------------------------------------------------------------ paged decode

@dataclass(frozen=True)
class PagedDecode:
    """Single-query decode over a paged KV cache: sequence b has seqlens[b]
    keys stored in pages of ``page_size`` tokens, the pages of all sequences
    scattered over the cache in a seeded random order."""
    name: str
    B: int
    Hq: int
    Hkv: int
    seqlens: tuple
    page_size: int
    d: int
    num_splits: int
    seed: int = 0
    spare_pages: int = 0  # pages in the cache that no sequence uses

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_pages(self) -> int:
        return max((n + self.page_size - 1) // self.page_size for n in self.seqlens)

    @property
    def num_pages(self) -> int:
        return sum((n + self.page_size - 1) // self.page_size for n in self.seqlens) + self.spare_pages


def make_paged_inputs(w: PagedDecode, device: str = "cpu"):
    """q [B][Hq][1][d], k_cache/v_cache [num_pages][page_size][Hkv][d] (bf16),
    block_table int32 [B][max_pages] (unused entries -1), seqlens int32 [B].
    Draw order: Q, K cache, V cache, then the page permutation."""
    gen = _gen(w.seed, device)
    q = _randn((w.B, w.Hq, 1, w.d), gen, device).to(torch.bfloat16)
    cs = (w.num_pages, w.page_size, w.Hkv, w.d)
    kc = _randn(cs, gen, device).to(torch.bfloat16)
    vc = _randn(cs, gen, device).to(torch.bfloat16)
    perm = torch.randperm(w.num_pages, generator=gen, device=device).to(torch.int32)
    table = torch.full((w.B, w.max_pages), -1, dtype=torch.int32, device=device)
    at = 0
    for b, n in enumerate(w.seqlens):
        np_b = (n + w.page_size - 1) // w.page_size
        table[b, :np_b] = perm[at:at + np_b]
        at += np_b
    seqlens = torch.tensor(w.seqlens, dtype=torch.int32, device=device)
    return {"q": q.contiguous(), "k_cache": kc.contiguous(), "v_cache": vc.contiguous(),
            "block_table": table, "seqlens": seqlens}


# ------------------------------------------------------ variable-length batch

@dataclass(frozen=True)
class Varlen:
    """Packed variable-length batch: the sequences are concatenated along the
    token axis (q [total][Hq][d], k/v [total][Hkv][d]) with cumulative offsets
    cu = [0, n0, n0+n1, ...]; queries and keys have the same lengths."""
    name: str
    seqlens: tuple
    Hq: int
    Hkv: int
    d: int
    causal: bool = True
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def total(self) -> int:
        return sum(self.seqlens)

    def fwd_flops(self) -> float:
        f = sum(4.0 * self.Hq * n * n * self.d for n in self.seqlens)
        return f * 0.5 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()


def make_varlen_inputs(w: Varlen, device: str = "cpu"):
    """q, do [total][Hq][d], k/v [total][Hkv][d] (bf16) and cu int32 [len+1].
    Draw order: Q, K, V, dO."""
    gen = _gen(w.seed, device)
    T = w.total
    q = _randn((T, w.Hq, w.d), gen, device).to(torch.bfloat16)
    k = _randn((T, w.Hkv, w.d), gen, device).to(torch.bfloat16)
    v = _randn((T, w.Hkv, w.d), gen, device).to(torch.bfloat16)
    do = _randn((T, w.Hq, w.d), gen, device).to(torch.bfloat16)
    cu = [0]
    for n in w.seqlens:
        cu.append(cu[-1] + n)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "do": do.contiguous(), "cu": torch.tensor(cu, dtype=torch.int32, device=device)}


PAGED = {
    "decode_paged": PagedDecode("decode_paged", 8, 32, 8, (131072,) * 8, 16, 128, 64,
                                seed=8307, spare_pages=1024),
}
VARLEN = {
    "varlen_bf16": Varlen("varlen_bf16", (7919, 509, 3061, 1021, 6143, 257, 2053, 4099, 1531, 5113),
                          16, 16, 128, causal=True, seed=8306),
}


# ---------------------------------------------------------- sliding window

@dataclass(frozen=True)
class Windowed(Workload):
    """A Workload with a sliding window: key j is visible to query i only if
    i - window_left <= j <= i + window_right (-1: unbounded)."""
    window_left: int = -1
    window_right: int = -1

    def visible_pairs(self) -> int:
        # keys visible per query row, summed over the rows
        n = self.Nq
        tot = 0
        for i in range(n):
            lo = 0 if self.window_left < 0 else max(0, i - self.window_left)
            hi = n - 1 if self.window_right < 0 else min(n - 1, i + self.window_right)
            if self.causal:
                hi = min(hi, i)
            tot += max(0, hi - lo + 1)
        return tot

    def fwd_flops(self) -> float:
        return 4.0 * self.B * self.Hq * self.d * self.visible_pairs()


WINDOWED = {
    "window_bf16": Windowed("window_bf16", 2, 16, 16, 8192, 8192, 128, "bf16", causal=True,
                            backward=True, seed=8308, window_left=4096, window_right=0),
}


# ----------------------------------------------------------- block-sparse

@dataclass(frozen=True)
class BlockSparse(Workload):
    """A Workload with a block-sparse pattern shared by every (b, head):
    query tile t (block_q rows) sees the key blocks (block_k keys) within
    `local` keys of the tile on either side, plus the first `global_blocks`
    key blocks (a local + global pattern)."""
    block_q: int = 256
    block_k: int = 64
    local: int = 1024
    global_blocks: int = 4

    def pattern(self):
        nq = -(-self.Nq // self.block_q)
        nk = -(-self.Nk // self.block_k)
        ptr, idx = [0], []
        for t in range(nq):
            lo = max(0, (t * self.block_q - self.local) // self.block_k)
            hi = min(nk, -(-((t + 1) * self.block_q + self.local) // self.block_k))
            blocks = sorted(set(range(min(self.global_blocks, nk))) | set(range(lo, hi)))
            idx += blocks
            ptr.append(len(idx))
        return ptr, idx

    def visible_pairs(self) -> int:
        ptr, idx = self.pattern()
        tot = 0
        for t in range(len(ptr) - 1):
            rows = min(self.block_q, self.Nq - t * self.block_q)
            for c in idx[ptr[t]:ptr[t + 1]]:
                cols = min(self.block_k, self.Nk - c * self.block_k)
                tot += rows * cols
        return tot

    def fwd_flops(self) -> float:
        return 4.0 * self.B * self.Hq * self.d * self.visible_pairs()


SPARSE = {
    "sparse_bf16": BlockSparse("sparse_bf16", 2, 16, 16, 8192, 8192, 128, "bf16", causal=False,
                               backward=True, seed=8309),
}
