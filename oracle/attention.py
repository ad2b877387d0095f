"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library and never
calls it.  Everything here is the plain mathematical definition, evaluated in
float64 with numpy; a matrix product is the only library step used.

Pages cited (by title and section):
  [CH18]  "第 18 章 FlashAttention" (AI algorithm guide, theaiera.top)
  [L21]   "CMU 11-868 L21 FlashAttention" lecture digest (quidproquo.cc)

Conventions (readings of the pages where they are silent or disagree):
  * scores are multiplied by ``scale`` (the library's argument, 1/sqrt(d) by
    default); [CH18] §18.2.1 writes the same thing as a division by sqrt(d_k).
  * GQA: query head hq reads KV head hq // (Hq // Hkv)  ([CH18] §18.2.2 requires
    Hq to be a multiple of Hkv; the contiguous-group map is our reading).
  * causal is top-left aligned and only defined for Nq == Nk: key j is allowed
    for query i iff j <= i  ([CH18] §18.2.2 item 3, mask M_ij).
  * the saved row statistic is LSE_i = m_i + ln(l_i) in natural-log units.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head(hq: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head ``hq`` (contiguous groups of Hq//Hkv)."""
    assert Hq % Hkv == 0
    return hq // (Hq // Hkv)


def allowed(Nq: int, Nk: int, causal: bool, rows=None, window=None) -> np.ndarray:
    """Boolean [len(rows)][Nk] mask of keys each query may attend.

    [CH18] §18.2.2 (3): M_ij = 0 for j <= i and -inf for j > i.
    ``window`` = (left, right) ([CH18] §18.7.1, window_size): key j is visible
    to query i only if i - left <= j <= i + right; -1 leaves that side
    unbounded, and (-1, -1) is global attention.
    """
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    ok = np.ones((len(rows), Nk), dtype=bool)
    j = np.arange(Nk)[None, :]
    i = rows[:, None]
    if causal or window is not None:
        assert Nq == Nk, "causal / windowed attention is defined here for Nq == Nk only"
    if causal:
        ok &= j <= i
    if window is not None:
        left, right = window
        if left >= 0:
            ok &= j >= i - left
        if right >= 0:
            ok &= j <= i + right
    return ok


def scores(q, k, scale, causal, rows=None, window=None):
    """S = scale * Q K^T for one head, with masked entries set to -inf.

    q: [Nq][d], k: [Nk][d]; ``rows`` selects query rows.  [CH18] §18.2.1 and
    §18.2.2 (3); ``window`` as in ``allowed``.
    """
    q = _f64(q)
    k = _f64(k)
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scale * (q[r] @ k.T)
    if causal or window is not None:
        s = np.where(allowed(q.shape[0], k.shape[0], causal, r, window), s, -np.inf)
    return s


def softmax_rows(s):
    """Row softmax with the row max subtracted first ([CH18] §18.4.2 (2), safe
    softmax).  Returns (P, m, l) with P = exp(s - m) / l."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def head_forward(q, k, v, scale, causal, rows=None, window=None):
    """O and LSE for one (b, head): O = softmax(scale Q K^T + M) V.

    [CH18] §18.2.1 (definition), §18.2.2 (causal mask); LSE as stored by the
    forward for the recomputation backward ([CH18] §18.2.4, Fig. 18-6).
    """
    s = scores(q, k, scale, causal, rows, window)
    p, m, l = softmax_rows(s)
    o = p @ _f64(v)
    return o, m + np.log(l)


def forward(q, k, v, scale, causal=False, rows=None, window=None):
    """Batched forward.  q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] -> (O, LSE) fp64.

    ``rows`` optionally restricts the queries evaluated (each row of O depends
    only on its own query row, so a subset is still the plain definition).
    """
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    nr = Nq if rows is None else len(rows)
    o = np.empty((B, Hq, nr, v.shape[-1]))
    lse = np.empty((B, Hq, nr))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, hk], v[b, hk], scale,
                                              causal, rows, window)
    return o, lse


def probabilities(q, k, scale, causal=False, window=None):
    """Full attention matrix P for one head (used by invariance checks)."""
    p, _, _ = softmax_rows(scores(q, k, scale, causal, window=window))
    return p


def softmax_backward(p, dp):
    """dS = P * (dP - rowsum(P * dP)): the softmax Jacobian applied row by row,
    [CH18] §18.2.4 (1)."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def head_backward(q, k, v, do, scale, causal, window=None):
    """Materialising backward for one head, [CH18] §18.2.4 (2):
    dV = P^T dO, dP = dO V^T, dS = softmax_backward(P, dP), dQ = scale dS K,
    dK = scale dS^T Q.  Returns (dq, dk, dv, delta) with delta_i = sum_j P_ij dP_ij.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _, _ = softmax_rows(scores(q, k, scale, causal, window=window))
    dv = p.T @ do
    dp = do @ v.T
    ds = softmax_backward(p, dp)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    delta = (p * dp).sum(axis=1)
    return dq, dk, dv, delta


def head_forward_backward(q, k, v, do, scale, causal, window=None):
    """head_forward and head_backward of one head from one evaluation of P
    (the same operations in the same order as those two functions, so the
    results are identical to calling them separately).
    Returns (o, lse, dq, dk, dv)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, m, l = softmax_rows(scores(q, k, scale, causal, window=window))
    o = p @ v
    lse = m + np.log(l)
    dv = p.T @ do
    dp = do @ v.T
    ds = softmax_backward(p, dp)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return o, lse, dq, dk, dv


def head_dq_rows(q, k, v, do, scale, causal, rows):
    """dQ of the listed query rows of one head, row by row ([CH18] §18.2.4
    (2) restricted to row i: P_i = softmax of row i's visible scores,
    dP_i = dO_i V^T, dS_i = P_i * (dP_i - sum(P_i * dP_i)), dQ_i = scale dS_i K),
    for sizes where the whole matrices do not fit.  q/do [Nq][d], k/v [Nk][d]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    r = np.asarray(rows)
    s = scores(q, k, scale, causal, rows=r)
    p, _, _ = softmax_rows(s)
    dp = do[r] @ v.T
    return scale * (softmax_backward(p, dp) @ k)


def backward(q, k, v, do, scale, causal=False, window=None):
    """Batched backward -> (dQ, dK, dV) fp64.  A KV head's gradient is the sum
    over the query heads that read it (GQA broadcast, [CH18] §18.2.2)."""
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            a, bk, bv, _ = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h],
                                         scale, causal, window)
            dq[b, h] = a
            dk[b, hk] += bk
            dv[b, hk] += bv
    return dq, dk, dv


def decode_split(q, k, v, scale, num_splits):
    """Flash-Decoding, [CH18] §18.8.2 (2): split the KV length into
    ``num_splits`` equal chunks, attend each chunk on its own, then merge.

    q [B][Hq][1][d], k/v [B][Hkv][Nk][d].  Each chunk's partial is stored as
    (O_c normalised, lse_c); the merge is lse = M + ln sum_c exp(lse_c - M),
    O = sum_c exp(lse_c - lse) O_c, which equals the page's
    sum_t O_t e^{m_t - m} / sum_t l_t e^{m_t - m} with unnormalised O_t.
    Returns (O [B][Hq][1][d], lse [B][Hq][1], O_parts [B][Hq][S][d],
    lse_parts [B][Hq][S]).
    """
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    assert Nq == 1
    Nk = k.shape[2]
    assert Nk % num_splits == 0
    c = Nk // num_splits
    o_parts = np.empty((B, Hq, num_splits, v.shape[-1]))
    lse_parts = np.empty((B, Hq, num_splits))
    for s in range(num_splits):
        o_s, l_s = forward(q, k[:, :, s * c:(s + 1) * c], v[:, :, s * c:(s + 1) * c],
                           scale, causal=False)
        o_parts[:, :, s] = o_s[:, :, 0]
        lse_parts[:, :, s] = l_s[:, :, 0]
    o, lse = combine(o_parts, lse_parts)
    return o[:, :, None, :], lse[:, :, None], o_parts, lse_parts


def decode_multi(q, k, v, scale, causal=False):
    """Decode with a few query tokens against a long KV ([L21] slides 57-60:
    decode queries are a few tokens against contexts up to 128k, and GQA
    packing extends from one query token to any number).  The Nq
    queries are the newest positions of each sequence, so with ``causal``
    token t (0-based among the Nq) sees keys j <= Nk - Nq + t (the mask is
    aligned to the end of the keys); without it every token sees all keys.
    q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] -> O [B][Hq][Nq][d], LSE
    [B][Hq][Nq] in fp64 (plain definition, no splitting)."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, Hq, Nq, v.shape[-1]))
    lse = np.full((B, Hq, Nq), -np.inf)
    vis = np.ones((Nq, Nk), dtype=bool)
    if causal:
        vis = np.arange(Nk)[None, :] <= (Nk - Nq + np.arange(Nq))[:, None]
    # With more tokens than keys the earliest tokens see no key at all: their
    # output is 0 and their LSE -inf (the sum over an empty set).
    live = vis.any(axis=1)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            s = np.where(vis[live], scale * (q[b, h][live] @ k[b, hk].T), -np.inf)
            p, m, l = softmax_rows(s)
            o[b, h][live] = p @ v[b, hk]
            lse[b, h][live] = m + np.log(l)
    return o, lse


def combine(o_parts, lse_parts):
    """Merge split partials with their log-sum-exp weights ([CH18] §18.8.2 (2),
    the reduction step).  o_parts [..][S][d], lse_parts [..][S].  A chunk
    with no visible key has lse_c = -inf and weight 0; a row whose chunks are
    all empty saw no key at all and gets O = 0, lse = -inf."""
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    M = lse_parts.max(axis=-1, keepdims=True)
    dead = np.isneginf(M)
    Mr = np.where(dead, 0.0, M)
    z = np.exp(lse_parts - Mr).sum(axis=-1)
    with np.errstate(divide="ignore"):
        lse = Mr[..., 0] + np.log(z)
    w = np.where(dead, 0.0, np.exp(lse_parts - np.where(dead, 0.0, lse[..., None])))
    o = (w[..., None] * o_parts).sum(axis=-2)
    return o, lse


def forward_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Packed variable-length forward ([CH18] §18.7.1, flash_attn_varlen_func):
    the sequences of a batch are concatenated along the token axis and
    sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
    cu_k[b] .. cu_k[b+1]-1; no query attends outside its own sequence, and the
    causal mask is applied within each sequence (top-left: requires equal
    query and key lengths per sequence, as for the dense forward).

    q [total_q][Hq][d], k/v [total_k][Hkv][d] (token-major, as on the page),
    cu_q/cu_k [batch+1] cumulative offsets starting at 0.
    Returns O [total_q][Hq][d] and LSE [Hq][total_q] in fp64.  A sequence with
    no keys gives O = 0 and LSE = -inf (no key is visible).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    o = np.zeros((total_q, Hq, v.shape[-1]))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        qb = q[q0:q1].transpose(1, 0, 2)[None]          # [1][Hq][Nq][d]
        kb = k[k0:k1].transpose(1, 0, 2)[None]
        vb = v[k0:k1].transpose(1, 0, 2)[None]
        ob, lb = forward(qb, kb, vb, scale, causal)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0]
    return o, lse


def backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal=False):
    """Gradients of forward_varlen: each sequence's backward on its own rows
    ([CH18] §18.4.4 per sequence; the packing couples nothing), -> (dQ, dK,
    dV) fp64 in the packed token-major layouts of q, k, v.  Rows of a sequence
    with no keys get dQ = 0; keys of a sequence with no queries dK = dV = 0."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        per_seq = [x.transpose(1, 0, 2)[None] for x in (q[q0:q1], k[k0:k1], v[k0:k1], do[q0:q1])]
        a, bk, bv = backward(*per_seq, scale, causal)
        dq[q0:q1] = a[0].transpose(1, 0, 2)
        dk[k0:k1] = bk[0].transpose(1, 0, 2)
        dv[k0:k1] = bv[0].transpose(1, 0, 2)
    return dq, dk, dv


def gather_pages(cache, block_table, seqlen, hk):
    """Logical rows 0 .. seqlen-1 of one KV head from a paged cache
    ([CH18] §18.8.2 (3), §18.8.3 (1): the KV cache lives in fixed-size
    physical pages and a per-request page table maps logical block j to
    physical page block_table[j]).  cache [num_pages][page_size][Hkv][d].
    Returns [seqlen][d]."""
    page_size = cache.shape[1]
    rows = [cache[int(block_table[t // page_size]), t % page_size, hk] for t in range(seqlen)]
    return _f64(np.stack(rows)) if rows else np.zeros((0, cache.shape[-1]))


def decode_paged(q, k_cache, v_cache, block_table, seqlens, scale):
    """Single-query decode over a paged KV cache: for batch entry b the keys
    are logical rows 0 .. seqlens[b]-1, gathered through block_table[b]; then
    the plain (unsplit) forward with Nq = 1, non-causal.
    q [B][Hq][1][d]; k_cache/v_cache [num_pages][page_size][Hkv][d];
    block_table [B][max_pages]; seqlens [B] (each >= 1).
    Returns O [B][Hq][1][d], LSE [B][Hq][1] (fp64)."""
    q = _f64(q)
    B, Hq, _, d = q.shape
    Hkv = k_cache.shape[2]
    o = np.empty((B, Hq, 1, v_cache.shape[-1]))
    lse = np.empty((B, Hq, 1))
    for b in range(B):
        n = int(seqlens[b])
        assert n >= 1
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            kb = gather_pages(k_cache, block_table[b], n, hk)
            vb = gather_pages(v_cache, block_table[b], n, hk)
            o[b, h], lse[b, h] = head_forward(q[b, h], kb, vb, scale, False)
    return o, lse


def decode_paged_multi(q, k_cache, v_cache, block_table, seqlens, scale, causal=False):
    """decode_multi over a paged KV cache: entry b's keys are the logical rows
    0 .. seqlens[b]-1 gathered through block_table[b] (as in decode_paged),
    and its Nq query tokens are the newest positions.  With seqlens[b] < Nq
    and ``causal`` the entry's first Nq - seqlens[b] tokens see no key
    (O = 0, LSE = -inf).
    q [B][Hq][Nq][d] -> O [B][Hq][Nq][d], LSE [B][Hq][Nq] (fp64)."""
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    Hkv = k_cache.shape[2]
    o = np.empty((B, Hq, Nq, v_cache.shape[-1]))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        n = int(seqlens[b])
        assert n >= 1
        kb = np.stack([gather_pages(k_cache, block_table[b], n, hk) for hk in range(Hkv)])[None]
        vb = np.stack([gather_pages(v_cache, block_table[b], n, hk) for hk in range(Hkv)])[None]
        o[b:b + 1], lse[b:b + 1] = decode_multi(q[b:b + 1], kb, vb, scale, causal)
    return o, lse


def block_sparse_allowed(Nq, Nk, q_ptr, kv_idx, block_q, block_k, causal=False):
    """Boolean [Nq][Nk] mask of a block-sparse pattern ([CH18] §18.8.1: query
    block i attends only to the key blocks kv_idx[q_ptr[i] .. q_ptr[i+1]-1];
    skipped blocks contribute nothing, as if their scores were -inf).  Query
    block i is rows i*block_q .. +block_q-1, key block j keys j*block_k ..
    +block_k-1 (clipped at the ends); causal additionally requires j <= i."""
    ok = np.zeros((Nq, Nk), dtype=bool)
    for i in range(len(q_ptr) - 1):
        r0, r1 = i * block_q, min((i + 1) * block_q, Nq)
        for j in kv_idx[int(q_ptr[i]):int(q_ptr[i + 1])]:
            c0, c1 = int(j) * block_k, min((int(j) + 1) * block_k, Nk)
            ok[r0:r1, c0:c1] = True
    if causal:
        assert Nq == Nk
        ok &= np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    return ok


def forward_block_sparse(q, k, v, scale, q_ptr, kv_idx, block_q, block_k, causal=False,
                         rows=None):
    """Block-sparse forward ([CH18] §18.8.1) with one pattern for every
    (b, head).  q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] -> (O, LSE) fp64 for
    the query rows ``rows`` (all by default).  A row that sees no key gets
    O = 0 and LSE = -inf."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    r = np.arange(Nq) if rows is None else np.asarray(rows)
    ok = block_sparse_allowed(Nq, Nk, q_ptr, kv_idx, block_q, block_k, causal)[r]
    live = ok.any(axis=1)
    o = np.zeros((B, Hq, len(r), v.shape[-1]))
    lse = np.full((B, Hq, len(r)), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            s = scale * (q[b, h][r[live]] @ k[b, hk].T)
            s = np.where(ok[live], s, -np.inf)
            p, m, l = softmax_rows(s)
            o[b, h][live] = p @ v[b, hk]
            lse[b, h][live] = m + np.log(l)
    return o, lse


def backward_block_sparse(q, k, v, do, scale, q_ptr, kv_idx, block_q, block_k, causal=False):
    """Gradients of forward_block_sparse ([CH18] §18.2.4 (2) with the
    block-sparse visible set of [CH18] §18.8.1; skipped blocks have P = 0, so
    they receive no gradient).  Returns (dQ, dK, dV) fp64; a row that sees no
    key gets dQ = 0 and a key that no row sees dK = dV = 0."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    ok = block_sparse_allowed(Nq, Nk, q_ptr, kv_idx, block_q, block_k, causal)
    live = ok.any(axis=1)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            s = np.where(ok[live], scale * (q[b, h][live] @ k[b, hk].T), -np.inf)
            p, _, _ = softmax_rows(s)
            dp = do[b, h][live] @ v[b, hk].T
            ds = softmax_backward(p, dp)
            dq[b, h][live] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h][live])
            dv[b, hk] += p.T @ do[b, h][live]
    return dq, dk, dv

