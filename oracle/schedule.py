"""Reference list scheduler for longest-first tile order -- TEST INFRASTRUCTURE ONLY.

[L21] "CMU 11-868 L21 FlashAttention" digest (quidproquo.cc), slides 27-46:
causal attention gives the query tiles unequal amounts of work; handing the
longest work out first (LPT) balances the workers.  The worked example there
(2 batches on 3 workers) reports per-worker loads [9, 5, 6] when tiles are
handed out in order and [7, 7, 6] when the longest go first.

Model: a free worker takes the next tile of the list; when several workers are
free at once, the lowest-numbered one goes first.
"""
from __future__ import annotations


def list_schedule(costs, workers: int):
    """Greedy earliest-free list scheduling.  Returns (loads, owner_of_item)."""
    loads = [0] * workers
    owner = []
    for c in costs:
        w = min(range(workers), key=lambda i: (loads[i], i))
        loads[w] += c
        owner.append(w)
    return loads, owner


def lpt_order(costs):
    """Indices of ``costs`` sorted longest first (stable among equal costs)."""
    return sorted(range(len(costs)), key=lambda i: -costs[i])


def causal_tile_costs(batch_heads: int, q_tiles: int, rows_per_q_tile: int,
                      keys_per_kv_tile: int):
    """Cost (number of KV tiles visited) of every (bh, i) query tile of a
    square causal problem, listed bh-major.  Query tile i covers rows
    [i*Br, (i+1)*Br) and visits every KV tile holding a key <= its last row."""
    out = []
    for _ in range(batch_heads):
        for i in range(q_tiles):
            last = (i + 1) * rows_per_q_tile - 1
            out.append(last // keys_per_kv_tile + 1)
    return out
