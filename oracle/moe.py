"""MoE dispatch and combine as all-to-alls (oracle side).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

"Networks and Collective Communication", section 7.4: with expert
parallelism every MoE layer runs two all-to-alls, dispatch (tokens to the
ranks holding their chosen experts) and combine (the reverse); each (token,
chosen expert) pair is one row of hidden-size activations. Section 4.2: an
all-to-all applied twice returns the data home, which is what makes
combine(dispatch(x)) == x.

Plan (integer only): rank i sends one row per (token t, slot k) pair to the
rank owning expert e = topk[t, k] (experts_per_rank consecutive ids per rank),
ordered by (destination rank, expert, token). ``src_rows`` names the token
row each sent row copies; ``dst_rows`` names the (token, slot) position
t * topk + k a returning row lands on at combine.
"""
from __future__ import annotations

import numpy as np

from .collectives import all_to_all


def plan(topk_ids: list, experts_per_rank: int):
    """Splits [p, p] (int64) and per-rank src_rows / dst_rows (int32)."""
    p = len(topk_ids)
    splits = np.zeros((p, p), dtype=np.int64)
    src_rows, dst_rows = [], []
    for i in range(p):
        ids = np.asarray(topk_ids[i])
        T, K = ids.shape
        pairs = []
        for t in range(T):
            for k in range(K):
                e = int(ids[t, k])
                pairs.append((e // experts_per_rank, e, t, k))
        pairs.sort()
        for dest, _, _, _ in pairs:
            splits[i, dest] += 1
        src_rows.append(np.array([t for _, _, t, _ in pairs], dtype=np.int32))
        dst_rows.append(np.array([t * K + k for _, _, t, k in pairs], dtype=np.int32))
    return splits, src_rows, dst_rows


def dispatch(tokens: list, splits, src_rows: list, dtype: str = "bf16"):
    """Gather each rank's rows in send order, then all-to-all. Returns
    (recv per rank, send buffers, ledger)."""
    send = [tokens[i][src_rows[i]] for i in range(len(tokens))]
    recv, ledger = all_to_all(send, splits, dtype)
    return recv, send, ledger


def combine(recv: list, splits, dst_rows: list, topk: int, tokens: int, dtype: str = "bf16"):
    """Reverse all-to-all (splits transposed), then scatter every returning row
    to its (token, slot) position. Returns (out per rank [tokens*topk, H],
    ledger)."""
    back, ledger = all_to_all(recv, np.asarray(splits).T, dtype)
    outs = []
    for i, rows in enumerate(back):
        out = np.zeros((tokens * topk, rows.shape[1]), dtype=rows.dtype)
        out[dst_rows[i]] = rows
        outs.append(out)
    return outs, ledger
