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

Dispatch variants (section 7.4 and exercise 10: DeepSeek-V3 sends a token
once to each place that needs it and then forwards it locally, and sends the
dispatch in FP8):

R18  per-destination deduplication: rank i sends each token once to every
     rank j that holds at least one of the token's chosen experts, rows
     ordered by token; rank j then copies each received row to every
     (expert, token) slot of the plain layout above (a local gather, no
     message), so the expanded buffer equals the plain dispatch bit for bit.
     Combine is the plain reverse all-to-all (the pages do not describe a
     deduplicated combine, which would have to sum expert outputs first).
R19  FP8 payload: the rows a rank sends are quantised once, at the sender,
     in the layout of fp8.py (R15-R17); the all-to-all moves those bytes.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .collectives import all_to_all
from .numerics import bf16_to_f32


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


def plan_dedup(topk_ids: list, experts_per_rank: int):
    """R18. Returns (splits_unique [p, p], src_unique per rank (token of
    each sent row), expand per receiving rank (for each row of the plain
    layout, the index of the deduplicated received row it copies))."""
    p = len(topk_ids)
    splits_u = np.zeros((p, p), dtype=np.int64)
    src_u = []
    uniq = {}                                        # (i, j) -> sorted unique tokens
    for i in range(p):
        ids = np.asarray(topk_ids[i])
        rows = []
        for j in range(p):
            toks = sorted({t for t in range(ids.shape[0]) for k in range(ids.shape[1])
                           if int(ids[t, k]) // experts_per_rank == j})
            uniq[(i, j)] = toks
            splits_u[i, j] = len(toks)
            rows += toks
        src_u.append(np.array(rows, dtype=np.int32))
    splits, src_rows, _ = plan(topk_ids, experts_per_rank)
    expand = []
    for j in range(p):
        base, idx = 0, []
        for i in range(p):
            pos = {t: base + n for n, t in enumerate(uniq[(i, j)])}
            # the plain block (i -> j) in send order: rows of src_rows[i]
            # from offset sum(splits[i, :j]), splits[i, j] of them
            s0 = int(splits[i, :j].sum())
            idx += [pos[int(t)] for t in src_rows[i][s0:s0 + int(splits[i, j])]]
            base += len(uniq[(i, j)])
        expand.append(np.array(idx, dtype=np.int32))
    return splits_u, src_u, expand


def dispatch_dedup(tokens: list, topk_ids: list, experts_per_rank: int, dtype: str = "bf16"):
    """R18: deduplicated all-to-all, then the local expansion. Returns
    (expanded recv per rank, deduplicated recv per rank, ledger)."""
    splits_u, src_u, expand = plan_dedup(topk_ids, experts_per_rank)
    send = [tokens[i][src_u[i]] for i in range(len(tokens))]
    recv_u, ledger = all_to_all(send, splits_u, dtype)
    return [recv_u[j][expand[j]] for j in range(len(tokens))], recv_u, ledger


def dispatch_fp8(tokens: list, splits, src_rows: list):
    """R19: quantise each sent row (bfloat16 tokens) at the sender, then the
    all-to-all of the byte rows. Returns (recv byte rows per rank, ledger)."""
    send = [fp8.quantize_rows(bf16_to_f32(tokens[i][src_rows[i]])) for i in range(len(tokens))]
    return all_to_all(send, splits, "u8")
