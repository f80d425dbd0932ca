"""Rooted collectives on the virtual cluster: broadcast and reduce.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

"Networks and Collective Communication" (semidirectx cs349e prerequisite
lecture 5), section 4.1: broadcast copies the root's data to every device;
reduce sums elementwise and leaves the result on the root only. Section 4.2:
broadcast can also be a scatter followed by an all-gather (Van de Geijn).
Section 5.5: the naive broadcast, the binomial tree and the pipelined chain
(k blocks passed down a chain of devices, p - 2 + k steps).

Readings where the pages leave a step open:

R9   root: every algorithm runs on ranks relative to the root, v = (r - root)
     mod p, so relative rank 0 is the root.
R10  naive broadcast: the root sends its whole vector to one device per
     step, relative ranks 1, 2, .., p-1 in turn (p - 1 steps; section 5.5's
     1.25 ms for 8 MB to 7 devices is 7 such sends).
R11  binomial broadcast: the broadcast half of the binary tree (R5 in
     collectives.py), masks descending: a relative rank that is a multiple
     of 2m sends to v + m when v + m < p.
R12  scatter + all-gather: the scatter is one step in which the root sends
     chunk v (balanced chunks, R1) to every relative rank v != 0 (the
     section 4.2 times, 16.1 and 49 us, come out only if the root's port
     carries the (p-1)/p share in one step); then the plain ring all-gather
     of R2 on relative ranks, step s: v sends chunk (v - s) mod p to v + 1.
     The root takes part like any rank, so it is sent the chunks it already
     holds; the time is the same either way.
R13  pipelined chain: the vector is cut into k balanced blocks (R1); in step
     t relative rank v (0 <= v <= p-2) passes block t - v, when it exists,
     to v + 1. Blocks that are empty (k > n) are still recorded, as 0-byte
     messages.
R14  reduce: the binomial reduce of R5 on relative ranks; the root's float32
     sum is rounded to bfloat16 once (R6).
"""
from __future__ import annotations

import numpy as np

from .cluster import ADD, COPY, Cluster, Ledger, Send
from .collectives import chunk_bounds
from .numerics import ELEM_BYTES, round_to_bf16, store, widen

BROADCAST_ALGOS = ("naive", "tree", "scatter_allgather", "chain")


def _masks(p: int) -> list:
    out, m = [], 1
    while m < p:
        out.append(m)
        m *= 2
    return out


def broadcast(x_root, p: int, algo: str, root: int = 0, k: int = 1, dtype: str = "f32"):
    """Broadcast of the root's storage words to all p ranks. Returns (one
    array per rank, ledger). Values are copied, never widened or rounded."""
    if not 0 <= root < p:
        raise ValueError("root out of range")
    x_root = np.asarray(x_root)
    n = len(x_root)
    ledger = Ledger(p, ELEM_BYTES[dtype])
    bufs = [np.zeros(n, dtype=x_root.dtype) for _ in range(p)]
    bufs[root] = x_root.copy()
    cl = Cluster(bufs, 0, ledger)

    def a(v):                                   # relative -> absolute rank
        return (v + root) % p

    if algo == "naive":
        for s in range(p - 1):
            cl.step(s, [Send(a(0), a(s + 1), 0, 0, n, COPY)])
    elif algo == "tree":
        for step, m in enumerate(reversed(_masks(p))):
            cl.step(step, [Send(a(v), a(v + m), 0, 0, n, COPY) for v in range(0, p, 2 * m) if v + m < p])
    elif algo == "scatter_allgather":
        offs = chunk_bounds(n, p)
        if p > 1:
            cl.step(0, [Send(a(0), a(v), offs[v], offs[v], offs[v + 1] - offs[v], COPY) for v in range(1, p)])
        for s in range(p - 1):
            sends = []
            for v in range(p):
                c = (v - s) % p
                sends.append(Send(a(v), a((v + 1) % p), offs[c], offs[c], offs[c + 1] - offs[c], COPY))
            cl.step(1 + s, sends)
    elif algo == "chain":
        if k < 1:
            raise ValueError("the chain needs k >= 1 blocks")
        offs = chunk_bounds(n, k)
        for t in range(p - 2 + k if p > 1 else 0):
            sends = []
            for v in range(p - 1):
                b = t - v
                if 0 <= b < k:
                    sends.append(Send(a(v), a(v + 1), offs[b], offs[b], offs[b + 1] - offs[b], COPY))
            cl.step(t, sends)
    else:
        raise ValueError(f"broadcast has no {algo} variant")
    return [b.copy() for b in cl.bufs], ledger


def reduce(x: list, root: int = 0, dtype: str = "f32", n: int | None = None, lo: int = 0):
    """Binomial-tree reduce to the root (R14). Returns (the root's result,
    ledger). In windowed mode x[r] holds elements [lo, lo+len) of vectors of
    n elements."""
    p = len(x)
    if not 0 <= root < p:
        raise ValueError("root out of range")
    n = len(x[0]) if n is None else n
    ledger = Ledger(p, ELEM_BYTES[dtype])
    cl = Cluster([widen(v, dtype) for v in x], lo, ledger)
    for step, m in enumerate(_masks(p)):
        # relative ranks whose lowest set bit is m send their vector to v - m
        cl.step(step, [Send((v + root) % p, (v - m + root) % p, 0, 0, n, ADD)
                       for v in range(p) if (v & -v) == m])
    out = cl.bufs[root]
    if dtype == "bf16":
        out = round_to_bf16(out)
    return store(out, dtype), ledger
