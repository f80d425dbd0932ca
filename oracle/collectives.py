"""Collective algorithms on the virtual cluster, one step at a time.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

Sources (page titles as published):

* P1 -- "LLM Distributed Training Collectives"
  (lukebest.github.io), section "Ring AllReduce".
* P2 -- "Networks and Collective Communication", semidirectx cs349e
  prerequisite lecture 5: semantics in section 4.1, identities in section
  4.2, per-device byte bounds in section 4.3, ring in section 5.1,
  recursive doubling / Rabenseifner / binary tree in section 5.2, MoE
  all-to-all in section 7.4, ring formula in exercise 2.
* P3 -- "11-1. Distributed training" (HPC101 notes), sections
  "Collective Communication Primitives" and "Ring Algorithm".

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes):

R1  chunk bounds when p does not divide n: balanced, the first n mod p chunks
    get one extra element.
R2  after the ring reduce-scatter rank c owns chunk c (P3: process k gets the
    k-th piece of the sum), so reduce-scatter step s has rank i send chunk
    (i-1-s) mod p and all-gather step s has it send chunk (i-s) mod p; the
    ring runs i -> i+1.
R3  recursive doubling for p not a power of two (outside the pages): the
    fold of Thakur, Rabenseifner and Gropp (cited in P2's reading list) --
    with p2 the largest power of two <= p and r = p - p2, even ranks below 2r
    first send their vector to the next rank, which adds; the odd ones and
    the ranks >= 2r run the power-of-two algorithm; the odd ones finally send
    the result back.
R4  Rabenseifner's recursive halving pairs at distance p/2 first, so rank c
    ends the reduce-scatter holding chunk c; the all-gather doubles the
    distance 1, 2, .., p/2. Non-power-of-two p uses the fold of R3 around it,
    with the vector cut into p2 chunks.
R5  binary tree: binomial reduce to root 0 (a rank whose lowest set bit is
    the mask sends to rank - mask, masks ascending), then the mirrored
    binomial broadcast; a partner beyond p-1 skips the step.
R6  bfloat16 storage: inputs widen exactly to float32, every add is a
    float32 add, and each result is rounded to bfloat16 once, when it is
    complete (end of the reduce phase); the ledger counts storage bytes.
R8  hierarchical and 2D all-reduce (P2 sections 6.1, 6.3): ranks form N
    groups of L consecutive ranks (nodes, or torus rows); the group
    reduce-scatter cuts the vector into L chunks, the cross-group ring cuts
    chunk l into N pieces, both balanced as in R1, rings run i -> i+1 with
    the piece owner rule of R2; every ring in a phase runs in lockstep.
R7  all-to-all: receive buffers hold the blocks in source-rank order (the
    transpose of section 4.1); the ledger follows the direct schedule, step
    s = 1..p-1 has rank i send its block for rank (i+s) mod p; the diagonal
    block is a local copy and no message.
"""
from __future__ import annotations

import numpy as np

from .cluster import ADD, COPY, Cluster, Ledger, Send
from .numerics import ELEM_BYTES, round_to_bf16, store, widen

ALGOS = ("ring", "rd", "rabenseifner", "tree")


# --------------------------------------------------------------------------
# partition and helpers


def chunk_bounds(n: int, p: int) -> list:
    """Offsets of the p chunks of an n-element vector (reading R1).

    Chunk c is [offs[c], offs[c+1]); the first n mod p chunks are one
    element longer than the rest.
    """
    q, r = divmod(n, p)
    return [c * q + min(c, r) for c in range(p + 1)]


def _is_pow2(p: int) -> bool:
    return p >= 1 and (p & (p - 1)) == 0


def _fold(p: int):
    """p2, r and the map new rank -> old rank of the fold (reading R3)."""
    p2 = 1 << (p.bit_length() - 1)
    r = p - p2

    def old(nr: int) -> int:
        return 2 * nr + 1 if nr < r else nr + r
    return p2, r, old


def _narrow(cl: Cluster, rank: int, off: int, count: int, dtype: str) -> None:
    """Round a finished float32 range of one rank to the storage type (R6)."""
    if dtype == "f32" or count == 0:
        return
    buf = cl.bufs[rank]
    a, b = max(off, cl.lo), min(off + count, cl.lo + len(buf))
    if b > a:
        buf[a - cl.lo:b - cl.lo] = round_to_bf16(buf[a - cl.lo:b - cl.lo])


def _start(x: list, dtype: str, lo: int):
    ledger = Ledger(len(x), ELEM_BYTES[dtype])
    return Cluster([widen(v, dtype) for v in x], lo, ledger), ledger


def _finish(cl: Cluster, dtype: str) -> list:
    return [store(v, dtype) for v in cl.bufs]


# --------------------------------------------------------------------------
# ring (P2 section 5.1; P1 "Ring AllReduce"; P3 "Ring Algorithm")


def _ring_reduce_scatter_steps(cl: Cluster, p: int, offs: list, step0: int) -> int:
    """p-1 steps; each rank passes one chunk of partial sums to its successor,
    which adds its own piece of that chunk. Afterwards rank c holds chunk c."""
    for s in range(p - 1):
        sends = []
        for i in range(p):
            c = (i - 1 - s) % p
            sends.append(Send(i, (i + 1) % p, offs[c], offs[c], offs[c + 1] - offs[c], ADD))
        cl.step(step0 + s, sends)
    return step0 + p - 1


def _ring_all_gather_steps(cl: Cluster, p: int, offs: list, step0: int) -> int:
    """p-1 steps; each rank forwards the complete chunk it received last."""
    for s in range(p - 1):
        sends = []
        for i in range(p):
            c = (i - s) % p
            sends.append(Send(i, (i + 1) % p, offs[c], offs[c], offs[c + 1] - offs[c], COPY))
        cl.step(step0 + s, sends)
    return step0 + p - 1


def _allreduce_ring(cl: Cluster, p: int, n: int, dtype: str) -> None:
    offs = chunk_bounds(n, p)
    step = _ring_reduce_scatter_steps(cl, p, offs, 0)
    for c in range(p):
        _narrow(cl, c, offs[c], offs[c + 1] - offs[c], dtype)
    _ring_all_gather_steps(cl, p, offs, step)


# --------------------------------------------------------------------------
# recursive doubling (P2 section 5.2), with the fold of R3


def _fold_pre(cl: Cluster, p: int, n: int, r: int, step: int) -> int:
    if r == 0:
        return step
    cl.step(step, [Send(2 * j, 2 * j + 1, 0, 0, n, ADD) for j in range(r)])
    return step + 1


def _fold_post(cl: Cluster, p: int, n: int, r: int, step: int) -> int:
    if r == 0:
        return step
    cl.step(step, [Send(2 * j + 1, 2 * j, 0, 0, n, COPY) for j in range(r)])
    return step + 1


def _allreduce_rd(cl: Cluster, p: int, n: int, dtype: str) -> None:
    p2, r, old = _fold(p)
    step = _fold_pre(cl, p, n, r, 0)
    k = 0
    while (1 << k) < p2:
        # step k: new rank i and i xor 2^k exchange their full vectors and add
        cl.step(step, [Send(old(nr), old(nr ^ (1 << k)), 0, 0, n, ADD) for nr in range(p2)])
        step += 1
        k += 1
    for nr in range(p2):
        _narrow(cl, old(nr), 0, n, dtype)
    _fold_post(cl, p, n, r, step)


# --------------------------------------------------------------------------
# Rabenseifner (P2 section 5.2): recursive-halving reduce-scatter followed by
# recursive-doubling all-gather (reading R4)


def _rab_reduce_scatter_steps(cl, p2, old, offs2, step):
    """Distance p2/2, p2/4, .., 1: each new rank keeps the half of its current
    range that holds its own chunk, sends the other half to its partner, and
    adds the half it receives. Afterwards new rank c holds chunk c."""
    d = p2 // 2
    while d >= 1:
        sends = []
        for nr in range(p2):
            base = nr & ~(2 * d - 1)           # first chunk of the current range
            keep_upper = bool(nr & d)
            lo_c = base if keep_upper else base + d   # first chunk of the half sent away
            off = offs2[lo_c]
            sends.append(Send(old(nr), old(nr ^ d), off, off, offs2[lo_c + d] - off, ADD))
        cl.step(step, sends)
        step += 1
        d //= 2
    return step


def _rab_all_gather_steps(cl, p2, old, offs2, step):
    """Distance 1, 2, .., p2/2: each new rank sends the complete range it holds
    (d chunks containing its own) to its partner."""
    d = 1
    while d < p2:
        sends = []
        for nr in range(p2):
            base = nr & ~(d - 1)
            off = offs2[base]
            sends.append(Send(old(nr), old(nr ^ d), off, off, offs2[base + d] - off, COPY))
        cl.step(step, sends)
        step += 1
        d *= 2
    return step


def _allreduce_rabenseifner(cl: Cluster, p: int, n: int, dtype: str) -> None:
    p2, r, old = _fold(p)
    offs2 = chunk_bounds(n, p2)
    step = _fold_pre(cl, p, n, r, 0)
    step = _rab_reduce_scatter_steps(cl, p2, old, offs2, step)
    for nr in range(p2):
        _narrow(cl, old(nr), offs2[nr], offs2[nr + 1] - offs2[nr], dtype)
    step = _rab_all_gather_steps(cl, p2, old, offs2, step)
    _fold_post(cl, p, n, r, step)


# --------------------------------------------------------------------------
# binary (binomial) tree (P2 section 5.2; P1 "Ring AllReduce" table), R5


def _masks(p: int) -> list:
    out, m = [], 1
    while m < p:
        out.append(m)
        m <<= 1
    return out


def _allreduce_tree(cl: Cluster, p: int, n: int, dtype: str) -> None:
    step = 0
    masks = _masks(p)
    for m in masks:
        # ranks whose lowest set bit is m send their full vector to rank - m
        sends = [Send(i, i - m, 0, 0, n, ADD) for i in range(p) if (i & -i) == m]
        cl.step(step, sends)
        step += 1
    _narrow(cl, 0, 0, n, dtype)
    for m in reversed(masks):
        sends = [Send(i, i + m, 0, 0, n, COPY) for i in range(0, p, 2 * m) if i + m < p]
        cl.step(step, sends)
        step += 1


# --------------------------------------------------------------------------
# hierarchical / 2D all-reduce (P2 sections 6.1 and 6.3): ranks form N groups
# of L (rank = g*L + l); reading R8 below


def allreduce_hierarchical_steps(cl: Cluster, nodes: int, local: int, n: int, dtype: str) -> None:
    """R8: (1) inside each group, a ring reduce-scatter over L chunks (group
    rank l ends with chunk l of the group's sum); (2) for every l, the N ranks
    with that index run a ring all-reduce on chunk l, cut into N pieces (ring
    reduce-scatter then all-gather); (3) inside each group a ring all-gather.
    All groups (and all same-index rings) run their steps together."""
    L, N = local, nodes
    chunks = chunk_bounds(n, L)
    cpieces = [(chunks[c], chunks[c + 1] - chunks[c]) for c in range(L)]
    sub = []                                       # sub[l][j] = piece j of chunk l
    for l in range(L):
        b = chunk_bounds(cpieces[l][1], N)
        sub.append([(cpieces[l][0] + b[j], b[j + 1] - b[j]) for j in range(N)])

    def together(step0, rings):
        """Run several rings in lockstep; rings = (members in ring order,
        their pieces, op, shift). Step s: member i sends piece
        (i - shift - s) mod m to member i+1 (shift 1 reduce-scatters so that
        member i finishes piece i; shift 0 all-gathers)."""
        steps = max(len(m) for m, _, _, _ in rings) - 1
        for s in range(steps):
            sends = []
            for members, pieces, op, shift in rings:
                m = len(members)
                for i in range(m):
                    off, cnt = pieces[(i - shift - s) % m]
                    sends.append(Send(members[i], members[(i + 1) % m], off, off, cnt, op))
            cl.step(step0 + s, sends)
        return step0 + steps

    groups = [[g * L + l for l in range(L)] for g in range(N)]
    same = [[g * L + l for g in range(N)] for l in range(L)]
    step = 0
    if L > 1:
        step = together(step, [(grp, cpieces, ADD, 1) for grp in groups])
    if N > 1:
        step = together(step, [(same[l], sub[l], ADD, 1) for l in range(L)])
    for l in range(L):                              # piece j of chunk l is complete on group j
        for j in range(N):
            off, cnt = sub[l][j]
            _narrow(cl, j * L + l, off, cnt, dtype)
    if N > 1:
        step = together(step, [(same[l], sub[l], COPY, 0) for l in range(L)])
    if L > 1:
        together(step, [(grp, cpieces, COPY, 0) for grp in groups])


def allreduce_hierarchical(x: list, nodes: int, local: int, dtype: str = "f32", n: int | None = None,
                           lo: int = 0):
    """Hierarchical all-reduce of nodes*local ranks; 2D torus all-reduce of an
    a x b grid is the same with nodes = a, local = b (rows first)."""
    p = len(x)
    if nodes * local != p:
        raise ValueError("p must equal nodes * local")
    n = len(x[0]) if n is None else n
    cl, ledger = _start(x, dtype, lo)
    allreduce_hierarchical_steps(cl, nodes, local, n, dtype)
    return _finish(cl, dtype), ledger


_AR = {
    "ring": _allreduce_ring,
    "rd": _allreduce_rd,
    "rabenseifner": _allreduce_rabenseifner,
    "tree": _allreduce_tree,
}


# --------------------------------------------------------------------------
# public entry points


def allreduce(x: list, algo: str, dtype: str = "f32", n: int | None = None, lo: int = 0):
    """All-reduce of the p rank vectors ``x`` with the given algorithm.

    ``x[r]`` holds storage values (float32, or uint16 bfloat16 patterns) of
    rank r. In windowed mode ``x[r]`` holds only elements [lo, lo+len) of
    vectors of ``n`` elements. Returns (outputs per rank, ledger).
    """
    p = len(x)
    n = len(x[0]) if n is None else n
    if p == 0:
        raise ValueError("p must be >= 1")
    cl, ledger = _start(x, dtype, lo)
    _AR[algo](cl, p, n, dtype)
    return _finish(cl, dtype), ledger


def reduce_scatter(x: list, algo: str, dtype: str = "f32", n: int | None = None, lo: int = 0):
    """Reduce-scatter: rank c receives chunk c of the sum (P3 primitives; P2
    section 4.1). Ring for any p; Rabenseifner's halving half for powers of
    two. Returns (per-rank chunk outputs restricted to the window, ledger)."""
    p = len(x)
    n = len(x[0]) if n is None else n
    if algo == "rabenseifner" and not _is_pow2(p):
        raise ValueError("Rabenseifner reduce-scatter needs a power-of-two p")
    if algo not in ("ring", "rabenseifner"):
        raise ValueError(f"reduce-scatter has no {algo} variant")
    cl, ledger = _start(x, dtype, lo)
    offs = chunk_bounds(n, p)
    if algo == "ring":
        _ring_reduce_scatter_steps(cl, p, offs, 0)
    else:
        _rab_reduce_scatter_steps(cl, p, lambda nr: nr, offs, 0)
    outs = []
    for c in range(p):
        _narrow(cl, c, offs[c], offs[c + 1] - offs[c], dtype)
        a, b = max(offs[c], lo), min(offs[c + 1], lo + len(cl.bufs[c]))
        piece = cl.bufs[c][a - lo:b - lo] if b > a else cl.bufs[c][:0]
        outs.append(store(piece, dtype))
    return outs, ledger


def all_gather(x: list, algo: str, dtype: str = "f32"):
    """All-gather of equal blocks of m elements: every rank ends with the
    concatenation block_0 .. block_{p-1} (P3 primitives; P2 section 4.1).
    Ring for any p, recursive doubling for powers of two. Values are copied
    as raw storage words."""
    p = len(x)
    m = len(x[0])
    if algo == "rd" and not _is_pow2(p):
        raise ValueError("recursive-doubling all-gather needs a power-of-two p")
    if algo not in ("ring", "rd"):
        raise ValueError(f"all-gather has no {algo} variant")
    ledger = Ledger(p, ELEM_BYTES[dtype])
    bufs = []
    for i in range(p):
        b = np.zeros(p * m, dtype=np.asarray(x[i]).dtype)
        b[i * m:(i + 1) * m] = x[i]            # own block: a local copy, no message
        bufs.append(b)
    cl = Cluster(bufs, 0, ledger)
    offs = [c * m for c in range(p + 1)]
    if algo == "ring":
        _ring_all_gather_steps(cl, p, offs, 0)
    else:
        _rab_all_gather_steps(cl, p, lambda nr: nr, offs, 0)
    return [b.copy() for b in cl.bufs], ledger


def block_offsets(splits: np.ndarray):
    """Row offsets of block (i -> j) in the sender's and in the receiver's buffer."""
    splits = np.asarray(splits, dtype=np.int64)
    p = splits.shape[0]
    send_off = np.zeros((p, p), dtype=np.int64)
    recv_off = np.zeros((p, p), dtype=np.int64)
    for i in range(p):
        for j in range(1, p):
            send_off[i, j] = send_off[i, j - 1] + splits[i, j - 1]
    for j in range(p):
        for i in range(1, p):
            recv_off[i, j] = recv_off[i - 1, j] + splits[i - 1, j]
    return send_off, recv_off


def all_to_all(send: list, splits, dtype: str = "bf16"):
    """Variable-split all-to-all (P2 section 4.1: device i's block j goes to
    device j, the transpose of the device x block matrix; reading R7).

    ``send[i]`` is a [rows_i, H] array holding blocks j = 0..p-1 in order,
    block (i -> j) having ``splits[i][j]`` rows. Returns (recv per rank, each
    [sum_i splits[i][j], H], ledger with offsets in elements)."""
    splits = np.asarray(splits, dtype=np.int64)
    p = splits.shape[0]
    H = send[0].shape[1] if send[0].ndim == 2 else 1
    for i in range(p):
        if send[i].shape[0] != splits[i].sum():
            raise ValueError(f"rank {i}: send rows {send[i].shape[0]} != splits sum {splits[i].sum()}")
    send_off, recv_off = block_offsets(splits)
    ledger = Ledger(p, ELEM_BYTES[dtype])
    recv = [np.zeros((int(splits[:, j].sum()), H), dtype=send[0].dtype) for j in range(p)]

    def move(i, j):
        s0, r0, k = send_off[i, j], recv_off[i, j], splits[i, j]
        recv[j][r0:r0 + k] = send[i][s0:s0 + k]

    for i in range(p):
        move(i, i)
    for s in range(1, p):
        for i in range(p):
            j = (i + s) % p
            ledger.record(s - 1, i, j, int(send_off[i, j] * H), int(recv_off[i, j] * H), int(splits[i, j] * H))
        for i in range(p):
            move(i, (i + s) % p)
    return recv, ledger
