"""The alpha-beta (Hockney) cost model over the collectives (oracle side).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

"Networks and Collective Communication", section 2.1: a message of n bytes
takes T = alpha + n / beta (alpha the start-up latency, beta the bandwidth in
bytes per second); the half-bandwidth size is n_1/2 = alpha * beta.
Section 5.1 and exercise 2 give the ring all-reduce time
2(p-1)(alpha + n/(p beta)); section 5.2 gives recursive doubling
log2(p)(alpha + n/beta), Rabenseifner 2 log2(p) alpha + 2(p-1)/p n/beta and
the binary tree 2 ceil(log2 p)(alpha + n/beta). Section 5.6: algbw = n/T,
busbw = algbw * 2(p-1)/p.

The simulated clock follows the lecture's comm_sim: every step of an
algorithm costs alpha plus the time the busiest port needs, each device
sending and receiving concurrently at beta (full duplex, one port each way).
"""
from __future__ import annotations

import math


def p2p_time(nbytes: float, alpha: float, beta: float) -> float:
    """Section 2.1: one message."""
    return alpha + nbytes / beta


def half_bandwidth_size(alpha: float, beta: float) -> float:
    return alpha * beta


def formula(algo: str, p: int, nbytes: float, alpha: float, beta: float) -> float:
    """Closed-form all-reduce time of sections 5.1 / 5.2 (p a power of two for
    recursive doubling and Rabenseifner; other p use the fold's two extra
    full-vector steps, a reading outside the pages)."""
    if p == 1:
        return 0.0
    if algo == "ring":
        return 2 * (p - 1) * (alpha + nbytes / (p * beta))
    if algo == "tree":
        return 2 * math.ceil(math.log2(p)) * (alpha + nbytes / beta)
    p2 = 1 << (p.bit_length() - 1)
    extra = 0.0 if p2 == p else 2 * (alpha + nbytes / beta)
    k = p2.bit_length() - 1
    if algo == "rd":
        return k * (alpha + nbytes / beta) + extra
    if algo == "rabenseifner":
        return 2 * k * alpha + 2 * (p2 - 1) / p2 * nbytes / beta + extra
    raise ValueError(algo)


def ring_all_gather_formula(p: int, nbytes_total: float, alpha: float, beta: float) -> float:
    """All-gather on a ring of the whole n-byte result: p-1 steps of n/p."""
    return (p - 1) * (alpha + nbytes_total / (p * beta))


def ledger_time(ledger, alpha: float, beta: float) -> float:
    """Simulated clock over a ledger: sum over steps of alpha plus the
    largest number of bytes any device sends or receives in that step,
    divided by beta. A step with no messages costs nothing."""
    per_step: dict = {}
    for m in ledger.msgs:
        sent, recv = per_step.setdefault(m.step, ({}, {}))
        sent[m.src] = sent.get(m.src, 0) + m.bytes
        recv[m.dst] = recv.get(m.dst, 0) + m.bytes
    t = 0.0
    for step in sorted(per_step):
        sent, recv = per_step[step]
        busiest = max(max(sent.values()), max(recv.values()))
        t += alpha + busiest / beta
    return t


def algbw(nbytes: float, t: float) -> float:
    return nbytes / t


def busbw(nbytes: float, t: float, p: int) -> float:
    return nbytes / t * 2 * (p - 1) / p


def ledger_time_nodes(ledger, local: int, alpha_in: float, beta_in: float, alpha_out: float,
                      beta_out: float) -> float:
    """Two-level clock (sections 2.3 and 6.3, exercise 6): ranks r and s share
    a node when r // local == s // local. A message inside a node costs
    (alpha_in, beta_in), one across nodes (alpha_out, beta_out). Every rank has
    one sending and one receiving port of each class; a step lasts as long as
    its slowest busy port, alpha + bytes / beta of that port's class."""
    per_step: dict = {}
    for m in ledger.msgs:
        ports = per_step.setdefault(m.step, {})
        cls = "out" if m.src // local != m.dst // local else "in"
        ports[(cls, "send", m.src)] = ports.get((cls, "send", m.src), 0) + m.bytes
        ports[(cls, "recv", m.dst)] = ports.get((cls, "recv", m.dst), 0) + m.bytes
    t = 0.0
    for step in sorted(per_step):
        slowest = 0.0
        for (cls, _, _), nbytes in per_step[step].items():
            a, b = (alpha_out, beta_out) if cls == "out" else (alpha_in, beta_in)
            slowest = max(slowest, a + nbytes / b)
        t += slowest
    return t


def broadcast_formula(algo: str, p: int, nbytes: float, alpha: float, beta: float, k: int = 1) -> float:
    """Closed-form broadcast times ("Networks and Collective Communication",
    sections 4.2 and 5.5): naive (p-1)(alpha + n/beta); binomial tree
    ceil(log2 p)(alpha + n/beta); pipelined chain of k blocks
    (p-2+k)(alpha + n/(k beta)); scatter + all-gather: one scatter step that
    puts (p-1)/p n through the root's port, then p-1 ring steps of n/p."""
    if p == 1:
        return 0.0
    if algo == "naive":
        return (p - 1) * (alpha + nbytes / beta)
    if algo == "tree":
        return math.ceil(math.log2(p)) * (alpha + nbytes / beta)
    if algo == "chain":
        return (p - 2 + k) * (alpha + nbytes / (k * beta))
    if algo == "scatter_allgather":
        return (alpha + (p - 1) / p * nbytes / beta) + (p - 1) * (alpha + nbytes / (p * beta))
    raise ValueError(algo)


def chain_optimum(p: int, nbytes: float, alpha: float, beta: float) -> tuple:
    """Section 5.5 / exercise 9: d/dk of (p-2+k)(alpha + n/(k beta)) = 0 gives
    k* = sqrt((p-2) n / (alpha beta)) and T* = (sqrt((p-2) alpha) + sqrt(n/beta))^2."""
    k = math.sqrt((p - 2) * nbytes / (alpha * beta))
    t = (math.sqrt((p - 2) * alpha) + math.sqrt(nbytes / beta)) ** 2
    return k, t
