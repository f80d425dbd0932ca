"""A virtual cluster: p ranks holding real arrays, plus a per-message ledger.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

This is the simulation style that "Networks and Collective Communication"
(semidirectx cs349e prerequisite lecture 5) describes for its comm_sim
module: real data on every simulated device and an account of every message
(code note at the top of the lecture; per-device byte counts in section 4.3).

One step of an algorithm is synchronous: every message of the step is formed
from the state the ranks hold *before* the step, and only then are all of them
delivered (copied into, or added onto, the receiver's buffer). Recursive
doubling partners "exchange" full vectors in the same step (section 5.2),
which only makes sense under this reading.

Windowed mode: a rank's buffer may hold only the element window [lo, hi) of
its logical vector of ``size`` elements. Messages are recorded in the ledger
with their full logical ranges, but only their intersection with the window
is moved. This lets the oracle check sampled elements of inputs too large to
hold on the host.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import NamedTuple

import numpy as np


class Msg(NamedTuple):
    """One ledger record. Offsets and count are in elements of the storage type."""
    step: int
    src: int
    dst: int
    src_off: int
    dst_off: int
    count: int
    bytes: int


ADD = "add"
COPY = "copy"


class Send(NamedTuple):
    src: int
    dst: int
    src_off: int
    dst_off: int
    count: int
    op: str


@dataclass
class Ledger:
    p: int
    elem_bytes: int
    msgs: list = field(default_factory=list)
    n_steps: int = 0

    def record(self, step: int, src: int, dst: int, src_off: int, dst_off: int, count: int) -> None:
        self.msgs.append(Msg(step, src, dst, src_off, dst_off, count, count * self.elem_bytes))
        self.n_steps = max(self.n_steps, step + 1)

    def sorted(self) -> list:
        return sorted(self.msgs, key=lambda m: (m.step, m.src, m.dst, m.src_off))

    def sent_bytes(self) -> list:
        out = [0] * self.p
        for m in self.msgs:
            out[m.src] += m.bytes
        return out

    def recv_bytes(self) -> list:
        out = [0] * self.p
        for m in self.msgs:
            out[m.dst] += m.bytes
        return out


class Cluster:
    """p ranks; ``bufs[r]`` holds elements [lo, lo + len) of rank r's vector."""

    def __init__(self, bufs: list, lo: int, ledger: Ledger):
        self.bufs = bufs
        self.lo = lo
        self.ledger = ledger

    def _window(self, off: int, count: int, length: int):
        a = max(off, self.lo)
        b = min(off + count, self.lo + length)
        return a, b

    def step(self, step: int, sends: list) -> None:
        # 1) form every message from the pre-step state
        pending = []
        for s in sends:
            self.ledger.record(step, s.src, s.dst, s.src_off, s.dst_off, s.count)
            src_buf = self.bufs[s.src]
            a, b = self._window(s.src_off, s.count, len(src_buf))
            if b <= a:
                continue
            payload = src_buf[a - self.lo:b - self.lo].copy()
            # every collective run on this cluster keeps a piece at the same
            # position in sender and receiver, so one window serves both
            assert s.src_off == s.dst_off
            pending.append((s.dst, a, payload, s.op))
        # 2) deliver
        for dst, da, payload, op in pending:
            dbuf = self.bufs[dst]
            sl = slice(da - self.lo, da - self.lo + len(payload))
            if op == ADD:
                dbuf[sl] = dbuf[sl] + payload
            else:
                dbuf[sl] = payload
