"""A process pool that runs the CPU oracle (and the seeded input generators)
over consecutive element windows of workloads too large for one thread.

Used by the GPU parity tests to compare every element of full-size outputs:
the workers are spawned Python processes that import only ``workloads``
(inputs) and ``oracle`` (expected values); they never touch the GPU. The
oracle's windowed mode computes elements [lo, hi) of every rank's all-reduce
output from the same elements of every rank's input, so the windows can be
checked independently and in any order.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle
import workloads

WORKERS = max(1, min(8, len(os.sched_getaffinity(0))))


def windows(n: int, w: int) -> list:
    """Consecutive [lo, hi) windows covering 0..n."""
    return [(lo, min(n, lo + w)) for lo in range(0, n, w)]


def window_len(p: int, budget: int = 1 << 24) -> int:
    """Elements per window so that one window of all p ranks holds about
    `budget` elements."""
    return max(4096, budget // p)


def _inputs(tag, p, lo, hi, dist, dtype):
    return np.stack([workloads.rank_window(tag, r, lo, hi, dist, dtype) for r in range(p)])


def gen_window(args):
    """(lo, hi, [p, hi-lo] input bits) of workload `tag`."""
    tag, p, lo, hi, dist, dtype = args
    return lo, hi, _inputs(tag, p, lo, hi, dist, dtype)


def oracle_window(args):
    """(lo, hi, {algo: [p, hi-lo] expected all-reduce bits}) on the
    workload's inputs, regenerated in the worker."""
    tag, p, n, lo, hi, dist, dtype, algos = args
    x = _inputs(tag, p, lo, hi, dist, dtype)
    out = {}
    for algo in algos:
        want, _ = oracle.allreduce(list(x), algo, dtype, n=n, lo=lo)
        out[algo] = np.stack(want).view(np.uint32 if dtype == "f32" else np.uint16)
    return lo, hi, out


def pool(workers: int = WORKERS):
    return mp.get_context("spawn").Pool(workers)
