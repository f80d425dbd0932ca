"""Seeded synthetic inputs for the single-GPU virtual cluster.

This module is shared *data* for both the CPU oracle and the HIP path: it
draws random numbers and lays them out, and holds none of the collectives'
arithmetic (no sums, no chunking, no schedules, no routing plans).

Every rank buffer is generated in blocks of ``BLOCK`` elements, block ``b`` of
rank ``r`` of workload tag ``t`` coming from ``numpy.random.default_rng([t,
r, b])`` (a tuple-seeded PCG64 stream), so any element window can be
regenerated on its own without materialising the rest of the buffer.

Floating-point draws are made in float64 and rounded once to the storage type:
float32 by numpy's round-to-nearest-even cast, bfloat16 by torch's CPU
conversion (also round-to-nearest-even); bfloat16 data is handed around as
``uint16`` bit patterns.

Workload shapes follow the pages' examples:

* worked example -- 4 devices, device d holds [10d, 10d+1, 10d+2, 10d+3]
  (Networks and Collective Communication, section 4.1);
* DDP gradient bucket -- 25 MB buckets (11-1 distributed training notes,
  "Communication-Computation Overlap", bucket_cap_mb=25);
* 16 ranks x 192 MiB gradients (LLM Distributed Training Collectives, the
  book chapters 6-7/10 summary on hierarchical gradients);
* DeepSeek-V3-sized MoE dispatch: hidden 7168, top-8 of 256 experts
  (Networks and Collective Communication, section 7.4);
* decode-like 10 KiB and prefill-like 80 MiB all-reduce messages (LLM
  Distributed Training Collectives, same summary).
"""
from __future__ import annotations

import numpy as np

BLOCK = 1 << 20

# Workload tags: the first element of every seed tuple.
TAG_RING_SMALL = 1      # p=8, 262,144 fp32 uniform[-1, 1]
TAG_DDP_BUCKET = 2      # p=8, 6,553,600 fp32 normal(0, 1e-3)
TAG_HIER_BF16 = 3       # p=16, 100,663,296 bf16 uniform[-1, 1]
TAG_MOE = 4             # p=8 MoE tokens + routing
TAG_SWEEP = 5           # message-size sweep, fp32 normal(0, 1)
TAG_TEST = 9            # small ad-hoc test buffers


def _to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _draw(rng: np.random.Generator, dist: tuple, size: int) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size)
    if kind == "int":      # integers in [lo, hi), exact in float32 when small
        return rng.integers(dist[1], dist[2], size).astype(np.float64)
    raise ValueError(f"unknown distribution {dist!r}")


def rank_window(tag: int, rank: int, lo: int, hi: int, dist: tuple,
                dtype: str = "f32") -> np.ndarray:
    """Elements [lo, hi) of rank ``rank``'s buffer of workload ``tag``.

    Returns float32 values for ``dtype='f32'`` and uint16 bfloat16 bit
    patterns for ``dtype='bf16'``.
    """
    if hi < lo:
        raise ValueError("hi < lo")
    out = np.empty(hi - lo, dtype=np.float32 if dtype == "f32" else np.uint16)
    b0, b1 = lo // BLOCK, (hi - 1) // BLOCK if hi > lo else lo // BLOCK - 1
    for b in range(b0, b1 + 1):
        rng = np.random.default_rng([tag, rank, b])
        vals = _draw(rng, dist, BLOCK)
        s, e = max(lo, b * BLOCK), min(hi, (b + 1) * BLOCK)
        piece = vals[s - b * BLOCK:e - b * BLOCK]
        out[s - lo:e - lo] = piece.astype(np.float32) if dtype == "f32" else _to_bf16_bits(piece)
    return out


def rank_buffers(tag: int, p: int, n: int, dist: tuple, dtype: str = "f32") -> list[np.ndarray]:
    """All p rank buffers of n elements each."""
    return [rank_window(tag, r, 0, n, dist, dtype) for r in range(p)]


def worked_example(p: int = 4, n: int = 4) -> list[np.ndarray]:
    """Device d holds [10d, 10d+1, ..., 10d+n-1] (section 4.1 demo)."""
    return [np.array([10 * d + k for k in range(n)], dtype=np.float32) for d in range(p)]


# --- named workloads -------------------------------------------------------

RING_SMALL = dict(tag=TAG_RING_SMALL, p=8, n=262_144, dist=("uniform", -1.0, 1.0), dtype="f32")
DDP_BUCKET = dict(tag=TAG_DDP_BUCKET, p=8, n=6_553_600, dist=("normal", 0.0, 1e-3), dtype="f32")
HIER_BF16 = dict(tag=TAG_HIER_BF16, p=16, n=100_663_296, dist=("uniform", -1.0, 1.0), dtype="bf16")
SWEEP_P = (2, 4, 8, 16, 72)
# per-rank bytes: 1 KiB .. 1 GiB in powers of 4, plus decode-like 10 KiB and prefill-like 80 MiB
SWEEP_BYTES = tuple(sorted([1024 * 4 ** k for k in range(11)] + [10 * 1024, 80 * 1024 * 1024]))
SWEEP_DIST = ("normal", 0.0, 1.0)

MOE = dict(p=8, tokens=4096, hidden=7168, experts=256, topk=8, zipf_s=1.1)


def moe_topk(rank: int, tokens: int = 4096, experts: int = 256, topk: int = 8,
             zipf_s: float = 1.1) -> np.ndarray:
    """Top-k expert ids per token of one rank, int32 [tokens, topk], ascending per row.

    Expert popularity is Zipf(s): weight (e+1)^-s for expert id e (ids map to
    popularity rank directly). Each token draws ``topk`` distinct experts
    without replacement in proportion to the weights, via Gumbel-top-k: the
    k largest of log w_e + Gumbel(0, 1).
    """
    rng = np.random.default_rng([TAG_MOE, rank])
    logw = -zipf_s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    keys = logw[None, :] + rng.gumbel(size=(tokens, experts))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :topk]
    return np.sort(order, axis=1).astype(np.int32)


def moe_tokens(rank: int, tokens: int = 4096, hidden: int = 7168) -> np.ndarray:
    """Token activations of one rank: bf16 bits [tokens, hidden], normal(0, 1)."""
    flat = rank_window(TAG_MOE * 100 + 1, rank, 0, tokens * hidden, ("normal", 0.0, 1.0), "bf16")
    return flat.reshape(tokens, hidden)


def tagged_rows(rows: np.ndarray, rank: int, token: np.ndarray, slot: np.ndarray | None = None) -> np.ndarray:
    """Copy of bf16 rows with (rank, token[, slot]) written as raw uint16 into
    the first elements, so that a misplaced row is visible even among equal rows."""
    out = rows.copy()
    out[:, 0] = np.uint16(rank)
    out[:, 1] = token.astype(np.uint16)
    if slot is not None:
        out[:, 2] = slot.astype(np.uint16)
    return out
