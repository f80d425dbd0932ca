"""CPU oracle for the virtual-cluster collectives.

TEST INFRASTRUCTURE. This package is a plain, slow, step-by-step CPU model of
each collective with an explicit message ledger. Only ``tests/``, the smoke
check in ``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may
import it. The library under ``collective_communication_algorithms_vcoll_amd``
never imports it and shares no code with it; the two meet only through the
seeded inputs of the ``workloads`` module.

Arithmetic: float32 adds, round to nearest even, in the order each
algorithm's steps produce (numpy float32 arrays, no fused multiply-add, no
flush-to-zero); bfloat16 values widen exactly and round once (numerics.py).
"""
from .cluster import ADD, COPY, Ledger, Msg
from .collectives import (ALGOS, all_gather, all_to_all, allreduce, allreduce_hierarchical,
                          block_offsets, chunk_bounds, reduce_scatter)
from .moe import combine as moe_combine
from .moe import dispatch as moe_dispatch
from .moe import plan as moe_plan
from .numerics import ELEM_BYTES, bf16_to_f32, f32_to_bf16, round_to_bf16

__all__ = [
    "ADD", "COPY", "Ledger", "Msg", "ALGOS", "all_gather", "all_to_all", "allreduce",
    "allreduce_hierarchical",
    "block_offsets", "chunk_bounds", "reduce_scatter", "moe_plan", "moe_dispatch",
    "moe_combine", "ELEM_BYTES", "bf16_to_f32", "f32_to_bf16", "round_to_bf16",
]
