"""Python binding of libvcoll, the single-GPU virtual-cluster collectives.

Functions carry the C names of ``include/vcoll.h`` and only marshal
arguments: tensors become device pointers, torch's current HIP stream becomes
the launch stream, and status codes become exceptions. Every collective runs
in libvcoll's HIP kernels; there is no other code path. If ``libvcoll.so``
has not been built this module raises on import.

Rank buffers are given either as one 2-D tensor [p, n] (row r is rank r) or
as a sequence of p 1-D tensors, all on the same GPU, contiguous, same dtype
(torch.float32 or torch.bfloat16).

Environment: VCOLL_DEBUG=1 synchronizes after every call (see _check).
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvcoll.so")

RING, RECURSIVE_DOUBLING, RABENSEIFNER, BINARY_TREE = 0, 1, 2, 3
NAIVE, SCATTER_ALLGATHER, PIPELINED_CHAIN = 4, 5, 6
ALGOS = {"ring": RING, "rd": RECURSIVE_DOUBLING, "recursive_doubling": RECURSIVE_DOUBLING,
         "rabenseifner": RABENSEIFNER, "tree": BINARY_TREE, "binary_tree": BINARY_TREE,
         "naive": NAIVE, "scatter_allgather": SCATTER_ALLGATHER, "chain": PIPELINED_CHAIN,
         "pipelined_chain": PIPELINED_CHAIN}
F32, BF16, U8 = 0, 1, 2
OP_ALLREDUCE, OP_REDUCE_SCATTER, OP_ALL_GATHER, OP_ALL_TO_ALL = 0, 1, 2, 3
OP_BROADCAST, OP_REDUCE = 4, 5
OPS = {"allreduce": OP_ALLREDUCE, "reduce_scatter": OP_REDUCE_SCATTER,
       "all_gather": OP_ALL_GATHER, "all_to_all": OP_ALL_TO_ALL,
       "broadcast": OP_BROADCAST, "reduce": OP_REDUCE}
MAX_RANKS = 128


class VcollError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = _lib()
        detail = lib.vcoll_status_str(status).decode()
        if status == 4:
            detail += f" ({lib.vcoll_last_hip_error().decode()})"
        super().__init__(f"{what}: {detail} (status {status})")
        self.status = status


class Msg(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("src", ctypes.c_int32), ("dst", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("src_off", ctypes.c_int64),
                ("dst_off", ctypes.c_int64), ("count", ctypes.c_int64), ("bytes", ctypes.c_int64)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        # torch ships its own copy of the HIP runtime under the same soname;
        # loading torch first makes libvcoll bind to that copy, so there is
        # one runtime in the process and torch's streams and memory are ours
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python collective_communication_algorithms_vcoll_amd/csrc/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64, VP = ctypes.POINTER, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        lib.vcoll_abi_version.restype = I
        lib.vcoll_status_str.restype = ctypes.c_char_p
        lib.vcoll_status_str.argtypes = [I]
        lib.vcoll_chunk.argtypes = [I, I64, I, P(I64), P(I64)]
        for name in ("vcoll_allreduce", "vcoll_reduce_scatter", "vcoll_all_gather"):
            getattr(lib, name).argtypes = [I, I, I64, I, P(VP), P(VP), VP]
            getattr(lib, name).restype = I
        lib.vcoll_all_to_all.argtypes = [I, I64, I, P(I64), P(VP), P(VP), P(VP), P(I64), P(VP),
                                         P(I64), VP]
        lib.vcoll_all_to_all.restype = I
        lib.vcoll_ledger.argtypes = [I, I, I, I64, I, P(I64), I64, P(Msg), I64, P(I64), P(I64),
                                     P(I64), P(ctypes.c_int32)]
        lib.vcoll_ledger.restype = I
        lib.vcoll_moe_plan.argtypes = [I, I64, I, I, P(ctypes.c_int32), P(I64),
                                       P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.vcoll_moe_plan.restype = I
        lib.vcoll_last_hip_error.restype = ctypes.c_char_p
        lib.vcoll_allreduce_hierarchical.argtypes = [I, I, I64, I, P(VP), P(VP), VP]
        lib.vcoll_allreduce_hierarchical.restype = I
        lib.vcoll_ledger_hierarchical.argtypes = [I, I, I64, I, P(Msg), I64, P(I64), P(I64), P(I64),
                                                  P(ctypes.c_int32)]
        lib.vcoll_ledger_hierarchical.restype = I
        lib.vcoll_model_ledger_time_nodes.argtypes = [I, I, I, I, I64, I, ctypes.c_double, ctypes.c_double,
                                                      ctypes.c_double, ctypes.c_double,
                                                      P(ctypes.c_double), P(ctypes.c_int32)]
        lib.vcoll_model_ledger_time_nodes.restype = I
        lib.vcoll_broadcast.argtypes = [I, I64, I, I, VP, P(VP), VP]
        lib.vcoll_broadcast.restype = I
        lib.vcoll_reduce.argtypes = [I, I, I64, I, I, P(VP), VP, VP]
        lib.vcoll_reduce.restype = I
        lib.vcoll_ledger_rooted.argtypes = [I, I, I, I64, I, I, I64, P(Msg), I64, P(I64), P(I64), P(I64),
                                            P(ctypes.c_int32)]
        lib.vcoll_ledger_rooted.restype = I
        D = ctypes.c_double
        lib.vcoll_model_broadcast_formula.argtypes = [I, I, D, I64, D, D, P(D)]
        lib.vcoll_model_broadcast_formula.restype = I
        lib.vcoll_model_chain_optimum.argtypes = [I, D, D, D, P(D), P(D)]
        lib.vcoll_model_chain_optimum.restype = I
        lib.vcoll_model_clock.argtypes = [P(Msg), I64, I, I, D, D, D, D, P(D)]
        lib.vcoll_model_clock.restype = I
        lib.vcoll_moe_slots.argtypes = [I, I64, I, P(I64), P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.vcoll_moe_slots.restype = I
        lib.vcoll_moe_expand_slots.argtypes = [I64, I, P(ctypes.c_int32), I64, P(ctypes.c_int32)]
        lib.vcoll_moe_expand_slots.restype = I
        lib.vcoll_moe_dedup_slots.argtypes = [I, I64, I, P(I64), P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.vcoll_moe_dedup_slots.restype = I
        lib.vcoll_moe_dispatch.argtypes = [I, I64, I, I64, I, I, P(VP), P(VP), P(VP), P(I64), VP]
        lib.vcoll_moe_dispatch.restype = I
        lib.vcoll_moe_combine.argtypes = [I, I64, I, I64, I, P(VP), P(I64), P(VP), P(VP), VP]
        lib.vcoll_moe_combine.restype = I
        lib.vcoll_moe_plan_dedup.argtypes = [I, I64, I, I, P(ctypes.c_int32), P(I64), P(ctypes.c_int32),
                                             P(ctypes.c_int32), P(I64)]
        lib.vcoll_moe_plan_dedup.restype = I
        lib.vcoll_moe_dispatch_fp8.argtypes = [I, I64, P(I64), P(VP), P(I64), P(VP), P(VP), VP]
        lib.vcoll_moe_dispatch_fp8.restype = I
        lib.vcoll_allreduce_stepwise.argtypes = [I, I, I64, I, P(VP), P(VP), VP, I64, P(ctypes.c_int32), VP]
        lib.vcoll_allreduce_stepwise_static.restype = I
        lib.vcoll_broadcast_stepwise.restype = I
        lib.vcoll_broadcast_stepwise.argtypes = [I, I, I64, I, I, I64, VP, P(VP), P(ctypes.c_int32), VP]
        lib.vcoll_allreduce_stepwise_static.argtypes = [I, I, I64, I, P(VP), P(VP), P(ctypes.c_int32), VP]
        lib.vcoll_allreduce_stepwise.restype = I
        D = ctypes.c_double
        lib.vcoll_model_formula.argtypes = [I, I, D, D, D, P(D)]
        lib.vcoll_model_formula.restype = I
        lib.vcoll_model_ledger_time.argtypes = [I, I, I, I64, I, P(I64), I64, D, D, P(D), P(ctypes.c_int32)]
        lib.vcoll_model_ledger_time.restype = I
        lib.vcoll_bench_copy.argtypes = [VP, VP, I64, VP]
        lib.vcoll_bench_copy.restype = I
        lib.vcoll_bench_stream.argtypes = [I, VP, VP, I64, VP]
        lib.vcoll_bench_stream.restype = I
        if lib.vcoll_abi_version() != 1:
            raise ImportError("libvcoll ABI version mismatch")
        _LIB = lib
    return _LIB


_lib()


# VCOLL_DEBUG=1: wait for the device after every successful call, so that a
# fault in a kernel surfaces at the call that launched it rather than at a
# later synchronization (slow; for debugging only)
_DEBUG = os.environ.get("VCOLL_DEBUG", "") not in ("", "0")


def _check(status: int, what: str) -> None:
    if status != 0:
        raise VcollError(status, what)
    if _DEBUG:
        import torch
        if torch.cuda.is_initialized():
            try:
                torch.cuda.synchronize()
            except RuntimeError as e:
                raise RuntimeError(f"{what}: the device reported an error after this call: {e}") from e


def _algo(algo) -> int:
    if isinstance(algo, str):
        if algo not in ALGOS:
            raise ValueError(f"unknown algorithm {algo!r}")
        return ALGOS[algo]
    return int(algo)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return U8                     # accepted by the all-to-all only
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ranks(bufs) -> list:
    import torch
    if isinstance(bufs, torch.Tensor):
        if bufs.dim() != 2:
            raise ValueError("a single tensor of rank buffers must be 2-D [p, n]")
        return [bufs[r] for r in range(bufs.shape[0])]
    return list(bufs)


def _on_current_gpu(t) -> None:
    """The library launches on the calling thread's current device, so every
    buffer whose address it receives must live there (a host or other-device
    address would fault inside a kernel)."""
    import torch
    if t.device.type != "cuda":
        raise ValueError(f"vcoll: buffer on {t.device}; every buffer must be a GPU tensor")
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"vcoll: buffer on {t.device}, but kernels run on the current device cuda:{cur}")


def _dptr(t) -> int:
    """Device address of a tensor on the current GPU."""
    _on_current_gpu(t)
    return t.data_ptr()


def _ptrs(ts: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        if t is not None and t.numel() > 0:
            _on_current_gpu(t)
            arr[i] = t.data_ptr()
        else:
            arr[i] = None
    return arr


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _validate(ts: list, what: str, n: int | None = None):
    import torch
    if not 1 <= len(ts) <= MAX_RANKS:
        raise ValueError(f"{what}: p={len(ts)} outside [1, {MAX_RANKS}]")
    dev, dt = ts[0].device, ts[0].dtype
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.device != dev or t.dtype != dt:
            raise ValueError(f"{what}: all rank buffers must be tensors on one device with one dtype")
        if dev.type != "cuda":
            raise ValueError(f"{what}: rank buffers must be on a GPU")
        if not t.is_contiguous():
            raise ValueError(f"{what}: rank buffers must be contiguous")
        if n is not None and t.numel() != n:
            raise ValueError(f"{what}: expected {n} elements per rank, got {t.numel()}")


def _span(t):
    return t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()


def _no_overlap(a: list, b: list, what: str, same_index_ok: bool = False) -> None:
    """Raise if a buffer of `a` overlaps a buffer of `b`. With same_index_ok,
    a[i] and b[i] may be the very same buffer (in place). Sorted sweep over
    the spans, so p = 128 rank buffers cost O(p log p), not O(p^2)."""
    import heapq
    spans = []
    for side, ts in ((0, a), (1, b)):
        for i, t in enumerate(ts):
            if t is not None and t.numel() > 0:
                s0, s1 = _span(t)
                spans.append((s0, s1, side, i))
    spans.sort()
    active = []                                   # (end, start, side, index)
    for s0, s1, side, i in spans:
        while active and active[0][0] <= s0:
            heapq.heappop(active)
        for e1, e0, oside, oi in active:
            if oside == side:
                continue
            if same_index_ok and oi == i and e0 == s0 and e1 == s1:
                continue
            raise ValueError(f"{what}: input and output buffers overlap")
        heapq.heappush(active, (s1, s0, side, i))


def _disjoint(ts: list, what: str) -> None:
    """Raise if two of the buffers overlap: every output of a collective gets
    its own data, so two outputs sharing bytes would race."""
    spans = sorted(_span(t) for t in ts if t is not None and t.numel() > 0)
    for (_, e0), (s1, _) in zip(spans, spans[1:]):
        if s1 < e0:
            raise ValueError(f"{what}: output buffers overlap")


# -----------------------------------------------------------------------------


def vcoll_chunk(p: int, n: int, c: int) -> tuple:
    off, cnt = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib().vcoll_chunk(p, n, c, ctypes.byref(off), ctypes.byref(cnt)), "vcoll_chunk")
    return off.value, cnt.value


def vcoll_allreduce(algo, send, recv=None):
    """All-reduce; returns recv (allocated like send when None; recv may be send)."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_allreduce")
    n = s[0].numel()
    _validate(s, "vcoll_allreduce", n)
    if recv is None:
        recv = torch.empty_like(send) if isinstance(send, torch.Tensor) else [torch.empty_like(t) for t in s]
    r = _ranks(recv)
    _validate(r, "vcoll_allreduce", n)
    if len(r) != len(s) or r[0].dtype != s[0].dtype or r[0].device != s[0].device:
        raise ValueError("vcoll_allreduce: send and recv must match in p, dtype and device")
    _no_overlap(s, r, "vcoll_allreduce", same_index_ok=True)
    _disjoint(r, "vcoll_allreduce")
    _check(_lib().vcoll_allreduce(_algo(algo), len(s), n, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                  _stream(s[0])), "vcoll_allreduce")
    return recv


def vcoll_allreduce_stepwise(algo, send, recv=None, workspace=None):
    """Stepwise all-reduce (one launch per algorithm step); returns
    (recv, launches). bf16 needs a float32 workspace of p*n elements, made
    when None."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_allreduce_stepwise")
    n = s[0].numel()
    _validate(s, "vcoll_allreduce_stepwise", n)
    if recv is None:
        recv = torch.empty_like(send) if isinstance(send, torch.Tensor) else [torch.empty_like(t) for t in s]
    r = _ranks(recv)
    _validate(r, "vcoll_allreduce_stepwise", n)
    _no_overlap(s, r, "vcoll_allreduce_stepwise", same_index_ok=True)
    _disjoint(r, "vcoll_allreduce_stepwise")
    ws_ptr, ws_bytes = None, 0
    if _dtype_code(s[0]) == BF16:
        if workspace is None:
            workspace = torch.empty(len(s) * n, dtype=torch.float32, device=s[0].device)
        if workspace.dtype != torch.float32 or workspace.numel() < len(s) * n:
            raise ValueError("vcoll_allreduce_stepwise: workspace must hold p*n float32")
        _no_overlap([workspace], s + r, "vcoll_allreduce_stepwise")
        ws_ptr, ws_bytes = _dptr(workspace), workspace.numel() * 4
    launches = ctypes.c_int32()
    _check(_lib().vcoll_allreduce_stepwise(_algo(algo), len(s), n, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                           ws_ptr, ws_bytes, ctypes.byref(launches), _stream(s[0])),
           "vcoll_allreduce_stepwise")
    return recv, launches.value


STEP_SCRATCH_BYTES = 64 * 1024 * 1024     # VCOLL_STEP_SCRATCH_BYTES


def vcoll_allreduce_stepwise_static(algo, send, recv=None):
    """vcoll_allreduce_stepwise without a workspace: bf16 partial sums live
    in the library's own per-GPU scratch array (p*n*4 bytes at most
    STEP_SCRATCH_BYTES). Returns (recv, launches). Calls on one GPU that
    are not ordered on one stream race on that array."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_allreduce_stepwise_static")
    n = s[0].numel()
    _validate(s, "vcoll_allreduce_stepwise_static", n)
    if recv is None:
        recv = torch.empty_like(send) if isinstance(send, torch.Tensor) else [torch.empty_like(t) for t in s]
    r = _ranks(recv)
    _validate(r, "vcoll_allreduce_stepwise_static", n)
    _no_overlap(s, r, "vcoll_allreduce_stepwise_static", same_index_ok=True)
    _disjoint(r, "vcoll_allreduce_stepwise_static")
    launches = ctypes.c_int32()
    _check(_lib().vcoll_allreduce_stepwise_static(_algo(algo), len(s), n, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                                  ctypes.byref(launches), _stream(s[0])),
           "vcoll_allreduce_stepwise_static")
    return recv, launches.value


def vcoll_broadcast(send, recv, root: int = 0):
    """Copy the root's buffer `send` into every rank's buffer of `recv` (a
    [p, n] tensor or a list of p tensors; recv[root] may be `send` itself)."""
    r = _ranks(recv)
    _validate(r, "vcoll_broadcast")
    n = r[0].numel()
    _validate(r, "vcoll_broadcast", n)
    if not 0 <= root < len(r):
        raise ValueError("vcoll_broadcast: root out of range")
    _validate([send], "vcoll_broadcast", n)
    if send.dtype != r[0].dtype or send.device != r[0].device:
        raise ValueError("vcoll_broadcast: send and recv differ in dtype or device")
    targets = [t for i, t in enumerate(r) if not (i == root and t.data_ptr() == send.data_ptr())]
    _no_overlap([send], targets, "vcoll_broadcast")
    for i, a in enumerate(targets):
        _no_overlap([a], targets[i + 1:], "vcoll_broadcast")
    _check(_lib().vcoll_broadcast(len(r), n, _dtype_code(send), root, _dptr(send) if n else None, _ptrs(r),
                                  _stream(send)), "vcoll_broadcast")
    return recv


def vcoll_broadcast_stepwise(algo, send, recv, root: int = 0, blocks: int = 1):
    """vcoll_broadcast executed one launch per step of the algorithm's
    schedule ('naive', 'tree', 'scatter_allgather', 'chain' with `blocks`
    blocks). Returns (recv, launches)."""
    r = _ranks(recv)
    _validate(r, "vcoll_broadcast_stepwise")
    n = r[0].numel()
    _validate(r, "vcoll_broadcast_stepwise", n)
    if not 0 <= root < len(r):
        raise ValueError("vcoll_broadcast_stepwise: root out of range")
    _validate([send], "vcoll_broadcast_stepwise", n)
    if send.dtype != r[0].dtype or send.device != r[0].device:
        raise ValueError("vcoll_broadcast_stepwise: send and recv differ in dtype or device")
    targets = [t for i, t in enumerate(r) if not (i == root and t.data_ptr() == send.data_ptr())]
    _no_overlap([send], targets, "vcoll_broadcast_stepwise")
    for i, a in enumerate(targets):
        _no_overlap([a], targets[i + 1:], "vcoll_broadcast_stepwise")
    launches = ctypes.c_int32()
    _check(_lib().vcoll_broadcast_stepwise(_algo(algo), len(r), n, _dtype_code(send), root, blocks,
                                           _dptr(send) if n else None, _ptrs(r), ctypes.byref(launches),
                                           _stream(send)), "vcoll_broadcast_stepwise")
    return recv, launches.value


def prepare_broadcast_stepwise(algo, send, recv, root: int = 0, blocks: int = 1) -> PreparedCall:
    r = _ranks(recv)
    vcoll_broadcast_stepwise(algo, send, recv, root, blocks)
    rp = _ptrs(r)
    args = (_algo(algo), len(r), r[0].numel(), _dtype_code(send), root, blocks, send.data_ptr(), rp, None,
            _stream(send))
    return PreparedCall("vcoll_broadcast_stepwise", _lib().vcoll_broadcast_stepwise, args, (send, recv, rp))


def vcoll_reduce(send, recv=None, root: int = 0, algo="tree"):
    """Sum the p rank buffers of `send` into the root's buffer `recv`
    (binomial tree on ranks relative to the root). Returns recv."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_reduce")
    n = s[0].numel()
    _validate(s, "vcoll_reduce", n)
    if not 0 <= root < len(s):
        raise ValueError("vcoll_reduce: root out of range")
    if recv is None:
        recv = torch.empty_like(s[0])
    _validate([recv], "vcoll_reduce", n)
    if recv.dtype != s[0].dtype or recv.device != s[0].device:
        raise ValueError("vcoll_reduce: send and recv differ in dtype or device")
    others = [t for i, t in enumerate(s) if not (i == root and t.data_ptr() == recv.data_ptr())]
    _no_overlap(others, [recv], "vcoll_reduce")
    _check(_lib().vcoll_reduce(_algo(algo), len(s), n, _dtype_code(s[0]), root, _ptrs(s),
                               _dptr(recv) if n else None, _stream(s[0])), "vcoll_reduce")
    return recv


def vcoll_ledger_rooted(op, algo, p: int, n: int, dtype: str = "f32", root: int = 0, blocks: int = 1):
    """Ledger of a broadcast or reduce: (messages, sent, received, steps)."""
    lib = _lib()
    opc = OPS[op] if isinstance(op, str) else int(op)
    dtc = {"f32": F32, "bf16": BF16}[dtype]
    count = ctypes.c_int64()
    _check(lib.vcoll_ledger_rooted(opc, _algo(algo), p, n, dtc, root, blocks, None, 0, ctypes.byref(count), None,
                                   None, None), "vcoll_ledger_rooted")
    msgs = (Msg * max(1, count.value))()
    sent, got, steps = (ctypes.c_int64 * p)(), (ctypes.c_int64 * p)(), ctypes.c_int32()
    _check(lib.vcoll_ledger_rooted(opc, _algo(algo), p, n, dtc, root, blocks, msgs, count.value,
                                   ctypes.byref(count), sent, got, ctypes.byref(steps)), "vcoll_ledger_rooted")
    out = [(m.step, m.src, m.dst, m.src_off, m.dst_off, m.count, m.bytes) for m in msgs[:count.value]]
    return out, list(sent), list(got), steps.value


def vcoll_model_broadcast_formula(algo, p: int, nbytes: float, alpha: float, beta: float, blocks: int = 1) -> float:
    t = ctypes.c_double()
    _check(_lib().vcoll_model_broadcast_formula(_algo(algo), p, float(nbytes), blocks, float(alpha), float(beta),
                                                ctypes.byref(t)), "vcoll_model_broadcast_formula")
    return t.value


def vcoll_model_chain_optimum(p: int, nbytes: float, alpha: float, beta: float) -> tuple:
    k, t = ctypes.c_double(), ctypes.c_double()
    _check(_lib().vcoll_model_chain_optimum(p, float(nbytes), float(alpha), float(beta), ctypes.byref(k),
                                            ctypes.byref(t)), "vcoll_model_chain_optimum")
    return k.value, t.value


def vcoll_model_clock(msgs, p: int, alpha: float, beta: float, local: int | None = None,
                      alpha_out: float | None = None, beta_out: float | None = None) -> float:
    """Simulated clock over a ledger given as (step, src, dst, src_off,
    dst_off, count, bytes) records; one link class unless `local` is set."""
    arr = (Msg * max(1, len(msgs)))()
    for i, m in enumerate(msgs):
        arr[i] = Msg(m[0], m[1], m[2], 0, m[3], m[4], m[5], m[6])
    t = ctypes.c_double()
    local = p if local is None else local
    _check(_lib().vcoll_model_clock(arr, len(msgs), p, local, float(alpha), float(beta),
                                    float(alpha if alpha_out is None else alpha_out),
                                    float(beta if beta_out is None else beta_out), ctypes.byref(t)),
           "vcoll_model_clock")
    return t.value


def vcoll_allreduce_hierarchical(nodes: int, local: int, send, recv=None):
    """Hierarchical (or 2D torus: nodes = rows, local = columns) all-reduce."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_allreduce_hierarchical")
    n = s[0].numel()
    _validate(s, "vcoll_allreduce_hierarchical", n)
    if len(s) != nodes * local:
        raise ValueError("vcoll_allreduce_hierarchical: p must equal nodes * local")
    if recv is None:
        recv = torch.empty_like(send) if isinstance(send, torch.Tensor) else [torch.empty_like(t) for t in s]
    r = _ranks(recv)
    _validate(r, "vcoll_allreduce_hierarchical", n)
    _no_overlap(s, r, "vcoll_allreduce_hierarchical", same_index_ok=True)
    _disjoint(r, "vcoll_allreduce_hierarchical")
    _check(_lib().vcoll_allreduce_hierarchical(nodes, local, n, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                               _stream(s[0])), "vcoll_allreduce_hierarchical")
    return recv


def vcoll_ledger_hierarchical(nodes: int, local: int, n: int, dtype: str = "f32"):
    """Ledger of the hierarchical all-reduce: (messages, sent, received, steps)."""
    lib = _lib()
    p = nodes * local
    dtc = {"f32": F32, "bf16": BF16}[dtype]
    count = ctypes.c_int64()
    _check(lib.vcoll_ledger_hierarchical(nodes, local, n, dtc, None, 0, ctypes.byref(count), None, None, None),
           "vcoll_ledger_hierarchical")
    msgs = (Msg * max(1, count.value))()
    sent, got, steps = (ctypes.c_int64 * p)(), (ctypes.c_int64 * p)(), ctypes.c_int32()
    _check(lib.vcoll_ledger_hierarchical(nodes, local, n, dtc, msgs, count.value, ctypes.byref(count), sent, got,
                                         ctypes.byref(steps)), "vcoll_ledger_hierarchical")
    out = [(m.step, m.src, m.dst, m.src_off, m.dst_off, m.count, m.bytes) for m in msgs[:count.value]]
    return out, list(sent), list(got), steps.value


def vcoll_model_ledger_time_nodes(algo, nodes: int, local: int, n: int, alpha_in: float, beta_in: float,
                                  alpha_out: float, beta_out: float, dtype: str = "f32") -> tuple:
    """Two-level alpha-beta clock; algo 'hierarchical' or a flat algorithm."""
    hier = algo == "hierarchical"
    t, steps = ctypes.c_double(), ctypes.c_int32()
    _check(_lib().vcoll_model_ledger_time_nodes(int(hier), 0 if hier else _algo(algo), nodes, local, n,
                                                {"f32": F32, "bf16": BF16}[dtype], alpha_in, beta_in,
                                                alpha_out, beta_out, ctypes.byref(t), ctypes.byref(steps)),
           "vcoll_model_ledger_time_nodes")
    return t.value, steps.value


def vcoll_reduce_scatter(algo, send, recv=None):
    """Reduce-scatter; recv[c] gets chunk c (vcoll_chunk(p, n, c) bounds)."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_reduce_scatter")
    n = s[0].numel()
    _validate(s, "vcoll_reduce_scatter", n)
    p = len(s)
    if recv is None:
        recv = [torch.empty(vcoll_chunk(p, n, c)[1], dtype=s[0].dtype, device=s[0].device) for c in range(p)]
    r = list(recv)
    if len(r) != p:
        raise ValueError("vcoll_reduce_scatter: need p output buffers")
    for c in range(p):
        if r[c].numel() != vcoll_chunk(p, n, c)[1] or r[c].dtype != s[0].dtype or not r[c].is_contiguous():
            raise ValueError(f"vcoll_reduce_scatter: output {c} must hold chunk {c}")
    _no_overlap(s, r, "vcoll_reduce_scatter")
    _disjoint(r, "vcoll_reduce_scatter")
    _check(_lib().vcoll_reduce_scatter(_algo(algo), p, n, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                       _stream(s[0])), "vcoll_reduce_scatter")
    return recv


def vcoll_all_gather(algo, send, recv=None):
    """All-gather of p equal blocks; recv[r] holds p*m elements."""
    import torch
    s = _ranks(send)
    _validate(s, "vcoll_all_gather")
    m = s[0].numel()
    _validate(s, "vcoll_all_gather", m)
    p = len(s)
    if recv is None:
        recv = torch.empty((p, p * m), dtype=s[0].dtype, device=s[0].device)
    r = _ranks(recv)
    _validate(r, "vcoll_all_gather", p * m)
    _no_overlap(s, r, "vcoll_all_gather")
    _disjoint(r, "vcoll_all_gather")
    _check(_lib().vcoll_all_gather(_algo(algo), p, m, _dtype_code(s[0]), _ptrs(s), _ptrs(r),
                                   _stream(s[0])), "vcoll_all_gather")
    return recv


def vcoll_all_to_all(send, splits, recv=None, src_rows=None, dst_rows=None, dst_table_rows=None):
    """Variable-split all-to-all of rows (see vcoll.h).

    send: p 2-D tensors [rows, H] (row-major, contiguous). splits: host
    [p, p] integers. src_rows / dst_rows: optional per-rank int32 GPU tensors
    (entries may be None) of gather / scatter indices. recv: p tensors, made
    when None ([sum_i splits[i][j], H], or [dst_table_rows[j], H] for ranks
    that scatter).
    """
    import torch
    s = list(send)
    p = len(s)
    sp = np.ascontiguousarray(np.asarray(splits, dtype=np.int64).reshape(p, p))
    H = s[0].shape[1] if s[0].dim() == 2 else 1
    dt = s[0].dtype
    dev = s[0].device
    for t in s:
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or (t.dim() == 2 and t.shape[1] != H):
            raise ValueError("vcoll_all_to_all: send buffers must share dtype, device, row width")
    scat = list(dst_rows) if dst_rows is not None else [None] * p
    gath = list(src_rows) if src_rows is not None else [None] * p
    if recv is None:
        recv = []
        for j in range(p):
            rows = int(sp[:, j].sum()) if scat[j] is None else int(dst_table_rows[j])
            recv.append(torch.empty((rows, H), dtype=dt, device=dev))
    r = list(recv)
    if len(r) != p:
        raise ValueError("vcoll_all_to_all: need p receive buffers")
    # the kernels trust the splits: every buffer must hold the rows they name
    for i in range(p):
        rows_i = s[i].shape[0] if s[i].dim() == 2 else s[i].numel()
        if gath[i] is None and rows_i < int(sp[i].sum()):
            raise ValueError(f"vcoll_all_to_all: send[{i}] has {rows_i} rows, splits send {int(sp[i].sum())}")
        if gath[i] is not None and gath[i].numel() < int(sp[i].sum()):
            raise ValueError(f"vcoll_all_to_all: src_rows[{i}] is shorter than the rows rank {i} sends")
        t = r[i]
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or (t.dim() == 2 and t.shape[1] != H):
            raise ValueError("vcoll_all_to_all: recv buffers must match send in dtype, device, row width")
        rows_r = t.shape[0] if t.dim() == 2 else t.numel()
        if scat[i] is None and rows_r < int(sp[:, i].sum()):
            raise ValueError(f"vcoll_all_to_all: recv[{i}] has {rows_r} rows, splits bring {int(sp[:, i].sum())}")
        if scat[i] is not None and scat[i].numel() < int(sp[:, i].sum()):
            raise ValueError(f"vcoll_all_to_all: dst_rows[{i}] is shorter than the rows rank {i} receives")
    _no_overlap(s, r, "vcoll_all_to_all")
    _disjoint(r, "vcoll_all_to_all")
    src_tab = (ctypes.c_int64 * p)(*[t.shape[0] if t.dim() == 2 else t.numel() for t in s])
    dst_tab = (ctypes.c_int64 * p)(*[t.shape[0] if t.dim() == 2 else t.numel() for t in r])
    for idx in gath + scat:
        if idx is not None and (idx.dtype != torch.int32 or idx.device != dev or not idx.is_contiguous()):
            raise ValueError("vcoll_all_to_all: row maps must be contiguous int32 tensors on the GPU")
    _check(_lib().vcoll_all_to_all(
        p, H, _dtype_code(s[0]), sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptrs(s), _ptrs(r),
        _ptrs(gath) if src_rows is not None else None, src_tab,
        _ptrs(scat) if dst_rows is not None else None, dst_tab, _stream(s[0])), "vcoll_all_to_all")
    return recv


def vcoll_ledger(op, algo, p: int, n: int, dtype: str = "f32", splits=None, row_elems: int = 0):
    """Messages of a collective: (list of (step, src, dst, src_off, dst_off,
    count, bytes), sent bytes per rank, received bytes per rank, step count)."""
    lib = _lib()
    opc = OPS[op] if isinstance(op, str) else int(op)
    dtc = {"f32": F32, "bf16": BF16, "u8": U8}[dtype] if isinstance(dtype, str) else int(dtype)
    sp = None
    if splits is not None:
        sp_arr = np.ascontiguousarray(np.asarray(splits, dtype=np.int64).reshape(p, p))
        sp = sp_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    count = ctypes.c_int64()
    _check(lib.vcoll_ledger(opc, _algo(algo), p, n, dtc, sp, row_elems, None, 0, ctypes.byref(count),
                            None, None, None), "vcoll_ledger")
    msgs = (Msg * max(1, count.value))()
    sent = (ctypes.c_int64 * p)()
    got = (ctypes.c_int64 * p)()
    steps = ctypes.c_int32()
    _check(lib.vcoll_ledger(opc, _algo(algo), p, n, dtc, sp, row_elems, msgs, count.value,
                            ctypes.byref(count), sent, got, ctypes.byref(steps)), "vcoll_ledger")
    out = [(m.step, m.src, m.dst, m.src_off, m.dst_off, m.count, m.bytes) for m in msgs[:count.value]]
    return out, list(sent), list(got), steps.value


def vcoll_ledger_summary(op, algo, p: int, n: int, dtype: str = "f32", splits=None, row_elems: int = 0):
    """Totals of a collective's ledger without its records: (message count,
    sent bytes per rank, received bytes per rank, step count). One call of
    vcoll_ledger with no record buffer."""
    lib = _lib()
    opc = OPS[op] if isinstance(op, str) else int(op)
    dtc = {"f32": F32, "bf16": BF16, "u8": U8}[dtype] if isinstance(dtype, str) else int(dtype)
    sp = None
    if splits is not None:
        sp_arr = np.ascontiguousarray(np.asarray(splits, dtype=np.int64).reshape(p, p))
        sp = sp_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    count = ctypes.c_int64()
    sent = (ctypes.c_int64 * p)()
    got = (ctypes.c_int64 * p)()
    steps = ctypes.c_int32()
    _check(lib.vcoll_ledger(opc, _algo(algo), p, n, dtc, sp, row_elems, None, 0, ctypes.byref(count),
                            sent, got, ctypes.byref(steps)), "vcoll_ledger")
    return count.value, list(sent), list(got), steps.value


def vcoll_model_formula(algo, p: int, nbytes: float, alpha: float, beta: float) -> float:
    """Closed-form alpha-beta all-reduce time in seconds (see vcoll.h)."""
    t = ctypes.c_double()
    _check(_lib().vcoll_model_formula(_algo(algo), p, float(nbytes), float(alpha), float(beta),
                                      ctypes.byref(t)), "vcoll_model_formula")
    return t.value


def vcoll_model_ledger_time(op, algo, p: int, n: int, alpha: float, beta: float, dtype: str = "f32",
                            splits=None, row_elems: int = 0) -> tuple:
    """Simulated alpha-beta clock over the ledger: (seconds, steps)."""
    opc = OPS[op] if isinstance(op, str) else int(op)
    dtc = {"f32": F32, "bf16": BF16, "u8": U8}[dtype] if isinstance(dtype, str) else int(dtype)
    sp = None
    if splits is not None:
        sp_arr = np.ascontiguousarray(np.asarray(splits, dtype=np.int64).reshape(p, p))
        sp = sp_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    t, steps = ctypes.c_double(), ctypes.c_int32()
    _check(_lib().vcoll_model_ledger_time(opc, _algo(algo), p, n, dtc, sp, row_elems, float(alpha),
                                          float(beta), ctypes.byref(t), ctypes.byref(steps)),
           "vcoll_model_ledger_time")
    return t.value, steps.value


def vcoll_moe_plan(topk_ids: np.ndarray, experts_per_rank: int):
    """topk_ids: int32 [p, tokens, topk]. Returns (splits [p, p] int64,
    src_rows [p, tokens*topk] int32, dst_rows [p, tokens*topk] int32)."""
    ids = np.ascontiguousarray(np.asarray(topk_ids, dtype=np.int32))
    p, tokens, topk = ids.shape
    splits = np.zeros((p, p), dtype=np.int64)
    src = np.zeros((p, tokens * topk), dtype=np.int32)
    dst = np.zeros((p, tokens * topk), dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    _check(_lib().vcoll_moe_plan(p, tokens, topk, experts_per_rank, ids.ctypes.data_as(i32),
                                 splits.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 src.ctypes.data_as(i32), dst.ctypes.data_as(i32)), "vcoll_moe_plan")
    return splits, src, dst


def vcoll_moe_slots(splits, dst_rows, topk: int) -> np.ndarray:
    """Token-major view of a vcoll_moe_plan: int32 [p, tokens*topk, 2]
    (destination rank, destination row) per (token, slot)."""
    sp = np.ascontiguousarray(np.asarray(splits, dtype=np.int64))
    dr = np.ascontiguousarray(np.asarray(dst_rows, dtype=np.int32))
    p, rows = dr.shape
    if rows % topk:
        raise ValueError("vcoll_moe_slots: dst_rows must hold tokens * topk entries per rank")
    slots = np.zeros((p, rows, 2), dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    _check(_lib().vcoll_moe_slots(p, rows // topk, topk, sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  dr.ctypes.data_as(i32), slots.ctypes.data_as(i32)), "vcoll_moe_slots")
    return slots


def vcoll_moe_dispatch(tokens, slots, recv_rows, topk: int, fp8: bool = False, recv=None):
    """Token-major dispatch (see vcoll.h): tokens p tensors [T, hidden];
    slots p int32 GPU tensors [T*topk, 2]; recv_rows the rows each rank
    receives. Returns recv (p tensors; uint8 rows of hidden + hidden//32
    bytes for FP8)."""
    import torch
    t = list(tokens)
    p = len(t)
    T, H = t[0].shape
    dev, dt = t[0].device, t[0].dtype
    for x in t:
        if x.shape != (T, H) or x.dtype != dt or x.device != dev or not x.is_contiguous():
            raise ValueError("vcoll_moe_dispatch: token tables must be contiguous [T, hidden] of one dtype")
    rr = [int(r) for r in recv_rows]
    if recv is None:
        if fp8:
            recv = [torch.empty((rr[j], H + H // 32), dtype=torch.uint8, device=dev) for j in range(p)]
        else:
            recv = [torch.empty((rr[j], H), dtype=dt, device=dev) for j in range(p)]
    r = list(recv)
    orb = H + H // 32 if fp8 else H * t[0].element_size()
    for j in range(p):
        if not r[j].is_contiguous() or r[j].numel() * r[j].element_size() < rr[j] * orb:
            raise ValueError(f"vcoll_moe_dispatch: recv[{j}] holds fewer than {rr[j]} rows")
    s = list(slots)
    for x in s:
        if x.dtype != torch.int32 or x.device != dev or x.numel() < 2 * T * topk:
            raise ValueError("vcoll_moe_dispatch: slots must be int32 GPU tensors of T*topk pairs")
    _no_overlap(t, r, "vcoll_moe_dispatch")
    _disjoint(r, "vcoll_moe_dispatch")
    rows = (ctypes.c_int64 * p)(*rr)
    _check(_lib().vcoll_moe_dispatch(p, T, topk, H, _dtype_code(t[0]), int(bool(fp8)), _ptrs(t), _ptrs(s),
                                     _ptrs(r), rows, _stream(t[0])), "vcoll_moe_dispatch")
    return recv


def vcoll_moe_combine(expert_out, slots, tokens: int, topk: int, out=None):
    """Token-major combine (see vcoll.h): expert_out p tensors [rows_j,
    hidden] in dispatch receive order; slots the dispatch's p int32 GPU
    tensors [tokens*topk, 2]. Returns out (p tensors [tokens*topk, hidden]),
    row t*topk + k of rank i being the expert output of token t's slot k."""
    import torch
    e = list(expert_out)
    p = len(e)
    H = e[0].shape[1]
    dev, dt = e[0].device, e[0].dtype
    for x in e:
        if x.dim() != 2 or x.shape[1] != H or x.dtype != dt or x.device != dev or not x.is_contiguous():
            raise ValueError("vcoll_moe_combine: expert outputs must be contiguous [rows, hidden] of one dtype")
    T = int(tokens)
    if out is None:
        out = [torch.empty((T * topk, H), dtype=dt, device=dev) for _ in range(p)]
    o = list(out)
    if len(o) != p:
        raise ValueError("vcoll_moe_combine: need p output buffers")
    for x in o:
        if x.dtype != dt or not x.is_contiguous() or x.numel() < T * topk * H:
            raise ValueError(f"vcoll_moe_combine: every output must hold {T * topk} rows of {H} {dt}")
    s = list(slots)
    if len(s) != p:
        raise ValueError("vcoll_moe_combine: need p slot tables")
    for x in s:
        if x.dtype != torch.int32 or x.device != dev or not x.is_contiguous() or x.numel() < 2 * T * topk:
            raise ValueError("vcoll_moe_combine: slots must be contiguous int32 GPU tensors of tokens*topk pairs")
    _no_overlap(e, o, "vcoll_moe_combine")
    for i, a in enumerate(o):
        _no_overlap([a], o[i + 1:], "vcoll_moe_combine")
    rows = (ctypes.c_int64 * p)(*[x.shape[0] for x in e])
    _check(_lib().vcoll_moe_combine(p, T, topk, H, _dtype_code(e[0]), _ptrs(e), rows, _ptrs(s), _ptrs(o),
                                    _stream(e[0])), "vcoll_moe_combine")
    return out


def vcoll_moe_plan_dedup(topk_ids: np.ndarray, experts_per_rank: int):
    """Deduplicated dispatch plan (see vcoll.h). Returns (splits_unique [p, p],
    src_unique: list of p int32 arrays (the token of each sent row), expand:
    list of p int32 arrays (for each plain-layout row, the deduplicated row))."""
    ids = np.ascontiguousarray(np.asarray(topk_ids, dtype=np.int32))
    p, tokens, topk = ids.shape
    rows = tokens * topk
    splits = np.zeros((p, p), dtype=np.int64)
    src = np.zeros((p, rows), dtype=np.int32)
    expand = np.zeros((p, p * rows), dtype=np.int32)
    count = np.zeros(p, dtype=np.int64)
    i32, i64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    _check(_lib().vcoll_moe_plan_dedup(p, tokens, topk, experts_per_rank, ids.ctypes.data_as(i32),
                                       splits.ctypes.data_as(i64), src.ctypes.data_as(i32),
                                       expand.ctypes.data_as(i32), count.ctypes.data_as(i64)),
           "vcoll_moe_plan_dedup")
    return (splits, [src[i, :int(splits[i].sum())].copy() for i in range(p)],
            [expand[j, :int(count[j])].copy() for j in range(p)])


def vcoll_moe_expand(recv_unique, expand, out=None):
    """Local expansion of a deduplicated dispatch: out[j][x] = recv_unique[j][expand[j][x]]
    (the diagonal blocks of one all-to-all; no message)."""
    p = len(recv_unique)
    counts = [int(e.numel()) for e in expand]
    return vcoll_all_to_all(recv_unique, np.diag(counts).astype(np.int64), recv=out, src_rows=expand)


def vcoll_moe_dedup_slots(splits_unique, src_unique, tokens: int, topk: int) -> np.ndarray:
    """Token-major form of a deduplicated plan (see vcoll.h): int32
    [p, tokens*topk, 2] for vcoll_moe_dispatch. src_unique: the p arrays of
    vcoll_moe_plan_dedup (each rank's sent rows' tokens)."""
    su = np.ascontiguousarray(np.asarray(splits_unique, dtype=np.int64))
    p = su.shape[0]
    src = np.zeros((p, tokens * topk), dtype=np.int32)
    for i in range(p):
        a = np.asarray(src_unique[i], dtype=np.int32)
        if a.size > tokens * topk:
            raise ValueError("vcoll_moe_dedup_slots: more sent rows than tokens*topk")
        src[i, :a.size] = a
    slots = np.zeros((p, max(1, tokens * topk), 2), dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    _check(_lib().vcoll_moe_dedup_slots(p, tokens, topk, su.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                        src.ctypes.data_as(i32), slots.ctypes.data_as(i32)), "vcoll_moe_dedup_slots")
    return slots[:, :tokens * topk]


def vcoll_moe_expand_slots(unique_rows: int, expand: np.ndarray, topk: int) -> np.ndarray:
    """Token-major form of one rank's expansion (see vcoll.h): int32
    [unique_rows*topk, 2], the plain rows copying each unique row as (0, x)."""
    e = np.ascontiguousarray(np.asarray(expand, dtype=np.int32))
    slots = np.zeros((max(1, unique_rows * topk), 2), dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    _check(_lib().vcoll_moe_expand_slots(unique_rows, topk, e.ctypes.data_as(i32), e.size,
                                         slots.ctypes.data_as(i32)), "vcoll_moe_expand_slots")
    return slots[:unique_rows * topk]


def vcoll_moe_expand_token_major(recv_unique, slots, counts, topk: int, out=None):
    """The expansion of vcoll_moe_expand, reading each unique row once:
    rank j's received unique rows are the token table of a one-rank
    vcoll_moe_dispatch whose slots come from vcoll_moe_expand_slots (int32
    GPU tensors [unique_rows*topk, 2]); counts[j] plain rows are written.
    Equal to vcoll_moe_expand bit for bit."""
    import torch
    u = list(recv_unique)
    p = len(u)
    if out is None:
        out = [torch.empty((int(counts[j]), u[j].shape[1]), dtype=u[j].dtype, device=u[j].device) for j in range(p)]
    _disjoint(list(out), "vcoll_moe_expand_token_major")

    def words(t):
        # byte rows (FP8 payloads) move as 2-byte words: the copy is bitwise
        if t.dtype != torch.uint8:
            return t
        if t.dim() != 2 or t.shape[1] % 2:
            raise ValueError("vcoll_moe_expand_token_major: byte rows must be [rows, even width]")
        return t.view(torch.bfloat16)
    for j in range(p):
        if u[j].shape[0] == 0 or int(counts[j]) == 0:
            continue
        vcoll_moe_dispatch([words(u[j])], [slots[j]], [int(counts[j])], topk, recv=[words(out[j])])
    return out


def vcoll_moe_dispatch_fp8(tokens, splits, src_rows, recv=None):
    """Dispatch bfloat16 token rows quantised to E4M3 with a power-of-two
    scale per 128 elements (see vcoll.h). tokens: p bfloat16 tensors
    [T_i, hidden]; src_rows: p int32 GPU tensors. Returns p uint8 tensors
    [rows_j, hidden + hidden // 32]."""
    import torch
    t = list(tokens)
    p = len(t)
    sp = np.ascontiguousarray(np.asarray(splits, dtype=np.int64).reshape(p, p))
    H = t[0].shape[1]
    dev = t[0].device
    for x in t:
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != H or not x.is_contiguous() or x.device != dev:
            raise ValueError("vcoll_moe_dispatch_fp8: tokens must be contiguous bfloat16 [T, hidden] on one GPU")
    if H % 128:
        raise ValueError("vcoll_moe_dispatch_fp8: hidden must be a multiple of 128")
    orb = H + H // 32
    if recv is None:
        recv = [torch.empty((int(sp[:, j].sum()), orb), dtype=torch.uint8, device=dev) for j in range(p)]
    r = list(recv)
    for j in range(p):
        if r[j].dtype != torch.uint8 or not r[j].is_contiguous() or r[j].numel() < int(sp[:, j].sum()) * orb:
            raise ValueError(f"vcoll_moe_dispatch_fp8: recv[{j}] too small or not contiguous uint8")
    g = list(src_rows)
    for i in range(p):
        if g[i].dtype != torch.int32 or g[i].device != dev or g[i].numel() < int(sp[i].sum()):
            raise ValueError(f"vcoll_moe_dispatch_fp8: src_rows[{i}] must be int32 on the GPU, one per sent row")
    _no_overlap(t, r, "vcoll_moe_dispatch_fp8")
    _disjoint(r, "vcoll_moe_dispatch_fp8")
    rows = (ctypes.c_int64 * p)(*[x.shape[0] for x in t])
    _check(_lib().vcoll_moe_dispatch_fp8(p, H, sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptrs(t), rows,
                                         _ptrs(g), _ptrs(r), _stream(t[0])), "vcoll_moe_dispatch_fp8")
    return recv


BENCH_KINDS = {"copy": 0, "read": 1, "write": 2, "copy_plain": 3}


def vcoll_bench_copy(dst, src) -> None:
    """Streaming copy of src into dst (equal byte sizes, 16-byte multiple)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("vcoll_bench_copy: size mismatch")
    _check(_lib().vcoll_bench_copy(_dptr(dst), _dptr(src), nbytes, _stream(src)),
           "vcoll_bench_copy")


def _bench_stream_args(kind: str, dst, src):
    if kind not in BENCH_KINDS:
        raise ValueError(f"vcoll_bench_stream: unknown kind {kind!r}")
    ref = src if kind != "write" else dst
    nbytes = ref.numel() * ref.element_size()
    if kind in ("copy", "copy_plain") and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("vcoll_bench_stream: size mismatch")
    if kind in ("copy", "copy_plain"):
        _no_overlap([dst], [src], "vcoll_bench_stream")
    return (BENCH_KINDS[kind], _dptr(dst), _dptr(src) if src is not None else None, nbytes, _stream(ref))


def vcoll_bench_stream(kind: str, dst, src=None) -> None:
    """One streaming pass: 'copy' / 'copy_plain' src -> dst, 'read' src (dst:
    a small sink tensor), 'write' dst."""
    _check(_lib().vcoll_bench_stream(*_bench_stream_args(kind, dst, src)), "vcoll_bench_stream")


class PreparedCall:
    """A collective whose arguments were validated and marshalled once; each
    call enqueues it again on the stream captured at preparation."""

    def __init__(self, name: str, fn, args: tuple, keep: tuple):
        self._name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self) -> None:
        _check(self._fn(*self._args), self._name)


def prepare_allreduce(algo, send, recv) -> PreparedCall:
    s, r = _ranks(send), _ranks(recv)
    vcoll_allreduce(algo, send, recv)            # validates (and runs) once
    sp, rp = _ptrs(s), _ptrs(r)
    args = (_algo(algo), len(s), s[0].numel(), _dtype_code(s[0]), sp, rp, _stream(s[0]))
    return PreparedCall("vcoll_allreduce", _lib().vcoll_allreduce, args, (send, recv, sp, rp))


def prepare_allreduce_hierarchical(nodes: int, local: int, send, recv) -> PreparedCall:
    s, r = _ranks(send), _ranks(recv)
    vcoll_allreduce_hierarchical(nodes, local, send, recv)
    sp, rp = _ptrs(s), _ptrs(r)
    args = (nodes, local, s[0].numel(), _dtype_code(s[0]), sp, rp, _stream(s[0]))
    return PreparedCall("vcoll_allreduce_hierarchical", _lib().vcoll_allreduce_hierarchical, args,
                        (send, recv, sp, rp))


def prepare_broadcast(send, recv, root: int = 0) -> PreparedCall:
    r = _ranks(recv)
    vcoll_broadcast(send, recv, root)
    rp = _ptrs(r)
    args = (len(r), r[0].numel(), _dtype_code(send), root, send.data_ptr(), rp, _stream(send))
    return PreparedCall("vcoll_broadcast", _lib().vcoll_broadcast, args, (send, recv, rp))


def prepare_reduce(send, recv, root: int = 0) -> PreparedCall:
    s = _ranks(send)
    vcoll_reduce(send, recv, root)
    sp = _ptrs(s)
    args = (BINARY_TREE, len(s), s[0].numel(), _dtype_code(s[0]), root, sp, recv.data_ptr(), _stream(s[0]))
    return PreparedCall("vcoll_reduce", _lib().vcoll_reduce, args, (send, recv, sp))


def prepare_reduce_scatter(algo, send, recv) -> PreparedCall:
    s, r = _ranks(send), list(recv)
    vcoll_reduce_scatter(algo, send, recv)
    sp, rp = _ptrs(s), _ptrs(r)
    args = (_algo(algo), len(s), s[0].numel(), _dtype_code(s[0]), sp, rp, _stream(s[0]))
    return PreparedCall("vcoll_reduce_scatter", _lib().vcoll_reduce_scatter, args, (send, recv, sp, rp))


def prepare_all_gather(algo, send, recv) -> PreparedCall:
    s, r = _ranks(send), _ranks(recv)
    vcoll_all_gather(algo, send, recv)
    sp, rp = _ptrs(s), _ptrs(r)
    args = (_algo(algo), len(s), s[0].numel(), _dtype_code(s[0]), sp, rp, _stream(s[0]))
    return PreparedCall("vcoll_all_gather", _lib().vcoll_all_gather, args, (send, recv, sp, rp))


def prepare_bench_copy(dst, src) -> PreparedCall:
    vcoll_bench_copy(dst, src)
    args = (dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(), _stream(src))
    return PreparedCall("vcoll_bench_copy", _lib().vcoll_bench_copy, args, (dst, src))


def prepare_bench_stream(kind: str, dst, src=None) -> PreparedCall:
    vcoll_bench_stream(kind, dst, src)
    return PreparedCall("vcoll_bench_stream", _lib().vcoll_bench_stream, _bench_stream_args(kind, dst, src),
                        (dst, src))


def prepare_allreduce_stepwise(algo, send, recv, workspace=None) -> PreparedCall:
    import torch
    s, r = _ranks(send), _ranks(recv)
    n = s[0].numel()
    if _dtype_code(s[0]) == BF16 and workspace is None:
        workspace = torch.empty(len(s) * n, dtype=torch.float32, device=s[0].device)
    vcoll_allreduce_stepwise(algo, send, recv, workspace)      # validates (and runs) once
    sp, rp = _ptrs(s), _ptrs(r)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * 4 if workspace is not None else 0
    args = (_algo(algo), len(s), n, _dtype_code(s[0]), sp, rp, ws_ptr, ws_bytes, None, _stream(s[0]))
    return PreparedCall("vcoll_allreduce_stepwise", _lib().vcoll_allreduce_stepwise, args,
                        (send, recv, workspace, sp, rp))
