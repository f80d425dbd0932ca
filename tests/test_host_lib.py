"""Host-side checks of libvcoll that need no GPU.

The library loads on a machine without a GPU; these tests call only its host
entry points (ledger, chunk bounds, MoE plan) and its argument validation,
which rejects bad calls before any device work is attempted.
"""
import ctypes
import re
import os

import numpy as np
import pytest

import oracle
import workloads

vc = pytest.importorskip("collective_communication_algorithms_vcoll_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALGOS = oracle.ALGOS
PS = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 72]


def declared_functions():
    names = []
    for h in ("vcoll.h", "vcoll_bench.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        names += re.findall(r"^(?:[a-z_]+\s*\*?\s+)(vcoll_[a-z_]+)\(", text, flags=re.M)
        names += re.findall(r"^const char\*\s+(vcoll_[a-z_]+)\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "vcoll_allreduce" in names and "vcoll_ledger" in names and "vcoll_moe_plan" in names
    lib = ctypes.CDLL(vc.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.vcoll_abi_version() == 1


def _oracle_ledger(op, algo, p, n, dtype="f32"):
    if op == "allreduce":
        x = [np.zeros(1, dtype=np.float32 if dtype == "f32" else np.uint16)] * p
        _, led = oracle.allreduce(x, algo, dtype, n=n, lo=0)
    elif op == "reduce_scatter":
        x = [np.zeros(1, dtype=np.float32)] * p
        _, led = oracle.reduce_scatter(x, algo, dtype, n=n, lo=0)
    else:
        x = [np.zeros(n, dtype=np.float32) for _ in range(p)]
        _, led = oracle.all_gather(x, algo, dtype)
    return led


@pytest.mark.parametrize("p", PS)
@pytest.mark.parametrize("algo", ALGOS)
def test_allreduce_ledger_matches_oracle(p, algo):
    for n in (0, 1, p, 3 * p + 2, 1000):
        for dtype in ("f32", "bf16"):
            led = _oracle_ledger("allreduce", algo, p, n, dtype)
            msgs, sent, got, steps = vc.vcoll_ledger("allreduce", algo, p, n, dtype)
            assert msgs == [tuple(m) for m in led.sorted()], (p, algo, n, dtype)
            assert sent == led.sent_bytes() and got == led.recv_bytes()
            assert steps == led.n_steps


@pytest.mark.parametrize("p", PS)
def test_reduce_scatter_and_all_gather_ledgers_match_oracle(p):
    for n in (1, p, 5 * p + 3):
        led = _oracle_ledger("reduce_scatter", "ring", p, n)
        msgs, sent, _, steps = vc.vcoll_ledger("reduce_scatter", "ring", p, n)
        assert msgs == [tuple(m) for m in led.sorted()] and steps == led.n_steps
        led = _oracle_ledger("all_gather", "ring", p, n)
        msgs, sent, _, steps = vc.vcoll_ledger("all_gather", "ring", p, n)
        assert msgs == [tuple(m) for m in led.sorted()] and steps == led.n_steps
        if p & (p - 1) == 0:
            led = _oracle_ledger("reduce_scatter", "rabenseifner", p, n)
            msgs, _, _, _ = vc.vcoll_ledger("reduce_scatter", "rabenseifner", p, n)
            assert msgs == [tuple(m) for m in led.sorted()]
            led = _oracle_ledger("all_gather", "rd", p, n)
            msgs, _, _, _ = vc.vcoll_ledger("all_gather", "rd", p, n)
            assert msgs == [tuple(m) for m in led.sorted()]


@pytest.mark.parametrize("p", [1, 2, 3, 8, 16])
def test_all_to_all_ledger_matches_oracle(p):
    rng = np.random.default_rng(p)
    splits = rng.integers(0, 6, size=(p, p))
    H = 5
    send = [np.zeros((int(splits[i].sum()), H), dtype=np.uint16) for i in range(p)]
    _, led = oracle.all_to_all(send, splits, "bf16")
    msgs, sent, got, steps = vc.vcoll_ledger("all_to_all", "ring", p, 0, "bf16", splits=splits, row_elems=H)
    assert msgs == [tuple(m) for m in led.sorted()]
    assert sent == led.sent_bytes() and got == led.recv_bytes() and steps == led.n_steps


def test_headline_ledger_closed_form():
    msgs, sent, got, steps = vc.vcoll_ledger("allreduce", "ring", 8, 6_553_600, "f32")
    assert sent == [45_875_200] * 8 and got == sent and steps == 14 and len(msgs) == 112
    msgs, sent, _, steps = vc.vcoll_ledger("allreduce", "rabenseifner", 16, 100_663_296, "bf16")
    assert sent == [377_487_360] * 16 and steps == 8
    msgs, sent, _, steps = vc.vcoll_ledger("allreduce", "ring", 16, 100_663_296, "bf16")
    assert sent == [377_487_360] * 16 and steps == 30


@pytest.mark.parametrize("op,algo,p", [("allreduce", "ring", 8), ("allreduce", "rabenseifner", 72),
                                       ("allreduce", "tree", 5), ("reduce_scatter", "ring", 16),
                                       ("all_gather", "rd", 4)])
def test_ledger_summary_equals_the_records(op, algo, p):
    """The record-free ledger call gives the totals of the full ledger."""
    n = 1000 * p + 7
    msgs, sent, got, steps = vc.vcoll_ledger(op, algo, p, n)
    assert vc.vcoll_ledger_summary(op, algo, p, n) == (len(msgs), sent, got, steps)

@pytest.mark.parametrize("p,n", [(1, 0), (1, 5), (4, 3), (8, 6_553_600), (72, 1000), (128, 129)])
def test_chunk_bounds_match_oracle(p, n):
    offs = oracle.chunk_bounds(n, p)
    for c in range(p):
        assert vc.vcoll_chunk(p, n, c) == (offs[c], offs[c + 1] - offs[c])


def test_moe_plan_matches_oracle():
    p, T, E, K = 8, 512, 256, 8
    topk = [workloads.moe_topk(r, T, E, K) for r in range(p)]
    splits, src, dst = vc.vcoll_moe_plan(np.stack(topk), E // p)
    o_splits, o_src, o_dst = oracle.moe_plan(topk, E // p)
    assert np.array_equal(splits, o_splits)
    for i in range(p):
        assert np.array_equal(src[i], o_src[i]) and np.array_equal(dst[i], o_dst[i])


def test_moe_plan_rejects_bad_expert_ids():
    ids = np.zeros((2, 4, 2), dtype=np.int32)
    ids[1, 2, 1] = 99
    with pytest.raises(vc.VcollError) as e:
        vc.vcoll_moe_plan(ids, 4)
    assert e.value.status == 1


# ------------------------------------------------------------- validation (no launch happens)

def _lib():
    return vc._lib()


def _ptrs(p, value=0x1000):
    arr = (ctypes.c_void_p * p)()
    for i in range(p):
        arr[i] = value + 256 * i
    return arr


@pytest.mark.parametrize("fn", ["vcoll_allreduce", "vcoll_reduce_scatter", "vcoll_all_gather"])
def test_reduce_validation_errors(fn):
    f = getattr(_lib(), fn)
    ok_algo = 0
    # p out of range, negative n, bad dtype, bad algo, NULL pointers
    assert f(ok_algo, 0, 8, 0, _ptrs(1), _ptrs(1), None) == 1
    assert f(ok_algo, 129, 8, 0, _ptrs(129), _ptrs(129), None) == 1
    assert f(ok_algo, 4, -1, 0, _ptrs(4), _ptrs(4), None) == 1
    assert f(ok_algo, 4, 8, 7, _ptrs(4), _ptrs(4), None) == 1
    assert f(9, 4, 8, 0, _ptrs(4), _ptrs(4), None) == 1
    assert f(ok_algo, 4, 8, 0, None, _ptrs(4), None) == 1
    holes = _ptrs(4)
    holes[2] = None
    assert f(ok_algo, 4, 8, 0, _ptrs(4), holes, None) == 1
    # n == 0 is a no-op and never touches the pointers
    assert f(ok_algo, 4, 0, 0, None, None, None) == 0


def test_unsupported_combinations():
    lib = _lib()
    P = _ptrs(8)
    assert lib.vcoll_reduce_scatter(1, 8, 64, 0, P, P, None) == 2      # RS + recursive doubling
    assert lib.vcoll_reduce_scatter(3, 8, 64, 0, P, P, None) == 2      # RS + tree
    assert lib.vcoll_reduce_scatter(2, 6, 64, 0, P, P, None) == 2      # RS + Rabenseifner, p = 6
    assert lib.vcoll_all_gather(2, 8, 64, 0, P, P, None) == 2          # AG + Rabenseifner
    assert lib.vcoll_all_gather(3, 8, 64, 0, P, P, None) == 2          # AG + tree
    assert lib.vcoll_all_gather(1, 6, 64, 0, P, P, None) == 2          # AG + RD, p = 6
    with pytest.raises(vc.VcollError):
        vc.vcoll_ledger("reduce_scatter", "rd", 8, 64)


def test_all_to_all_validation_errors():
    lib = _lib()
    p = 3
    sp = (ctypes.c_int64 * 9)(*([1] * 9))
    P = _ptrs(p)
    tab = (ctypes.c_int64 * p)(1, 1, 1)
    assert lib.vcoll_all_to_all(p, 4, 0, None, P, P, None, tab, None, tab, None) == 1   # no splits
    neg = (ctypes.c_int64 * 9)(*([1] * 8 + [-1]))
    assert lib.vcoll_all_to_all(p, 4, 0, neg, P, P, None, tab, None, tab, None) == 1
    assert lib.vcoll_all_to_all(p, -4, 0, sp, P, P, None, tab, None, tab, None) == 1
    holes = _ptrs(p)
    holes[1] = None
    assert lib.vcoll_all_to_all(p, 4, 0, sp, holes, P, None, tab, None, tab, None) == 1
    gather = (ctypes.c_void_p * p)(0x2000, None, None)
    assert lib.vcoll_all_to_all(p, 4, 0, sp, P, P, gather, None, None, tab, None) == 1   # no table rows
    zero = (ctypes.c_int64 * 9)()
    assert lib.vcoll_all_to_all(p, 4, 0, zero, None, None, None, None, None, None, None) == 0


def test_ledger_two_call_protocol_and_errors():
    lib = _lib()
    n = ctypes.c_int64()
    assert lib.vcoll_ledger(0, 0, 4, 16, 0, None, 0, None, 0, ctypes.byref(n), None, None, None) == 0
    assert n.value == 24
    small = (vc.Msg * 3)()
    assert lib.vcoll_ledger(0, 0, 4, 16, 0, None, 0, small, 3, ctypes.byref(n), None, None, None) == 3
    assert n.value == 24
    assert lib.vcoll_ledger(0, 0, 0, 16, 0, None, 0, None, 0, ctypes.byref(n), None, None, None) == 1
    assert lib.vcoll_ledger(3, 0, 4, 16, 0, None, 0, None, 0, ctypes.byref(n), None, None, None) == 1
    assert lib.vcoll_ledger(0, 0, 4, 16, 0, None, 0, None, 0, None, None, None, None) == 1


def test_chunk_validation():
    with pytest.raises(vc.VcollError):
        vc.vcoll_chunk(4, 10, 4)
    with pytest.raises(vc.VcollError):
        vc.vcoll_chunk(0, 10, 0)


def test_status_strings():
    lib = _lib()
    for s in range(5):
        assert lib.vcoll_status_str(s)
    assert lib.vcoll_status_str(42) == b"unknown status"


def test_one_hip_runtime_in_the_process():
    # torch bundles its own HIP runtime under the same soname as the system
    # one; libvcoll must bind to the copy torch uses, never load a second one
    import torch  # noqa: F401
    vc._lib()
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    assert len(paths) == 1, paths


def test_stepwise_validation():
    lib = _lib()
    P = _ptrs(4)
    # bf16 needs a float32 workspace of p*n*4 bytes
    assert lib.vcoll_allreduce_stepwise(0, 4, 16, 1, P, P, None, 0, None, None) == 1
    assert lib.vcoll_allreduce_stepwise(0, 4, 16, 1, P, P, 0x9000, 4 * 16 * 4 - 1, None, None) == 3
    assert lib.vcoll_allreduce_stepwise(0, 0, 16, 0, P, P, None, 0, None, None) == 1
    assert lib.vcoll_allreduce_stepwise(5, 4, 16, 0, P, P, None, 0, None, None) == 1
    assert lib.vcoll_allreduce_stepwise(0, 4, 0, 0, None, None, None, 0, None, None) == 0


def test_overlap_check_allows_in_place_and_rejects_cross_overlap():
    import torch
    t = torch.zeros(4, 16)
    other = torch.zeros(4, 16)
    rows = [t[r] for r in range(4)]
    vc._no_overlap(rows, rows, "x", same_index_ok=True)                 # in place
    vc._no_overlap(rows, [other[r] for r in range(4)], "x")              # disjoint
    with pytest.raises(ValueError):
        vc._no_overlap(rows, [t[1], t[0], t[2], t[3]], "x", same_index_ok=True)   # rank 0 writes rank 1's input
    with pytest.raises(ValueError):
        vc._no_overlap(rows, rows, "x")                                   # in place not allowed here
    flat = torch.zeros(64)
    with pytest.raises(ValueError):
        vc._no_overlap([flat[0:16]], [flat[8:24]], "x")                   # partial overlap
    big = [torch.zeros(8) for _ in range(128)]
    vc._no_overlap(big[:64], big[64:], "x")                               # many disjoint buffers


def test_outputs_must_not_overlap_each_other():
    import torch
    t = torch.zeros(4, 16)
    vc._disjoint([t[r] for r in range(4)], "x")                          # rows of one tensor
    vc._disjoint([t[0], torch.zeros(0), t[1]], "x")                      # empty buffers are ignored
    with pytest.raises(ValueError, match="output buffers overlap"):
        vc._disjoint([t[0], t[1], t[0]], "x")                             # one buffer twice
    flat = torch.zeros(64)
    with pytest.raises(ValueError, match="output buffers overlap"):
        vc._disjoint([flat[0:16], flat[32:48], flat[15:20]], "x")         # one element shared
    vc._disjoint([flat[0:16], flat[16:32]], "x")                          # adjacent, not shared


def test_debug_flag_is_read_from_the_environment():
    """VCOLL_DEBUG=1 turns on a device synchronization after every call; a
    host-only call in a process that never touched the GPU must still work."""
    import subprocess
    import sys
    code = ("import collective_communication_algorithms_vcoll_amd as vc; assert vc._DEBUG; "
            "assert vc.vcoll_chunk(4, 10, 1) == (3, 3); print('ok')")
    env = dict(os.environ, VCOLL_DEBUG="1", PYTHONPATH=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr[-2000:]


def test_widened_entry_points_validate_before_launching():
    """Every error below is returned before anything is enqueued (no GPU here)."""
    lib = _lib()
    P8 = _ptrs(8)
    one = ctypes.c_void_p(0x1000)
    # broadcast: root out of range, bad dtype, missing receive buffer
    assert lib.vcoll_broadcast(8, 64, 0, 8, one, P8, None) == 1
    assert lib.vcoll_broadcast(8, 64, 5, 0, one, P8, None) == 1
    holes = _ptrs(8)
    holes[3] = None
    assert lib.vcoll_broadcast(8, 64, 0, 0, one, holes, None) == 1
    assert lib.vcoll_broadcast(8, 0, 0, 0, None, None, None) == 0                # n = 0: no-op
    # reduce: only the binomial tree; root range; NULL output
    assert lib.vcoll_reduce(0, 8, 64, 0, 0, P8, one, None) == 2
    assert lib.vcoll_reduce(3, 8, 64, 0, 8, P8, one, None) == 1
    assert lib.vcoll_reduce(3, 8, 64, 0, 0, P8, None, None) == 1
    assert lib.vcoll_reduce(99, 8, 64, 0, 0, P8, one, None) == 1
    # hierarchical: shapes
    assert lib.vcoll_allreduce_hierarchical(0, 8, 64, 0, P8, P8, None) == 1
    assert lib.vcoll_allreduce_hierarchical(16, 16, 64, 0, _ptrs(256), _ptrs(256), None) == 1
    assert lib.vcoll_allreduce_hierarchical(2, 4, 64, 2, P8, P8, None) == 1     # U8 is for the all-to-all only
    # nodes x local would wrap around int: each factor is bounded on its own
    n = ctypes.c_int64()
    for nodes, local in ((4, 2 ** 30 + 1), (65536, 65536), (2 ** 30 + 1, 4)):
        assert lib.vcoll_allreduce_hierarchical(nodes, local, 64, 0, P8, P8, None) == 1
        assert lib.vcoll_ledger_hierarchical(nodes, local, 64, 0, None, 0, ctypes.byref(n), None, None, None) == 1
        t = ctypes.c_double()
        assert lib.vcoll_model_ledger_time_nodes(1, 0, nodes, local, 64, 0, 1e-6, 1e9, 1e-6, 1e9,
                                                 ctypes.byref(t), None) == 1
    # tokens x topk would overflow int64: refused by division, before the product
    ids = (ctypes.c_int32 * 8)()
    out64 = (ctypes.c_int64 * 4)()
    out32 = (ctypes.c_int32 * 8)()
    assert lib.vcoll_moe_plan(2, 1 << 48, 2 ** 31 - 1, 4, ids, out64, out32, out32) == 1
    assert lib.vcoll_moe_slots(2, 1 << 48, 2 ** 31 - 1, out64, out32, out32) == 1
    assert lib.vcoll_moe_expand_slots(1 << 48, 2 ** 31 - 1, out32, 1, out32) == 1
    # the all-to-all takes raw bytes, the reductions do not
    assert lib.vcoll_allreduce(0, 8, 64, 2, P8, P8, None) == 1
    # FP8 dispatch: hidden must be a positive multiple of 128; token tables aligned
    sp = (ctypes.c_int64 * 4)(1, 0, 0, 1)
    rows = (ctypes.c_int64 * 2)(4, 4)
    idx = (ctypes.c_void_p * 2)(0x3000, 0x3000)
    assert lib.vcoll_moe_dispatch_fp8(2, 100, sp, _ptrs(2), rows, idx, _ptrs(2), None) == 1
    unaligned = (ctypes.c_void_p * 2)(0x1008, 0x2000)
    assert lib.vcoll_moe_dispatch_fp8(2, 128, sp, unaligned, rows, idx, _ptrs(2), None) == 1
    # token-major dispatch: FP8 needs bf16 and hidden % 128 == 0
    rr = (ctypes.c_int64 * 2)(1, 1)
    assert lib.vcoll_moe_dispatch(2, 4, 1, 100, 1, 1, _ptrs(2), idx, _ptrs(2), rr, None) == 1
    assert lib.vcoll_moe_dispatch(2, 4, 1, 128, 0, 1, _ptrs(2), idx, _ptrs(2), rr, None) == 1
    bad_rows = (ctypes.c_int64 * 2)(-1, 1)
    assert lib.vcoll_moe_dispatch(2, 4, 1, 128, 1, 0, _ptrs(2), idx, _ptrs(2), bad_rows, None) == 1
    # models
    t = ctypes.c_double()
    assert lib.vcoll_model_chain_optimum(2, 1e6, 1e-6, 1e9, ctypes.byref(t), ctypes.byref(t)) == 1
    assert lib.vcoll_model_broadcast_formula(6, 8, 1e6, 0, 1e-6, 1e9, ctypes.byref(t)) == 1   # chain, 0 blocks
    assert lib.vcoll_model_clock(None, 3, 8, 8, 1e-6, 1e9, 1e-6, 1e9, ctypes.byref(t)) == 1


def test_static_stepwise_refuses_sizes_beyond_its_scratch_array():
    """vcoll_allreduce_stepwise_static keeps bf16 partial sums in the
    library's own 64 MiB array: a call needing more is refused before any
    HIP call (so this runs without a GPU), and n = 0 is a no-op."""
    lib = _lib()
    P8 = _ptrs(8)
    launches = ctypes.c_int32(-1)
    over = (64 * 2 ** 20) // (8 * 4) + 1
    assert lib.vcoll_allreduce_stepwise_static(0, 8, over, 1, P8, P8, ctypes.byref(launches), None) == 5
    assert launches.value == 0
    assert lib.vcoll_allreduce_stepwise_static(0, 8, 1 << 48, 1, P8, P8, None, None) == 5
    assert lib.vcoll_allreduce_stepwise_static(0, 8, 0, 1, None, None, None, None) == 0
    assert lib.vcoll_allreduce_stepwise_static(0, 129, 10, 1, P8, P8, None, None) == 1
    assert b"static scratch" in lib.vcoll_status_str(5)


def test_stepwise_broadcast_validation():
    """vcoll_broadcast_stepwise checks its schedule before any launch (no GPU
    needed): the algorithm must be a broadcast one, the chain needs 1..65536
    blocks, the root must be a rank; n = 0 is a no-op."""
    lib = _lib()
    P8 = _ptrs(8)
    one = ctypes.c_void_p(0x1000)
    launches = ctypes.c_int32(-1)
    assert lib.vcoll_broadcast_stepwise(0, 8, 64, 0, 0, 1, one, P8, ctypes.byref(launches), None) == 2   # ring
    assert launches.value == 0
    assert lib.vcoll_broadcast_stepwise(6, 8, 64, 0, 0, 0, one, P8, None, None) == 1        # chain, 0 blocks
    assert lib.vcoll_broadcast_stepwise(6, 8, 64, 0, 0, 65537, one, P8, None, None) == 1
    assert lib.vcoll_broadcast_stepwise(3, 8, 64, 0, 8, 1, one, P8, None, None) == 1        # root out of range
    assert lib.vcoll_broadcast_stepwise(3, 8, 64, 2, 0, 1, one, P8, None, None) == 1        # U8
    assert lib.vcoll_broadcast_stepwise(3, 8, 0, 0, 0, 1, None, None, None, None) == 0      # n = 0
    holes = _ptrs(8)
    holes[5] = None
    assert lib.vcoll_broadcast_stepwise(4, 8, 64, 0, 0, 1, one, holes, None, None) == 1


def test_oversized_counts_and_buffers_are_refused():
    """Element counts above 2^48 and buffers above 2^56 bytes are refused
    before anything is enqueued, so no byte offset can overflow int64."""
    lib = _lib()
    P8 = _ptrs(8)
    one = ctypes.c_void_p(0x1000)
    big = (1 << 48) + 1
    assert lib.vcoll_allreduce(0, 8, big, 0, P8, P8, None) == 1
    assert lib.vcoll_reduce_scatter(0, 8, big, 0, P8, P8, None) == 1
    assert lib.vcoll_all_gather(0, 8, big, 0, P8, P8, None) == 1
    assert lib.vcoll_broadcast(8, big, 0, 0, one, P8, None) == 1
    assert lib.vcoll_reduce(3, 8, big, 0, 0, P8, one, None) == 1
    assert lib.vcoll_allreduce_hierarchical(2, 4, big, 0, P8, P8, None) == 1
    ws = ctypes.c_void_p(0x4000)
    assert lib.vcoll_allreduce_stepwise(0, 8, big, 1, P8, P8, ws, ctypes.c_int64(1 << 62), None, None) == 1
    n = ctypes.c_int64()
    assert lib.vcoll_ledger(0, 0, 8, big, 0, None, 0, None, 0, ctypes.byref(n), None, None, None) == 1
    # all-to-all: rows x row bytes above 2^56 (each factor within its own bound)
    sp = (ctypes.c_int64 * 4)(1 << 21, 0, 0, 1)
    P2 = _ptrs(2)
    assert lib.vcoll_all_to_all(2, 1 << 35, 1, sp, P2, P2, None, None, None, None, None) == 1
    assert lib.vcoll_all_to_all(2, big, 2, sp, P2, P2, None, None, None, None, None) == 1
    # the all-to-all ledger takes the same split limits as the all-to-all:
    # a block or a rank's total beyond INT32_MAX rows, or beyond 2^56 bytes
    for bad in ((1 << 62, 0, 0, 1), (2 ** 31 - 1, 1, 0, 1), (1 << 21, 0, 0, 1)):
        spb = (ctypes.c_int64 * 4)(*bad)
        assert lib.vcoll_ledger(3, 0, 2, 0, 1, spb, 1 << 35, None, 0, ctypes.byref(n), None, None, None) == 1
        assert lib.vcoll_all_to_all(2, 1 << 35, 1, spb, P2, P2, None, None, None, None, None) == 1
    assert lib.vcoll_ledger(3, 0, 2, 0, 1, sp, 1, None, 0, ctypes.byref(n), None, None, None) == 0
    # token-major dispatch: tokens x row bytes above 2^56
    idx = (ctypes.c_void_p * 2)(0x3000, 0x3000)
    rr = (ctypes.c_int64 * 2)(1, 1)
    assert lib.vcoll_moe_dispatch(2, 1 << 30, 1, 1 << 26, 0, 0, P2, idx, P2, rr, None) == 1
    # FP8 dispatch: hidden beyond the row bound
    rows = (ctypes.c_int64 * 2)(4, 4)
    sp1 = (ctypes.c_int64 * 4)(1, 0, 0, 1)
    assert lib.vcoll_moe_dispatch_fp8(2, 1 << 40, sp1, P2, rows, idx, P2, None) == 1


def test_binding_refuses_host_tensors_before_calling_the_library():
    """Host (CPU) tensors never reach a kernel: every entry point that takes
    device buffers refuses them, including the MoE paths whose tensors are
    only compared with one another."""
    import torch
    toks = [torch.zeros((4, 128), dtype=torch.bfloat16) for _ in range(2)]
    splits = np.array([[2, 2], [2, 2]])
    idx = [torch.zeros(4, dtype=torch.int32) for _ in range(2)]
    with pytest.raises(ValueError):
        vc.vcoll_all_to_all(toks, splits)
    with pytest.raises(ValueError):
        vc.vcoll_moe_dispatch_fp8(toks, splits, idx)
    slots = [torch.zeros((4, 2), dtype=torch.int32) for _ in range(2)]
    with pytest.raises(ValueError):
        vc.vcoll_moe_dispatch(toks, slots, [4, 4], 1)
    with pytest.raises(ValueError):
        vc.vcoll_allreduce("ring", torch.zeros((2, 64)))
    with pytest.raises(ValueError):
        vc.vcoll_bench_copy(torch.zeros(16), torch.zeros(16))


def test_combine_validates_before_launching():
    lib = _lib()
    P2 = _ptrs(2)
    rows = (ctypes.c_int64 * 2)(4, 4)
    idx = (ctypes.c_void_p * 2)(0x3000, 0x3000)
    assert lib.vcoll_moe_combine(2, 4, 1, 64, 7, P2, rows, idx, P2, None) == 1          # bad dtype
    assert lib.vcoll_moe_combine(2, 4, 0, 64, 0, P2, rows, idx, P2, None) == 1          # topk 0
    assert lib.vcoll_moe_combine(2, 4, 1, 64, 0, P2, None, idx, P2, None) == 1          # no row counts
    bad = (ctypes.c_int64 * 2)(-1, 4)
    assert lib.vcoll_moe_combine(2, 4, 1, 64, 0, P2, bad, idx, P2, None) == 1
    holes = _ptrs(2)
    holes[1] = None
    assert lib.vcoll_moe_combine(2, 4, 1, 64, 0, holes, rows, idx, P2, None) == 1     # missing expert buffer
    assert lib.vcoll_moe_combine(2, 4, 1, 64, 0, P2, rows, idx, holes, None) == 1     # missing output
    assert lib.vcoll_moe_combine(2, 1 << 30, 1, 1 << 26, 0, P2, rows, idx, P2, None) == 1  # > 2^56 bytes
    assert lib.vcoll_moe_combine(2, 0, 1, 64, 0, None, rows, None, None, None) == 0   # no tokens: no-op
