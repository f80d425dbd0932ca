"""Planted mistakes: each test copies the oracle package, plants one
plausible mistake in the copy's source (on the CPU, never in the real
oracle), and checks that the battery of pins -- the pages' worked example,
the hand-derived order probes, integer sums, the all-reduce = reduce-scatter
+ all-gather identity, the ledger closed forms, the all-to-all worked example
and round trip, and bfloat16 rounding against torch -- catches it, while the
unmodified oracle passes the same battery."""
import importlib
import json
import os
import shutil
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = json.load(open(os.path.join(ROOT, "tests", "golden", "order_probes.json")))
ALGOS = ("ring", "rd", "rabenseifner", "tree")

# (name, file, text in the oracle, planted replacement)
MUTANTS = [
    ("ring sends to the predecessor", "collectives.py",
     "            c = (i - 1 - s) % p\n            sends.append(Send(i, (i + 1) % p,",
     "            c = (i - 1 - s) % p\n            sends.append(Send(i, (i - 1) % p,"),
    ("ring reduce-scatter chunk index off by one", "collectives.py",
     "            c = (i - 1 - s) % p\n", "            c = (i - s) % p\n"),
    ("ring all-gather chunk index off by one", "collectives.py",
     "            c = (i - s) % p\n            sends.append(Send(i, (i + 1) % p, offs[c], offs[c], offs[c + 1] - offs[c], COPY))",
     "            c = (i - 1 - s) % p\n            sends.append(Send(i, (i + 1) % p, offs[c], offs[c], offs[c + 1] - offs[c], COPY))"),
    ("Rabenseifner halves at distance 1 first", "collectives.py",
     "    d = p2 // 2\n    while d >= 1:\n        sends = []\n        for nr in range(p2):\n            base = nr & ~(2 * d - 1)",
     "    d = 1\n    while d < p2:\n        sends = []\n        for nr in range(p2):\n            base = nr & ~(2 * d - 1)"),
    ("recursive doubling pairs by shift instead of xor", "collectives.py",
     "old(nr ^ (1 << k))", "old((nr + (1 << k)) % p2)"),
    ("fold pairs odd into even", "collectives.py",
     "Send(2 * j, 2 * j + 1, 0, 0, n, ADD)", "Send(2 * j + 1, 2 * j, 0, 0, n, ADD)"),
    ("binomial reduce with masks descending", "collectives.py",
     "    masks = _masks(p)\n    for m in masks:", "    masks = _masks(p)\n    for m in reversed(masks):"),
    ("bfloat16 narrowing truncates", "numerics.py",
     "((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16))", "((u) >> np.uint64(16))"),
    ("all-to-all receiver uses the sender's block offset", "collectives.py",
     "s0, r0, k = send_off[i, j], recv_off[i, j], splits[i, j]",
     "s0, r0, k = send_off[i, j], send_off[j, i], splits[i, j]"),
    ("ring ledger forgets the chunk size", "cluster.py",
     "m.bytes", "m.count"),
]


# a mistake that needs a second edit to stay a terminating program
FOLLOW_UPS = {
    "Rabenseifner halves at distance 1 first": ("collectives.py", "        step += 1\n        d //= 2\n    return step",
                                                "        step += 1\n        d *= 2\n    return step"),
}


def load_copy(tmp_path, name, patch=None, follow_up=None):
    """Import a copy of the oracle package under another name, optionally
    with textual changes."""
    dst = tmp_path / name
    shutil.copytree(os.path.join(ROOT, "oracle"), dst)
    for change in (patch, follow_up):
        if not change:
            continue
        fname, old, new = change
        path = dst / fname
        text = path.read_text()
        assert old in text, f"mutation target not found in {fname}: {old!r}"
        path.write_text(text.replace(old, new, 1))
    sys.path.insert(0, str(tmp_path))
    try:
        return importlib.import_module(name)
    finally:
        sys.path.remove(str(tmp_path))


def battery(o) -> list:
    """Names of the pins a given oracle fails (an exception counts as a failure)."""
    fails = []

    def check(name, fn):
        try:
            if not fn():
                fails.append(name)
        except Exception:                        # noqa: BLE001  -- a crash is a caught mistake too
            fails.append(name)

    x = workloads.worked_example()
    check("worked example", lambda: all(
        all(v.tolist() == [60, 64, 68, 72] for v in o.allreduce(x, a)[0]) for a in ALGOS))
    check("worked example reduce-scatter", lambda: [v.tolist() for v in o.reduce_scatter(x, "ring")[0]]
          == [[60.0], [64.0], [68.0], [72.0]])
    check("worked example all-gather", lambda: all(
        v.tolist() == [0, 1, 2, 3, 10, 11, 12, 13, 20, 21, 22, 23, 30, 31, 32, 33]
        for v in o.all_gather(x, "ring")[0]))
    probe = [np.full(4, v, np.float32) for v in PROBES["probe"]]
    check("order probes", lambda: all(
        o.allreduce(probe, a)[0][0].tolist() == PROBES["expected"][a]["value"] for a in ALGOS))
    for p in (3, 5, 6, 8):
        rng = np.random.default_rng(p)
        xi = [rng.integers(-100, 100, size=2 * p + 3).astype(np.float32) for _ in range(p)]
        want = np.sum(np.stack(xi).astype(np.int64), axis=0).tolist()
        check(f"integer sums p={p}", lambda xi=xi, want=want: all(
            all(v.astype(np.int64).tolist() == want for v in o.allreduce(xi, a)[0]) for a in ALGOS))
    xr = [np.random.default_rng([9, r]).normal(size=37).astype(np.float32) for r in range(8)]

    def ar_is_rs_ag():
        ar, _ = o.allreduce(xr, "ring")
        rs, _ = o.reduce_scatter(xr, "ring")
        return all(np.concatenate(rs).tobytes() == v.tobytes() for v in ar)
    check("AR = AG o RS", ar_is_rs_ag)
    check("all ranks bitwise equal", lambda: all(
        all(v.tobytes() == o.allreduce(xr, a)[0][0].tobytes() for v in o.allreduce(xr, a)[0]) for a in ALGOS))

    def rd_exchanges_xor_partners():
        # [NCC] 5.2: in step k ranks i and i xor 2^k exchange (p = 8, no fold)
        _, led = o.allreduce([np.zeros(8, np.float32)] * 8, "rd")
        pairs = {(m.step, m.src, m.dst) for m in led.msgs}
        return all((s, d, r) in pairs and r == d ^ (1 << s) for s, d, r in pairs)
    check("recursive doubling partners", rd_exchanges_xor_partners)

    def ledger_closed_form():
        p, n = 8, 8 * 1024
        _, led = o.allreduce([np.zeros(n, np.float32)] * p, "ring")
        ok = led.sent_bytes() == [2 * (p - 1) * (n // p) * 4] * p and led.n_steps == 2 * (p - 1)
        _, led = o.allreduce([np.zeros(n, np.float32)] * p, "rd")
        ok = ok and led.sent_bytes() == [3 * n * 4] * p
        _, led = o.allreduce([np.zeros(n, np.float32)] * p, "tree")
        return ok and led.sent_bytes() == [k * n * 4 for k in (3, 1, 2, 1, 3, 1, 2, 1)]
    check("ledger closed forms", ledger_closed_form)

    def a2a():
        send = [np.array([[10 * i + j] for j in range(4)], np.float32) for i in range(4)]
        recv, _ = o.all_to_all(send, np.ones((4, 4), np.int64), "f32")
        ok = [r.ravel().tolist() for r in recv] == [[j, 10 + j, 20 + j, 30 + j] for j in range(4)]
        sp = np.array([[2, 0, 1], [1, 3, 0], [0, 2, 2]])
        rows = [np.arange(sp[i].sum() * 2, dtype=np.float32).reshape(-1, 2) + 100 * i for i in range(3)]
        there, _ = o.all_to_all(rows, sp, "f32")
        back, _ = o.all_to_all(there, sp.T, "f32")
        return ok and all(np.array_equal(a, b) for a, b in zip(back, rows))
    check("all-to-all", a2a)

    def bf16_vs_torch():
        import torch
        u = np.random.default_rng(3).integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
        f = u.view(np.float32)
        f = f[np.isfinite(f)]
        want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return np.array_equal(o.f32_to_bf16(f), want)
    check("bf16 rounding", bf16_vs_torch)
    return fails


@pytest.mark.timeout(120)
def test_unmodified_oracle_passes_the_battery(tmp_path):
    assert battery(load_copy(tmp_path, "oracle_copy")) == []


@pytest.mark.timeout(120)
@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, idx):
    name, fname, old, new = MUTANTS[idx]
    o = load_copy(tmp_path, f"oracle_mutant_{idx}", (fname, old, new), FOLLOW_UPS.get(name))
    fails = battery(o)
    assert fails, f"planted mistake not caught: {name}"


# ---------------------------------------------------------------- the widened rows' oracles

WIDE_MUTANTS = [
    ("hierarchical cross-node ring runs backwards", "collectives.py",
     "    same = [[g * L + l for g in range(N)] for l in range(L)]",
     "    same = [[g * L + l for g in reversed(range(N))] for l in range(L)]"),
    ("hierarchical in-node reduce-scatter owner shifted", "collectives.py",
     "        step = together(step, [(grp, cpieces, ADD, 1) for grp in groups])",
     "        step = together(step, [(grp, cpieces, ADD, 2) for grp in groups])"),
    ("reduce relabels ranks the other way round", "rooted.py",
     "        cl.step(step, [Send((v + root) % p, (v - m + root) % p, 0, 0, n, ADD)",
     "        cl.step(step, [Send((root - v) % p, (root - v + m) % p, 0, 0, n, ADD)"),
    ("binomial broadcast with masks ascending", "rooted.py",
     "        for step, m in enumerate(reversed(_masks(p))):",
     "        for step, m in enumerate(_masks(p)):"),
    ("E4M3 rounds half up", "fp8.py",
     "    q = np.rint(np.ldexp(a[nor], -(e[nor] - 3))).astype(np.int64)",
     "    q = np.floor(np.ldexp(a[nor], -(e[nor] - 3)) + 0.5).astype(np.int64)"),
    ("FP8 scale aims at 480 instead of 448", "fp8.py", "MAX_E4M3 = 448.0", "MAX_E4M3 = 480.0"),
    ("deduplicated blocks in descending token order", "moe.py",
     "                           if int(ids[t, k]) // experts_per_rank == j})",
     "                           if int(ids[t, k]) // experts_per_rank == j}, reverse=True)"),
    ("plan blocks ordered by (destination, token, expert)", "moe.py",
     "        pairs.sort()\n", "        pairs.sort(key=lambda x: (x[0], x[2], x[1], x[3]))\n"),
    ("plan blocks with experts descending", "moe.py",
     "        pairs.sort()\n", "        pairs.sort(key=lambda x: (x[0], -x[1], x[2], x[3]))\n"),
    ("plan combine slot index transposed", "moe.py",
     "dst_rows.append(np.array([t * K + k for _, _, t, k in pairs], dtype=np.int32))",
     "dst_rows.append(np.array([k * T + t for _, _, t, k in pairs], dtype=np.int32))"),
]


def wide_battery(o) -> list:
    from oracle import fp8 as _unused  # noqa: F401  (the real module stays importable)
    fails = []

    def check(name, fn):
        try:
            if not fn():
                fails.append(name)
        except Exception:                        # noqa: BLE001
            fails.append(name)

    big = 2.0 ** 24
    # hierarchical: the hand-worked probes of the inner and the outer chain
    check("hierarchical inner probe", lambda: o.allreduce_hierarchical(
        [np.full(6, v, np.float32) for v in (big, 1.0, -big, 0.0, 0.0, 0.0)], 2, 3)[0][0].tolist() == [1, 1, 1, 1, 0, 0])
    check("hierarchical outer probe", lambda: o.allreduce_hierarchical(
        [np.full(6, v, np.float32) for v in (big, 0.0, 1.0, 0.0, -big, 0.0)], 3, 2)[0][0].tolist() == [1, 1, 0, 1, 1, 0])

    def hier_ledger_cross_node_bytes():
        _, led = o.allreduce_hierarchical([np.zeros(1, np.float32)] * 16, 2, 8, n=16 * 64, lo=0)
        cross = [m for m in led.msgs if m.src // 8 != m.dst // 8]
        return sum(m.bytes for m in cross) == 16 * 2 * (128 // 2) * 4 and all(m.dst == m.src ^ 8 for m in cross)
    check("hierarchical cross-node ring", hier_ledger_cross_node_bytes)
    # rooted: the reduce probe by root, broadcast delivery and causality
    x3 = [np.full(3, v, np.float32) for v in (big, 1.0, -big)]
    check("reduce probe", lambda: [o.rooted.reduce(x3, r)[0].tolist()[0] for r in range(3)] == [0.0, 1.0, 1.0])

    def broadcast_causal():
        for p in (5, 8):
            for root in (0, 3):
                led = o.rooted.broadcast(np.zeros(9, np.float32), p, "tree", root)[1]
                have = {root}
                for s in range(led.n_steps):
                    msgs = [m for m in led.msgs if m.step == s]
                    if any(m.src not in have for m in msgs):
                        return False
                    have |= {m.dst for m in msgs}
                if have != set(range(p)) or led.n_steps != (p - 1).bit_length():
                    return False
        return True
    check("broadcast causality", broadcast_causal)

    # FP8: codes against torch's float8_e4m3fn, and the scale's binade
    def e4m3_vs_torch():
        import torch
        v = np.random.default_rng(1).uniform(-448, 448, 50_000).astype(np.float32)
        v = np.concatenate([v, np.float32([1.0625, 1.1875, 2 ** -10, 1.5 * 2 ** -10])])
        return np.array_equal(o.fp8.e4m3_encode(v),
                              torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    check("E4M3 vs torch", e4m3_vs_torch)

    def scale_binade():
        x = np.random.default_rng(2).normal(size=(4, 256)).astype(np.float32)
        x[0, 7] = 460 * 2.0 ** -7                 # amax between 448 and 480 times a power of two
        b = o.fp8.quantize_rows(x)
        s = np.ascontiguousarray(b[:, 256:]).view(np.float32)
        amax = np.abs(x).reshape(4, 2, 128).max(axis=2)
        return bool(np.all(amax / s <= 448) and np.all(amax / s > 224))
    check("FP8 scale", scale_binade)

    # deduplicated dispatch: expansion equals the plain dispatch; blocks by token
    def dedup():
        topk = [np.stack([np.sort(np.random.default_rng([7, i, t]).choice(16, 3, replace=False))
                          for t in range(20)]).astype(np.int32) for i in range(4)]
        toks = [workloads.tagged_rows(np.zeros((20, 8), np.uint16), i, np.arange(20)) for i in range(4)]
        splits, src, _ = o.moe_plan(topk, 4)
        plain, _, _ = o.moe_dispatch(toks, splits, src)
        expanded, _, _ = o.moe.dispatch_dedup(toks, topk, 4)
        su, src_u, _ = o.moe.plan_dedup(topk, 4)
        ordered = all(np.all(np.diff(src_u[i][int(su[i, :j].sum()):int(su[i, :j + 1].sum())]) > 0)
                      for i in range(4) for j in range(4))
        return ordered and all(np.array_equal(a, b) for a, b in zip(plain, expanded))
    check("dedup dispatch", dedup)

    # the plan's row order inside each block, worked by hand
    def plan_order():
        g = json.load(open(os.path.join(ROOT, "tests", "golden", "moe_plan_order.json")))
        topk = [np.array(t, dtype=np.int32) for t in g["topk_ids"]]
        splits, src, dst = o.moe_plan(topk, g["experts_per_rank"])
        return (splits.tolist() == g["splits"] and [x.tolist() for x in src] == g["src_rows"]
                and [x.tolist() for x in dst] == g["dst_rows"])
    check("MoE plan row order", plan_order)
    return fails


def load_wide(tmp_path, name, patch=None):
    o = load_copy(tmp_path, name, patch)
    for sub in ("rooted", "fp8", "moe"):
        setattr(o, sub, importlib.import_module(f"{name}.{sub}"))
    return o


@pytest.mark.timeout(120)
def test_unmodified_widened_oracles_pass_their_battery(tmp_path):
    sys.path.insert(0, str(tmp_path))
    try:
        assert wide_battery(load_wide(tmp_path, "oracle_wide_copy")) == []
    finally:
        sys.path.remove(str(tmp_path))


@pytest.mark.timeout(120)
@pytest.mark.parametrize("idx", range(len(WIDE_MUTANTS)), ids=[m[0] for m in WIDE_MUTANTS])
def test_planted_mistake_in_a_widened_oracle_is_caught(tmp_path, idx):
    name, fname, old, new = WIDE_MUTANTS[idx]
    sys.path.insert(0, str(tmp_path))
    try:
        o = load_wide(tmp_path, f"oracle_wide_mutant_{idx}", (fname, old, new))
        assert wide_battery(o), f"planted mistake not caught: {name}"
    finally:
        sys.path.remove(str(tmp_path))
