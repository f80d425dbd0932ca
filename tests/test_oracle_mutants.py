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
