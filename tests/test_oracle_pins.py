"""Pins of the CPU oracle to facts fixed by the pages and by arithmetic.

Nothing here compares the oracle with itself: every expected value is a
printed input with a hand-derived output (golden files), a closed form, a
structural rule derived from an algorithm's definition independently of the
oracle's message passing, an exact integer sum, an error bound, or a library
routine (torch's bfloat16 conversion).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALGOS = oracle.ALGOS
BIG = np.float32(2.0 ** 24)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example

def test_worked_example_all_collectives():
    g = load("worked_example.json")
    x = [np.array(v, dtype=np.float32) for v in g["inputs"]]
    assert [v.tolist() for v in workloads.worked_example()] == [v.tolist() for v in x]
    for algo in ALGOS:
        out, _ = oracle.allreduce(x, algo)
        for r in range(4):
            assert out[r].tolist() == g["allreduce"], (algo, r)
    rs, _ = oracle.reduce_scatter(x, "ring")
    assert [v.tolist() for v in rs] == g["reduce_scatter"]
    rs, _ = oracle.reduce_scatter(x, "rabenseifner")
    assert [v.tolist() for v in rs] == g["reduce_scatter"]
    for algo in ("ring", "rd"):
        ag, _ = oracle.all_gather(x, algo)
        for r in range(4):
            assert ag[r].tolist() == g["all_gather"]
    recv, _ = oracle.all_to_all([v.reshape(4, 1) for v in x], np.ones((4, 4), dtype=np.int64), "f32")
    assert [v.ravel().tolist() for v in recv] == g["all_to_all"]


def test_worked_example_ring_ledger():
    g = load("worked_example.json")["ring_allreduce_ledger"]
    x = workloads.worked_example()
    _, led = oracle.allreduce(x, "ring")
    assert led.n_steps == g["n_steps"]
    assert len(led.msgs) == g["n_msgs"]
    assert all(m.bytes == g["bytes_per_msg"] for m in led.msgs)
    assert led.sent_bytes() == [g["sent_per_rank"]] * 4
    assert led.recv_bytes() == [g["sent_per_rank"]] * 4


def test_worked_example_ring_reduce_scatter_owner():
    g = load("worked_example.json")
    x = workloads.worked_example()
    rs, _ = oracle.reduce_scatter(x, "ring")
    owner = g["ring_trace_after_reduce_scatter"]["owner_of_chunk"]
    for c, r in enumerate(owner):
        assert rs[r].tolist() == [g["allreduce"][c]]


# ---------------------------------------------------------------- order probes

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order_probes_p4(dtype):
    g = load("order_probes.json")
    x = [np.full(4, v, dtype=np.float32) for v in g["probe"]]
    if dtype == "bf16":
        x = [oracle.f32_to_bf16(v) for v in x]
        assert all((oracle.bf16_to_f32(v) == np.float32(w)).all() for v, w in zip(x, g["probe"]))
    for algo, exp in g["expected"].items():
        out, _ = oracle.allreduce(x, algo, dtype)
        for r in range(4):
            got = out[r] if dtype == "f32" else oracle.bf16_to_f32(out[r])
            assert got.tolist() == exp["value"], (algo, r)


def _lca_height_rd(u, v):          # partners differ in bit 0 first
    return (u ^ v).bit_length()


def _lca_height_rab(u, v, k):      # partners differ in the top bit first
    x = u ^ v
    low = (x & -x).bit_length() - 1
    return k - low


def _new_rank(u, p):
    p2 = 1 << (p.bit_length() - 1)
    r = p - p2
    return u // 2 if u < 2 * r else u - r


def _height(algo, p, u, v, chunk):
    """Height at which leaves u and v first meet in the summation order.
    Derived from the step definitions, without simulating messages."""
    if algo == "ring":
        seq = [(chunk + 1 + k) % p for k in range(p)]        # chain: later position meets later
        return max(seq.index(u), seq.index(v))
    if algo == "tree":                                       # binomial == padded perfect tree
        return _lca_height_rd(u, v)
    nu, nv = _new_rank(u, p), _new_rank(v, p)
    if nu == nv:                                             # folded pair: added before anything else
        return 0
    k = (1 << (p.bit_length() - 1)).bit_length() - 1
    if algo == "rd":
        return 1 + _lca_height_rd(nu, nv)
    return 1 + _lca_height_rab(nu, nv, k)


def _triple_expect(algo, p, a, b, c, chunk):
    """x_a = 2^24, x_b = x_c = 1, rest 0: the two ones survive only if they
    meet each other before either meets 2^24."""
    hbc = _height(algo, p, b, c, chunk)
    hab = _height(algo, p, a, b, chunk)
    hac = _height(algo, p, a, c, chunk)
    return float(BIG + 2) if hbc < min(hab, hac) else float(BIG)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p", [3, 4, 5, 6, 7, 8, 12, 16])
def test_triple_probes(algo, p):
    n = p                                          # chunk c = element c
    triples = list(itertools.permutations(range(p), 3))
    rng = np.random.default_rng(p)
    if len(triples) > 400:
        triples = [triples[i] for i in rng.choice(len(triples), 400, replace=False)]
    for a, b, c in triples:
        x = [np.zeros(n, dtype=np.float32) for _ in range(p)]
        x[a][:] = BIG
        x[b][:] = 1.0
        x[c][:] = 1.0
        out, _ = oracle.allreduce(x, algo)
        for e in range(n):
            exp = _triple_expect(algo, p, a, b, c, e)
            assert float(out[0][e]) == exp, (algo, p, a, b, c, e)
        for r in range(1, p):
            assert np.array_equal(out[r], out[0])


def test_rd_and_tree_differ_when_p_is_not_a_power_of_two():
    # p=5: the fold gives ((x0+x1)+x2)+(x3+x4); the binomial tree ((x0+x1)+(x2+x3))+x4
    x = [np.full(1, v, dtype=np.float32) for v in (0.0, 0.0, 1.0, 1.0, float(BIG))]
    x[0][:] = 0.0
    rd, _ = oracle.allreduce(x, "rd")
    tr, _ = oracle.allreduce(x, "tree")
    assert rd[0][0] == BIG            # 1 + 2^24 rounds away before the second 1 arrives
    assert tr[0][0] == BIG + 2        # the two ones meet first


# ---------------------------------------------------------------- identities

@pytest.mark.parametrize("p,n", [(4, 4), (8, 64), (8, 1024), (16, 320), (2, 6)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_is_reduce_scatter_then_all_gather(p, n, dtype):
    rng = np.random.default_rng(p * 1000 + n)
    x = [rng.normal(size=n).astype(np.float32) for _ in range(p)]
    if dtype == "bf16":
        x = [oracle.f32_to_bf16(v) for v in x]
    for rs_algo, ag_algo, ar_algo in (("ring", "ring", "ring"), ("rabenseifner", "rd", "rabenseifner")):
        rs, rs_led = oracle.reduce_scatter(x, rs_algo, dtype)
        ag, ag_led = oracle.all_gather(rs, ag_algo, dtype)
        ar, ar_led = oracle.allreduce(x, ar_algo, dtype)
        for r in range(p):
            assert np.array_equal(ag[r].view(np.uint8), ar[r].view(np.uint8)), (rs_algo, r)
        # ledger(AR) = ledger(RS) followed by ledger(AG) shifted by the RS step count
        shifted = [m._replace(step=m.step + rs_led.n_steps) for m in ag_led.msgs]
        assert sorted(ar_led.msgs) == sorted(rs_led.msgs + shifted)


@pytest.mark.parametrize("p", [2, 3, 4, 8])
def test_all_to_all_twice_is_identity(p):
    rng = np.random.default_rng(p)
    splits = rng.integers(0, 5, size=(p, p))
    splits[0, :] = 0                       # a rank that sends nothing
    splits[p - 1, 0] = 0
    H = 3
    send = [rng.integers(0, 2 ** 16, size=(int(splits[i].sum()), H)).astype(np.uint16) for i in range(p)]
    recv, led = oracle.all_to_all(send, splits, "bf16")
    for j in range(p):
        assert recv[j].shape[0] == splits[:, j].sum()
    back, _ = oracle.all_to_all(recv, splits.T, "bf16")
    for i in range(p):
        assert np.array_equal(back[i], send[i])
    # ledger: p(p-1) messages, diagonal excluded, sent = off-diagonal rows * row bytes
    assert len(led.msgs) == p * (p - 1)
    assert all(m.src != m.dst for m in led.msgs)
    for i in range(p):
        assert led.sent_bytes()[i] == sum(int(splits[i, j]) * H * 2 for j in range(p) if j != i)


def test_all_to_all_tagged_rows_in_source_order():
    p, H = 3, 4
    splits = np.array([[1, 2, 0], [3, 0, 1], [2, 2, 2]])
    send = []
    for i in range(p):
        rows = np.zeros((int(splits[i].sum()), H), dtype=np.uint16)
        k = 0
        for j in range(p):
            for q in range(splits[i, j]):
                rows[k] = (i, j, q, 7)
                k += 1
        send.append(rows)
    recv, _ = oracle.all_to_all(send, splits, "bf16")
    for j in range(p):
        expect = [(i, j, q, 7) for i in range(p) for q in range(splits[i, j])]
        assert [tuple(r) for r in recv[j].tolist()] == expect


# ---------------------------------------------------------------- ledger closed forms

def _S(n, dtype):
    return n * oracle.ELEM_BYTES[dtype]


@pytest.mark.parametrize("p", [2, 4, 8, 16])
def test_ledger_ring_and_rabenseifner_meet_the_bound(p):
    n = 64 * p
    x = [np.zeros(n, dtype=np.float32) for _ in range(p)]
    S = _S(n, "f32")
    for algo in ("ring", "rabenseifner"):
        _, led = oracle.allreduce(x, algo)
        assert led.sent_bytes() == [2 * (p - 1) * S // p] * p, algo
        assert led.recv_bytes() == [2 * (p - 1) * S // p] * p, algo
    _, led = oracle.allreduce(x, "ring")
    assert led.n_steps == 2 * (p - 1)
    _, led = oracle.allreduce(x, "rabenseifner")
    assert led.n_steps == 2 * (p.bit_length() - 1)


def test_ledger_p8_bytes_per_device():
    # section 5.3: ring and Rabenseifner send 1.75 n per device at p = 8, recursive doubling 3 n
    n = 8 * 1000
    S = _S(n, "f32")
    x = [np.zeros(n, dtype=np.float32) for _ in range(8)]
    for algo, factor in (("ring", 1.75), ("rabenseifner", 1.75), ("rd", 3.0)):
        _, led = oracle.allreduce(x, algo)
        assert led.sent_bytes() == [int(factor * S)] * 8, algo
    _, led = oracle.allreduce(x, "tree")
    assert led.sent_bytes() == [3 * S, S, 2 * S, S, 3 * S, S, 2 * S, S]
    assert led.n_steps == 6


@pytest.mark.parametrize("p", [1, 2, 3, 5, 6, 7, 8, 12, 16, 72])
def test_ledger_closed_forms_any_p(p):
    n = 3 * p + 1 if p > 1 else 5                    # p does not divide n
    x = [np.zeros(n, dtype=np.float32) for _ in range(p)]
    S = _S(n, "f32")
    offs = oracle.chunk_bounds(n, p)
    cnt = [offs[c + 1] - offs[c] for c in range(p)]
    _, led = oracle.allreduce(x, "ring")
    assert led.sent_bytes() == [2 * S - (cnt[i] + cnt[(i + 1) % p]) * 4 if p > 1 else 0 for i in range(p)]
    assert led.n_steps == 2 * (p - 1)
    p2 = 1 << (p.bit_length() - 1)
    r = p - p2
    lg = p2.bit_length() - 1
    _, led = oracle.allreduce(x, "rd")
    exp = [S if (i < 2 * r and i % 2 == 0) else (lg * S + S if i < 2 * r else lg * S) for i in range(p)]
    assert led.sent_bytes() == exp
    assert led.n_steps == lg + (2 if r else 0)
    _, led = oracle.allreduce(x, "tree")
    assert sum(led.sent_bytes()) == 2 * (p - 1) * S
    assert led.sent_bytes()[0] == (p - 1).bit_length() * S
    assert led.n_steps == 2 * (p - 1).bit_length()
    # bandwidth bound of section 4.3 holds for the busiest device of every algorithm
    for algo in ALGOS:
        _, led = oracle.allreduce(x, algo)
        assert max(led.sent_bytes()) * p >= 2 * (p - 1) * S, algo


def test_ledger_rabenseifner_fold():
    p, n = 12, 8 * 40                                # p2 = 8, r = 4
    x = [np.zeros(n, dtype=np.float32) for _ in range(p)]
    S = _S(n, "f32")
    _, led = oracle.allreduce(x, "rabenseifner")
    base = 2 * 7 * S // 8
    exp = [S if (i < 8 and i % 2 == 0) else (base + S if i < 8 else base) for i in range(p)]
    assert led.sent_bytes() == exp
    assert led.n_steps == 2 * 3 + 2


def test_ledger_bytes_count_storage_type():
    p, n = 8, 800
    x = [np.zeros(n, dtype=np.uint16) for _ in range(p)]
    _, led = oracle.allreduce(x, "ring", "bf16")
    assert led.sent_bytes() == [2 * 7 * n * 2 // 8] * p


def test_ledger_headline_closed_forms():
    # ring over 8 ranks: 2(p-1)/p of the bytes per rank; 14 steps, 112 messages
    for n, per_rank, msg in ((262_144, 1_835_008, 131_072), (6_553_600, 45_875_200, 3_276_800)):
        x = [np.zeros(8, dtype=np.float32)] * 8
        _, led = oracle.allreduce([v for v in x], "ring", n=n, lo=0)
        assert led.sent_bytes() == [per_rank] * 8
        assert led.n_steps == 14 and len(led.msgs) == 112
        assert {m.bytes for m in led.msgs} == {msg}


# ---------------------------------------------------------------- sums

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p", [1, 2, 3, 5, 6, 7, 8, 9, 12, 16, 72])
def test_integer_inputs_give_the_exact_sum(algo, p):
    n = 2 * p + 3
    rng = np.random.default_rng(p)
    xi = [rng.integers(-1000, 1000, size=n) for _ in range(p)]
    out, _ = oracle.allreduce([v.astype(np.float32) for v in xi], algo)
    exact = np.sum(np.stack(xi), axis=0)
    for r in range(p):
        assert np.array_equal(out[r].astype(np.int64), exact), (algo, r)


def test_p1_is_identity_and_p2_is_one_add():
    rng = np.random.default_rng(0)
    a = rng.normal(size=17).astype(np.float32)
    b = rng.normal(size=17).astype(np.float32)
    for algo in ALGOS:
        out, led = oracle.allreduce([a], algo)
        assert np.array_equal(out[0], a) and led.msgs == [] and led.n_steps == 0
        out, _ = oracle.allreduce([a, b], algo)
        assert np.array_equal(out[0], a + b) and np.array_equal(out[1], a + b)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p", [2, 5, 8, 16])
def test_error_bound_against_float64(algo, p):
    n = 4096
    rng = np.random.default_rng(p + 17)
    x = [rng.normal(size=n).astype(np.float32) for _ in range(p)]
    out, _ = oracle.allreduce(x, algo)
    ref = np.sum(np.stack(x).astype(np.float64), axis=0)
    bound = 2 * (p - 1) * 2.0 ** -24 * np.sum(np.abs(np.stack(x).astype(np.float64)), axis=0)
    assert np.all(np.abs(out[0].astype(np.float64) - ref) <= bound)


def test_bf16_output_error_bound():
    p, n = 16, 4096
    x = workloads.rank_buffers(workloads.TAG_TEST, p, n, ("uniform", -1.0, 1.0), "bf16")
    xf = np.stack([oracle.bf16_to_f32(v) for v in x]).astype(np.float64)
    ref = xf.sum(axis=0)
    for algo in ALGOS:
        out, _ = oracle.allreduce(x, algo, "bf16")
        got = oracle.bf16_to_f32(out[0]).astype(np.float64)
        bound = 2 * (p - 1) * 2.0 ** -24 * np.abs(xf).sum(axis=0) + 2.0 ** -8 * (np.abs(ref) + 2 * (p - 1) * 2.0 ** -24 * np.abs(xf).sum(axis=0))
        assert np.all(np.abs(got - ref) <= bound), algo


# ---------------------------------------------------------------- bfloat16 rounding

def test_bf16_rounding_matches_torch():
    import torch
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    structured = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(5).integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([structured, rnd])
    f = u.view(np.float32)
    mine = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(mine[~nan], ref[~nan])
    back = oracle.bf16_to_f32(mine[nan])
    assert np.all(np.isnan(back))
    # widening is exact
    w = oracle.bf16_to_f32(np.arange(1 << 16, dtype=np.uint16))
    assert np.array_equal(w.view(np.uint32) >> 16, np.arange(1 << 16, dtype=np.uint32))


def test_bf16_accumulates_in_float32_once_rounded():
    # x_r = 1 + r * 2^-7 is exact in bf16 and every partial sum is exact in
    # float32, so each order gives 8 + 28 * 2^-7 = 8.21875; rounded once to
    # bf16 (spacing 2^-4 above 8) that is a tie, which goes to even: 8.25
    x = [oracle.f32_to_bf16(np.full(8, 1 + r * 2.0 ** -7, dtype=np.float32)) for r in range(8)]
    for algo in ALGOS:
        out, _ = oracle.allreduce(x, algo, "bf16")
        assert np.all(oracle.bf16_to_f32(out[0]) == np.float32(8.25)), algo


# ---------------------------------------------------------------- windows

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p", [3, 8, 72])
def test_windowed_run_equals_full_run(algo, p):
    n = 40 * p + 7
    rng = np.random.default_rng(p)
    x = [rng.normal(size=n).astype(np.float32) for _ in range(p)]
    full, fled = oracle.allreduce(x, algo)
    for lo, hi in ((0, 5), (n // 3, n // 3 + 61), (n - 9, n)):
        win, wled = oracle.allreduce([v[lo:hi] for v in x], algo, n=n, lo=lo)
        for r in range(p):
            assert np.array_equal(win[r], full[r][lo:hi])
        assert wled.sorted() == fled.sorted()
    if algo == "ring":
        rs_full, _ = oracle.reduce_scatter(x, "ring")
        offs = oracle.chunk_bounds(n, p)
        lo, hi = offs[1] - 3, offs[1] + 4
        rs_win, _ = oracle.reduce_scatter([v[lo:hi] for v in x], "ring", n=n, lo=lo)
        assert np.array_equal(rs_win[0], rs_full[0][lo - offs[0]:])
        assert np.array_equal(rs_win[1], rs_full[1][:hi - offs[1]])


# ---------------------------------------------------------------- MoE

def test_moe_plan_dispatch_combine_round_trip():
    p, T, H, E, K = 4, 64, 8, 32, 4
    epr = E // p
    topk = [workloads.moe_topk(r, T, E, K) for r in range(p)]
    for ids in topk:
        assert ids.shape == (T, K)
        assert all(len(set(row)) == K for row in ids.tolist())
    toks = [workloads.rank_window(workloads.TAG_TEST, r, 0, T * H, ("normal", 0, 1), "bf16").reshape(T, H)
            for r in range(p)]
    toks = [workloads.tagged_rows(t, r, np.arange(T)) for r, t in enumerate(toks)]
    splits, src_rows, dst_rows = oracle.moe_plan(topk, epr)
    assert np.all(splits.sum(axis=1) == T * K)
    recv, send, led = oracle.moe_dispatch(toks, splits, src_rows)
    # every received row belongs to an expert held by the receiving rank
    for j in range(p):
        for row in recv[j]:
            src, t = int(row[0]), int(row[1])
            assert any(e // epr == j for e in topk[src][t])
    outs, _ = oracle.moe_combine(recv, splits, dst_rows, K, T)
    for i in range(p):
        assert np.array_equal(outs[i], np.repeat(toks[i], K, axis=0))


def test_moe_plan_row_order_hand_worked():
    """The plan's row order inside each (i -> j) block, worked by hand
    (tests/golden/moe_plan_order.json): by expert, then token, then slot."""
    g = json.load(open(os.path.join(GOLDEN, "moe_plan_order.json")))
    topk = [np.array(t, dtype=np.int32) for t in g["topk_ids"]]
    splits, src_rows, dst_rows = oracle.moe_plan(topk, g["experts_per_rank"])
    assert splits.tolist() == g["splits"]
    assert [s.tolist() for s in src_rows] == g["src_rows"]
    assert [d.tolist() for d in dst_rows] == g["dst_rows"]
    # the expert of each row rank j receives (source blocks in order), from
    # the sender's (token, slot) of that row
    for j in range(g["p"]):
        exp = []
        for i in range(g["p"]):
            s0 = int(splits[i, :j].sum())
            for q in range(int(splits[i, j])):
                t, k = divmod(int(dst_rows[i][s0 + q]), g["topk"])
                exp.append(int(topk[i][t, k]))
        assert exp == g["received_expert_per_row"][j]


def test_moe_plan_blocks_are_expert_major_on_the_full_workload():
    """On the cfg-sized routing (8 ranks x 4096 tokens, top-8 of 256): inside
    every block the (expert, token) keys of the rows strictly increase, and
    every row's expert lives on the block's destination."""
    p, T, E, K = 8, 4096, 256, 8
    epr = E // p
    topk = [workloads.moe_topk(r, T, E, K) for r in range(p)]
    splits, src_rows, dst_rows = oracle.moe_plan(topk, epr)
    for i in range(p):
        t, k = np.divmod(dst_rows[i].astype(np.int64), K)
        assert np.array_equal(t, src_rows[i])
        e = topk[i][t, k].astype(np.int64)
        bounds = np.concatenate([[0], np.cumsum(splits[i])])
        for j in range(p):
            eb, tb = e[bounds[j]:bounds[j + 1]], t[bounds[j]:bounds[j + 1]]
            assert np.all(eb // epr == j)
            key = eb * T + tb
            assert np.all(np.diff(key) > 0)


def test_moe_workload_skew_and_conservation():
    p, T, E, K = 8, 4096, 256, 8
    topk = [workloads.moe_topk(r, T, E, K) for r in range(p)]
    splits, _, _ = oracle.moe_plan(topk, E // p)
    assert splits.sum() == p * T * K == 262_144
    assert np.all(splits.sum(axis=1) == T * K)
    # Zipf(1.1) over ids with the identity id mapping: rank 0's 32 experts
    # carry most of the draws
    frac0 = splits[:, 0].sum() / splits.sum()
    assert 0.55 < frac0 < 0.75


def test_moe_routing_draws_follow_the_zipf_weights():
    """Gumbel-top-k with k = 1 is a draw with P(e) = w_e / sum(w) (the
    Gumbel-max property), w_e = (e+1)^-1.1: expert frequencies over many
    tokens match within 4 standard deviations, and rank 0's 32 experts
    carry 72.8 % of the single-draw mass."""
    E, T = 256, 200_000
    w = (np.arange(E) + 1.0) ** -1.1
    prob = w / w.sum()
    assert round(prob[:32].sum(), 3) == 0.728
    ids = workloads.moe_topk(0, T, E, 1)[:, 0]
    counts = np.bincount(ids, minlength=E)
    sd = np.sqrt(T * prob * (1 - prob))
    assert np.all(np.abs(counts - T * prob) <= 4 * sd + 1)
    # top-k draws are distinct and sorted
    ids8 = workloads.moe_topk(1, 1000, E, 8)
    assert np.all(np.diff(ids8, axis=1) > 0)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p", [2, 3, 5, 8, 12, 16])
def test_every_rank_holds_the_same_bits(algo, p):
    """An all-reduce leaves one value per element, the same bits on every
    rank ([NCC] 4.1); a schedule that sums in a rank-dependent order (for
    example a dissemination pattern) fails this on random inputs."""
    x = [np.random.default_rng([p, r, 5]).normal(size=3 * p + 1).astype(np.float32) for r in range(p)]
    out, _ = oracle.allreduce(x, algo)
    assert all(v.tobytes() == out[0].tobytes() for v in out)


@pytest.mark.parametrize("p", [2, 4, 8, 16])
def test_recursive_doubling_exchanges_with_xor_partners(p):
    """[NCC] 5.2: in step k, ranks i and i xor 2^k exchange their vectors."""
    _, led = oracle.allreduce([np.zeros(p, np.float32)] * p, "rd")
    pairs = {(m.step, m.src, m.dst) for m in led.msgs}
    assert len(pairs) == p * (p.bit_length() - 1)
    for s, a, b in pairs:
        assert b == a ^ (1 << s) and (s, b, a) in pairs
