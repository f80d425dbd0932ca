"""GPU parity of the MoE dispatch variants: the FP8-payload dispatch against
the oracle's quantiser, byte for byte (codes and scales), and the
deduplicated dispatch plus local expansion against the plain dispatch, bit
for bit, up to the full MoE workload."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import fp8, moe
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


def sync():
    import torch
    torch.cuda.synchronize()


def to_gpu_bf16(rows):
    import torch
    return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).cuda().view(torch.bfloat16)


def gpu_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def small_routing(p, T, K, E, seed):
    return [np.stack([np.sort(np.random.default_rng([seed, i, t]).choice(E, K, replace=False))
                      for t in range(T)]).astype(np.int32) for i in range(p)]


def check_fp8(vc, toks, topk, epr, what):
    p = len(toks)
    splits, src, _ = vc.vcoll_moe_plan(np.stack(topk), epr)
    say(f"vcoll_moe_dispatch_fp8 {what}")
    recv = vc.vcoll_moe_dispatch_fp8([to_gpu_bf16(t) for t in toks], splits, [gpu_i32(s) for s in src])
    sync()
    want, _ = moe.dispatch_fp8(toks, splits, list(src))
    for j in range(p):
        got = recv[j].cpu().numpy()
        assert got.shape == want[j].shape
        bad = np.argwhere(got != want[j])
        assert bad.size == 0, f"{what}: rank {j}: {len(bad)} bytes differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("H", [128, 384, 7168])
def test_fp8_dispatch_matches_oracle(vc, H):
    p, T, K, E = 4, 48, 3, 16
    topk = small_routing(p, T, K, E, H)
    toks = [workloads.rank_window(workloads.TAG_TEST * 1000 + 950, i, 0, T * H, ("normal", 0.0, 1.0),
                                  "bf16").reshape(T, H) for i in range(p)]
    check_fp8(vc, toks, topk, E // p, f"H={H}")


def test_fp8_dispatch_special_values(vc):
    """Rounding ties, the subnormal grid, zero and negative zero, group
    maxima exactly at 448 * 2^k, all-zero groups, tiny and huge groups, and
    non-finite elements."""
    p, T, H = 2, 8, 256
    rng = np.random.default_rng(5)
    rows = np.zeros((T, H), np.float32)
    rows[0] = rng.normal(0, 1, H)
    rows[1, :128] = np.ldexp(rng.integers(1, 16, 128) * (1 + rng.integers(0, 2, 128) / 16.0), -12)   # ties below 2^-6
    rows[1, 128:] = 448.0 * np.ldexp(1.0, rng.integers(-20, 20))
    rows[2, :128] = 0.0
    rows[2, 128:] = -0.0
    rows[3] = np.ldexp(rng.normal(0, 1, H), 100)
    rows[4] = np.ldexp(rng.normal(0, 1, H), -100)
    rows[5, :128] = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 1.5 * 2.0 ** -10, 448.0] + [0.0] * 122)
    rows[6, :5] = [np.nan, np.inf, -np.inf, 1.0, -np.nan]
    rows[7] = rng.uniform(-1, 1, H)
    bf = oracle.f32_to_bf16(rows)
    toks = [bf, bf[::-1].copy()]
    topk = [np.array([[0], [1], [0], [1], [0], [1], [0], [1]], np.int32)] * p
    check_fp8(vc, toks, topk, 1, "special values")


def every_bf16_pattern_rows():
    """bfloat16 rows of 128 (one scale group each) that hold every bit
    pattern: (a) each in-domain pattern (finite, |x| <= 448) in a group led
    by 448, so the group's scale is 2^0 and the encoder sees the pattern
    itself; (b) every non-finite pattern, also behind 448; (c) all 65536
    patterns in plain order, 128 consecutive patterns being one binade of
    one sign, so every group exponent from -126 to 126 and the clamps
    occur."""
    pats = np.arange(65536, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    anchor = np.uint16(0x43E0)                           # 448.0
    assert (np.uint32(anchor) << 16).view(np.float32) == 448.0
    rows = []
    for sel in (np.isfinite(vals) & (np.abs(vals) <= 448.0), ~np.isfinite(vals)):
        body = pats[sel].astype(np.uint16)
        pad = (-len(body)) % 127
        body = np.concatenate([body, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        rows.append(np.concatenate([np.full((body.shape[0], 1), anchor, np.uint16), body], axis=1))
    rows.append(pats.astype(np.uint16).reshape(-1, 128))
    return np.concatenate(rows)


def test_fp8_dispatch_every_bf16_pattern(vc):
    """Both FP8 dispatch forms (row-major gather and token-major push)
    against the oracle's quantiser on every bfloat16 bit pattern."""
    import torch
    rows = every_bf16_pattern_rows()
    T, H, p = rows.shape[0], 128, 2
    toks = [rows, rows[::-1].copy()]
    topk = [(np.arange(T) % 2).astype(np.int32).reshape(T, 1)] * p
    check_fp8(vc, toks, topk, 1, "every bf16 pattern")
    splits, src, dst = vc.vcoll_moe_plan(np.stack(topk), 1)
    got = vc.vcoll_moe_dispatch([to_gpu_bf16(t) for t in toks], slots_gpu(vc, splits, dst, 1), splits.sum(axis=0),
                                1, fp8=True)
    sync()
    want, _ = moe.dispatch_fp8(toks, splits, list(src))
    for j in range(p):
        assert np.array_equal(got[j].cpu().numpy(), want[j]), f"token-major, rank {j}"


def test_fp8_dispatch_skips_out_of_range_rows(vc):
    import torch
    p, T, H = 2, 4, 128
    toks = [to_gpu_bf16(np.zeros((T, H), np.uint16)) for _ in range(p)]
    recv = [torch.full((2, H + 4), 7, dtype=torch.uint8, device="cuda") for _ in range(p)]
    splits = np.array([[1, 1], [1, 1]])
    src = [gpu_i32([0, 99]), gpu_i32([-1, 3])]
    vc.vcoll_moe_dispatch_fp8(toks, splits, src, recv)
    sync()
    assert torch.all(recv[0][0, :H] == 0) and torch.all(recv[0][1] == 7)      # row 1 came from index -1
    assert torch.all(recv[1][0] == 7) and torch.all(recv[1][1, :H] == 0)      # index 99 skipped


def test_dedup_dispatch_and_expand_equal_plain(vc):
    """Full MoE workload (p = 8, 4096 tokens x 7168 bf16, top-8 of 256):
    the deduplicated all-to-all plus the local expansion equals the plain
    dispatch bit for bit."""
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    say("plans")
    splits, src, _ = vc.vcoll_moe_plan(topk, E // p)
    su, src_u, expand = vc.vcoll_moe_plan_dedup(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(11)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    say("plain dispatch")
    plain = vc.vcoll_all_to_all(toks, splits, src_rows=[gpu_i32(s) for s in src])
    say("deduplicated dispatch + expansion")
    recv_u = vc.vcoll_all_to_all(toks, su, src_rows=[gpu_i32(s) for s in src_u])
    out = vc.vcoll_moe_expand(recv_u, [gpu_i32(e) for e in expand])
    say("token-major expansion")
    slots = [gpu_i32(vc.vcoll_moe_expand_slots(int(su[:, j].sum()), expand[j], K)) for j in range(p)]
    out_tm = vc.vcoll_moe_expand_token_major(recv_u, slots, [len(e) for e in expand], K)
    say("token-major deduplicated dispatch")
    dslots = vc.vcoll_moe_dedup_slots(su, src_u, T, K)
    recv_tm = vc.vcoll_moe_dispatch(toks, [gpu_i32(dslots[i]) for i in range(p)], su.sum(axis=0), K)
    sync()
    for j in range(p):
        assert torch.equal(out[j].view(torch.int16), plain[j].view(torch.int16))
        assert torch.equal(out_tm[j].view(torch.int16), plain[j].view(torch.int16))
        assert torch.equal(recv_tm[j].view(torch.int16), recv_u[j].view(torch.int16))
    assert int(su.sum()) < int(splits.sum())


def test_fp8_dedup_combination(vc):
    """FP8 payload over the deduplicated plan, then the byte-row expansion,
    equals the FP8 dispatch over the plain plan."""
    import torch
    p, T, K, E, H = 8, 200, 8, 256, 7168
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, _ = vc.vcoll_moe_plan(topk, E // p)
    su, src_u, expand = vc.vcoll_moe_plan_dedup(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(12)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    plain = vc.vcoll_moe_dispatch_fp8(toks, splits, [gpu_i32(s) for s in src])
    recv_u = vc.vcoll_moe_dispatch_fp8(toks, su, [gpu_i32(s) for s in src_u])
    out = vc.vcoll_moe_expand(recv_u, [gpu_i32(e) for e in expand])
    slots = [gpu_i32(vc.vcoll_moe_expand_slots(int(su[:, j].sum()), expand[j], K)) for j in range(p)]
    out_tm = vc.vcoll_moe_expand_token_major(recv_u, slots, [len(e) for e in expand], K)
    dslots = vc.vcoll_moe_dedup_slots(su, src_u, T, K)
    recv_tm = vc.vcoll_moe_dispatch(toks, [gpu_i32(dslots[i]) for i in range(p)], su.sum(axis=0), K, fp8=True)
    sync()
    for j in range(p):
        assert torch.equal(out[j], plain[j])
        assert torch.equal(out_tm[j], plain[j])
        assert torch.equal(recv_tm[j], recv_u[j])                   # FP8 quantised once per token


def test_fp8_full_workload_sampled_rows(vc):
    """Full MoE workload in FP8: 64 sampled received rows per rank against
    the oracle's quantiser applied to the token row each one carries."""
    M = workloads.MOE
    p, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, _ = vc.vcoll_moe_plan(topk, E // p)
    say("generating MoE tokens")
    toks = [workloads.moe_tokens(r, T, H) for r in range(p)]
    recv = vc.vcoll_moe_dispatch_fp8([to_gpu_bf16(t) for t in toks], splits, [gpu_i32(s) for s in src])
    sync()
    # received row x of rank j: from sender i with recv offset, token src[i][so + r]
    send_off = np.concatenate([np.zeros((p, 1), np.int64), np.cumsum(splits, axis=1)[:, :-1]], axis=1)
    rng = np.random.default_rng(1)
    for j in range(p):
        base = 0
        rows, want_tok = [], []
        for i in range(p):
            n = int(splits[i, j])
            for r in rng.choice(n, size=min(8, n), replace=False) if n else []:
                rows.append(base + int(r))
                want_tok.append((i, int(src[i][send_off[i, j] + r])))
            base += n
        got = recv[j][rows].cpu().numpy()
        want = fp8.quantize_rows(np.stack([oracle.bf16_to_f32(toks[i][t]) for i, t in want_tok]))
        assert np.array_equal(got, want), f"rank {j}"


# --------------------------------------------------------------------------- token-major dispatch

def slots_gpu(vc, splits, dst, topk):
    import torch
    s = vc.vcoll_moe_slots(splits, np.stack(dst), topk)
    return [torch.from_numpy(np.ascontiguousarray(s[i])).cuda() for i in range(len(dst))]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_major_dispatch_equals_gather_dispatch(vc, dtype):
    """Full MoE workload: reading each token once and writing it to its 8
    slots gives the plain dispatch's receive buffers bit for bit."""
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    if dtype == "f32":
        T, H = 1024, 2048 + 6                           # rows of 8216 bytes: the element path
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(13)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
            for _ in range(p)]
    say(f"gather dispatch {dtype}")
    want = vc.vcoll_all_to_all(toks, splits, src_rows=[gpu_i32(s) for s in src])
    say(f"token-major dispatch {dtype}")
    got = vc.vcoll_moe_dispatch(toks, slots_gpu(vc, splits, dst, K), splits.sum(axis=0), K)
    sync()
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for j in range(p):
        assert torch.equal(got[j].view(iv), want[j].view(iv))


def test_token_major_fp8_dispatch_equals_oracle_and_row_major(vc):
    import torch
    p, T, K, E, H = 4, 64, 3, 16, 384
    topk = small_routing(p, T, K, E, 3)
    toks = [workloads.rank_window(workloads.TAG_TEST * 1000 + 960, i, 0, T * H, ("normal", 0.0, 1.0),
                                  "bf16").reshape(T, H) for i in range(p)]
    splits, src, dst = vc.vcoll_moe_plan(np.stack(topk), E // p)
    got = vc.vcoll_moe_dispatch([to_gpu_bf16(t) for t in toks], slots_gpu(vc, splits, dst, K), splits.sum(axis=0),
                                K, fp8=True)
    sync()
    want, _ = moe.dispatch_fp8(toks, splits, list(src))
    for j in range(p):
        assert np.array_equal(got[j].cpu().numpy(), want[j]), f"rank {j}"


def test_token_major_fp8_full_workload_equals_row_major(vc):
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(14)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    want = vc.vcoll_moe_dispatch_fp8(toks, splits, [gpu_i32(s) for s in src])
    got = vc.vcoll_moe_dispatch(toks, slots_gpu(vc, splits, dst, K), splits.sum(axis=0), K, fp8=True)
    sync()
    for j in range(p):
        assert torch.equal(got[j], want[j])


def test_token_major_dispatch_skips_bad_slots(vc):
    import torch
    p, T, H, K = 2, 3, 64, 2
    toks = [torch.arange(T * H, device="cuda", dtype=torch.float32).reshape(T, H) + 1000 * i for i in range(p)]
    # rank 0: token 0 -> (1, 0) and an out-of-range rank; token 1 -> (0, 0), row 9 (too big); token 2 -> (0, 1), (1, 1)
    s0 = torch.tensor([[1, 0], [5, 0], [0, 0], [0, 9], [0, 1], [1, 1]], dtype=torch.int32, device="cuda")
    s1 = torch.full((T * K, 2), -1, dtype=torch.int32, device="cuda")
    recv = [torch.full((2, H), -7.0, device="cuda") for _ in range(p)]
    vc.vcoll_moe_dispatch(toks, [s0, s1], [2, 2], K, recv=recv)
    sync()
    assert torch.equal(recv[1][0], toks[0][0]) and torch.equal(recv[0][0], toks[0][1])
    assert torch.equal(recv[0][1], toks[0][2]) and torch.equal(recv[1][1], toks[0][2])


# --------------------------------------------------------------------------- token-major combine

@pytest.mark.parametrize("dtype,H", [("bf16", 384), ("f32", 133)])
def test_token_major_combine_matches_oracle(vc, dtype, H):
    """Pulling every (token, slot) row from the expert outputs equals the
    oracle's combine (reverse all-to-all, then the scatter to (token, slot)
    positions); f32 rows of 532 bytes take the 2-byte path."""
    import torch
    p, T, K, E = 4, 64, 3, 16
    topk = small_routing(p, T, K, E, 21)
    splits, _, dst = vc.vcoll_moe_plan(np.stack(topk), E // p)
    rows = splits.sum(axis=0)
    eo = [workloads.rank_window(workloads.TAG_TEST * 1000 + 970, j, 0, int(rows[j]) * H, ("normal", 0.0, 1.0),
                                dtype).reshape(-1, H) for j in range(p)]
    if dtype == "bf16":
        teo = [to_gpu_bf16(x) for x in eo]
    else:
        teo = [torch.from_numpy(x).cuda() for x in eo]
    say(f"vcoll_moe_combine {dtype} H={H}")
    got = vc.vcoll_moe_combine(teo, slots_gpu(vc, splits, dst, K), T, K)
    sync()
    want, _ = moe.combine(eo, splits, list(dst), K, T, dtype)
    for i in range(p):
        g = got[i].cpu()
        g = g.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else g.numpy()
        assert np.array_equal(g.view(np.uint8), want[i].view(np.uint8)), f"rank {i}"


def test_token_major_combine_full_workload(vc):
    """Full MoE workload: the token-major combine equals the scattering
    combine bit for bit, and combine(dispatch(x)) puts token t in every one
    of its topk rows."""
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(15)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    say("dispatch (gather)")
    recv = vc.vcoll_all_to_all(toks, splits, src_rows=[gpu_i32(s) for s in src])
    say("combine (scatter)")
    want = vc.vcoll_all_to_all(recv, splits.T, dst_rows=[gpu_i32(d) for d in dst], dst_table_rows=[T * K] * p)
    say("combine (token-major)")
    got = vc.vcoll_moe_combine(recv, slots_gpu(vc, splits, dst, K), T, K)
    sync()
    for i in range(p):
        assert torch.equal(got[i].view(torch.int16), want[i].view(torch.int16)), f"rank {i}"
        assert torch.equal(got[i].view(T, K, H).view(torch.int16),
                           toks[i].view(torch.int16).unsqueeze(1).expand(T, K, H)), f"identity, rank {i}"


def test_token_major_combine_skips_bad_slots(vc):
    import torch
    p, T, H, K = 2, 2, 64, 2
    eo = [torch.arange(3 * H, device="cuda", dtype=torch.float32).reshape(3, H) + 1000 * j for j in range(p)]
    # rank 0: (t0,k0) <- (1, 2); (t0,k1) <- rank 5 (no such rank); (t1,k0) <- (0, 3) (row too big); (t1,k1) <- (0, 0)
    s0 = torch.tensor([[1, 2], [5, 0], [0, 3], [0, 0]], dtype=torch.int32, device="cuda")
    s1 = torch.full((T * K, 2), -1, dtype=torch.int32, device="cuda")
    out = [torch.full((T * K, H), -7.0, device="cuda") for _ in range(p)]
    vc.vcoll_moe_combine(eo, [s0, s1], T, K, out=out)
    sync()
    assert torch.equal(out[0][0], eo[1][2]) and torch.equal(out[0][3], eo[0][0])
    assert torch.all(out[0][1] == -7.0) and torch.all(out[0][2] == -7.0) and torch.all(out[1] == -7.0)
