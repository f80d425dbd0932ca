"""The collectives under HIP graph capture: the library enqueues kernels only
(no allocation, no memset, no synchronisation), so a captured sequence
replays with the same results. Each replay is checked against the eager
result, with eager work and synchronisations between replays."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


def test_captured_allreduces_replay_exactly(vc):
    import torch
    p, n = 8, 2560                                       # 10 KiB per rank: decode-sized
    g = torch.Generator(device="cuda").manual_seed(21)
    x = torch.randn((p, n), device="cuda", generator=g)
    y = torch.randn((16, 1 << 16), device="cuda", generator=g).to(torch.bfloat16)
    # the two-phase ring kernel (chunks one element apart) and a broadcast fan-out
    z = torch.randn((8, 3_276_804), device="cuda", generator=g)
    bsrc = torch.randn(1 << 20, device="cuda", generator=g)
    outs = {a: torch.empty_like(x) for a in ("ring", "rd", "rabenseifner", "tree")}
    oy, oz = torch.empty_like(y), torch.empty_like(z)
    ob = torch.empty((8, 1 << 20), device="cuda")
    # eager results
    want = {a: vc.vcoll_allreduce(a, x).clone() for a in outs}
    want_y = vc.vcoll_allreduce("rabenseifner", y).clone()
    want_z = vc.vcoll_allreduce("ring", z).clone()
    stepwise_want, _ = vc.vcoll_allreduce_stepwise("ring", x)
    stepwise_want = stepwise_want.clone()
    so = torch.empty_like(x)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vc.vcoll_allreduce("ring", x, outs["ring"])          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    say("capturing")
    with torch.cuda.graph(graph):
        for a, o in outs.items():
            vc.vcoll_allreduce(a, x, o)
        vc.vcoll_allreduce("rabenseifner", y, oy)
        vc.vcoll_allreduce_stepwise("ring", x, so)
        vc.vcoll_allreduce("ring", z, oz)
        vc.vcoll_broadcast(bsrc, ob, 0)
    for rep in range(4):
        for o in list(outs.values()) + [oy, so, oz, ob]:
            o.fill_(float("nan"))                        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, o in outs.items():
            assert torch.equal(o.view(torch.int32), want[a].view(torch.int32)), (rep, a)
        assert torch.equal(oy.view(torch.int16), want_y.view(torch.int16)), rep
        assert torch.equal(so.view(torch.int32), stepwise_want.view(torch.int32)), rep
        assert torch.equal(oz.view(torch.int32), want_z.view(torch.int32)), rep
        assert all(torch.equal(ob[r].view(torch.int32), bsrc.view(torch.int32)) for r in range(8)), rep


def test_captured_all_to_all_and_moe_dispatch_replay(vc):
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], 256, 512, M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    slots = vc.vcoll_moe_slots(splits, dst, K)
    g = torch.Generator(device="cuda").manual_seed(22)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    srcg = [torch.from_numpy(s).cuda() for s in src]
    dstg = [torch.from_numpy(d).cuda() for d in dst]
    slg = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in slots]
    recv = vc.vcoll_all_to_all(toks, splits, src_rows=srcg)
    back = vc.vcoll_all_to_all(recv, splits.T, dst_rows=dstg, dst_table_rows=[T * K] * p)
    push = vc.vcoll_moe_dispatch(toks, slg, splits.sum(axis=0), K)
    f8 = vc.vcoll_moe_dispatch(toks, slg, splits.sum(axis=0), K, fp8=True)
    want = [r.clone() for r in recv] + [b.clone() for b in back] + [q.clone() for q in push] + [q.clone() for q in f8]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vc.vcoll_all_to_all(toks, splits, recv=recv, src_rows=srcg)
        vc.vcoll_all_to_all(recv, splits.T, recv=back, dst_rows=dstg)
        vc.vcoll_moe_dispatch(toks, slg, splits.sum(axis=0), K, recv=push)
        vc.vcoll_moe_dispatch(toks, slg, splits.sum(axis=0), K, fp8=True, recv=f8)
    got = recv + back + push + f8
    for rep in range(3):
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep


def test_captured_plain_all_to_all_combine_and_dedup_replay(vc):
    """The index-free all-to-all (1024-thread path), the token-major combine,
    the token-major deduplicated dispatch (bf16 and FP8) and the token-major
    expansion (one launch per rank), captured once and replayed three times
    with the outputs cleared in between: every replay equals the eager run."""
    import torch
    M = workloads.MOE
    p, T, H, E, K = M["p"], 256, 512, M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    slots = vc.vcoll_moe_slots(splits, dst, K)
    su, src_u, expand = vc.vcoll_moe_plan_dedup(topk, E // p)
    g = torch.Generator(device="cuda").manual_seed(23)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p)]
    plain_send = [torch.randn((int(splits[i].sum()), H), device="cuda", generator=g).to(torch.bfloat16)
                  for i in range(p)]
    slg = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in slots]
    dsl = vc.vcoll_moe_dedup_slots(su, src_u, T, K)
    dslg = [torch.from_numpy(np.ascontiguousarray(dsl[i])).cuda() for i in range(p)]
    urows = su.sum(axis=0)
    xsl = [torch.from_numpy(vc.vcoll_moe_expand_slots(int(urows[j]), expand[j], K)).cuda() for j in range(p)]
    counts = [len(e) for e in expand]
    plain = vc.vcoll_all_to_all(plain_send, splits)
    push = vc.vcoll_moe_dispatch(toks, slg, splits.sum(axis=0), K)
    comb = vc.vcoll_moe_combine(push, slg, T, K)
    du = vc.vcoll_moe_dispatch(toks, dslg, urows, K)
    du8 = vc.vcoll_moe_dispatch(toks, dslg, urows, K, fp8=True)
    ex = vc.vcoll_moe_expand_token_major(du, xsl, counts, K)
    want = [t.clone() for t in plain + comb + du + du8 + ex]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vc.vcoll_all_to_all(plain_send, splits, recv=plain)
        vc.vcoll_moe_combine(push, slg, T, K, out=comb)
        vc.vcoll_moe_dispatch(toks, dslg, urows, K, recv=du)
        vc.vcoll_moe_dispatch(toks, dslg, urows, K, fp8=True, recv=du8)
        vc.vcoll_moe_expand_token_major(du, xsl, counts, K, out=ex)
    got = plain + comb + du + du8 + ex
    for rep in range(3):
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
