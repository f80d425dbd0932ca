"""Every point of the message-size sweep (p in {2, 4, 8, 16, 72}, 1 KiB to
1 GiB per rank, four algorithms) against the oracle.

Every element is compared wherever a point's p*n is at most 1.6e9 elements
(6.4 GB of inputs): the seeded inputs and the oracle's outputs are produced
window by window by a pool of CPU workers. Beyond that (p = 8 and 16 at
1 GiB per rank, p = 72 at 256 MiB and 1 GiB) the inputs come from torch's
device generator and every chunk boundary plus 16 random windows of 1024
elements are copied back and compared; each test states the fraction of
elements it verified, and with VCOLL_PARITY_LOG set appends one JSON line
per point to that file."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pool
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

FULL_LIMIT = 1_600_000_000     # p*n elements verified in full up to here (p = 72 x 80 MiB: 1.5e9)
IN_PROCESS = 2 ** 22           # below this the oracle runs in the test process


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


@pytest.fixture(scope="module")
def pool():
    with oracle_pool.pool() as pl:
        yield pl


SIZE_GROUPS = {
    "to_4MiB": [b for b in workloads.SWEEP_BYTES if b <= 4 * 2 ** 20],
    "16_to_80MiB": [b for b in workloads.SWEEP_BYTES if 4 * 2 ** 20 < b <= 80 * 2 ** 20],
    "256MiB_to_1GiB": [b for b in workloads.SWEEP_BYTES if b > 80 * 2 ** 20],
}


def _record(p, nbytes, algo, verified, total):
    say(f"sweep p={p} {nbytes} B {algo}: verified {verified:,} of {total:,} elements "
        f"({100.0 * verified / total:.4g} %)")
    path = os.environ.get("VCOLL_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"p": p, "bytes_per_rank": nbytes, "algo": algo, "verified": verified,
                                "total": total}) + "\n")


def _full(vc, pool, p, n, nbytes):
    """Seeded workloads inputs, every element of every algorithm's output."""
    import torch
    tag, dist = workloads.TAG_SWEEP, workloads.SWEEP_DIST
    if p * n <= IN_PROCESS:
        x = np.stack([workloads.rank_window(tag, r, 0, n, dist, "f32") for r in range(p)])
        t = torch.from_numpy(x).cuda()
    else:
        t = torch.empty((p, n), dtype=torch.float32, device="cuda")
        wins = oracle_pool.windows(n, oracle_pool.window_len(p))
        for lo, hi, xw in pool.imap(oracle_pool.gen_window, [(tag, p, lo, hi, dist, "f32") for lo, hi in wins]):
            t[:, lo:hi].copy_(torch.from_numpy(xw))
    outs = {}
    for algo in oracle.ALGOS:
        outs[algo] = vc.vcoll_allreduce(algo, t)
    torch.cuda.synchronize()
    checked = {a: 0 for a in oracle.ALGOS}
    if p * n <= IN_PROCESS:
        for algo in oracle.ALGOS:
            want, _ = oracle.allreduce(list(x), algo, "f32")
            got = outs[algo].cpu().numpy().view(np.uint32)
            bad = np.flatnonzero(got.ravel() != np.stack(want).view(np.uint32).ravel())
            assert bad.size == 0, f"p={p} {nbytes} B {algo}: {bad.size} differ, first {bad[:3]}"
            checked[algo] = p * n
    else:
        jobs = [(tag, p, n, lo, hi, dist, "f32", oracle.ALGOS) for lo, hi in wins]
        for lo, hi, want in pool.imap(oracle_pool.oracle_window, jobs):
            for algo in oracle.ALGOS:
                got = outs[algo][:, lo:hi].cpu().numpy().view(np.uint32)
                bad = np.flatnonzero(got.ravel() != want[algo].ravel())
                assert bad.size == 0, f"p={p} {nbytes} B {algo} window [{lo},{hi}): {bad.size} differ"
                checked[algo] += p * (hi - lo)
    for algo in oracle.ALGOS:
        assert checked[algo] == p * n
        _record(p, nbytes, algo, checked[algo], p * n)
    del t, outs


def _sampled(vc, p, n, nbytes):
    """Device-generated inputs; every chunk boundary and 16 random windows."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(workloads.TAG_SWEEP * 10 ** 6 + p * 1000 + nbytes % 997)
    t = torch.randn((p, n), device="cuda", generator=g)
    o = torch.empty_like(t)
    w = min(1024, n)
    rng = np.random.default_rng([p, nbytes])
    offs = oracle.chunk_bounds(n, p)
    wins = sorted({(max(0, min(b - w // 2, n - w)), max(0, min(b - w // 2, n - w)) + w) for b in offs[1:-1]} |
                  {(int(s0), int(s0) + w) for s0 in rng.integers(0, n - w + 1, size=16)})
    covered = np.zeros(0, dtype=np.int64)
    for lo, hi in wins:
        covered = np.union1d(covered, np.arange(lo, hi))
    for algo in oracle.ALGOS:
        vc.vcoll_allreduce(algo, t, o)
        torch.cuda.synchronize()
        for r in range(1, p):
            assert torch.equal(o[r].view(torch.int32), o[0].view(torch.int32)), f"p={p} {algo}: rank {r} != 0"
        for lo, hi in wins:
            xw = [t[r, lo:hi].cpu().numpy() for r in range(p)]
            want, _ = oracle.allreduce(xw, algo, "f32", n=n, lo=lo)
            got = o[:, lo:hi].cpu().numpy().view(np.uint32)
            assert np.array_equal(got, np.stack(want).view(np.uint32)), f"p={p} {nbytes} B {algo} window [{lo},{hi})"
        _record(p, nbytes, algo, p * covered.size, p * n)
    del t, o


@pytest.mark.parametrize("sizes", list(SIZE_GROUPS))
@pytest.mark.parametrize("p", workloads.SWEEP_P)
def test_sweep_points_match_oracle(vc, pool, p, sizes):
    import torch
    for nbytes in SIZE_GROUPS[sizes]:
        n = nbytes // 4
        say(f"sweep parity p={p} bytes={nbytes}")
        if p * n <= FULL_LIMIT:
            _full(vc, pool, p, n, nbytes)
        else:
            _sampled(vc, p, n, nbytes)
        torch.cuda.empty_cache()
