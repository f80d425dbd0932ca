"""Every point of the message-size sweep (p in {2, 4, 8, 16, 72}, 1 KiB to
1 GiB per rank, four algorithms) against the oracle: the whole vector where
p*n <= 2^25 elements, else every chunk boundary plus 16 random windows of
1024 elements (inputs too large to draw on the host come from torch's
device generator and are copied back window by window)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


SIZE_GROUPS = {
    "to_4MiB": [b for b in workloads.SWEEP_BYTES if b <= 4 * 2 ** 20],
    "16_to_80MiB": [b for b in workloads.SWEEP_BYTES if 4 * 2 ** 20 < b <= 80 * 2 ** 20],
    "256MiB_to_1GiB": [b for b in workloads.SWEEP_BYTES if b > 80 * 2 ** 20],
}


@pytest.mark.parametrize("sizes", list(SIZE_GROUPS))
@pytest.mark.parametrize("p", workloads.SWEEP_P)
def test_sweep_points_match_oracle(vc, p, sizes):
    import torch
    for nbytes in SIZE_GROUPS[sizes]:
        n = nbytes // 4
        host = p * n <= 2 ** 25
        say(f"sweep parity p={p} bytes={nbytes}")
        if host:
            x = [workloads.rank_window(workloads.TAG_SWEEP, r, 0, n, workloads.SWEEP_DIST, "f32") for r in range(p)]
            t = torch.from_numpy(np.stack(x)).cuda()
        else:
            g = torch.Generator(device="cuda").manual_seed(workloads.TAG_SWEEP * 10 ** 6 + p * 1000 + nbytes % 997)
            t = torch.randn((p, n), device="cuda", generator=g)
        o = torch.empty_like(t)
        w = min(1024, n)
        rng = np.random.default_rng([p, nbytes])
        offs = oracle.chunk_bounds(n, p)
        wins = sorted({(max(0, min(b - w // 2, n - w)), max(0, min(b - w // 2, n - w)) + w) for b in offs[1:-1]} |
                      {(int(s0), int(s0) + w) for s0 in rng.integers(0, n - w + 1, size=16)})
        for algo in oracle.ALGOS:
            vc.vcoll_allreduce(algo, t, o)
            torch.cuda.synchronize()
            if host:
                want, _ = oracle.allreduce(x, algo, "f32")
                got = o.cpu().numpy().view(np.uint32)
                bad = np.flatnonzero(got.ravel() != np.stack(want).view(np.uint32).ravel())
                assert bad.size == 0, f"p={p} {nbytes} B {algo}: {bad.size} differ, first {bad[:3]}"
            else:
                for lo, hi in wins:
                    xw = [t[r, lo:hi].cpu().numpy() for r in range(p)]
                    want, _ = oracle.allreduce(xw, algo, "f32", n=n, lo=lo)
                    got = o[:, lo:hi].cpu().numpy().view(np.uint32)
                    assert np.array_equal(got, np.stack(want).view(np.uint32)), \
                        f"p={p} {nbytes} B {algo} window [{lo},{hi})"
        del t, o
        torch.cuda.empty_cache()
