"""The windowed oracle pool used by the full-size GPU parity tests: its
windows, regenerated inputs and expected values put together equal one
oracle run over the whole vectors (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pool


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_windows_equal_the_whole_vector_oracle(dtype):
    p, n, tag, dist = 5, 30_011, workloads.TAG_TEST, ("uniform", -1.0, 1.0)
    x = [workloads.rank_window(tag, r, 0, n, dist, dtype) for r in range(p)]
    wins = oracle_pool.windows(n, 4093)
    assert wins[0][0] == 0 and wins[-1][1] == n
    assert all(a[1] == b[0] for a, b in zip(wins, wins[1:]))
    with oracle_pool.pool(2) as pool:
        gen = list(pool.imap(oracle_pool.gen_window, [(tag, p, lo, hi, dist, dtype) for lo, hi in wins]))
        res = list(pool.imap(oracle_pool.oracle_window,
                             [(tag, p, n, lo, hi, dist, dtype, oracle.ALGOS) for lo, hi in wins]))
    assert np.array_equal(np.concatenate([g[2] for g in gen], axis=1), np.stack(x))
    for algo in oracle.ALGOS:
        want, _ = oracle.allreduce(x, algo, dtype)
        got = np.concatenate([r[2][algo] for r in res], axis=1)
        assert np.array_equal(got, np.stack(want).view(got.dtype)), algo
