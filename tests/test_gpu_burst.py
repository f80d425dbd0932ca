"""The two-phase ring all-reduce (every workgroup reads its tile of all p
ranks, then writes it to all p outputs), which the library selects for ring
all-reduces whose whole vector fits in one generation of workgroups: bit for
bit against the oracle on every element, at shapes chosen to land in that
regime -- tiles that divide their chunk and tiles that do not, p that does
and does not divide the 256 compute units, float32 and bfloat16, in place
and out of place, special values."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_bits_equal, bits, download, say, upload, upload_list

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


def burst_tile(p, n, dtype, cus=256):
    """Vectors per tile the library picks, or 0 if it takes the one-pass kernel
    (the same rule as the host library, restated for the test's shapes): the
    largest count of 16-byte vectors lying wholly inside one chunk, spread
    over the compute units a chunk gets, in whole 128-byte lines. (The
    library also moves each chunk's first tile up to a 128-byte boundary,
    which can shorten a chunk by up to 7 vectors; the shapes below are far
    from the thresholds.)"""
    ve = 4 if dtype == "f32" else 8
    per_chunk = cus // p
    q, r = divmod(n, p)
    cv = 0
    for c in range(p):
        e0 = c * q + min(c, r)
        e1 = e0 + q + (c < r)
        cv = max(cv, e1 // ve - -(-e0 // ve))
    t = (-(-cv // per_chunk) + 7) // 8 * 8
    tmax = (25 if dtype == "f32" else 16) * 256
    return t if 3072 <= t <= tmax else 0


# (p, n, dtype): every shape lands in the two-phase regime on a 256-CU MI355X
CASES = [
    (8, 6_553_600, "f32"),              # the DDP bucket: 32 tiles of 6400 vectors per chunk
    (8, 4_194_304 + 8 * 4 * 37, "f32"),  # tiles that do not divide their chunk
    (2, 4_194_304, "f32"),              # 128 tiles per chunk
    (16, 4_999_936, "f32"),             # 16 tiles per chunk
    (3, 4_800_000, "f32"),              # 85 tiles per chunk, 1 compute unit left over
    (72, 4_320_000, "f32"),             # 3 tiles per chunk, run-time rank count
    (8, 7_168_000, "bf16"),             # bfloat16: 16 vectors (128 elements) per thread
    (16, 6_825_984, "bf16"),
    # chunks that are not whole vectors: each chunk's end elements go one by one
    (72, 4_194_304, "f32"),             # 16 MiB per rank: 58,254 or 58,255 elements per chunk
    (8, 6_553_604, "f32"),              # 4 chunks one element longer
    (3, 4_800_004, "f32"),
    (16, 6_826_008, "bf16"),
    (5, 7_000_008, "bf16"),
]


@pytest.mark.parametrize("p,n,dtype", CASES, ids=[f"p{p}-n{n}-{d}" for p, n, d in CASES])
def test_two_phase_ring_matches_oracle(vc, p, n, dtype):
    import torch
    assert burst_tile(p, n, dtype) > 0
    x = [workloads.rank_window(workloads.TAG_TEST * 1000 + 700 + p, r, 0, n, ("normal", 0.0, 1.0), dtype)
         for r in range(p)]
    want, _ = oracle.allreduce(x, "ring", dtype)
    want = np.stack([bits(w, dtype) for w in want])
    t = upload(x, dtype)
    say(f"two-phase ring p={p} n={n} {dtype}: out of place")
    out = vc.vcoll_allreduce("ring", t)
    torch.cuda.synchronize()
    assert_bits_equal(download(out, dtype), want, f"ring p={p} n={n} {dtype}")
    say(f"two-phase ring p={p} n={n} {dtype}: in place")
    vc.vcoll_allreduce("ring", t, t)
    torch.cuda.synchronize()
    assert_bits_equal(download(t, dtype), want, f"in-place ring p={p} n={n} {dtype}")


# separately allocated rank buffers whose length is not a whole number of
# 16-byte vectors: the last chunk's final elements share no vector with a
# neighbour and still go one by one
LIST_CASES = [(8, 6_553_601, "f32"), (8, 6_553_603, "f32"), (16, 6_825_989, "bf16"), (72, 4_194_307, "f32")]


@pytest.mark.parametrize("p,n,dtype", LIST_CASES, ids=[f"p{p}-n{n}-{d}" for p, n, d in LIST_CASES])
def test_two_phase_ring_ragged_buffer_lengths(vc, p, n, dtype):
    import torch
    assert burst_tile(p, n, dtype) > 0
    x = [workloads.rank_window(workloads.TAG_TEST * 1000 + 760 + p, r, 0, n, ("normal", 0.0, 1.0), dtype)
         for r in range(p)]
    want, _ = oracle.allreduce(x, "ring", dtype)
    send = upload_list(x, dtype)
    recv = [torch.empty_like(t) for t in send]
    say(f"two-phase ring, separate buffers, p={p} n={n} {dtype}")
    vc.vcoll_allreduce("ring", send, recv)
    torch.cuda.synchronize()
    for r in range(p):
        assert_bits_equal(download(recv[r], dtype), bits(want[r], dtype), f"rank {r}")


def test_two_phase_ring_special_values(vc):
    """Signed zeros, infinities, NaN and denormals through the two-phase
    kernel: -0 + -0 stays -0 only if the first leaf is copied, not added to 0."""
    import torch
    p, n = 8, 6_553_600
    x = [workloads.rank_window(workloads.TAG_TEST * 1000 + 750, r, 0, n, ("normal", 0.0, 1.0), "f32") for r in range(p)]
    specials = np.array([-0.0, 0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1.17e-38], dtype=np.float32)
    rng = np.random.default_rng(9)
    for r in range(p):
        idx = rng.integers(0, n, size=4096)
        x[r][idx] = specials[rng.integers(0, len(specials), size=idx.size)]
        x[r][:64] = -0.0                       # an all-negative-zero stretch
    want, _ = oracle.allreduce(x, "ring", "f32")
    say("two-phase ring with special values")
    out = vc.vcoll_allreduce("ring", upload(x, "f32"))
    torch.cuda.synchronize()
    got = download(out, "f32")
    w = np.stack(want)
    nan = np.isnan(w)
    assert np.array_equal(np.isnan(got.view(np.float32)), nan)
    assert_bits_equal(got[~nan], w.view(np.uint32)[~nan], "specials")
    assert np.all(got[:, :64] == np.uint32(0x80000000))
