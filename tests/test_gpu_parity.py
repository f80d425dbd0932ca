"""GPU parity: libvcoll's HIP kernels against the CPU oracle, bit for bit.

Every collective result is compared element by element with the oracle on
the same seeded inputs: small cases that span several tiles of every kernel
with ragged chunk edges, the pages' worked example and order probes, and the
full-size workloads (all elements where the oracle finishes in seconds,
sampled windows of the oracle's windowed mode beyond that).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_bits_equal, bits, dev, download, say, upload

pytestmark = pytest.mark.gpu

ALGOS = oracle.ALGOS


@pytest.fixture(scope="module")
def vc():
    import torch
    assert torch.cuda.is_available()
    import collective_communication_algorithms_vcoll_amd as m
    return m


def sync():
    import torch
    torch.cuda.synchronize()


def ragged_n(p: int) -> int:
    # each chunk spans three 2048-element tiles plus a tail, and chunk starts
    # are not multiples of the 16-byte vector width
    return p * (3 * 2048 + 13) + p // 2 + 1


def rand_inputs(p, n, dtype, seed, dist=("normal", 0.0, 1.0)):
    return [workloads.rank_window(workloads.TAG_TEST * 1000 + seed, r, 0, n, dist, dtype) for r in range(p)]


def gpu_allreduce(vc, algo, x, dtype):
    t = upload(x, dtype)
    say(f"vcoll_allreduce algo={algo} p={len(x)} n={len(x[0])} dtype={dtype}")
    out = vc.vcoll_allreduce(algo, t)
    sync()
    return download(out, dtype)


# --------------------------------------------------------------------------- pages' examples

def test_worked_example(vc):
    x = workloads.worked_example()
    for algo in ALGOS:
        got = gpu_allreduce(vc, algo, x, "f32")
        for r in range(4):
            assert got[r].view(np.float32).tolist() == [60, 64, 68, 72], algo
    t = upload(x, "f32")
    rs = vc.vcoll_reduce_scatter("ring", t)
    ag = vc.vcoll_all_gather("ring", t)
    send = [t[r].reshape(4, 1) for r in range(4)]
    recv = vc.vcoll_all_to_all(send, np.ones((4, 4), dtype=np.int64))
    sync()
    assert [r.cpu().tolist() for r in rs] == [[60.0], [64.0], [68.0], [72.0]]
    for r in range(4):
        assert ag[r].cpu().tolist() == [float(v) for v in [0, 1, 2, 3, 10, 11, 12, 13, 20, 21, 22, 23, 30, 31, 32, 33]]
    assert [r.cpu().ravel().tolist() for r in recv] == [[j, 10 + j, 20 + j, 30 + j] for j in range(4)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order_probes(vc, dtype):
    probe = [2.0 ** 24, 1.0, -(2.0 ** 24), 1.0]
    expect = {"ring": [2, 2, 0, 1], "rd": [1, 1, 1, 1], "tree": [1, 1, 1, 1], "rabenseifner": [2, 2, 2, 2]}
    x = [np.full(4, v, dtype=np.float32) for v in probe]
    if dtype == "bf16":
        x = [oracle.f32_to_bf16(v) for v in x]
    for algo, want in expect.items():
        got = gpu_allreduce(vc, algo, x, dtype)
        vals = got.view(np.float32) if dtype == "f32" else oracle.bf16_to_f32(got)
        for r in range(4):
            assert vals[r].tolist() == want, (algo, r)


# --------------------------------------------------------------------------- all-reduce parity

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 72])
@pytest.mark.parametrize("algo", ALGOS)
def test_allreduce_matches_oracle(vc, algo, p, dtype):
    n = ragged_n(p) if p <= 16 else 72 * 2500 + 41
    x = rand_inputs(p, n, dtype, seed=p)
    want, _ = oracle.allreduce(x, algo, dtype)
    got = gpu_allreduce(vc, algo, x, dtype)
    for r in range(p):
        assert_bits_equal(got[r], bits(want[r], dtype), f"{algo} p={p} rank {r}")


@pytest.mark.parametrize("p", [9, 10, 11, 13, 15, 17, 24, 31, 33, 63, 100, 127])
def test_allreduce_run_time_programs_over_many_p(vc, p):
    """p without a compiled program, chosen so that the fold of recursive
    doubling and Rabenseifner pairs 1, 2, 3, 5, 7, 8, 15, 17, 31, 36 and 63
    ranks (p - 2^floor(log2 p)); chunks of about 1500 elements (the vector
    path, heads and tails ragged) and of about 300 (the LDS-staged path);
    float32 and bfloat16; every algorithm and the ring reduce-scatter."""
    for n in (p * 1500 + 13, p * 300 + 5):
        for dtype in ("f32", "bf16"):
            x = rand_inputs(p, n, dtype, seed=600 + p)
            t = upload(x, dtype)
            for algo in ALGOS:
                say(f"vcoll_allreduce p={p} n={n} {algo} {dtype}")
                want, _ = oracle.allreduce(x, algo, dtype)
                got = download(vc.vcoll_allreduce(algo, t), dtype)
                assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"{algo} p={p} n={n} {dtype}")
            rs = vc.vcoll_reduce_scatter("ring", t)
            sync()
            want, _ = oracle.reduce_scatter(x, "ring", dtype)
            for c in range(p):
                assert_bits_equal(download(rs[c], dtype), bits(want[c], dtype), f"rs p={p} chunk {c}")


@pytest.mark.parametrize("p,n", [(8, 1), (8, 7), (8, 8), (16, 9), (72, 5), (3, 2), (128, 300)])
def test_allreduce_tiny_and_max_p(vc, p, n):
    for dtype in ("f32", "bf16"):
        x = rand_inputs(p, n, dtype, seed=n)
        for algo in ALGOS:
            want, _ = oracle.allreduce(x, algo, dtype)
            got = gpu_allreduce(vc, algo, x, dtype)
            assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"{algo} p={p} n={n}")


# element path: compiled p, run-time p (batches of 16 ranks), several tiles
# per chunk with a ragged end
UNALIGNED_SHAPES = [(8, 5000), (5, 70001), (16, 100003), (72, 30011)]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("p,n", UNALIGNED_SHAPES, ids=[f"p{p}-n{n}" for p, n in UNALIGNED_SHAPES])
def test_allreduce_unaligned_buffers_use_element_path(vc, algo, p, n):
    import torch
    if algo == "rabenseifner" and p & (p - 1):
        pytest.skip("halving and doubling need a power-of-two p")
    for dtype in ("f32", "bf16"):
        x = rand_inputs(p, n, dtype, seed=11 + p)
        want, _ = oracle.allreduce(x, algo, dtype)
        big = upload([np.concatenate([v[:1], v]) for v in x], dtype)
        send = [big[r, 1:] for r in range(p)]                 # 1 element off 16-byte alignment
        out_big = torch.zeros_like(big)
        recv = [out_big[r, 1:] for r in range(p)]
        say(f"unaligned vcoll_allreduce algo={algo} p={p} n={n} dtype={dtype}")
        vc.vcoll_allreduce(algo, send, recv)
        sync()
        got = download(out_big, dtype)
        assert_bits_equal(got[:, 1:], np.stack([bits(w, dtype) for w in want]), f"unaligned {algo} {dtype}")
        assert not got[:, 0].any(), "element before the buffers written"


@pytest.mark.parametrize("algo", ["ring", "rabenseifner"])
@pytest.mark.parametrize("p,n", UNALIGNED_SHAPES, ids=[f"p{p}-n{n}" for p, n in UNALIGNED_SHAPES])
def test_reduce_scatter_unaligned_buffers_use_element_path(vc, algo, p, n):
    import torch
    if algo == "rabenseifner" and p & (p - 1):
        pytest.skip("halving and doubling need a power-of-two p")
    for dtype in ("f32", "bf16"):
        x = rand_inputs(p, n, dtype, seed=23 + p)
        want, _ = oracle.reduce_scatter(x, algo, dtype)
        big = upload([np.concatenate([v[:1], v]) for v in x], dtype)
        send = [big[r, 1:] for r in range(p)]
        outs = [torch.zeros(len(w) + 1, dtype=big.dtype, device=big.device) for w in want]
        recv = [o[1:] for o in outs]
        say(f"unaligned vcoll_reduce_scatter algo={algo} p={p} n={n} dtype={dtype}")
        vc.vcoll_reduce_scatter(algo, send, recv)
        sync()
        for r in range(p):
            got = download(outs[r], dtype)
            assert_bits_equal(got[1:], bits(want[r], dtype), f"unaligned RS {algo} rank {r} {dtype}")
            assert got[0] == 0, "element before the output written"


@pytest.mark.parametrize("algo", ALGOS)
def test_allreduce_in_place(vc, algo):
    p, n = 8, ragged_n(8)
    x = rand_inputs(p, n, "f32", seed=3)
    want, _ = oracle.allreduce(x, algo, "f32")
    t = upload(x, "f32")
    say(f"in-place vcoll_allreduce algo={algo}")
    vc.vcoll_allreduce(algo, t, t)
    sync()
    assert_bits_equal(download(t, "f32"), np.stack([bits(w, "f32") for w in want]), f"in place {algo}")


def test_special_values(vc):
    # denormals stay denormal, infinities and signed zeros follow IEEE
    p, n = 4, 4096
    rng = np.random.default_rng(7)
    specials = np.array([1e-40, -1e-40, 1.4e-45, -0.0, 0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-38],
                        dtype=np.float32)
    x = [specials[rng.integers(0, len(specials), n)] for _ in range(p)]
    for algo in ALGOS:
        want, _ = oracle.allreduce(x, algo, "f32")
        got = gpu_allreduce(vc, algo, x, "f32")
        w = np.stack(want)
        nan = np.isnan(w)
        assert_bits_equal(got[~nan], bits(w[~nan], "f32"), f"specials {algo}")
        assert np.all(np.isnan(got.view(np.float32)[nan]))


def test_bf16_rounding_of_kernel_matches_oracle(vc):
    # float32 sums whose lower halves sit at and around the rounding
    # midpoint, for every upper half: the kernel's one rounding to bf16 must
    # match the oracle's routine
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    f = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    f = f[~np.isnan(f)]
    # bf16 inputs can only hold bf16 values; split each float32 into two bf16
    # parts a + b with a = RNE(f) and b = RNE(f - a); the kernel sums them in
    # float32 (exact when no overflow) and rounds once, like the oracle
    a = oracle.f32_to_bf16(f)
    f = f[np.isfinite(oracle.bf16_to_f32(a))]          # keep inf - inf (NaN payloads) out
    a = oracle.f32_to_bf16(f)
    b = oracle.f32_to_bf16((f - oracle.bf16_to_f32(a)).astype(np.float32))
    x = [a, b]
    for algo in ("ring", "tree"):
        want, _ = oracle.allreduce(x, algo, "bf16")
        got = gpu_allreduce(vc, algo, x, "bf16")
        assert_bits_equal(got[0], want[0], f"bf16 rounding {algo}")


def test_determinism(vc):
    p, n = 16, ragged_n(16)
    x = rand_inputs(p, n, "bf16", seed=5)
    t = upload(x, "bf16")
    ref = None
    for algo in ALGOS:
        outs = []
        for _ in range(3):
            say(f"repeat vcoll_allreduce {algo}")
            outs.append(download(vc.vcoll_allreduce(algo, t), "bf16"))
        sync()
        assert all(np.array_equal(o, outs[0]) for o in outs)
        ref = outs[0]
    assert ref is not None


def test_guard_bands_and_poison(vc):
    import torch
    p, n = 8, ragged_n(8)
    x = rand_inputs(p, n, "f32", seed=9)
    want, _ = oracle.allreduce(x, "ring", "f32")
    guard = 64
    t = upload(x, "f32")
    out = torch.full((p, n + 2 * guard), float("nan"), device=dev())
    out[:, :guard] = 1234.5
    out[:, -guard:] = -4321.5
    recv = [out[r, guard:guard + n] for r in range(p)]
    say("guarded vcoll_allreduce ring")
    vc.vcoll_allreduce("ring", t, recv)
    sync()
    o = out.cpu().numpy()
    assert np.all(o[:, :guard] == 1234.5) and np.all(o[:, -guard:] == -4321.5)
    assert_bits_equal(o[:, guard:guard + n].view(np.uint32), np.stack([bits(w, "f32") for w in want]), "guarded")


# --------------------------------------------------------------------------- reduce-scatter / all-gather

# Rabenseifner's reduce-scatter and recursive doubling's all-gather exist for
# powers of two only (other p return VCOLL_ERR_UNSUPPORTED, tested below)
RS_CASES = [("ring", p) for p in (1, 2, 3, 4, 8, 16, 72)] + [("rabenseifner", p) for p in (1, 2, 4, 8, 16)]
AG_CASES = [("ring", p) for p in (1, 2, 3, 4, 8, 16, 72)] + [("rd", p) for p in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo,p", RS_CASES)
def test_reduce_scatter_matches_oracle(vc, algo, p, dtype):
    for n in (ragged_n(p) if p <= 16 else 72 * 2500 + 41, p * 2048 * 3):   # ragged and aligned chunks
        x = rand_inputs(p, n, dtype, seed=p + 100)
        want, _ = oracle.reduce_scatter(x, algo, dtype)
        t = upload(x, dtype)
        say(f"vcoll_reduce_scatter algo={algo} p={p} n={n} dtype={dtype}")
        got = vc.vcoll_reduce_scatter(algo, t)
        sync()
        for c in range(p):
            assert_bits_equal(download(got[c], dtype), bits(want[c], dtype), f"RS {algo} p={p} chunk {c}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [3, 5, 12, 24, 72, 128])
def test_reduce_scatter_with_unaligned_chunk_starts(vc, p, dtype):
    """Ring reduce-scatter at a p without a compiled program where chunk
    starts are not 16-byte aligned: the vector path realigns every rank's
    loads to the output (every shift of 1..VE-1 elements occurs across the
    chunks), the last vectors and the ragged end go through the element path."""
    ve = 4 if dtype == "f32" else 8
    for n in (p * (3 * 1024 + 5) + 3, p * 777 + p - 1, p * 2 * ve + 1):
        x = rand_inputs(p, n, dtype, seed=p + 500 + n % 97)
        want, _ = oracle.reduce_scatter(x, "ring", dtype)
        offs = oracle.chunk_bounds(n, p)
        assert {o % ve for o in offs[:-1]} - {0}, "no unaligned chunk start"
        t = upload(x, dtype)
        say(f"vcoll_reduce_scatter ring p={p} n={n} dtype={dtype} (unaligned chunk starts)")
        got = vc.vcoll_reduce_scatter("ring", t)
        sync()
        for c in range(p):
            assert_bits_equal(download(got[c], dtype), bits(want[c], dtype), f"RS ring p={p} n={n} chunk {c}")


@pytest.mark.parametrize("pad", [20, 4], ids=["common-line-phase", "phases-differ"])
def test_reduce_scatter_unaligned_chunk_starts_line_aligned_waves(vc, pad):
    """The same at a size whose grid spans many workgroup generations, where
    f32 takes the wave shape that starts every wave on a 128-byte line of the
    inputs (pad 20: rows a whole number of lines apart, so every row has the
    same address mod 128) or, when the rows' phases differ (pad 4: rows 64
    bytes apart mod 128), on 16-byte bounds."""
    import torch
    p, n = 24, 16_777_216 + 12                       # 64 MiB per rank, chunks of 699,051 or 699,050
    x = rand_inputs(p, n, "f32", seed=611 + pad)
    want, _ = oracle.reduce_scatter(x, "ring", "f32")
    offs = oracle.chunk_bounds(n, p)
    assert {o % 4 for o in offs[:-1]} - {0}, "no unaligned chunk start"
    big = torch.zeros((p, n + pad), dtype=torch.float32, device="cuda")
    big[:, :n].copy_(torch.from_numpy(np.stack(x)))
    send = [big[r, :n] for r in range(p)]
    say(f"vcoll_reduce_scatter ring p={p} n={n} row pad {pad} (line-aligned waves)")
    got = vc.vcoll_reduce_scatter("ring", send)
    sync()
    for c in range(p):
        assert_bits_equal(download(got[c], "f32"), bits(want[c], "f32"), f"RS ring p={p} pad {pad} chunk {c}")


def test_allreduce_rows_sharing_only_a_line_phase(vc):
    """Rank rows 128 bytes apart mod 256 (a [8, n] tensor with n = 32 mod
    64): the tiles start on a 128-byte line of every row instead; every
    algorithm against the oracle."""
    p, n = 8, 4_194_304 + 32
    x = rand_inputs(p, n, "f32", 651)
    t = upload(x, "f32")
    assert t.stride(0) * 4 % 256 == 128
    for algo in ALGOS:
        say(f"all-reduce p={p} n={n} {algo}, rows sharing a line phase only")
        want, _ = oracle.allreduce(x, algo, "f32")
        got = download(vc.vcoll_allreduce(algo, t), "f32")
        assert_bits_equal(got, np.stack([bits(w, "f32") for w in want]), f"{algo} p={p}")


@pytest.mark.parametrize("pad", [20, 4], ids=["common-line-phase", "phases-differ"])
def test_reduce_scatter_aligned_chunk_starts_line_aligned_waves(vc, pad):
    """Chunks that all start on 16-byte bounds, at a size with as many waves
    (f32, run-time p): they take the same line-aligned wave shape with no
    shift (every output vector is a lane's own sum), the chunk's last vector
    and ragged end element by element."""
    import torch
    p, n = 24, 24 * 4 * 174_763                      # chunks of 699,052 elements, all 16-byte aligned
    x = rand_inputs(p, n, "f32", seed=631 + pad)
    want, _ = oracle.reduce_scatter(x, "ring", "f32")
    offs = oracle.chunk_bounds(n, p)
    assert all(o % 4 == 0 for o in offs), "an unaligned chunk start"
    big = torch.zeros((p, n + pad), dtype=torch.float32, device="cuda")
    big[:, :n].copy_(torch.from_numpy(np.stack(x)))
    send = [big[r, :n] for r in range(p)]
    say(f"vcoll_reduce_scatter ring p={p} n={n} row pad {pad} (aligned, line-aligned waves)")
    got = vc.vcoll_reduce_scatter("ring", send)
    sync()
    for c in range(p):
        assert_bits_equal(download(got[c], "f32"), bits(want[c], "f32"), f"RS ring p={p} pad {pad} chunk {c}")


def test_non_power_of_two_halving_and_doubling_are_refused(vc):
    import torch
    t = torch.zeros(3, 96, device="cuda")
    with pytest.raises(vc.VcollError, match="unsupported"):
        vc.vcoll_reduce_scatter("rabenseifner", t)
    with pytest.raises(vc.VcollError, match="unsupported"):
        vc.vcoll_all_gather("rd", t)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo,p", AG_CASES)
def test_all_gather_matches_oracle(vc, algo, p, dtype):
    for m in (1, 37, 4096, 5 * 2048 + 8):
        x = rand_inputs(p, m, dtype, seed=m)
        want, _ = oracle.all_gather(x, algo, dtype)
        t = upload(x, dtype)
        say(f"vcoll_all_gather algo={algo} p={p} m={m} dtype={dtype}")
        got = download(vc.vcoll_all_gather(algo, t), dtype)
        sync()
        assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"AG {algo} p={p} m={m}")


@pytest.mark.parametrize("m_extra", [4, 1])
def test_all_gather_beyond_1gib_written(vc, m_extra):
    """The all-gather's shape for launches that write more than 1 GiB (one
    vector per thread, cached stores): p = 8 float32 blocks of 2^22 + m_extra
    elements, 16-byte multiples (vector path, last tile partial) and an odd
    count (element path). Every output block of every rank is compared with
    its source block at both ends and at random windows."""
    p, m = 8, (1 << 22) + m_extra
    assert p * p * m * 4 > 1 << 30
    x = rand_inputs(p, m, "f32", seed=90 + m_extra)
    t = upload(x, "f32")
    say(f"vcoll_all_gather ring p={p} m={m} f32 (more than 1 GiB written)")
    out = vc.vcoll_all_gather("ring", t)
    sync()
    rng = np.random.default_rng(7)
    w = 4099
    for r in range(p):
        for b in range(p):
            for lo in (0, m - w, *rng.integers(0, m - w, size=3)):
                lo = int(lo)
                got = out[r, b * m + lo: b * m + lo + w].cpu().numpy().view(np.uint32)
                assert_bits_equal(got, bits(x[b][lo:lo + w], "f32"), f"AG rank {r} block {b} at {lo}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [4, 8, 16])
def test_allreduce_is_reduce_scatter_then_all_gather_on_gpu(vc, p, dtype):
    n = p * 4096
    x = rand_inputs(p, n, dtype, seed=21)
    t = upload(x, dtype)
    for rs_algo, ag_algo, ar_algo in (("ring", "ring", "ring"), ("rabenseifner", "rd", "rabenseifner")):
        say(f"identity {ar_algo} p={p} {dtype}")
        rs = vc.vcoll_reduce_scatter(rs_algo, t)
        ag = vc.vcoll_all_gather(ag_algo, rs)
        ar = vc.vcoll_allreduce(ar_algo, t)
        sync()
        assert_bits_equal(download(ag, dtype), download(ar, dtype), f"AR == AG o RS ({ar_algo})")


# --------------------------------------------------------------------------- all-to-all

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p,H", [(2, 8), (3, 5), (4, 256), (8, 7168), (8, 33), (16, 64), (72, 24), (128, 8),
                                 (72, 5)])
def test_all_to_all_matches_oracle(vc, p, H, dtype):
    rng = np.random.default_rng(p * H)
    splits = rng.integers(0, 40 if p <= 16 else 4, size=(p, p))    # large p: many empty blocks
    splits[0, 1 % p] = 0
    splits[p - 1, :] = 0 if p > 2 else splits[p - 1, :]
    send = [rand_inputs(1, int(splits[i].sum()) * H, dtype, seed=i + 31)[0].reshape(-1, H) for i in range(p)]
    want, _ = oracle.all_to_all(send, splits, dtype)
    tsend = [upload([s.ravel()], dtype)[0].reshape(-1, H) for s in send]
    say(f"vcoll_all_to_all p={p} H={H} dtype={dtype}")
    got = vc.vcoll_all_to_all(tsend, splits)
    back = vc.vcoll_all_to_all(got, splits.T)
    sync()
    for j in range(p):
        assert_bits_equal(download(got[j], dtype), bits(want[j], dtype), f"A2A recv {j}")
        assert_bits_equal(download(back[j], dtype), bits(send[j], dtype), f"A2A round trip {j}")


def _moe_case(vc, p, T, H, E, K, seed_tag, tagged):
    import torch
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p)])
    splits, src, dst = vc.vcoll_moe_plan(topk, E // p)
    toks = [workloads.moe_tokens(r, T, H) for r in range(p)]
    if tagged:
        toks = [workloads.tagged_rows(t, r, np.arange(T)) for r, t in enumerate(toks)]
    want_recv, _, _ = oracle.moe_dispatch(toks, *oracle.moe_plan(list(topk), E // p)[:2])
    ttok = [upload([t.ravel()], "bf16")[0].reshape(T, H) for t in toks]
    tsrc = [torch.from_numpy(src[i]).to(dev()) for i in range(p)]
    tdst = [torch.from_numpy(dst[i]).to(dev()) for i in range(p)]
    say(f"MoE dispatch p={p} T={T} H={H} E={E} K={K}")
    recv = vc.vcoll_all_to_all(ttok, splits, src_rows=tsrc)
    say("MoE combine")
    out = vc.vcoll_all_to_all(recv, splits.T, dst_rows=tdst, dst_table_rows=[T * K] * p)
    sync()
    for j in range(p):
        assert_bits_equal(download(recv[j], "bf16"), want_recv[j], f"dispatch recv {j}")
    for i in range(p):
        # combine(dispatch(x)) == x: every (token, slot) row is the token row
        o = out[i].view(T, K, H)
        assert torch.equal(o.view(torch.int16), ttok[i].view(torch.int16).unsqueeze(1).expand(T, K, H)), i


def test_moe_dispatch_combine_small(vc):
    _moe_case(vc, p=4, T=96, H=264, E=32, K=4, seed_tag=1, tagged=True)


def test_all_to_all_skips_out_of_range_indices(vc):
    import torch
    p, H = 2, 16
    splits = np.array([[2, 1], [0, 2]])
    tab = upload(rand_inputs(1, 4 * H, "bf16", seed=77), "bf16")[0].reshape(4, H)
    tab2 = upload(rand_inputs(1, 2 * H, "bf16", seed=78), "bf16")[0].reshape(2, H)
    idx0 = torch.tensor([0, 9, 3], dtype=torch.int32, device=dev())      # 9 is outside the 4-row table
    recv = [torch.full((2, H), 7.0, dtype=torch.bfloat16, device=dev()),
            torch.full((3, H), 7.0, dtype=torch.bfloat16, device=dev())]
    say("A2A with an out-of-range gather index")
    vc.vcoll_all_to_all([tab, tab2], splits, recv=recv, src_rows=[idx0, None])
    sync()
    assert torch.equal(recv[0][0], tab[0])
    assert torch.all(recv[0][1] == 7.0)                # skipped row left untouched
    assert torch.equal(recv[1][0], tab[3]) and torch.equal(recv[1][1:], tab2)


# --------------------------------------------------------------------------- full-size workloads

def test_ring_small_workload(vc):
    cfg = workloads.RING_SMALL
    p, n = cfg["p"], cfg["n"]
    x = workloads.rank_buffers(cfg["tag"], p, n, cfg["dist"], cfg["dtype"])
    want, led = oracle.allreduce(x, "ring", "f32")
    got = gpu_allreduce(vc, "ring", x, "f32")
    assert_bits_equal(got, np.stack([bits(w, "f32") for w in want]), "p=8 n=262144 ring")
    msgs, sent, _, steps = vc.vcoll_ledger("allreduce", "ring", p, n, "f32")
    assert sent == led.sent_bytes() == [1_835_008] * 8 and steps == 14
    assert len(msgs) == 112 and {m[6] for m in msgs} == {131_072}


def test_ddp_bucket_headline_workload(vc):
    """p=8, 25 MiB fp32 per rank, ring: every element, in the launch the benchmark times."""
    cfg = workloads.DDP_BUCKET
    p, n = cfg["p"], cfg["n"]
    x = workloads.rank_buffers(cfg["tag"], p, n, cfg["dist"], cfg["dtype"])
    want, led = oracle.allreduce(x, "ring", "f32")
    got = gpu_allreduce(vc, "ring", x, "f32")
    assert_bits_equal(got, np.stack([bits(w, "f32") for w in want]), "DDP bucket ring")
    xs = np.stack(x).astype(np.float64)
    err = np.abs(got[0].view(np.float32).astype(np.float64) - xs.sum(axis=0))
    assert np.all(err <= 2 * (p - 1) * 2.0 ** -24 * np.abs(xs).sum(axis=0))
    assert led.sent_bytes() == [45_875_200] * 8


def test_hierarchy_bf16_workload_every_element(vc):
    """p=16, 192 MiB bf16 per rank (100,663,296 elements), ring and
    Rabenseifner: every element of every rank compared with the oracle,
    streamed over consecutive windows by a pool of CPU workers; and
    reduce-scatter + all-gather equal to the fused all-reduce at full size."""
    import torch
    from tests import oracle_pool
    cfg = workloads.HIER_BF16
    p, n, tag, dist = cfg["p"], cfg["n"], cfg["tag"], cfg["dist"]
    algos = ("ring", "rabenseifner")
    wins = oracle_pool.windows(n, oracle_pool.window_len(p))
    t = torch.empty((p, n), dtype=torch.bfloat16, device="cuda")
    with oracle_pool.pool() as pool:
        say(f"generating {p} x {n} bf16 inputs in {len(wins)} windows")
        for lo, hi, xw in pool.imap(oracle_pool.gen_window, [(tag, p, lo, hi, dist, "bf16") for lo, hi in wins]):
            t[:, lo:hi].copy_(torch.from_numpy(xw.view(np.int16)).view(torch.bfloat16))
        outs = {}
        for algo in algos:
            say(f"vcoll_allreduce {algo} p=16 n={n} bf16")
            outs[algo] = vc.vcoll_allreduce(algo, t)
        sync()
        checked = {a: 0 for a in algos}
        jobs = [(tag, p, n, lo, hi, dist, "bf16", algos) for lo, hi in wins]
        for lo, hi, want in pool.imap(oracle_pool.oracle_window, jobs):
            for algo in algos:
                got = download(outs[algo][:, lo:hi], "bf16")
                assert_bits_equal(got, want[algo], f"{algo} window [{lo},{hi})")
                checked[algo] += p * (hi - lo)
    for algo in algos:
        assert checked[algo] == p * n
        say(f"cfg3 {algo}: 100 % of {n:,} elements x {p} ranks equal to the oracle")
    for algo, ag_algo in (("ring", "ring"), ("rabenseifner", "rd")):
        say(f"vcoll_reduce_scatter {algo} + vcoll_all_gather {ag_algo} at full size")
        rs = vc.vcoll_reduce_scatter(algo, t)
        ag_out = torch.empty_like(t)
        vc.vcoll_all_gather(ag_algo, rs, ag_out)
        sync()
        assert torch.equal(ag_out.view(torch.int16), outs[algo].view(torch.int16))
        del rs, ag_out
    del t, outs
    torch.cuda.empty_cache()


def test_moe_full_workload(vc):
    """p=8, 4096 tokens/rank, hidden 7168 bf16, top-8 of 256 Zipf(1.1) experts."""
    m = workloads.MOE
    _moe_case(vc, p=m["p"], T=m["tokens"], H=m["hidden"], E=m["experts"], K=m["topk"], seed_tag=4, tagged=False)


@pytest.mark.parametrize("p", workloads.SWEEP_P)
def test_message_size_sweep(vc, p):
    """Every algorithm at every sweep p, sizes up to 4 MiB per rank in full."""
    for nbytes in [b for b in workloads.SWEEP_BYTES if b <= 4 * 1024 * 1024]:
        n = nbytes // 4
        x = [workloads.rank_window(workloads.TAG_SWEEP, r, 0, n, workloads.SWEEP_DIST, "f32") for r in range(p)]
        t = upload(x, "f32")
        for algo in ALGOS:
            want, _ = oracle.allreduce(x, algo, "f32")
            say(f"sweep p={p} bytes={nbytes} {algo}")
            got = download(vc.vcoll_allreduce(algo, t), "f32")
            assert_bits_equal(got, np.stack([bits(w, "f32") for w in want]), f"sweep p={p} {nbytes}B {algo}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_max_p_with_vector_chunks(vc, dtype):
    """p = 128, the largest p, with chunks of about 5000 elements: the
    run-time order program's 16-byte vector path (chunk heads and tails
    ragged), every algorithm, and the reduce-scatter and all-gather."""
    p = 128
    n = p * 5000 + 77
    x = rand_inputs(p, n, dtype, 400)
    t = upload(x, dtype)
    for algo in ALGOS:
        say(f"vcoll_allreduce p={p} n={n} {algo} {dtype}")
        want, _ = oracle.allreduce(x, algo, dtype)
        got = download(vc.vcoll_allreduce(algo, t), dtype)
        assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"{algo} p={p}")
    rs = vc.vcoll_reduce_scatter("ring", t)
    sync()
    want, _ = oracle.reduce_scatter(x, "ring", dtype)
    for c in range(p):
        assert_bits_equal(download(rs[c], dtype), bits(want[c], dtype), f"rs chunk {c}")
    m = 4099
    y = rand_inputs(p, m, dtype, 401)
    want, _ = oracle.all_gather(y, "ring", dtype)
    got = download(vc.vcoll_all_gather("ring", upload(y, dtype)), dtype)
    assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"AG p={p} m={m}")


# chunks of 1025-4096 elements on at most 3072 workgroups also take the
# LDS-staged path; (72, 72 * 3641) is past the workgroup bound (per-thread path)
MID_SHAPES = [(24, 24 * 2731 + 5), (33, 33 * 3972 + 7), (72, 72 * 1820 + 11), (100, 100 * 1310 + 3),
              (72, 72 * 3641)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p,n", MID_SHAPES, ids=[f"p{p}-n{n}" for p, n in MID_SHAPES])
def test_mid_chunks_of_the_run_time_program(vc, p, n, dtype):
    """The staged path's larger chunks (ragged, 29-63 tiles of 64 elements)
    and the per-thread path just past its bound: all-reduce with every
    algorithm, ring reduce-scatter, and a reduce to a root of a vector of at
    most 4096 elements."""
    from oracle import rooted
    x = rand_inputs(p, n, dtype, 400 + p)
    t = upload(x, dtype)
    for algo in ALGOS:
        say(f"mid-chunk all-reduce p={p} n={n} {algo} {dtype}")
        want, _ = oracle.allreduce(x, algo, dtype)
        got = download(vc.vcoll_allreduce(algo, t), dtype)
        assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"{algo} p={p}")
    say(f"mid-chunk reduce-scatter p={p} n={n} {dtype}")
    rs = vc.vcoll_reduce_scatter("ring", t)
    sync()
    want, _ = oracle.reduce_scatter(x, "ring", dtype)
    for c in range(p):
        assert_bits_equal(download(rs[c], dtype), bits(want[c], dtype), f"rs chunk {c}")
    xs = [r[:4000] for r in x]
    say(f"reduce to a root p={p} n=4000 {dtype}")
    red = vc.vcoll_reduce(upload(xs, dtype), root=p - 1)
    sync()
    want, _ = rooted.reduce(xs, p - 1, dtype)
    assert_bits_equal(download(red, dtype), bits(want, dtype), "reduce")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [3, 12, 72, 128])
def test_small_chunks_of_the_run_time_program(vc, p, dtype):
    """p not compiled in, chunks of at most 1024 elements: the LDS-staged
    path (64-element tiles, the last one ragged) for all-reduce, ring
    reduce-scatter and reduce to a root."""
    from oracle import rooted
    n = p * 1000 + p // 2 + 3
    x = rand_inputs(p, n, dtype, 300 + p)
    t = upload(x, dtype)
    for algo in ALGOS:
        say(f"small-chunk all-reduce p={p} n={n} {algo} {dtype}")
        want, _ = oracle.allreduce(x, algo, dtype)
        got = download(vc.vcoll_allreduce(algo, t), dtype)
        assert_bits_equal(got, np.stack([bits(w, dtype) for w in want]), f"{algo} p={p}")
    rs = vc.vcoll_reduce_scatter("ring", t)
    sync()
    want, _ = oracle.reduce_scatter(x, "ring", dtype)
    for c in range(p):
        assert_bits_equal(download(rs[c], dtype), bits(want[c], dtype), f"rs chunk {c}")
    root = p // 2
    red = vc.vcoll_reduce(t, root=root)
    sync()
    want, _ = rooted.reduce(x, root, dtype)
    assert_bits_equal(download(red, dtype), bits(want, dtype), "reduce")
