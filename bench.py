#!/usr/bin/env python
"""Benchmark of the single-GPU virtual-cluster collectives on MI355X.

Headline: the DDP gradient-bucket all-reduce -- p = 8 logical ranks, 25 MiB
of float32 per rank (6,553,600 elements, normal(0, 1e-3), 25 MB buckets as in
PyTorch DDP's bucket_cap_mb), ring order rank 0 -> 1 -> .. -> 7, reduce-scatter
and all-gather fused into one HBM pass. One step is one such all-reduce.

value: whole-job effective HBM bandwidth = algorithmic bytes per step
(p*S read + p*S written = 419,430,400 B) x steps / wall time of the timed
steps. Inputs live in HBM; the steps cycle through several input/output
sets whose total exceeds the 256 MB Infinity Cache, so no step reads what
the previous one left in cache.

roofline.achieved: the same algorithmic bytes / the kernel's mean launch
duration: HIP events on the launch stream around the timed region, divided
by the number of launches; roofline.launch_us: median, p10 and p90 of 60
launches timed one by one, each after a 1 GiB copy that evicts the
Infinity Cache. roofline.traffic: HBM bytes per launch from rocprofv3
counters (profiles/traffic.json, valid while the kernel's machine code is
unchanged), or null.

cpu_baseline: the CPU oracle (step-by-step numpy ring with its message
ledger) on the same workload, on this host, one thread; its result is
compared with the GPU's bit for bit (parity_vs_oracle).

Extras (not the headline), each kernel with algorithmic bytes, microseconds
and fraction of 8 TB/s, each configuration with its oracle baseline and
parity check:
  ceilings -- read-only, write-only and copy streams of this GPU;
  cfg1 -- the pages' 4-device worked example and p = 8 x 262,144 float32;
  other algorithms, hierarchical orders, broadcast, reduce and the unfused
  reduce-scatter + all-gather on the bucket; stepwise execution;
  decode-like 10 KiB and prefill-like 80 MiB messages (and from a HIP graph);
  cfg3 -- p = 16 x 192 MiB bfloat16, ring and Rabenseifner;
  cfg4 -- MoE dispatch/combine (p = 8, 4096 tokens, hidden 7168, top-8);
  moe_variants -- row-major, FP8 and deduplicated dispatch forms;
  cfg5 -- the sweep's p in {2, 4, 8, 16, 72} at 64 MiB and 1 KiB per rank;
  host_schedule_and_ledger -- the host rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "all-reduce effective HBM GB/s (p=8, 25 MB/rank fp32) + % of HBM roofline"
PEAK_GBPS = 8000.0           # MI355X HBM3E, AMD public spec
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
# the headline kernel in libvcoll.so: the two-phase ring all-reduce, float32, 25 vectors per thread
HEADLINE_SYMBOL = "burst_ring_kernelILi0ELi25ELi0EE"


def _elf_sections(data: bytes) -> list:
    """(name, type, addr, offset, size, link) of every section of an ELF64
    little-endian image, in header order."""
    import struct
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    raw = [struct.unpack_from("<IIQQQQI", data, shoff + i * shentsize) for i in range(shnum)]
    strtab = raw[shstrndx][4]

    def name(o):
        return data[strtab + o:data.index(b"\0", strtab + o)].decode()
    return [(name(r[0]), r[1], r[3], r[4], r[5], r[6]) for r in raw]


def kernel_code_hash(symbol: str = HEADLINE_SYMBOL) -> str | None:
    """Hash of the gfx950 machine code of one kernel of the built libvcoll.so
    (read from the library's own offload bundles), or None. Counter traffic
    measured for a kernel stays valid exactly as long as this hash does."""
    import struct
    lib = os.path.join(ROOT, "collective_communication_algorithms_vcoll_amd", "libvcoll.so")
    if not os.path.exists(lib):
        return None
    data = open(lib, "rb").read()
    fats = [x for x in _elf_sections(data) if x[0] == ".hip_fatbin"]
    if not fats:
        return None
    _, _, _, off, size, _ = fats[0]
    fat = data[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    pos = fat.find(magic)
    while pos >= 0:
        count = struct.unpack_from("<Q", fat, pos + 24)[0]
        q = pos + 32
        for _ in range(count):
            e_off, e_size, id_len = struct.unpack_from("<QQQ", fat, q)
            ident = fat[q + 24:q + 24 + id_len]
            q += 24 + id_len
            if b"gfx950" not in ident:
                continue
            code = fat[pos + e_off:pos + e_off + e_size]
            csec = _elf_sections(code)
            symtabs = [x for x in csec if x[1] == 2]            # SHT_SYMTAB
            texts = [x for x in csec if x[0] == ".text"]
            if not symtabs or not texts:
                continue
            _, _, _, so, ss, link = symtabs[0]
            strtab = csec[link][3]

            for k in range(ss // 24):
                st_name, st_info, _, _, st_value, st_size = struct.unpack_from("<IBBHQQ", code, so + 24 * k)
                nm = code[strtab + st_name:code.index(b"\0", strtab + st_name)].decode()
                if symbol in nm and not nm.endswith(".kd") and st_size > 0:
                    text = texts[0]
                    start = text[3] + (st_value - text[2])
                    return hashlib.sha256(code[start:start + st_size]).hexdigest()[:16]
        pos = fat.find(magic, pos + len(magic))
    return None


def counter_traffic(kernel_key: str):
    """HBM bytes per launch measured by rocprofv3 for this kernel source, if any."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_key)
    code = kernel_code_hash()
    if not entry or code is None or entry.get("code_hash") != code:
        return None
    return entry.get("bytes_per_launch")


def time_launches(calls, steps, warmup):
    """Run calls[k % len(calls)] steps times after warmup, back to back on
    the current stream. Returns (wall seconds of the timed steps, mean launch
    ms): HIP events recorded on the launch stream at the start and end of
    the timed region, divided by the number of launches. (An event pair
    around every launch would add its own ~7 us per launch on this GPU.)"""
    import torch
    for k in range(warmup):
        calls[k % len(calls)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for k in range(steps):
        calls[k % len(calls)]()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def device_info(torch) -> dict:
    """The GPU the numbers were taken on."""
    prop = torch.cuda.get_device_properties(0)
    return {"name": prop.name, "arch": getattr(prop, "gcnArchName", ""),
            "compute_units": prop.multi_processor_count, "memory_bytes": prop.total_memory}


def rate(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def sets_for(bytes_per_set: int) -> int:
    """Input/output sets to cycle so that consecutive reuse is out of cache."""
    return max(2, -(-4 * MALL_BYTES // bytes_per_set))


def headline(vc, torch, args):
    import numpy as np
    import workloads
    cfg = workloads.DDP_BUCKET
    p, n = cfg["p"], cfg["n"]
    x = workloads.rank_buffers(cfg["tag"], p, n, cfg["dist"], cfg["dtype"])
    base = torch.from_numpy(np.stack(x)).cuda()
    S = n * 4
    nbytes = 2 * p * S
    R = sets_for(nbytes)
    ins = [base.clone() for _ in range(R)]
    outs = [torch.empty_like(base) for _ in range(R)]
    calls = [vc.prepare_allreduce("ring", ins[i], outs[i]) for i in range(R)]
    wall, mean_ms = time_launches(calls, args.steps, args.warmup)
    result = outs[(args.steps - 1) % R].cpu().numpy()       # written by the last timed launch
    scrub = Scrub(vc, torch)
    dist = launch_distribution(torch, calls, scrub)
    return dict(x=x, p=p, n=n, S=S, nbytes=nbytes, sets=R, wall=wall, mean_ms=mean_ms,
                result=result, base=base, scrub=scrub, dist=dist)


def cpu_baseline(h, seconds):
    import numpy as np
    import oracle
    reps, t0 = 0, time.perf_counter()
    out = None
    while True:
        out, _ = oracle.allreduce(h["x"], "ring", "f32")
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    parity = all(np.array_equal(out[r].view(np.uint32), h["result"][r].view(np.uint32)) for r in range(h["p"]))
    return {
        "value": round(h["nbytes"] * reps / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{reps} full ring all-reduces of the same bucket (p=8 x 6,553,600 fp32), "
                  f"{el:.1f} s, numpy single thread, host has {len(os.sched_getaffinity(0))} cores",
    }, parity


def roof(kernel: str, nbytes: int, ms: float, **more) -> dict:
    """Roofline record of one kernel: algorithmic bytes per launch over its
    mean launch duration, against MI355X's 8 TB/s."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    rec = {"kernel": kernel, "algorithmic_bytes": int(nbytes), "us": round(ms * 1e3, 2),
           "achieved_GBps": round(gbps, 1), "peak_GBps": PEAK_GBPS, "frac": round(gbps / PEAK_GBPS, 4)}
    rec.update(more)
    return rec


class Scrub:
    """A 1 GiB streaming copy that evicts the 256 MB Infinity Cache between
    timed launches (run outside the timed events). It uses the plain copy
    shape, so that the fast copy stays the only kernel of its kind in a run
    (its counter readings scale the other kernels')."""

    def __init__(self, vc, torch):
        half = 512 * 2 ** 20
        self.src = torch.empty(half // 4, device="cuda")
        self.dst = torch.empty(half // 4, device="cuda")
        self.call = vc.prepare_bench_stream("copy_plain", self.dst, self.src)

    def __call__(self):
        self.call()


def launch_distribution(torch, calls, scrub, iters: int = 60) -> dict:
    """Per-launch durations: for each of `iters` launches, scrub the cache,
    then time the launch alone between two HIP events on its stream;
    median, p10 and p90 in microseconds (each includes one event pair's own
    cost, reported once as event_pair_floor_us)."""
    import numpy as np
    ts = []
    for k in range(iters + 3):
        scrub()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        calls[k % len(calls)]()
        e.record()
        e.synchronize()
        if k >= 3:
            ts.append(s.elapsed_time(e) * 1e3)
    q = np.percentile(ts, [10, 50, 90])
    return {"p10": round(float(q[0]), 2), "median": round(float(q[1]), 2), "p90": round(float(q[2]), 2),
            "iterations": iters, "cache_scrubbed": True}


def event_pair_floor(vc, torch) -> float:
    """Median time between two HIP events around a 16-byte copy: the floor
    every per-launch event measurement includes."""
    import numpy as np
    a, b = torch.zeros(4, device="cuda"), torch.zeros(4, device="cuda")
    call = vc.prepare_bench_stream("copy", b, a)
    ts = []
    for _ in range(53):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        call()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e) * 1e3)
    return round(float(np.median(ts[3:])), 2)


def oracle_seconds(fn, seconds: float):
    """Run fn repeatedly for about `seconds` (at least once); returns
    (result of the last run, runs, elapsed seconds)."""
    reps, t0, out = 0, time.perf_counter(), None
    while True:
        out = fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return out, reps, el


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def ceilings(vc, torch, nbytes: int) -> dict:
    """Streaming ceilings of this GPU measured in the same run: read-only,
    write-only, the fastest copy shape and the earlier plain copy, each over
    `nbytes` read and/or written per launch, cycled through buffer sets that
    exceed the Infinity Cache."""
    R = sets_for(2 * nbytes)
    src = [torch.empty(nbytes // 4, device="cuda") for _ in range(R)]
    dst = [torch.empty(nbytes // 4, device="cuda") for _ in range(R)]
    sink = torch.zeros(4, device="cuda")
    out = {}
    for kind, moved, mk in (
            ("read", nbytes, lambda i: vc.prepare_bench_stream("read", sink, src[i])),
            ("write", nbytes, lambda i: vc.prepare_bench_stream("write", dst[i])),
            ("copy", 2 * nbytes, lambda i: vc.prepare_bench_stream("copy", dst[i], src[i])),
            ("copy_plain", 2 * nbytes, lambda i: vc.prepare_bench_stream("copy_plain", dst[i], src[i]))):
        calls = [mk(i) for i in range(R)]
        _, ms = time_launches(calls, 60, 5)
        out[kind] = roof({"read": "read_kernel<4, 256>", "write": "write_kernel<4, 64>",
                          "copy": "copy_kernel<2, 64, sc0 sc1 nt>", "copy_plain": "copy_kernel<4, 256, nt>"}[kind],
                         moved, ms)
    del src, dst
    torch.cuda.empty_cache()
    return out


def cfg1(vc, torch, scrub, cpu_seconds, cpu_leg: bool) -> dict:
    """The pages' 4-device worked example, then p = 8 x 262,144 float32
    (uniform[-1, 1]): ring all-reduce, reduce-scatter + all-gather identity,
    ledger, latency."""
    import numpy as np
    import workloads
    res = {"workload": "worked example p=4 x 4 (device d holds 10d..10d+3); ring all-reduce p=8 x 262,144 fp32"}
    x4 = workloads.worked_example()
    t4 = torch.from_numpy(np.stack(x4)).cuda()
    ar4 = {a: vc.vcoll_allreduce(a, t4).cpu().numpy() for a in ("ring", "rd", "rabenseifner", "tree")}
    rs4 = vc.vcoll_reduce_scatter("ring", t4)
    ag4 = vc.vcoll_all_gather("ring", rs4).cpu().numpy()
    res["worked_example_allreduce"] = ar4["ring"][0].tolist()
    res["worked_example_rs_then_ag_equals_allreduce"] = bool(np.array_equal(ag4, ar4["ring"]))
    msgs, sent, _, steps = vc.vcoll_ledger("allreduce", "ring", 4, 4, "f32")
    res["worked_example_ledger"] = {"steps": steps, "messages": len(msgs), "sent_bytes_per_rank": sent}

    cfg = workloads.RING_SMALL
    p, n = cfg["p"], cfg["n"]
    x = workloads.rank_buffers(cfg["tag"], p, n, cfg["dist"], cfg["dtype"])
    base = torch.from_numpy(np.stack(x)).cuda()
    S = n * 4
    R = sets_for(2 * p * S)
    ins = [base.clone() for _ in range(R)]
    outs = [torch.empty_like(base) for _ in range(R)]
    calls = [vc.prepare_allreduce("ring", ins[i], outs[i]) for i in range(R)]
    _, ms = time_launches(calls, 200, 20)
    res["roofline"] = roof("reduce_kernel<f32, ring, p=8, 4 vectors per thread>", 2 * p * S, ms,
                           bound="latency (16 MiB moved per call)",
                           launch_us=launch_distribution(torch, calls, scrub))
    rs = vc.vcoll_reduce_scatter("ring", base)
    ag = vc.vcoll_all_gather("ring", rs)
    ar = vc.vcoll_allreduce("ring", base)
    torch.cuda.synchronize()
    res["rs_then_ag_equals_allreduce"] = bool(torch.equal(ag.view(torch.int32), ar.view(torch.int32)))
    msgs, sent, _, steps = vc.vcoll_ledger("allreduce", "ring", p, n, "f32")
    res["ledger"] = {"steps": steps, "messages": len(msgs), "bytes_per_message": sorted({m[6] for m in msgs}),
                     "sent_bytes_per_rank": sorted(set(sent)),
                     "closed_form_2(p-1)/p*S": 2 * (p - 1) * S // p}
    if cpu_leg:
        import oracle
        got = ar.cpu().numpy().view(np.uint32)
        (want, _), reps, el = oracle_seconds(lambda: oracle.allreduce(x, "ring", "f32"), cpu_seconds)
        ok4 = all(np.array_equal(ar4[a], np.stack(oracle.allreduce(x4, a, "f32")[0]))
                  for a in ("ring", "rd", "rabenseifner", "tree"))
        res["parity_vs_oracle"] = "bit-exact" if (np.array_equal(got, np.stack(want).view(np.uint32)) and ok4) \
            else "MISMATCH"
        res["cpu_baseline"] = {"value": round(2 * p * S * reps / el / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} full ring all-reduces of p=8 x 262,144 fp32, {el:.1f} s, numpy "
                                         f"single thread, host has {host_cores()} cores; worked example all four "
                                         f"algorithms"}
    del ins, outs, base
    torch.cuda.empty_cache()
    return res


def cfg3(vc, torch, scrub, cpu_leg: bool) -> dict:
    """p = 16 x 192 MiB bf16 per rank, float32 accumulation: fused ring and
    Rabenseifner all-reduces, their reduce-scatter and all-gather halves,
    and the 2 x 8 / 4 x 4 hierarchical orders."""
    import numpy as np
    P16, N16 = 16, 100_663_296
    S16 = N16 * 2
    res = {"workload": "p=16 x 192 MiB bf16 per rank (100,663,296 elements), uniform[-1,1], fp32 accumulation, "
                       "bf16 output; inputs drawn on the GPU (seeded torch generator)"}
    g = torch.Generator(device="cuda").manual_seed(3)
    t16 = (torch.rand((P16, N16), device="cuda", generator=g) * 2 - 1).to(torch.bfloat16)
    o16 = {a: torch.empty_like(t16) for a in ("ring", "rabenseifner")}
    for algo in ("ring", "rabenseifner"):
        call = vc.prepare_allreduce(algo, t16, o16[algo])
        _, ms = time_launches([call], 30, 5)
        res[f"{algo}_allreduce"] = roof(f"reduce_kernel<bf16, {algo}, p=16, 1 vector per thread, 64 threads>",
                                        2 * P16 * S16, ms, launch_us=launch_distribution(torch, [call], scrub, 50))
    tmp = torch.empty_like(t16)
    for nodes, local in ((2, 8), (4, 4)):
        call = vc.prepare_allreduce_hierarchical(nodes, local, t16, tmp)
        _, ms = time_launches([call], 30, 5)
        res[f"hierarchical_{nodes}x{local}_allreduce"] = roof(f"hier_kernel<bf16, {nodes}, {local}>", 2 * P16 * S16, ms)
    rs16 = [torch.empty(N16 // P16, dtype=torch.bfloat16, device="cuda") for _ in range(P16)]
    for algo, ag_algo in (("ring", "ring"), ("rabenseifner", "rd")):
        call = vc.prepare_reduce_scatter(algo, t16, rs16)
        _, ms = time_launches([call], 30, 5)
        res[f"{algo}_reduce_scatter"] = roof(f"reduce_kernel<bf16, {algo}, p=16, reduce-scatter>",
                                             P16 * S16 + S16, ms)
        call = vc.prepare_all_gather(ag_algo, rs16, tmp)
        _, ms = time_launches([call], 30, 5)
        res[f"{ag_algo}_all_gather"] = roof("all_gather_kernel<bf16, 1 vector per thread, 64 threads>",
                                            S16 + P16 * S16, ms)
    del tmp, rs16
    if cpu_leg:
        import oracle
        w = 1 << 20
        lo = N16 // P16 - w // 2                     # straddles the chunk 0 / chunk 1 boundary
        xw = [t16[r, lo:lo + w].view(torch.int16).cpu().numpy().view(np.uint16) for r in range(P16)]
        ok, reps, t_or = True, 0, 0.0
        for algo in ("ring", "rabenseifner"):
            (want, _), k, el = oracle_seconds(lambda: oracle.allreduce(xw, algo, "bf16", n=N16, lo=lo), 1.5)
            t_or += el
            reps += k
            got = o16[algo][:, lo:lo + w].view(torch.int16).cpu().numpy().view(np.uint16)
            ok = ok and np.array_equal(got, np.stack(want))
        res["parity_vs_oracle"] = "bit-exact" if ok else "MISMATCH"
        res["parity_fraction"] = round(w / N16, 6)
        res["cpu_baseline"] = {"value": round(2 * P16 * w * 2 * reps / t_or / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"windowed oracle, ring and Rabenseifner, elements [{lo}, {lo + w}) of all "
                                         f"16 ranks ({100 * w / N16:.2f} % of the vector), {t_or:.1f} s, numpy single "
                                         f"thread, host has {host_cores()} cores; every element of the full vector is "
                                         f"compared with the oracle by the GPU tests"}
    del t16, o16
    torch.cuda.empty_cache()
    return res


def cfg4(vc, torch, cpu_leg: bool) -> dict:
    """MoE dispatch/combine: p = 8, 4096 tokens per rank, hidden 7168 bf16,
    top-8 of 256 Zipf(1.1) experts."""
    import numpy as np
    import workloads
    M = workloads.MOE
    p8, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p8)])
    splits, src_rows, dst_rows = vc.vcoll_moe_plan(topk, E // p8)
    rb, orb = H * 2, H + H // 32
    rows = int(splits.sum())
    res = {"workload": "MoE dispatch/combine p=8, 4096 tokens/rank, hidden 7168 bf16, top-8 of 256 experts "
                       "(32/rank), Zipf(1.1) popularity; tokens normal(0,1) drawn on the GPU",
           "rows": rows, "rows_to_rank0": round(float(splits[:, 0].sum() / rows), 4)}
    g = torch.Generator(device="cuda").manual_seed(4)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p8)]
    slots = vc.vcoll_moe_slots(splits, dst_rows, K)
    slots_g = [torch.from_numpy(np.ascontiguousarray(slots[i])).cuda() for i in range(p8)]
    recv_rows = splits.sum(axis=0)
    # dispatch: token-major (each token row read once, written to each of its slots)
    recv = vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K)
    push = lambda: vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, recv=recv)          # noqa: E731
    _, ms = time_launches([push], 10, 2)
    res["dispatch"] = roof("dispatch_push_kernel<false, 64> (bf16, 2 KiB row segments)", p8 * T * rb + rows * rb, ms)
    # combine: token-major (each (token, slot) row pulled from its expert output)
    back = vc.vcoll_moe_combine(recv, slots_g, T, K)
    pull = lambda: vc.vcoll_moe_combine(recv, slots_g, T, K, out=back)                    # noqa: E731
    _, ms = time_launches([pull], 10, 2)
    res["combine"] = roof("combine_pull_kernel<64> (1 KiB row segments)", 2 * rows * rb, ms)
    torch.cuda.synchronize()
    res["combine_of_dispatch_is_identity"] = all(
        torch.equal(back[i].view(T, K, H).view(torch.int16), toks[i].view(torch.int16).unsqueeze(1).expand(T, K, H))
        for i in range(p8))
    # FP8 payload, token-major
    f8 = vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, fp8=True)
    push8 = lambda: vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, fp8=True, recv=f8)  # noqa: E731
    _, ms = time_launches([push8], 10, 2)
    res["dispatch_fp8"] = roof("dispatch_push_kernel<true, 512> (FP8)", p8 * T * rb + rows * orb, ms)
    del f8
    # the plain block transpose on the same splits (send buffers already in
    # destination-block order)
    plain_send = [torch.randn((int(splits[i].sum()), H), device="cuda", generator=g).to(torch.bfloat16)
                  for i in range(p8)]
    plain_recv = vc.vcoll_all_to_all(plain_send, splits)
    a2a = lambda: vc.vcoll_all_to_all(plain_send, splits, recv=plain_recv)                # noqa: E731
    _, ms = time_launches([a2a], 10, 2)
    res["all_to_all_plain"] = roof("all_to_all_kernel<1024>", 2 * rows * rb, ms)
    del plain_send, plain_recv
    torch.cuda.empty_cache()
    if cpu_leg:
        import oracle
        t_h = [x.view(torch.int16).cpu().numpy().view(np.uint16) for x in toks]
        o_splits, o_src, o_dst = oracle.moe_plan(list(topk), E // p8)
        t0 = time.perf_counter()
        want_recv, _, _ = oracle.moe_dispatch(t_h, o_splits, o_src)
        t_d = time.perf_counter() - t0
        ok = all(np.array_equal(recv[j].view(torch.int16).cpu().numpy().view(np.uint16), want_recv[j])
                 for j in range(p8))
        t0 = time.perf_counter()
        want_back, _ = oracle.moe_combine(want_recv, o_splits, o_dst, K, T)
        t_c = time.perf_counter() - t0
        ok = ok and np.array_equal(o_splits, splits)
        ok = ok and all(np.array_equal(back[i].view(torch.int16).cpu().numpy().view(np.uint16), want_back[i])
                        for i in range(p8))
        del want_recv, want_back, t_h
        moved = (p8 * T * rb + rows * rb) + 2 * rows * rb
        res["parity_vs_oracle"] = "bit-exact" if ok else "MISMATCH"
        res["cpu_baseline"] = {"value": round(moved / (t_d + t_c) / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"one full dispatch ({t_d:.1f} s) and combine ({t_c:.1f} s) of the workload "
                                         f"(262,144 rows of 14,336 B each way), numpy single thread, host has "
                                         f"{host_cores()} cores; bytes as the GPU figures (dispatch: tokens read "
                                         f"once + rows written; combine: rows read + written)"}
    del toks, recv, back
    torch.cuda.empty_cache()
    return res


def cfg5(vc, torch, cpu_leg: bool) -> dict:
    """The message-size sweep in the driver's run: every p at 64 MiB per rank
    (the largest oracle-timed size) for all four algorithms, and at 1 KiB per
    rank (latency). The full 260-point sweep is `bench.py --sweep`."""
    import numpy as np
    import workloads
    res = {"workload": "p in {2,4,8,16,72}, fp32 normal(0,1) drawn on the GPU; 64 MiB and 1 KiB per rank"}
    for p in workloads.SWEEP_P:
        for nbytes in (2 ** 10, 64 * 2 ** 20):
            n = nbytes // 4
            g = torch.Generator(device="cuda").manual_seed(workloads.TAG_SWEEP * 10 ** 6 + p * 1000 + nbytes % 997)
            t = torch.randn((p, n), device="cuda", generator=g)
            sets = 1 if 2 * p * nbytes > 4 * MALL_BYTES else min(64, sets_for(2 * p * nbytes))
            ins = [t] + [t.clone() for _ in range(sets - 1)]
            outs = [torch.empty_like(t) for _ in range(sets)]
            for algo in ("ring", "rd", "rabenseifner", "tree"):
                calls = [vc.prepare_allreduce(algo, ins[i], outs[i]) for i in range(sets)]
                K = 200 if nbytes < 2 ** 20 else 15
                _, ms = time_launches(calls, K, 3)
                key = f"p{p}_{'1KiB' if nbytes < 2 ** 20 else '64MiB'}_{algo}"
                res[key] = roof(f"reduce_kernel<f32, {algo}, p={p}>", 2 * p * nbytes, ms)
            if cpu_leg and nbytes > 2 ** 20:
                import oracle
                w = min(n, 1 << 18)
                offs = [c * (n // p) + min(c, n % p) for c in range(p + 1)]
                lo = max(0, offs[1] - w // 2)
                xw = [t[r, lo:lo + w].cpu().numpy() for r in range(p)]
                ok, t_or, reps = True, 0.0, 0
                for algo in ("ring", "rd", "rabenseifner", "tree"):
                    vc.vcoll_allreduce(algo, t, outs[0])
                    (want, _), k, el = oracle_seconds(lambda: oracle.allreduce(xw, algo, "f32", n=n, lo=lo), 0.3)
                    t_or += el
                    reps += k
                    ok = ok and np.array_equal(outs[0][:, lo:lo + w].cpu().numpy().view(np.uint32),
                                               np.stack(want).view(np.uint32))
                res[f"p{p}_64MiB_parity_vs_oracle"] = "bit-exact" if ok else "MISMATCH"
                res[f"p{p}_64MiB_cpu_baseline"] = {
                    "value": round(reps * 2 * p * w * 4 / t_or / 1e9, 3), "unit": "GB/s", "cores": 1,
                    "kind": "oracle",
                    "sample": f"windowed oracle, all four algorithms, {reps} runs over elements [{lo}, {lo + w}) "
                              f"of all {p} ranks ({100 * w / n:.2f} % of the vector), {t_or:.1f} s, numpy single "
                              f"thread"}
            del t, ins, outs
            torch.cuda.empty_cache()
    return res


EXTRA_SECTIONS = ("ceilings", "cfg1", "bucket", "stepwise", "decode_prefill", "graphs", "cfg3", "cfg4",
                  "moe_variants", "cfg5", "layouts", "host")


def extras(vc, torch, h, args):
    import numpy as np
    import workloads
    cpu_leg = not args.no_cpu_baseline
    only = set(args.only.split(",")) if args.only else set(EXTRA_SECTIONS)
    ex = {}
    p, n, S = h["p"], h["n"], h["S"]
    base = h["base"]
    steps, warm = max(20, args.steps // 4), 5
    scrub = h["scrub"]
    ex["event_pair_floor_us"] = event_pair_floor(vc, torch)
    if "ceilings" in only:
        ex["ceilings"] = ceilings(vc, torch, p * S)
    if "cfg1" in only:
        ex["cfg1"] = cfg1(vc, torch, scrub, min(3.0, args.cpu_seconds), cpu_leg)
    if "bucket" in only:
        bucket_extras(vc, torch, h, ex, steps, warm)
    if "stepwise" in only:
        stepwise_extras(vc, torch, ex, steps, warm)
        stepwise_broadcast_extras(vc, torch, ex, steps, warm)
    if "decode_prefill" in only:
        decode_prefill_extras(vc, torch, ex, steps, warm)
    if "graphs" in only:
        graph_extras(vc, torch, ex)
    if "cfg3" in only:
        ex["cfg3"] = cfg3(vc, torch, scrub, cpu_leg)
    if "cfg4" in only:
        ex["cfg4"] = cfg4(vc, torch, cpu_leg)
    if "moe_variants" in only:
        ex["moe_variants"] = moe_variants(vc, torch)
    if "cfg5" in only:
        ex["cfg5"] = cfg5(vc, torch, cpu_leg)
    if "layouts" in only:                 # last: its many allocations must not shift the configurations' buffers
        ex["layouts"] = layout_extras(vc, torch, steps, warm)
    if "host" in only:
        ex["host_schedule_and_ledger"] = host_rows(vc)
    return ex


def bucket_extras(vc, torch, h, ex, steps, warm):
    """Other algorithms, hierarchical orders, broadcast, reduce, the warm
    cache and the unfused pair on the DDP bucket."""
    p, n, S = h["p"], h["n"], h["S"]
    base = h["base"]
    # other algorithms on the same bucket (fused, one pass each)
    R = sets_for(2 * p * S)
    ins = [base.clone() for _ in range(R)]
    outs = [torch.empty_like(base) for _ in range(R)]
    for algo in ("rd", "rabenseifner", "tree"):
        calls = [vc.prepare_allreduce(algo, ins[i], outs[i]) for i in range(R)]
        _, mean_ms = time_launches(calls, steps, warm)
        ex[f"ddp_bucket_{algo}_fused"] = roof(f"reduce_kernel<f32, {algo}, p=8>", 2 * p * S, mean_ms)
    # hierarchical (2 groups of 4, and 4 of 2) on the same bucket
    for nodes, local in ((2, 4), (4, 2)):
        calls = [vc.prepare_allreduce_hierarchical(nodes, local, ins[i], outs[i]) for i in range(R)]
        _, mean_ms = time_launches(calls, steps, warm)
        ex[f"ddp_bucket_hierarchical_{nodes}x{local}_fused"] = roof(f"hier_kernel<f32, {nodes}, {local}>",
                                                                   2 * p * S, mean_ms)
    # rooted collectives on the same bucket: broadcast of one rank's 25 MiB to
    # 8 receive buffers (S read + 8 S written), reduce to rank 0 (8 S + S)
    bsrc = [base[i % p].clone() for i in range(R)]
    calls = [vc.prepare_broadcast(bsrc[i], outs[i], 0) for i in range(R)]
    _, mean_ms = time_launches(calls, steps, warm)
    ex["ddp_bucket_broadcast_p8"] = roof("broadcast_kernel<f32, 4 vectors per thread, 64 threads>", (p + 1) * S,
                                         mean_ms)
    rout = [torch.empty(n, device="cuda") for _ in range(R)]
    calls = [vc.prepare_reduce(ins[i], rout[i], 0) for i in range(R)]
    _, mean_ms = time_launches(calls, steps, warm)
    ex["ddp_bucket_reduce_tree_p8"] = roof("reduce_kernel<f32, tree, p=8, reduce>", (p + 1) * S, mean_ms)
    del bsrc, rout
    # warm: one set reused back to back (partly served by the Infinity Cache)
    call = vc.prepare_allreduce("ring", ins[0], outs[0])
    _, mean_ms = time_launches([call], steps, warm)
    ex["ddp_bucket_ring_fused_warm_cache"] = roof("ring all-reduce, one buffer set (warm)", 2 * p * S, mean_ms)
    # unfused ring: reduce-scatter kernel then all-gather kernel
    rs_out = [[torch.empty(n // p, device="cuda") for _ in range(p)] for _ in range(R)]
    rs = [vc.prepare_reduce_scatter("ring", ins[i], rs_out[i]) for i in range(R)]
    ag = [vc.prepare_all_gather("ring", rs_out[i], outs[i]) for i in range(R)]
    pair = [lambda i=i: (rs[i](), ag[i]()) for i in range(R)]
    _, mean_ms = time_launches(pair, steps, warm)
    ex["ddp_bucket_ring_unfused_rs_then_ag"] = roof("reduce-scatter kernel + all-gather kernel",
                                                    2 * p * S + 2 * S, mean_ms)
    del ins, outs, rs_out
    torch.cuda.empty_cache()


def stepwise_extras(vc, torch, ex, steps, warm):
    """Stepwise execution (one launch per algorithm step, messages through
    memory) against the fused kernels: the per-step latency and the memory
    round trips that fusion removes."""
    for label, nbytes in (("10KiB", 10 * 1024), ("25MiB", 25 * 2 ** 20)):
        m = nbytes // 4
        g = torch.Generator(device="cuda").manual_seed(6)
        t = torch.randn((8, m), device="cuda", generator=g)
        R2 = min(64, sets_for(2 * 8 * nbytes))
        ts = [t.clone() for _ in range(R2)]
        os_ = [torch.empty_like(t) for _ in range(R2)]
        for algo in ("ring", "rd", "rabenseifner", "tree"):
            _, launches = vc.vcoll_allreduce_stepwise(algo, ts[0], os_[0])
            calls = [vc.prepare_allreduce_stepwise(algo, ts[i], os_[i]) for i in range(R2)]
            _, ms_step = time_launches(calls, steps if nbytes < 2 ** 20 else 20, warm)
            calls = [vc.prepare_allreduce(algo, ts[i], os_[i]) for i in range(R2)]
            _, ms_fused = time_launches(calls, steps if nbytes < 2 ** 20 else 20, warm)
            ex[f"stepwise_p8_{label}_{algo}"] = {
                "us": round(ms_step * 1e3, 2), "launches": launches,
                "us_per_launch": round(ms_step * 1e3 / launches, 2),
                "fused_us": round(ms_fused * 1e3, 2), "slowdown_vs_fused": round(ms_step / ms_fused, 2)}
        del t, ts, os_
    torch.cuda.empty_cache()


def stepwise_broadcast_extras(vc, torch, ex, steps, warm):
    """The broadcast family executed one launch per schedule step ([NCC] 5.5:
    naive, binomial tree, pipelined chain; 4.2 scatter + all-gather), p = 8,
    for the lecture's 8 MB example and a decode-sized 10 KiB message, beside
    the one-pass broadcast and the lecture's own clock for the same
    schedule (TPU ICI links: alpha = 1 us, 45 GB/s; ici_model_us)."""
    p = 8
    for label, nbytes in (("8MB", 8_000_000), ("10KiB", 10 * 1024)):
        n = nbytes // 4
        g = torch.Generator(device="cuda").manual_seed(11)
        src = torch.randn(n, device="cuda", generator=g)
        R2 = min(64, sets_for((p + 1) * nbytes))
        outs = [torch.empty((p, n), device="cuda") for _ in range(R2)]
        calls = [vc.prepare_broadcast(src, outs[i], 0) for i in range(R2)]
        _, ms_one = time_launches(calls, steps, warm)
        rec = {"one_pass_us": round(ms_one * 1e3, 2)}
        for algo, k in (("naive", 1), ("tree", 1), ("scatter_allgather", 1), ("chain", 8), ("chain", 32)):
            _, launches = vc.vcoll_broadcast_stepwise(algo, src, outs[0], 0, k)
            calls = [vc.prepare_broadcast_stepwise(algo, src, outs[i], 0, k) for i in range(R2)]
            _, ms = time_launches(calls, steps if nbytes < 2 ** 20 else 20, warm)
            msgs, _, _, nsteps = vc.vcoll_ledger_rooted("broadcast", algo, p, n, "f32", 0, k)
            rec[f"{algo}{k if algo == 'chain' else ''}"] = {
                "us": round(ms * 1e3, 2), "steps": nsteps, "launches": launches,
                "us_per_launch": round(ms * 1e3 / launches, 2),
                "ici_model_us": round(vc.vcoll_model_clock(msgs, p, 1e-6, 45e9) * 1e6, 2)}
        ex[f"stepwise_broadcast_p8_{label}"] = rec
        del src, outs
    torch.cuda.empty_cache()


def decode_prefill_extras(vc, torch, ex, steps, warm):
    """Decode-like (10 KiB) and prefill-like (80 MiB) messages, p = 8."""
    for label, nbytes in (("decode_10KiB", 10 * 1024), ("prefill_80MiB", 80 * 2 ** 20)):
        m = nbytes // 4
        g = torch.Generator(device="cuda").manual_seed(5)
        t = torch.randn((8, m), device="cuda", generator=g)
        R2 = min(64, sets_for(2 * 8 * nbytes))
        ts = [t.clone() for _ in range(R2)]
        os_ = [torch.empty_like(t) for _ in range(R2)]
        for algo in ("ring", "rd", "rabenseifner", "tree"):
            calls = [vc.prepare_allreduce(algo, ts[i], os_[i]) for i in range(R2)]
            _, mean_ms = time_launches(calls, steps, warm)
            ex[f"p8_{label}_{algo}"] = roof(f"reduce_kernel<f32, {algo}, p=8>", 2 * 8 * nbytes, mean_ms)
        del t, ts, os_
    torch.cuda.empty_cache()


def layout_extras(vc, torch, steps, warm) -> dict:
    """The ring all-reduce at p = 8 and p = 72, 16 MiB per rank, in four rank
    buffer layouts: rows of one [p, n] tensor a whole number of cache lines
    apart; separately allocated rows whose length is not a multiple of
    p * 4 elements (ragged chunks, common address phase); rows of one
    [p, n] tensor 16 bytes off a line apart (address phases differ mod 128);
    and rows of odd length (not 16-byte aligned: the element path)."""
    out = {}
    g = torch.Generator(device="cuda").manual_seed(9)
    for p in (8, 72):
        n0 = 16 * 2 ** 20 // 4
        for label, n, separate in (("lines_apart", n0, False), ("ragged_chunks", n0 + 4, True),
                                   ("phases_differ", n0 + 4, False), ("unaligned_rows", n0 + 1, False)):
            sets = []
            for _ in range(2):
                if separate:
                    x = [torch.randn(n, device="cuda", generator=g) for _ in range(p)]
                    y = [torch.empty(n, device="cuda") for _ in range(p)]
                else:
                    x = torch.randn((p, n), device="cuda", generator=g)
                    y = torch.empty_like(x)
                sets.append((x, y))
            calls = [vc.prepare_allreduce("ring", x, y) for x, y in sets]
            _, ms = time_launches(calls, max(10, steps // 2), warm)
            kernel = "burst_ring_kernel" if label in ("lines_apart", "ragged_chunks", "phases_differ") else "reduce_kernel"
            out[f"p{p}_{label}"] = roof(f"{kernel} (ring, n = {n:,})", 2 * p * n * 4, ms)
            del sets, calls
            torch.cuda.empty_cache()
    return out


def graph_extras(vc, torch, ex):
    """Decode-sized all-reduces replayed from a HIP graph: the per-call cost
    without the host's launch path (100 captured calls per replay)."""
    g = torch.Generator(device="cuda").manual_seed(7)
    t = torch.randn((8, 2560), device="cuda", generator=g)
    o = torch.empty_like(t)
    for algo in ("ring", "rd", "rabenseifner", "tree"):
        vc.vcoll_allreduce(algo, t, o)
        vc.vcoll_allreduce_stepwise(algo, t, o)
    torch.cuda.synchronize()
    for label, fn in (("fused", vc.vcoll_allreduce), ("stepwise", lambda a, x, y: vc.vcoll_allreduce_stepwise(a, x, y))):
        for algo in ("ring", "rd", "rabenseifner", "tree"):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(100):
                    fn(algo, t, o)
            _, ms = time_launches([graph.replay], 20, 3)
            ex[f"p8_decode_10KiB_{algo}_{label}_graph"] = {"us_per_allreduce": round(ms * 1e3 / 100, 2)}
            del graph
    del t, o
    torch.cuda.empty_cache()


def host_rows(vc) -> dict:
    """The host rows: partition + step schedule + ledger of a collective (the
    record-free ledger call builds every message and sums it per rank) and
    the MoE routing plan, through the Python binding, median of repeated calls."""
    import numpy as np
    import workloads

    def host_us(fn, reps):
        t = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return round(float(np.median(t)) * 1e6, 1)
    M = workloads.MOE
    topk = np.stack([workloads.moe_topk(r, M["tokens"], M["experts"], M["topk"]) for r in range(M["p"])])
    n8 = workloads.DDP_BUCKET["n"]
    host = {"ledger_ring_p8_ddp_bucket_us": host_us(lambda: vc.vcoll_ledger_summary("allreduce", "ring", 8, n8), 200)}
    for algo in ("ring", "rd", "rabenseifner", "tree"):
        host[f"ledger_{algo}_p72_us"] = host_us(lambda: vc.vcoll_ledger_summary("allreduce", algo, 72, 72 << 20), 50)
    host["ledger_ring_p72_messages"] = vc.vcoll_ledger_summary("allreduce", "ring", 72, 72 << 20)[0]
    host["moe_plan_8x4096x8_us"] = host_us(lambda: vc.vcoll_moe_plan(topk, M["experts"] // M["p"]), 20)
    return host


def moe_variants(vc, torch) -> dict:
    """The other MoE dispatch/combine forms on the same workload: the
    row-major gathering dispatch and scattering combine (generic all-to-all
    with index maps), the row-major FP8 dispatch, and the per-destination
    deduplicated dispatch with its local expansion."""
    import numpy as np
    import workloads
    M = workloads.MOE
    p8, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
    topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p8)])
    splits, src_rows, dst_rows = vc.vcoll_moe_plan(topk, E // p8)
    g = torch.Generator(device="cuda").manual_seed(4)
    toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p8)]
    srcs = [torch.from_numpy(src_rows[i]).cuda() for i in range(p8)]
    dsts = [torch.from_numpy(dst_rows[i]).cuda() for i in range(p8)]
    rb, orb = H * 2, H + H // 32
    rows = int(splits.sum())
    uniq = p8 * T * rb                              # every token row once: the algorithmic read of a dispatch
    res = {}
    recv = vc.vcoll_all_to_all(toks, splits, src_rows=srcs)
    back = vc.vcoll_all_to_all(recv, splits.T, dst_rows=dsts, dst_table_rows=[T * K] * p8)
    disp = lambda: vc.vcoll_all_to_all(toks, splits, recv=recv, src_rows=srcs)          # noqa: E731
    comb = lambda: vc.vcoll_all_to_all(recv, splits.T, recv=back, dst_rows=dsts)         # noqa: E731
    _, ms = time_launches([disp], 10, 2)
    res["dispatch_row_major_gather"] = roof("all_to_all_kernel<256> with gather map", uniq + rows * rb, ms,
                                            note="reads each token row once per (token, expert) pair: 8x the "
                                                 "unique token bytes")
    _, ms = time_launches([comb], 10, 2)
    res["combine_row_major_scatter"] = roof("all_to_all_kernel<256> with scatter map", 2 * rows * rb, ms)
    src_g = [torch.from_numpy(src_rows[i][:int(splits[i].sum())].copy()).cuda() for i in range(p8)]
    f8 = vc.vcoll_moe_dispatch_fp8(toks, splits, src_g)
    fp8_call = lambda: vc.vcoll_moe_dispatch_fp8(toks, splits, src_g, f8)               # noqa: E731
    _, ms = time_launches([fp8_call], 10, 2)
    res["dispatch_fp8_row_major_gather"] = roof("dispatch_fp8_kernel", uniq + rows * orb, ms,
                                                note="reads each token row once per (token, expert) pair")
    del f8, recv, back
    su, src_u, expand = vc.vcoll_moe_plan_dedup(topk, E // p8)
    src_ug = [torch.from_numpy(x).cuda() for x in src_u]
    exp_g = [torch.from_numpy(x).cuda() for x in expand]
    ru = vc.vcoll_all_to_all(toks, su, src_rows=src_ug)
    ex_out = vc.vcoll_moe_expand(ru, exp_g)
    rows_u = int(su.sum())
    d1 = lambda: vc.vcoll_all_to_all(toks, su, recv=ru, src_rows=src_ug)         # noqa: E731
    d2 = lambda: vc.vcoll_moe_expand(ru, exp_g, ex_out)                           # noqa: E731
    _, ms_u = time_launches([d1], 10, 2)
    _, ms_x = time_launches([d2], 10, 2)
    xslots = [torch.from_numpy(vc.vcoll_moe_expand_slots(int(su[:, j].sum()), expand[j], K)).cuda()
              for j in range(p8)]
    xcounts = [len(e) for e in expand]
    ex_tm = vc.vcoll_moe_expand_token_major(ru, xslots, xcounts, K)
    tm_x_ok = all(torch.equal(ex_tm[j].view(torch.int16), ex_out[j].view(torch.int16)) for j in range(p8))
    d3 = lambda: vc.vcoll_moe_expand_token_major(ru, xslots, xcounts, K, out=ex_tm)  # noqa: E731
    _, ms_xt = time_launches([d3], 10, 2)
    dsl = vc.vcoll_moe_dedup_slots(su, src_u, T, K)
    dsl_g = [torch.from_numpy(np.ascontiguousarray(dsl[i])).cuda() for i in range(p8)]
    urows = su.sum(axis=0)
    ru_tm = vc.vcoll_moe_dispatch(toks, dsl_g, urows, K)
    ru8 = vc.vcoll_moe_dispatch_fp8(toks, su, src_ug)
    ru8_tm = vc.vcoll_moe_dispatch(toks, dsl_g, urows, K, fp8=True)
    dd_ok = all(torch.equal(ru_tm[j].view(torch.int16), ru[j].view(torch.int16)) and torch.equal(ru8_tm[j], ru8[j])
                for j in range(p8))
    d4 = lambda: vc.vcoll_moe_dispatch(toks, dsl_g, urows, K, recv=ru_tm)            # noqa: E731
    d5 = lambda: vc.vcoll_moe_dispatch(toks, dsl_g, urows, K, fp8=True, recv=ru8_tm)  # noqa: E731
    _, ms_dt = time_launches([d4], 10, 2)
    _, ms_d8t = time_launches([d5], 10, 2)
    offrank = lambda sp: int(sp.sum() - np.trace(sp))                              # noqa: E731
    res["dispatch_dedup_token_major"] = roof("dispatch_push_kernel<false, 64>, deduplicated plan",
                                             uniq + rows_u * rb, ms_dt)
    res["dispatch_dedup_token_major_fp8"] = roof("dispatch_push_kernel<true, 512> (FP8), deduplicated plan",
                                                 uniq + rows_u * orb, ms_d8t)
    res["dedup"] = {
        "rows": rows_u, "rows_plain": rows, "offrank_rows": offrank(su), "offrank_rows_plain": offrank(splits),
        "all_to_all_gather_us": round(ms_u * 1e3, 1), "expand_us": round(ms_x * 1e3, 1),
        "expand_token_major_us": round(ms_xt * 1e3, 1), "expand_token_major_equal": bool(tm_x_ok),
        "token_major_equal_row_major": bool(dd_ok),
        "message_bytes_bf16": offrank(su) * rb, "message_bytes_fp8": offrank(su) * orb,
        "message_bytes_plain_bf16": offrank(splits) * rb}
    del toks, ru, ex_out, ex_tm, ru_tm, ru8, ru8_tm
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# rocprofv3 summaries

def _csv_rows(root: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


HEADLINE_KERNEL = "burst_ring_kernel<0, 25, 0>"
COPY_KERNEL = "copy_kernel<2, 64"


def summarize_profile(trace_dir: str, fetch_dir: str, write_dir: str, command: str) -> int:
    """Kernel-trace statistics and FETCH_SIZE / WRITE_SIZE counters of the
    headline kernel, scaled by the same counters of the plain copy kernel of
    known size, written to profiles/. If TRACE_DIR holds bench.json (the JSON
    line the profiled command printed), the events-based mean launch time of
    that same run is set beside rocprof's."""
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = [f"# rocprofv3 kernel statistics: headline ring all-reduce (p=8, 25 MiB fp32/rank)", "",
             f"Command: `{command}`", "", "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    bench_json = os.path.join(trace_dir, "bench.json")
    code_hash = None                                # of the library the profiled run loaded
    if os.path.exists(bench_json):
        with open(bench_json) as f:
            code_hash = json.loads(f.read().strip().splitlines()[-1])["roofline"].get("kernel_code")
    rocprof_avg = None
    for r in stats:
        name = r.get('Name', r.get('KernelName', '?'))
        lines.append(f"| {name[:90]} | {r.get('Calls')} | "
                     f"{r.get('AverageNs')} | {r.get('MinNs')} | {r.get('MaxNs')} |")
        if HEADLINE_KERNEL in name:
            rocprof_avg = float(r["AverageNs"]) / 1e3
    if rocprof_avg is not None and os.path.exists(bench_json):
        with open(bench_json) as f:
            run = json.loads(f.read().strip().splitlines()[-1])
        ev = run["roofline"]["mean_launch_us"]
        lines += ["", f"Same run: bench.py events mean launch {ev} us, rocprofv3 average {rocprof_avg:.2f} us "
                      f"(the profiler's average includes the {run['warmup']} warm-up launches); "
                      f"roofline.achieved {run['roofline']['achieved']} GB/s by events, "
                      f"{419430400 / (rocprof_avg * 1e-6) / 1e9:.1f} GB/s by rocprofv3."]

    trace = [r for r in _csv_rows(trace_dir, "kernel_trace.csv") if HEADLINE_KERNEL in r.get("Kernel_Name", "")]
    if trace:
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace)

        def pct(q):
            return d[min(len(d) - 1, int(q * (len(d) - 1) + 0.5))]
        r0 = trace[0]
        lines += ["", f"Headline launches in the kernel trace: {len(d)} (warm-up included); duration "
                      f"p10 {pct(0.1):.2f} us, median {pct(0.5):.2f} us, p90 {pct(0.9):.2f} us. Per dispatch: "
                      f"{r0.get('VGPR_Count')} VGPRs, {r0.get('SGPR_Count')} SGPRs, {r0.get('LDS_Block_Size')} B LDS, "
                      f"{r0.get('Scratch_Size')} B scratch, workgroup {r0.get('Workgroup_Size_X')} work-items, "
                      f"grid {r0.get('Grid_Size_X')} x {r0.get('Grid_Size_Y')} work-items."]

    def per_dispatch(root, counter):
        out = {}
        for r in _csv_rows(root, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            if "vcoll::" not in name:               # torch's own kernels (direct_copy_kernel_cuda, ...)
                continue
            key = "headline" if HEADLINE_KERNEL in name else ("copy" if COPY_KERNEL in name else None)
            if key:
                out.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in out.items()}

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    traffic = None
    if "headline" in fetch and "copy" in fetch and "headline" in write and "copy" in write:
        p, n = 8, 6_553_600
        copy_bytes = p * n * 4                      # read, and again written, by one copy launch
        f_scale = copy_bytes / fetch["copy"]
        w_scale = copy_bytes / write["copy"]
        traffic = round(fetch["headline"] * f_scale + write["headline"] * w_scale)
        lines += ["", "## HBM traffic from counters (per launch)", "",
                  f"FETCH_SIZE headline {fetch['headline']:.0f}, copy {fetch['copy']:.0f} "
                  f"(copy reads {copy_bytes} B: scale {f_scale:.2f} B/unit)",
                  f"WRITE_SIZE headline {write['headline']:.0f}, copy {write['copy']:.0f} "
                  f"(copy writes {copy_bytes} B: scale {w_scale:.2f} B/unit)",
                  f"headline traffic {traffic} B per launch vs 419430400 algorithmic "
                  f"({traffic / 419430400:.3f}x)"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "ring_allreduce_f32_p8_25MiB.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(tpath)) if os.path.exists(tpath) else {}
    data["ring_f32_p8_ddp_bucket"] = {"code_hash": code_hash, "bytes_per_launch": traffic,
                                      "fetch_units": fetch, "write_units": write}
    with open(tpath, "w") as f:
        json.dump(data, f, indent=1)
    print("\n".join(lines))
    return 0


def summarize_stats(trace_dir: str, name: str, title: str, command: str) -> int:
    """rocprofv3 --kernel-trace --stats output as a table in profiles/<name>.md:
    one row per libvcoll kernel instantiation (calls, average, min and max
    duration), plus p10 / median / p90 of each from the kernel trace."""
    stats = [r for r in _csv_rows(trace_dir, "kernel_stats.csv") if "vcoll::" in r.get("Name", r.get("KernelName", ""))]
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    lines = [f"# rocprofv3 kernel statistics: {title}", "", f"Command: `{command}`", "",
             "Template arguments of reduce_kernel: dtype (0 f32, 1 bf16), algorithm (0 ring, 1 recursive doubling, "
             "2 Rabenseifner, 3 tree), p (0: read at run time), vectors per thread, reduce-scatter, large-grid "
             "variant, workgroup size; of burst_ring_kernel: dtype, vectors per thread, store cache policy "
             "(0 through L2, 2 streamed); of reduce_small_kernel: dtype, algorithm, reduce-scatter, slots per "
             "wave.", "",
             "| kernel | calls | average us | min us | max us | p10 us | median us | p90 us |",
             "|---|---|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0) or 0)):
        full = r.get("Name", r.get("KernelName", "?"))
        short = full.replace("vcoll::(anonymous namespace)::", "")
        short = short.split("(vcoll::")[0].split("(")[0] if short.startswith(("reduce", "burst", "hier")) else short
        d = sorted((int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3
                   for t in trace if t.get("Kernel_Name") == full)

        def pct(q):
            return d[min(len(d) - 1, int(q * (len(d) - 1) + 0.5))] if d else float("nan")
        lines.append(f"| {short[:100]} | {r.get('Calls')} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {pct(0.1):.2f} | "
                     f"{pct(0.5):.2f} | {pct(0.9):.2f} |")
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


# Counter-traffic workloads, in launch order. Each entry: (label, kernel
# name substring as rocprofv3 prints it, algorithmic bytes per launch or
# None when the routing decides them, printed by the run). A one-workgroup
# marker launch separates consecutive workloads in the counter records.
TRAFFIC_GROUPS = {
    "hot": [
        ("two-phase ring all-reduce, p=8 x 25 MiB f32 (headline)", "burst_ring_kernel<0, 25, 0>", 419_430_400),
        ("hierarchical 2x4 all-reduce, p=8 x 25 MiB f32", "hier_kernel<0, 2, 4, true>", 419_430_400),
        ("tree reduce to one root, p=8 x 25 MiB f32", "reduce_kernel<0, 3, 8, 4, true, false, 256>", 235_929_600),
        ("broadcast of 25 MiB f32 to 8 buffers", "broadcast_kernel<4, 4, 64, true>", 235_929_600),
        ("copy, 200 MiB read + 200 MiB written (counter scale)", "copy_kernel<2, 64", 419_430_400),
        ("fused ring all-reduce, p=16 x 192 MiB bf16", "reduce_kernel<1, 0, 16, 1, false, true, 64>", 6_442_450_944),
        ("ring reduce-scatter, p=16 x 192 MiB bf16", "reduce_kernel<1, 0, 16, 1, true, false, 64>", 3_422_552_064),
        ("all-gather of 12 MiB bf16 blocks, p=16", "all_gather_kernel<2, 1, 64, false>", 3_422_552_064),
        ("variable-split all-to-all of the MoE splits (plain)", "all_to_all_kernel<1024>", None),
        ("token-major MoE dispatch, bf16", "dispatch_push_kernel<false, 64>", None),
        ("token-major MoE dispatch, FP8", "dispatch_push_kernel<true, 512>", None),
        ("token-major MoE combine", "combine_pull_kernel<64>", None),
        ("row-major MoE dispatch, gather map (all-to-all)", "all_to_all_kernel<256>", None),
        ("row-major FP8 dispatch (gather + quantise)", "dispatch_fp8_kernel", None),
    ],
    "sweep": [
        ("copy, 200 MiB read + 200 MiB written (counter scale)", "copy_kernel<2, 64", 419_430_400),
        ("ring all-reduce, p=72 x 16 MiB f32 (two-phase, ragged chunks)", "burst_ring_kernel<0, 25, 0>",
         2 * 72 * 16 * 2 ** 20),
        ("tree all-reduce, p=72 x 16 MiB f32 (run-time order)", "reduce_kernel<0, 3, 0, 1, false, false, 64>",
         2 * 72 * 16 * 2 ** 20),
        ("ring all-reduce, p=72 x 256 MiB f32 (run-time order)", "reduce_kernel<0, 0, 0, 1, false, false, 64>",
         2 * 72 * 256 * 2 ** 20),
        ("tree all-reduce, p=72 x 256 MiB f32 (run-time order)", "reduce_kernel<0, 3, 0, 1, false, false, 64>",
         2 * 72 * 256 * 2 ** 20),
        ("ring reduce-scatter, p=72 x 64 MiB f32 (unaligned chunk starts)",
         "reduce_scatter_shifted_kernel<0, true>", 73 * 64 * 2 ** 20),
        ("ring all-reduce, p=16 x 16 MiB f32", "burst_ring_kernel<0, 25, 0>", 2 * 16 * 16 * 2 ** 20),
        ("ring all-reduce, p=16 x 64 MiB f32", "reduce_kernel<0, 0, 16, 1, false, true, 64>", 2 * 16 * 64 * 2 ** 20),
        ("ring all-reduce, p=8 x 1 GiB f32", "reduce_kernel<0, 0, 8, 4, false, true, 256>", 2 * 8 * 2 ** 30),
    ],
}


def traffic_set(vc, torch, launches: int, group: str) -> int:
    """Launch each workload of TRAFFIC_GROUPS[group] `launches` times (after
    one warm-up), a marker launch before each, for rocprofv3 --pmc
    FETCH_SIZE / WRITE_SIZE runs. Prints the group's manifest (labels,
    kernels, algorithmic bytes, the routing-dependent ones filled in) as one
    JSON line."""
    import numpy as np
    import workloads

    marker_buf = torch.empty(4 * 64, device="cuda")
    marker = vc.prepare_bench_stream("write", marker_buf)          # one workgroup of 64

    def run(call):
        torch.cuda.synchronize()
        marker()
        for _ in range(launches + 1):
            call()
        torch.cuda.synchronize()

    def copy_ref():
        src, dst = torch.empty(8 * 6_553_600, device="cuda"), torch.empty(8 * 6_553_600, device="cuda")
        run(vc.prepare_bench_stream("copy", dst, src))

    filled = {}
    g = torch.Generator(device="cuda").manual_seed(9)
    if group == "hot":
        p, n = 8, workloads.DDP_BUCKET["n"]
        t = torch.randn((p, n), device="cuda", generator=g) * 1e-3
        o = torch.empty_like(t)
        run(vc.prepare_allreduce("ring", t, o))
        run(vc.prepare_allreduce_hierarchical(2, 4, t, o))
        root_out = torch.empty(n, device="cuda")
        run(vc.prepare_reduce(t, root_out, 0))
        run(vc.prepare_broadcast(t[0].clone(), o, 0))
        copy_ref()
        del t, o, root_out
        torch.cuda.empty_cache()
        P16, N16 = 16, 100_663_296
        t16 = (torch.rand((P16, N16), device="cuda", generator=g) * 2 - 1).to(torch.bfloat16)
        o16 = torch.empty_like(t16)
        run(vc.prepare_allreduce("ring", t16, o16))
        rs16 = [torch.empty(N16 // P16, dtype=torch.bfloat16, device="cuda") for _ in range(P16)]
        run(vc.prepare_reduce_scatter("ring", t16, rs16))
        run(vc.prepare_all_gather("ring", rs16, o16))
        del t16, o16, rs16
        torch.cuda.empty_cache()
        M = workloads.MOE
        p8, T, H, E, K = M["p"], M["tokens"], M["hidden"], M["experts"], M["topk"]
        topk = np.stack([workloads.moe_topk(r, T, E, K) for r in range(p8)])
        splits, src_rows, dst_rows = vc.vcoll_moe_plan(topk, E // p8)
        toks = [torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16) for _ in range(p8)]
        rb, orb, rows = 2 * H, H + H // 32, int(splits.sum())
        plain_send = [torch.randn((int(splits[i].sum()), H), device="cuda", generator=g).to(torch.bfloat16)
                      for i in range(p8)]
        plain_recv = vc.vcoll_all_to_all(plain_send, splits)
        run(lambda: vc.vcoll_all_to_all(plain_send, splits, recv=plain_recv))
        del plain_send, plain_recv
        slots = vc.vcoll_moe_slots(splits, dst_rows, K)
        slots_g = [torch.from_numpy(np.ascontiguousarray(slots[i])).cuda() for i in range(p8)]
        recv_rows = splits.sum(axis=0)
        tm = vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K)
        run(lambda: vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, recv=tm))
        tm8 = vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, fp8=True)
        run(lambda: vc.vcoll_moe_dispatch(toks, slots_g, recv_rows, K, fp8=True, recv=tm8))
        tc = vc.vcoll_moe_combine(tm, slots_g, T, K)
        run(lambda: vc.vcoll_moe_combine(tm, slots_g, T, K, out=tc))
        srcs = [torch.from_numpy(src_rows[i]).cuda() for i in range(p8)]
        run(lambda: vc.vcoll_all_to_all(toks, splits, recv=tm, src_rows=srcs))
        src_g = [torch.from_numpy(src_rows[i][:int(splits[i].sum())].copy()).cuda() for i in range(p8)]
        run(lambda: vc.vcoll_moe_dispatch_fp8(toks, splits, src_g, tm8))
        uniq = p8 * T * rb                          # every token row once
        filled = {"all_to_all_kernel<1024>": 2 * rows * rb, "dispatch_push_kernel<false, 64>": uniq + rows * rb,
                  "dispatch_push_kernel<true, 512>": uniq + rows * orb, "combine_pull_kernel<64>": 2 * rows * rb,
                  "all_to_all_kernel<256>": uniq + rows * rb, "dispatch_fp8_kernel": uniq + rows * orb}
    else:
        copy_ref()
        for p, mib, algos in ((72, 16, ("ring", "tree")), (72, 256, ("ring", "tree"))):
            n = mib * 2 ** 18
            t = torch.randn((p, n), device="cuda", generator=g)
            o = torch.empty_like(t)
            for algo in algos:
                run(vc.prepare_allreduce(algo, t, o))
            del t, o
            torch.cuda.empty_cache()
        n = 64 * 2 ** 18
        t = torch.randn((72, n), device="cuda", generator=g)
        rs = vc.vcoll_reduce_scatter("ring", t)
        run(vc.prepare_reduce_scatter("ring", t, rs))
        del t, rs
        torch.cuda.empty_cache()
        for p, mib in ((16, 16), (16, 64), (8, 1024)):
            n = mib * 2 ** 18
            t = torch.randn((p, n), device="cuda", generator=g)
            o = torch.empty_like(t)
            run(vc.prepare_allreduce("ring", t, o))
            del t, o
            torch.cuda.empty_cache()
    manifest = [{"label": lab, "kernel": k, "algorithmic_bytes": b if b is not None else filled[k],
                 "dispatches": launches + 1} for lab, k, b in TRAFFIC_GROUPS[group]]
    print(json.dumps({"traffic_manifest": manifest, "group": group}), flush=True)
    return 0


def summarize_traffic(fetch_dir: str, write_dir: str, manifest_log: str, command: str) -> int:
    """Per-workload HBM bytes per launch from the two counter runs of
    --traffic-set (FETCH_SIZE, WRITE_SIZE), scaled by the copy's readings,
    against each workload's algorithmic bytes: a table in profiles/. The
    counter records are cut into workloads at the marker launches."""
    with open(manifest_log) as f:
        info = json.loads([ln for ln in f.read().splitlines() if "traffic_manifest" in ln][-1])
    manifest, group = info["traffic_manifest"], info["group"]

    def segments(root, counter):
        recs = [r for r in _csv_rows(root, "counter_collection.csv")
                if r.get("Counter_Name") == counter and "vcoll::" in r.get("Kernel_Name", "")]
        recs.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        segs, cur = [], None
        for r in recs:
            name = r["Kernel_Name"]
            if "write_kernel<4, 64>" in name and int(r.get("Grid_Size", 0)) == 64:
                cur = []
                segs.append(cur)
            elif cur is not None:
                cur.append(r)
        # the marker launch made while preparing the markers opens an extra
        # first segment; a workload's own preparation call runs before its
        # marker, so it ends the previous segment: take the first `dispatches`
        # matching records of each of the last len(manifest) segments
        out = []
        for seg, m in zip(segs[-len(manifest):], manifest):
            vals = [float(r["Counter_Value"]) for r in seg if m["kernel"] in r["Kernel_Name"]][:m["dispatches"]]
            out.append((sum(vals) / len(vals), len(vals)) if vals else (None, 0))
        return out

    fetch = segments(fetch_dir, "FETCH_SIZE")
    write = segments(write_dir, "WRITE_SIZE")
    ci = next(i for i, m in enumerate(manifest) if m["kernel"].startswith("copy_kernel"))
    half = manifest[ci]["algorithmic_bytes"] // 2
    f_scale, w_scale = half / fetch[ci][0], half / write[ci][0]
    lines = [f"# HBM traffic per launch from rocprofv3 counters: {group} kernels", "",
             f"Command: `{command}`", "",
             f"FETCH_SIZE and WRITE_SIZE per dispatch, averaged over each workload's dispatches (warm-up "
             f"included), scaled by the copy's readings for {half} B read and written: {f_scale:.2f} B per "
             f"FETCH_SIZE unit, {w_scale:.2f} B per WRITE_SIZE unit. Algorithmic bytes are the bytes each "
             f"operation must move (inputs read once, outputs written once).", "",
             "| workload | kernel | dispatches | read B | written B | algorithmic B | traffic / algorithmic |",
             "|---|---|---|---|---|---|---|"]
    out = {}
    for m, (fv, nf), (wv, _) in zip(manifest, fetch, write):
        if fv is None or wv is None:
            lines.append(f"| {m['label']} | {m['kernel']} | 0 | - | - | {m['algorithmic_bytes']:,} | - |")
            continue
        rd, wr = fv * f_scale, wv * w_scale
        ratio = (rd + wr) / m["algorithmic_bytes"]
        out[m["label"]] = {"read": round(rd), "written": round(wr), "ratio": round(ratio, 4)}
        lines.append(f"| {m['label']} | {m['kernel']} | {nf} | {rd:,.0f} | {wr:,.0f} | "
                     f"{m['algorithmic_bytes']:,} | {ratio:.3f} |")
    name = "traffic_hot_kernels.md" if group == "hot" else "traffic_sweep_kernels.md"
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def sweep(vc, torch, out_path: str, max_bytes: int) -> int:
    """Message-size sweep of the fused all-reduce: every p in SWEEP_P, every
    per-rank size in SWEEP_BYTES up to max_bytes, every algorithm. Each point
    is timed (events over back-to-back launches on one buffer set, so points
    whose 2*p*S fits the 256 MB Infinity Cache run partly from it) and
    checked on every element: all ranks equal to rank 0 and, where memory
    allows, equal to the stepwise (one launch per step) execution of the
    same algorithm. (Parity of every point with the oracle is the GPU test
    tests/test_gpu_sweep.py.) One JSON line per point goes to out_path."""
    import workloads
    fails = 0
    with open(out_path, "w") as out:
        for p in workloads.SWEEP_P:
            for nbytes in workloads.SWEEP_BYTES:
                if nbytes > max_bytes:
                    continue
                n = nbytes // 4
                g = torch.Generator(device="cuda").manual_seed(workloads.TAG_SWEEP * 10 ** 6 + p * 1000 + nbytes % 997)
                t = torch.randn((p, n), device="cuda", generator=g)
                o = torch.empty_like(t)
                step_ok = 3 * p * nbytes <= 64 * 2 ** 30
                for algo in ("ring", "rd", "rabenseifner", "tree"):
                    call = vc.prepare_allreduce(algo, t, o)
                    K = int(min(200, max(5, 4e9 / (2 * p * nbytes))))
                    _, ms = time_launches([call], K, 3)
                    rec = {"p": p, "bytes_per_rank": nbytes, "algo": algo, "us": round(ms * 1e3, 2),
                           "GBps": rate(2 * p * nbytes, ms), "launches": K}
                    call()
                    torch.cuda.synchronize()
                    rec["ranks_equal"] = all(torch.equal(o[r].view(torch.int32), o[0].view(torch.int32))
                                             for r in range(1, p))
                    if step_ok:
                        st = torch.empty_like(t)
                        vc.vcoll_allreduce_stepwise(algo, t, st)
                        torch.cuda.synchronize()
                        rec["stepwise_equal"] = bool(torch.equal(st.view(torch.int32), o.view(torch.int32)))
                        del st
                    good = rec["ranks_equal"] and rec.get("stepwise_equal", True)
                    fails += 0 if good else 1
                    out.write(json.dumps(rec) + "\n")
                    out.flush()
                    print(f"sweep p={p} {nbytes} B {algo}: {rec['us']} us {rec['GBps']} GB/s "
                          f"{'ok' if good else 'MISMATCH'}", file=sys.stderr, flush=True)
                del t, o
                torch.cuda.empty_cache()
    return 1 if fails else 0


def summarize_sweep(jsonl: str, command: str, parity_jsonl: str = "") -> int:
    """The sweep's JSON lines as a table in profiles/: microseconds where the
    whole all-reduce moves less than 64 MiB (latency-bound), GB/s above;
    with parity_jsonl (the VCOLL_PARITY_LOG of tests/test_gpu_sweep.py), the
    fraction of every point's elements compared with the oracle."""
    recs = [json.loads(x) for x in open(jsonl)]
    sizes = sorted({r["bytes_per_rank"] for r in recs})

    def label(b):
        return f"{b >> 30} GiB" if b >= 2 ** 30 else (f"{b >> 20} MiB" if b >= 2 ** 20 else f"{b >> 10} KiB")
    bad = [r for r in recs if not (r["ranks_equal"] and r.get("stepwise_equal", True))]
    lines = ["# Fused all-reduce message-size sweep (float32, one buffer set; the ring takes the two-phase burst_ring_kernel where the whole vector fits one generation of workgroups, reduce_kernel elsewhere)", "",
             f"Command: `{command}`", "",
             f"{len(recs)} points, {len(bad)} mismatches on the GPU-side checks: all ranks equal on every "
             f"point, and the stepwise execution equal on every element for "
             f"{sum('stepwise_equal' in r for r in recs)} points. Parity of every point with the oracle "
             f"(whole vectors up to 2^25 elements, windows beyond) is tests/test_gpu_sweep.py.", "",
             "Cells: microseconds per all-reduce when 2*p*S < 64 MiB, else GB/s of algorithmic bytes (2*p*S). "
             "Buffers are reused, so points whose 2*p*S fits the 256 MB Infinity Cache run partly from it.", ""]
    for algo in ("ring", "rd", "rabenseifner", "tree"):
        lines += [f"## {algo}", "", "| p | " + " | ".join(label(b) for b in sizes) + " |",
                  "|---|" + "---|" * len(sizes)]
        for p in sorted({r["p"] for r in recs}):
            cells = []
            for b in sizes:
                r = [x for x in recs if x["p"] == p and x["bytes_per_rank"] == b and x["algo"] == algo]
                if not r:
                    cells.append("")
                elif 2 * p * b < 64 * 2 ** 20:
                    cells.append(f"{r[0]['us']:.1f} us")
                else:
                    cells.append(f"{r[0]['GBps']:.0f}")
            lines.append(f"| {p} | " + " | ".join(cells) + " |")
        lines.append("")
    # the virtual cluster read through the pages' alpha-beta model (T = alpha
    # + bytes / beta, half-performance length n_1/2 = alpha * beta): alpha is
    # the fastest point moving under 1 MiB in all (the launch floor), beta the
    # least-squares slope over the points moving at least 512 MiB (out of the
    # Infinity Cache); bytes are the algorithmic 2*p*S
    import numpy as np
    lines += ["## alpha-beta reading", "",
              "T = alpha + 2pS / beta: alpha = fastest point moving < 1 MiB in all (launch floor), beta = "
              "least-squares slope of time against 2pS over the points moving >= 512 MiB; "
              "n_1/2 = alpha * beta, the per-call bytes at which half of beta is reached.", "",
              "| algorithm | p | alpha (us) | beta (TB/s) | n_1/2 (MiB moved) |", "|---|---|---|---|---|"]
    for algo in ("ring", "rd", "rabenseifner", "tree"):
        for p in sorted({r["p"] for r in recs}):
            pts = [r for r in recs if r["p"] == p and r["algo"] == algo]
            small = [r["us"] for r in pts if 2 * p * r["bytes_per_rank"] < 2 ** 20]
            big = [(2 * p * r["bytes_per_rank"], r["us"]) for r in pts if 2 * p * r["bytes_per_rank"] >= 2 ** 29]
            if not small or len(big) < 2:
                continue
            alpha = min(small)
            slope = float(np.polyfit([b for b, _ in big], [t for _, t in big], 1)[0])      # us per byte
            beta = 1e6 / slope                                                             # bytes per second
            lines.append(f"| {algo} | {p} | {alpha:.1f} | {beta / 1e12:.2f} | "
                         f"{alpha * 1e-6 * beta / 2 ** 20:.0f} |")
    lines.append("")
    if parity_jsonl:
        par = [json.loads(x) for x in open(parity_jsonl)]
        frac = {}
        for r in par:
            frac.setdefault((r["p"], r["bytes_per_rank"]), []).append(r["verified"] / r["total"])
        lines += ["## Elements compared with the oracle (tests/test_gpu_sweep.py, every algorithm)", "",
                  f"{sum(1 for r in par if r['verified'] == r['total'])} of {len(par)} (p, size, algorithm) points "
                  f"compared on every element; the others on every chunk boundary plus 16 random 1024-element "
                  f"windows, the fraction below.", "",
                  "| p | " + " | ".join(label(b) for b in sizes) + " |", "|---|" + "---|" * len(sizes)]
        for p in sorted({r["p"] for r in recs}):
            cells = []
            for b in sizes:
                f = frac.get((p, b))
                cells.append("" if not f else ("100 %" if min(f) == 1 else f"{100 * min(f):.3g} %"))
            lines.append(f"| {p} | " + " | ".join(cells) + " |")
        lines.append("")
    with open(os.path.join(ROOT, "profiles", "reduce_kernel_sweep_p2-72_1KiB-1GiB.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 1 if bad else 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--only", default="", help="comma-separated extras sections to run (default all): "
                    + ", ".join(EXTRA_SECTIONS))
    ap.add_argument("--copy-reference", type=int, default=0, metavar="K",
                    help="after the headline, launch the plain copy K times over the headline's "
                         "bytes (a known-size kernel to scale hardware counter readings)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 output directories into profiles/ summaries and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summaries")
    ap.add_argument("--sweep", metavar="OUT_JSONL", help="run the message-size sweep instead, one JSON line per "
                    "(p, size, algorithm) point written to OUT_JSONL, and exit")
    ap.add_argument("--sweep-max-bytes", type=int, default=2 ** 30, help="largest per-rank size of the sweep")
    ap.add_argument("--traffic-group", default="hot", choices=sorted(TRAFFIC_GROUPS),
                    help="which workloads --traffic-set launches")
    ap.add_argument("--traffic-set", type=int, default=0, metavar="K",
                    help="launch each hot kernel K times (plus a warm-up) for counter runs, then exit")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRAFFIC_SET_LOG"),
                    help="turn the counter runs of --traffic-set into a table in profiles/ and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("TRACE_DIR", "NAME", "TITLE"),
                    help="turn a rocprofv3 --kernel-trace --stats directory into profiles/NAME.md and exit")
    ap.add_argument("--parity-log", default="", help="with --summarize-sweep: the JSON lines tests/test_gpu_sweep.py "
                    "writes to VCOLL_PARITY_LOG")
    ap.add_argument("--summarize-sweep", metavar="SWEEP_JSONL", help="turn a sweep's JSON lines into a table in "
                    "profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_profile:
        return summarize_profile(*args.summarize_profile, args.profile_command)
    if args.summarize_stats:
        return summarize_stats(*args.summarize_stats, args.profile_command)
    if args.summarize_sweep:
        return summarize_sweep(args.summarize_sweep, args.profile_command, args.parity_log)
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.profile_command)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py: --gpus {args.gpus} requested; this build runs its p logical ranks inside one "
                  "GPU's HBM (a single-GPU virtual cluster) and measures one GPU only.", file=sys.stderr)
        return 2

    import torch
    import collective_communication_algorithms_vcoll_amd as vc

    torch.cuda.set_device(0)
    if args.sweep:
        return sweep(vc, torch, args.sweep, args.sweep_max_bytes)
    if args.traffic_set:
        return traffic_set(vc, torch, args.traffic_set, args.traffic_group)
    h = headline(vc, torch, args)
    value = h["nbytes"] * args.steps / h["wall"] / 1e9
    achieved = h["nbytes"] / (h["mean_ms"] * 1e-3) / 1e9
    traffic = counter_traffic("ring_f32_p8_ddp_bucket")
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["wall"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded normal(0, 1e-3) float32 rank buffers",
        "config": {
            "workload": "DDP gradient-bucket all-reduce: p=8 logical ranks x 25 MiB fp32 "
                        "(6,553,600 elements) per rank, ring order 0->1->..->7, "
                        "reduce-scatter + all-gather fused in one pass",
            "p": h["p"], "elements_per_rank": h["n"], "algorithm": "ring",
            "algorithmic_bytes_per_step": h["nbytes"], "buffer_sets_cycled": h["sets"],
        },
        "device": device_info(torch),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
            "kernel": "burst_ring_kernel<f32, 25 vectors per thread> (two-phase ring, 256 workgroups)",
            "mean_launch_us": round(h["mean_ms"] * 1e3, 2), "launch_us": h["dist"],
            "kernel_code": kernel_code_hash(),
        },
    }
    if args.copy_reference:
        p, n = h["p"], h["n"]
        src, dst = torch.empty(p * n, device="cuda"), torch.empty(p * n, device="cuda")
        call = vc.prepare_bench_copy(dst, src)
        time_launches([call], args.copy_reference, 1)
        line["copy_reference"] = {"bytes_read": p * n * 4, "bytes_written": p * n * 4,
                                  "launches": args.copy_reference + 1}
    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline(h, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity_vs_oracle"] = "bit-exact" if parity else "MISMATCH"
    if not args.no_extras:
        line["extras"] = extras(vc, torch, h, args)
    print(json.dumps(line), flush=True)
    return 0 if line.get("parity_vs_oracle", "bit-exact") == "bit-exact" else 1


if __name__ == "__main__":
    sys.exit(main())
