#!/usr/bin/env python3
"""Reduce-scatter throughput on one MI355X: effective HBM GB/s and % of peak.

Workload: reduce-scatter sum, fp32, W = 8 virtual ranks of 67,108,864
elements (256 MiB) each, N(0, 1e-3) from per-rank seeds; each block of
8,388,608 elements folded in ring order (k+1)%8, ..., k.  One step = one
reduce-scatter launch over inputs already resident in HBM.

Effective bytes per step = every input read once + every output written once
= 8 * 256 MiB + 8 * 32 MiB = 2,415,919,104 B.  Peak HBM3E bandwidth of the
MI355X: 8 TB/s.

Layout: the W rank buffers are consecutive slices of one HBM allocation, as
a flat gradient buffer per virtual rank would be (``--layout separate`` puts
each rank in its own PyTorch allocation instead).

Prints ONE JSON line on stdout; progress goes to stderr.

``--calibrate-copy`` instead runs a plain 1 GiB device copy (the library's
all-gather over one rank) a few times: the reference kernel of known size that
rocprofv3's FETCH_SIZE / WRITE_SIZE counters are scaled by.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_reduce_scatter_w8_64Mi_f32.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, if the
    kernel sources are unchanged since they were taken; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    sys.path.insert(0, ROOT)
    from collective_reduction_ring_amd.profiling import kernel_source_digest

    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(xs, reps_budget_s: float):
    """Time the oracle on the host (single-threaded NumPy) over the same workload."""
    import numpy as np  # noqa: F401

    import oracle

    times, out = [], None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        out = oracle.reduce_scatter(xs, "sum", "f32")
        times.append(time.perf_counter() - t0)
        if len(times) % 10 == 1:
            log(f"oracle pass {len(times)}: {times[-1]:.2f} s")
        if time.perf_counter() - t_start >= reps_budget_s or len(times) >= 500:
            break
    return out, statistics.median(times), len(times)


def cpu_baseline_threaded(xs, reps_budget_s: float):
    """The same oracle, with each segment's fold cut into per-thread ranges and
    run in a thread pool (NumPy releases the GIL in its ufuncs).  Every element
    is still the oracle's fold of that element, in ring order."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    threads = cpu_threads()[0]
    w = len(xs)
    s = len(xs[0]) // w
    step = -(-s // threads)
    tasks = [(k, lo, min(lo + step, (k + 1) * s)) for k in range(w) for lo in range(k * s, (k + 1) * s, step)]

    def one(t):
        k, lo, hi = t
        return oracle.fold(xs, oracle.ring_fold_order(k, w), "sum", "f32", lo, hi)

    times, out = [], None
    t_start = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            t0 = time.perf_counter()
            parts = list(ex.map(one, tasks))
            out = [np.concatenate([p for (k, _, _), p in zip(tasks, parts) if k == kk]) for kk in range(w)]
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= reps_budget_s or len(times) >= 500:
                break
    return out, statistics.median(times), len(times), threads


def cpu_threads() -> tuple:
    """(threads to use, cores in this process's affinity mask).  The threaded
    baselines use every core of the mask, capped at the CPU share the machine
    declares for this job in OMP_NUM_THREADS when that is set."""
    aff = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    used = min(aff, int(share)) if share.isdigit() and int(share) > 0 else aff
    return max(1, used), aff


def threaded_folds(ex, threads: int, xs, segs, op: str, dtype: str) -> list:
    """The oracle's fold of each segment (order, lo, hi), every segment's
    element range cut into `threads` chunks run in the pool `ex`; each element
    is still the oracle's fold of that element in the segment's order."""
    import numpy as np

    import oracle

    tasks = []
    for si, (order, lo, hi) in enumerate(segs):
        step = max(1, -(-(hi - lo) // threads))
        tasks += [(si, order, a, min(a + step, hi)) for a in range(lo, hi, step)] or [(si, order, lo, hi)]
    parts = list(ex.map(lambda t: oracle.fold(xs, t[1], op, dtype, t[2], t[3]), tasks))
    return [np.concatenate([p for t, p in zip(tasks, parts) if t[0] == si]) for si in range(len(segs))]


def ring_segments(count: int, world: int) -> list:
    import oracle
    return [(oracle.ring_fold_order(k, world), lo, hi)
            for k, (lo, hi) in enumerate(oracle.segment_bounds(count, world))]


def oracle_baseline(single, threaded, nbytes: int, budget_s: float, sample: str, same=None) -> dict:
    """Time the oracle on the host: `single()` (NumPy on one thread) in whole
    passes for about `budget_s`, then `threaded(ex, threads)` on every core of
    the job's share for about a third of that; medians.  `same(a, b)` checks
    the two results agree bit for bit."""
    from concurrent.futures import ThreadPoolExecutor

    def passes(fn, budget):
        times, out = [], None
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            out = fn()
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= budget or len(times) >= 200:
                return out, statistics.median(times), len(times)

    out1, t1, n1 = passes(single, budget_s)
    threads, aff = cpu_threads()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        out_t, t_t, n_t = passes(lambda: threaded(ex, threads), max(1.0, budget_s / 3))
    res = {"value": round(nbytes / t1 / 1e9, 3), "unit": "GB/s", "us_per_call": round(t1 * 1e6, 1),
           "cores": 1, "kind": "oracle", "sample": f"{sample}; {n1} passes, median {t1:.4f} s, "
                                                   "single-threaded NumPy",
           "cpu_model": cpu_model(),
           "threaded": {"value": round(nbytes / t_t / 1e9, 3), "unit": "GB/s",
                        "us_per_call": round(t_t * 1e6, 1), "cores": threads, "affinity_cores": aff,
                        "sample": f"the same, split over {threads} threads; {n_t} passes, "
                                  f"median {t_t:.4f} s"}}
    if same is not None:
        res["threaded"]["bit_identical_to_single"] = bool(same(out1, out_t))
    return res


def _same_arrays(a, b) -> bool:
    import numpy as np
    return len(a) == len(b) and all(np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
                                    for x, y in zip(a, b))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibrate_copy(rsx, torch) -> int:
    """Plain copy of 1 GiB (one-rank all-gather), 20 launches: counter calibration."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(20):
        rsx.all_gather([src], [dst])
    torch.cuda.synchronize()
    ok = bool(torch.equal(src, dst))
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": 20, "copy_ok": ok}), flush=True)
    return 0 if ok else 1


def time_launches(fn, reps: int, warmup: int, torch) -> list:
    """Per-call durations (ms) of `fn`, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        st[i].record()
        fn()
        en[i].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(st, en)]


def time_from_state(fn, reset, reps: int, warmup: int, torch) -> list:
    """Per-call durations (ms) of `fn`, each call started from the same state:
    `reset()` runs before every call, outside the events."""
    for _ in range(warmup):
        reset()
        fn()
    torch.cuda.synchronize()
    st = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        reset()
        st[i].record()
        fn()
        en[i].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(st, en)]


def capture(fn, torch, reset=None):
    """`fn` captured once in a HIP graph (after warm-up calls on a side stream,
    each after `reset()` when given, so that every call starts from the same
    state)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            if reset is not None:
                reset()
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def graph_us_per_call(fn, inner: int, reps: int, torch) -> float:
    """Device time per call: `inner` calls captured in one HIP graph, replayed
    `reps` times; the median replay divided by `inner`."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    ms = time_launches(g.replay, reps, 2, torch)
    return round(statistics.median(ms) * 1e3 / inner, 3)


def _stat(ms: list, nbytes: int) -> dict:
    avg = statistics.mean(ms)
    return {"avg_us": round(avg * 1e3, 2), "median_us": round(statistics.median(ms) * 1e3, 2),
            "min_us": round(min(ms) * 1e3, 2), "bytes": nbytes,
            "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
            "pct_of_peak_hbm": round(100 * nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}


def _arena(torch, dtype, world, n):
    a = torch.empty(world * n, dtype=dtype, device="cuda:0")
    return a, [a[r * n:(r + 1) * n] for r in range(world)]


def other_workload(name: str, args, rsx, wl, torch, np) -> dict:
    """Timings of the workloads other than the headline one (one JSON line each)."""
    reps, warm = args.steps, args.warmup
    if name == "small":  # W=4, 4096 fp32 per rank: latency
        xs = wl.rank_inputs(1)
        _, dev = _arena(torch, torch.float32, 4, 4096)
        for d, x in zip(dev, xs):
            d.copy_(torch.from_numpy(x))
        _, out = _arena(torch, torch.float32, 4, 1024)
        _, ar = _arena(torch, torch.float32, 4, 4096)
        rs = rsx.ReduceScatter(dev, out, "sum")
        arp = rsx.AllReduce(dev, ar, "sum", "ring")
        res = {"workload": "rs+ar sum fp32, W=4, 4096/rank",
               "reduce_scatter": _stat(time_launches(rs, reps, warm, torch), 4 * 4096 * 4 + 4 * 1024 * 4),
               "all_reduce": _stat(time_launches(arp, reps, warm, torch), 2 * 4 * 4096 * 4)}
        res["reduce_scatter"]["graph_us_per_call"] = graph_us_per_call(rs, 100, 20, torch)
        res["all_reduce"]["graph_us_per_call"] = graph_us_per_call(arp, 100, 20, torch)
        if not args.no_cpu_baseline:
            import oracle
            rs_segs = [(oracle.ring_fold_order(k, 4), k * 1024, (k + 1) * 1024) for k in range(4)]
            res["reduce_scatter"]["cpu_baseline"] = oracle_baseline(
                lambda: oracle.reduce_scatter(xs, "sum", "f32"),
                lambda ex, t: threaded_folds(ex, t, xs, rs_segs, "sum", "f32"),
                4 * 4096 * 4 + 4 * 1024 * 4, min(3.0, args.cpu_seconds), "the whole workload", _same_arrays)
            res["all_reduce"]["cpu_baseline"] = oracle_baseline(
                lambda: oracle.all_reduce(xs, "sum", "f32"),
                lambda ex, t: oracle.all_gather(threaded_folds(ex, t, xs, ring_segments(4096, 4), "sum", "f32")),
                2 * 4 * 4096 * 4, min(3.0, args.cpu_seconds), "the whole workload", _same_arrays)
        return res
    if name == "bf16_bucketed":
        w = wl.WORKLOADS[3]
        world, n, bucket = w.world, w.n, w.extra["bucket_elems"]
        log("generating bf16 inputs")
        xs = wl.rank_inputs(3)
        _, dev = _arena(torch, torch.bfloat16, world, n)
        for d, x in zip(dev, xs):
            d.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        sample = [x[:2 * bucket].copy() for x in xs]      # the first two buckets, for the oracle
        del xs
        _, out = _arena(torch, torch.bfloat16, world, n)
        nbuckets = rsx.bucket_count(n, bucket)

        def bucketed(algo):
            return rsx.AllReduceBucketed(dev, out, bucket, "avg", algo)
        nb = 2 * world * n * 2
        step = bucketed("ring")
        res = {"workload": "all-reduce avg bf16 (fp32 accumulate), W=8, 134,217,728/rank, "
                           f"{nbuckets} buckets of <= 25 MiB in sequence on one stream; "
                           "ring = RSX_ALGO_RING (two passes at this shape; the full buckets share "
                           "one launch per pass)",
               "ring": _stat(time_launches(step, reps // 4 or 1, warm, torch), nb)}
        res["ring"]["graph_us_per_step"] = graph_us_per_call(step, 1, 10, torch)
        # The two-pass form (reduce-scatter, then all-gather); the same bits.
        st = _stat(time_launches(bucketed("ring_split"), reps // 4 or 1, warm, torch), nb)
        # reduce-scatter W*n*2 in, n*2 out; all-gather n*2 in, (W-1)*n*2 out
        st["actual_bytes"] = nb + n * 2
        res["ring_split_two_pass"] = st
        # For comparison only: the same bytes as one all-reduce without buckets.
        whole = rsx.AllReduce(dev, out, "avg", "ring")
        res["unbucketed_one_call"] = _stat(time_launches(whole, reps // 4 or 1, warm, torch), nb)
        if not args.no_cpu_baseline:
            import oracle

            def threaded(ex, t):
                outs = [np.empty_like(x) for x in sample]
                for b0 in (0, bucket):
                    part = [x[b0:b0 + bucket] for x in sample]
                    for r, o in enumerate(oracle.all_gather(
                            threaded_folds(ex, t, part, ring_segments(bucket, world), "avg", "bf16"))):
                        outs[r][b0:b0 + bucket] = o
                return outs
            del dev, out, whole, step
            torch.cuda.empty_cache()
            log("oracle baseline: two buckets")
            res["ring"]["cpu_baseline"] = oracle_baseline(
                lambda: oracle.bucketed_all_reduce(sample, bucket, "avg", "bf16"), threaded,
                2 * world * 2 * bucket * 2, args.cpu_seconds,
                f"the first 2 of the {nbuckets} buckets (2 x {bucket} bf16 per rank, W={world}), "
                "bytes scaled to that sample", _same_arrays)
        return res
    if name == "int32_w16":
        w = wl.WORKLOADS[4]
        world, n = w.world, w.n
        seg = n // world
        xs = wl.rank_inputs(4)
        _, dev = _arena(torch, torch.int32, world, n)
        for d, x in zip(dev, xs):
            d.copy_(torch.from_numpy(x))
        _, out = _arena(torch, torch.int32, world, seg)
        _, ar = _arena(torch, torch.int32, world, n)
        res = {"workload": "int32 W=16, 33,554,432/rank"}
        for op in ("sum", "max"):
            res[f"reduce_scatter_{op}"] = _stat(time_launches(rsx.ReduceScatter(dev, out, op), reps, warm, torch),
                                                world * n * 4 + world * seg * 4)
            res[f"all_reduce_{op}"] = _stat(time_launches(rsx.AllReduce(dev, ar, op, "ring"), reps, warm, torch),
                                            2 * world * n * 4)
        res["all_reduce_sum_two_pass"] = _stat(time_launches(rsx.AllReduce(dev, ar, "sum", "ring_split"), reps,
                                                             warm, torch), 2 * world * n * 4)
        if not args.no_cpu_baseline:
            import oracle
            rs_segs = [(oracle.ring_fold_order(k, world), k * seg, (k + 1) * seg) for k in range(world)]
            for op in ("sum", "max"):
                log(f"oracle baseline: int32 W=16 {op}")
                res[f"reduce_scatter_{op}"]["cpu_baseline"] = oracle_baseline(
                    lambda: oracle.reduce_scatter(xs, op, "i32"),
                    lambda ex, t: threaded_folds(ex, t, xs, rs_segs, op, "i32"),
                    world * n * 4 + world * seg * 4, args.cpu_seconds / 2, "the whole workload", _same_arrays)
                res[f"all_reduce_{op}"]["cpu_baseline"] = oracle_baseline(
                    lambda: oracle.all_reduce(xs, op, "i32"),
                    lambda ex, t: oracle.all_gather(threaded_folds(ex, t, xs, ring_segments(n, world), op, "i32")),
                    2 * world * n * 4, args.cpu_seconds / 2, "the whole workload", _same_arrays)
        return res
    if name == "fused":
        world = 4
        sizes = wl.fused_sizes()
        per_rank = wl.fused_tensors(world, sizes)
        tens = [[torch.from_numpy(t).to("cuda:0") for t in ts] for ts in per_rank]
        total = int(sizes.sum())
        stride = (total + 63) // 64 * 64        # 256-byte aligned fusion buffers
        fz = torch.empty(world * stride, dtype=torch.float32, device="cuda:0")
        fused = [fz[r * stride:r * stride + total] for r in range(world)]
        plan = rsx.FusedAllReduce(tens, fused, None, "sum", "ring")
        pack = lambda: [p() for p in plan.packs]  # noqa: E731
        arp = plan.reduce
        unpack = lambda: [u() for u in plan.unpacks]  # noqa: E731
        e2e = plan
        nb = world * total * 4
        direct = rsx.TensorFusionAllReduce(tens, None, "sum", "ring")
        grouped = rsx.GroupedAllReduce(tens, None, "sum", "ring", 64 * 2 ** 20)
        res = {"workload": f"fused: W=4, {len(sizes)} fp32 tensors, {total} elements/rank",
                "direct_tensor_fusion_all_reduce": _stat(time_launches(direct, reps, warm, torch), 2 * nb),
                "grouped_64MiB_threshold": dict(
                    _stat(time_launches(grouped, reps, warm, torch), 2 * nb), groups=len(grouped.groups)),
                "pack": _stat(time_launches(pack, reps, warm, torch), 2 * nb),
                "all_reduce": _stat(time_launches(arp, reps, warm, torch), 2 * nb),
                "unpack": _stat(time_launches(unpack, reps, warm, torch), 2 * nb),
                "end_to_end": _stat(time_launches(e2e, reps, warm, torch), 6 * nb)}
        if not args.no_cpu_baseline:
            import oracle
            counts = [int(c) for c in sizes]

            def threaded(ex, t):
                fused_h = list(ex.map(oracle.fuse_pack, per_rank))
                red = oracle.all_gather(threaded_folds(ex, t, fused_h, ring_segments(total, world), "sum", "f32"))
                return list(ex.map(lambda f: oracle.fuse_unpack(f, counts), red))
            log("oracle baseline: pack, all-reduce, unpack")
            res["end_to_end"]["cpu_baseline"] = oracle_baseline(
                lambda: oracle.fused_all_reduce(per_rank, "sum", "f32"), threaded, 6 * nb, args.cpu_seconds,
                "the whole workload: pack, all-reduce and unpack of every rank",
                lambda a, b: all(_same_arrays(x, y) for x, y in zip(a, b)))
        return res
    if name == "all_gather":
        # W = 8 pieces of 8,388,608 fp32 (32 MiB) gathered into 8 outputs of 256 MiB
        world, n = 8, 8388608
        gen = np.random.default_rng((8, 0))
        pieces_h = [gen.standard_normal(n, dtype=np.float32) for _ in range(world)]
        _, pieces = _arena(torch, torch.float32, world, n)
        for d, x in zip(pieces, pieces_h):
            d.copy_(torch.from_numpy(x))
        _, out = _arena(torch, torch.float32, world, world * n)
        in_place_src = [out[k][k * n:(k + 1) * n] for k in range(world)]
        res = {"workload": "all-gather fp32, W=8, pieces of 8,388,608 (32 MiB) into outputs of 256 MiB",
               "out_of_place": _stat(time_launches(lambda: rsx.all_gather(pieces, out), reps, warm, torch),
                                     world * n * 4 + world * world * n * 4),
               "in_place": _stat(time_launches(lambda: rsx.all_gather(in_place_src, out), reps, warm, torch),
                                 world * n * 4 + world * (world - 1) * n * 4)}
        got = out[world - 1].cpu().numpy()
        res["check_last_rank_equals_concatenation"] = bool(np.array_equal(got, np.concatenate(pieces_h)))
        if not args.no_cpu_baseline:
            import oracle

            def threaded(ex, t):
                return list(ex.map(lambda r: np.concatenate(pieces_h), range(world)))
            res["out_of_place"]["cpu_baseline"] = oracle_baseline(
                lambda: oracle.all_gather(pieces_h), threaded, world * n * 4 + world * world * n * 4,
                args.cpu_seconds / 2, "the whole workload (the oracle concatenates the pieces once per rank)",
                _same_arrays)
        return res
    if name == "sweep":
        res = {"workload": "all-reduce sum fp32, W=4, 1-32 KiB per rank: naive vs ring"}
        for kib in wl.SWEEP_KIB:
            xs = wl.sweep_inputs(kib)
            n = len(xs[0])
            _, dev = _arena(torch, torch.float32, 4, n)
            for d, x in zip(dev, xs):
                d.copy_(torch.from_numpy(x))
            _, out = _arena(torch, torch.float32, 4, n)
            row = {}
            for algo in ("naive", "ring"):
                p = rsx.AllReduce(dev, out, "sum", algo)
                row[algo] = _stat(time_launches(p, 200, 20, torch), 2 * 4 * n * 4)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(1000):
                    p()
                torch.cuda.synchronize()
                row[algo]["wall_us_per_call"] = round((time.perf_counter() - t0) * 1e3, 2)
                row[algo]["graph_us_per_call"] = graph_us_per_call(p, 100, 20, torch)
                if not args.no_cpu_baseline:
                    import oracle
                    segs = ring_segments(n, 4) if algo == "ring" else [(list(range(4)), 0, n)]
                    whole = oracle.all_reduce if algo == "ring" else oracle.naive_all_reduce
                    row[algo]["cpu_baseline"] = oracle_baseline(
                        lambda: whole(xs, "sum", "f32"),
                        lambda ex, t: oracle.all_gather(threaded_folds(ex, t, xs, segs, "sum", "f32"))
                        if algo == "ring" else [threaded_folds(ex, t, xs, segs, "sum", "f32")[0]] * 4,
                        2 * 4 * n * 4, 0.5, "the whole call", _same_arrays)
            res[f"{kib}KiB"] = row
        return res
    if name == "sparse":
        world, n = wl.SPARSE_WORLD, wl.SPARSE_N
        log("generating sparse inputs")
        grads, accs = wl.sparse_inputs()
        _, g = _arena(torch, torch.float32, world, n)
        a0_all, a0 = _arena(torch, torch.float32, world, n)
        for d, x in zip(g, grads):
            d.copy_(torch.from_numpy(x))
        for d, x in zip(a0, accs):
            d.copy_(torch.from_numpy(x))
        a_all, a = _arena(torch, torch.float32, world, n)
        _, out = _arena(torch, torch.float32, world, n)
        res = {"workload": f"sparsified all-reduce with error feedback, W={world}, {n} fp32/rank, "
                           "N(0,1e-3) gradients and residuals",
               "algorithmic_bytes": "W*n*16 (read grad and accum, write accum and output) "
                                    "+ 16 per message entry (written once, read once)"}
        modes = (("topk", {"fraction": wl.SPARSE_TOPK_FRACTION}),
                 ("threshold", {"threshold": wl.SPARSE_THRESHOLD}))

        def reset():   # every call starts from the same residual, as one training step would
            a_all.copy_(a0_all)
        for mode, kw in modes:
            plan = rsx.SparseAllReduce(g, a, out, mode, **kw)
            ms = time_from_state(plan, reset, reps, warm, torch)
            nnz = plan.nnz_host()
            st = _stat(ms, world * n * 16 + 16 * sum(nnz))
            st.update(k=plan.k, nnz_rank0=nnz[0], nnz_total=sum(nnz), params=kw)
            # the whole call captured in one HIP graph (its ~15 launches replayed at once)
            graph = capture(plan, torch, reset)
            ms_g = time_from_state(graph.replay, reset, reps, warm, torch)
            st["graph_replay_median_us"] = round(statistics.median(ms_g) * 1e3, 2)
            res[mode] = st
        if not args.no_cpu_baseline:
            import oracle
            k = oracle.topk_count(n, wl.SPARSE_TOPK_FRACTION)
            for mode in ("threshold", "topk"):
                fn, arg = ((oracle.sparsify_threshold, wl.SPARSE_THRESHOLD) if mode == "threshold"
                           else (oracle.sparsify_topk, k))
                nnz = res[mode]["nnz_total"]

                def threaded(ex, t, fn=fn, arg=arg):
                    per = list(ex.map(lambda r: fn(grads[r], accs[r], arg), range(world)))
                    return [oracle.sparse_combine([(i, v) for i, v, _ in per], n)]
                if mode == "threshold":
                    single = lambda: oracle.sparse_all_reduce(grads, accs, "threshold",  # noqa: E731
                                                              wl.SPARSE_THRESHOLD)[0][:1]
                    sample, nbytes, budget = "the whole workload", world * n * 16 + 16 * nnz, args.cpu_seconds
                else:
                    # one rank's selection (a stable sort of 64 Mi values takes ~15 s) and the
                    # combine of its message; the threaded leg runs all 8 ranks, one per thread
                    single = lambda: [oracle.sparse_combine(  # noqa: E731
                        [oracle.sparsify_topk(grads[0], accs[0], k)[:2]], n)]
                    sample, nbytes, budget = ("rank 0 only (its sort, residual and combine); bytes "
                                              "scaled to one rank", n * 16 + 16 * k, 1.0)
                log(f"oracle baseline: sparse {mode}")
                cb = oracle_baseline(single, threaded, nbytes, budget, sample)
                if mode == "topk":   # the threaded leg did all W ranks: its bytes are W times one rank's
                    cb["threaded"]["value"] = round(cb["threaded"]["value"] * world, 3)
                    cb["threaded"]["sample"] = ("all 8 ranks, one per thread, then the combine; "
                                                + cb["threaded"]["sample"].split("; ", 1)[1])
                res[mode]["cpu_baseline"] = cb
        return res
    if name == "sparse_sweep":
        # The sparsified all-reduce across selection sizes and rank counts, at
        # the same total bytes as the sparse workload (W * n = 8 * 64 Mi):
        # N(0, 1e-3) gradients and residuals drawn on the GPU with
        # torch.Generator(8).
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(8)
        points = [(8, "topk", {"fraction": f}) for f in (0.001, 0.01, 0.05, 0.1)]
        points += [(8, "threshold", {"threshold": t}) for t in (3.6e-3, 2.6e-3)]
        points += [(w, "topk", {"fraction": 0.01}) for w in (2, 16)]
        points += [(w, "threshold", {"threshold": 3.6e-3}) for w in (2, 16)]
        rows = []
        for world in (2, 8, 16):
            n = 8 * (64 << 20) // world
            g_all, g = _arena(torch, torch.float32, world, n)
            a0_all, _ = _arena(torch, torch.float32, world, n)
            g_all.normal_(0.0, 1e-3, generator=gen)
            a0_all.normal_(0.0, 1e-3, generator=gen)
            a_all, a = _arena(torch, torch.float32, world, n)
            _, out = _arena(torch, torch.float32, world, n)

            def reset():
                a_all.copy_(a0_all)
            for w, mode, kw in points:
                if w != world:
                    continue
                log(f"sparse sweep: W={world} n={n} {mode} {kw}")
                plan = rsx.SparseAllReduce(g, a, out, mode, **kw)
                ms = time_from_state(plan, reset, reps, warm, torch)
                nnz = plan.nnz_host()
                st = _stat(ms, world * n * 16 + 16 * sum(nnz))
                st.update(world=world, n=n, mode=mode, params=kw, k=plan.k, sent_fraction=sum(nnz) / (world * n))
                rows.append(st)
                del plan
            del g_all, g, a0_all, a_all, a, out
            torch.cuda.empty_cache()
        return {"workload": "sparsified all-reduce with error feedback, W * n = 8 * 64 Mi fp32, "
                            "N(0,1e-3) gradients and residuals",
                "algorithmic_bytes": "W*n*16 + 16 per message entry", "points": rows}
    if name == "overlap":
        # bucketed all-reduce beside a stand-in backward pass: per bucket, one
        # fp32 matmul on the main stream, then that bucket's all-reduce
        w = wl.WORKLOADS[3]
        world, n, bucket = w.world, w.n, w.extra["bucket_elems"]
        log("generating bf16 inputs")
        xs = wl.rank_inputs(3)
        _, dev = _arena(torch, torch.bfloat16, world, n)
        for d, x in zip(dev, xs):
            d.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        del xs
        _, out = _arena(torch, torch.bfloat16, world, n)
        plan = rsx.BucketedAllReduce(dev, out, bucket, "avg")
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(3)
        m = 1536
        a = torch.randn(m, m, device="cuda:0", generator=gen)
        c = torch.empty(m, m, device="cuda:0")

        def compute(b):
            torch.mm(a, a, out=c)

        def serial():
            for b in range(len(plan)):
                compute(b)
                plan.plans[b]()

        def overlapped():
            for b in range(len(plan)):
                compute(b)
                plan.ready(b)
            plan.wait()

        def compute_only():
            for b in range(len(plan)):
                compute(b)
        nb = 2 * world * n * 2
        res = {"workload": f"bucketed all-reduce avg bf16, W=8, 134,217,728/rank, {len(plan)} buckets; "
                           f"per bucket one {m}x{m}x{m} fp32 matmul on the main stream first; "
                           "side-stream reductions without the occupancy caps unless named",
               "compute_only": _stat(time_launches(compute_only, reps // 4 or 1, warm, torch), 0),
               "all_reduce_only": _stat(time_launches(plan, reps // 4 or 1, warm, torch), nb),
               "serial_one_stream": _stat(time_launches(serial, reps // 4 or 1, warm, torch), nb),
               "overlapped_side_stream": _stat(time_launches(overlapped, reps // 4 or 1, warm, torch), nb)}
        # the same with the library's occupancy caps left on for the side-stream launches
        plan.occupancy_caps = True
        res["overlapped_side_stream_caps_on"] = _stat(time_launches(overlapped, reps // 4 or 1, warm, torch), nb)
        plan.occupancy_caps = False
        for k in ("compute_only",):
            for f in ("GBps", "pct_of_peak_hbm", "bytes"):
                res[k].pop(f)
        return res
    if name == "size_sweep":
        # reduce-scatter and ring all-reduce, W = 8 fp32, 4 KiB .. 1 GiB per rank
        world = 8
        top = 2 ** 30 // 4
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(11)
        ins_all = torch.randn(world * top, device="cuda:0", generator=gen) * 1e-3
        outs_all = torch.empty(world * top, device="cuda:0")
        res = {"workload": "reduce-scatter and ring all-reduce sum fp32 (one pass, and two passes for "
                           "comparison; and an in-place avg all-reduce), all-gather of the W blocks, W=8, "
                           "per-rank size sweep; "
                           "below 64 MiB graph-timed device time (50 calls per graph), above HIP events per call"}
        kib = 4
        while kib * 1024 <= 2 ** 30:
            n = kib * 1024 // 4
            ins = [ins_all[r * n:(r + 1) * n] for r in range(world)]
            seg = n // world
            rs_out = [outs_all[k * seg:(k + 1) * seg] for k in range(world)]
            ar_out = [outs_all[r * n:(r + 1) * n] for r in range(world)]
            rs = rsx.ReduceScatter(ins, rs_out, "sum")
            ar = rsx.AllReduce(ins, ar_out, "sum", "ring")
            # in place (8 buffers instead of 16); avg keeps repeated calls' values bounded
            ar_in = rsx.AllReduce(ins, None, "avg", "ring")
            # the two-pass form (reduce-scatter, then all-gather), for comparison
            ar_two = rsx.AllReduce(ins, ar_out, "sum", "ring_split")
            # all-gather of W blocks of n/W elements (taken from the input arena) into the
            # W full-size outputs, out of place
            ag_in = [ins_all[k * seg:(k + 1) * seg] for k in range(world)]
            ag = lambda: rsx.all_gather(ag_in, ar_out)  # noqa: E731
            row = {}
            for what, fn, nbytes in (("reduce_scatter", rs, world * n * 4 + world * seg * 4),
                                     ("all_reduce", ar, 2 * world * n * 4),
                                     ("all_reduce_two_pass", ar_two, 2 * world * n * 4),
                                     ("all_gather", ag, n * 4 + world * n * 4),
                                     ("all_reduce_in_place_avg", ar_in, 2 * world * n * 4)):
                if kib * 1024 < 64 * 2 ** 20:
                    us = graph_us_per_call(fn, 50, 20, torch)
                else:
                    us = statistics.median(time_launches(fn, max(5, reps // 4), warm, torch)) * 1e3
                row[what] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
            res[f"{kib}KiB"] = row
            kib *= 4
        return res
    if name == "dtypes":
        world, rank_bytes = 8, 256 * 2 ** 20
        arena_in = torch.empty(world * rank_bytes, dtype=torch.uint8, device="cuda:0")
        arena_out = torch.empty(rank_bytes, dtype=torch.uint8, device="cuda:0")
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(7)
        res = {"workload": "reduce-scatter sum, W=8, 256 MiB per rank, every element type "
                           "(inputs: seeded N(0,1) for floats, uniform bits for integers)"}
        cases = (("f32", torch.float32, None), ("bf16", torch.bfloat16, None), ("f16", torch.float16, None),
                 ("f64", torch.float64, None), ("i32", torch.int32, None), ("i64", torch.int64, None),
                 ("u64", torch.uint64, None), ("i8", torch.int8, None), ("f32_half_wire", torch.float32, "f16"))
        for name_, dt, wire in cases:
            flat = arena_in.view(dt)
            if dt.is_floating_point:
                flat.copy_(torch.randn(flat.numel(), generator=gen, device="cuda:0").to(dt))
            else:
                arena_in.copy_(torch.randint(0, 256, (arena_in.numel(),), generator=gen, device="cuda:0",
                                             dtype=torch.int32).to(torch.uint8))
            n = flat.numel() // world
            ins = [flat[r * n:(r + 1) * n] for r in range(world)]
            seg = n // world
            outs = [arena_out.view(dt)[k * seg:(k + 1) * seg] for k in range(world)]
            p = rsx.ReduceScatter(ins, outs, "sum", wire)
            es = flat.element_size()
            res[name_] = _stat(time_launches(p, reps, warm, torch), world * n * es + world * seg * es)
        return res
    raise SystemExit(f"unknown workload {name}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget of the oracle baseline (whole passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=("arena", "separate"), default="arena")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--workload", default="rs_w8_f32",
                    choices=("rs_w8_f32", "small", "bf16_bucketed", "int32_w16", "fused", "sweep", "all_gather",
                             "sparse", "sparse_sweep", "dtypes", "overlap", "size_sweep", "ceilings"),
                    help="rs_w8_f32 (default) is the headline line; the others print timings only")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py measures one GPU only: the W ranks are buffers of a single MI355X; "
            f"--gpus {args.gpus} is not supported")
        return 2

    if args.workload == "ceilings":
        # A child process of its own, started before this one touches the GPU.
        import subprocess
        tool = os.path.join(ROOT, "collective_reduction_ring_amd", "tools", "hbm_ceiling")
        if not os.path.exists(tool):
            log(f"{tool} is not built; run `python -m collective_reduction_ring_amd.build`")
            return 2
        return subprocess.run([tool]).returncode

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import collective_reduction_ring_amd as rsx
    from collective_reduction_ring_amd import workloads as wl

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 2

    if args.calibrate_copy:
        return calibrate_copy(rsx, torch)
    if args.workload != "rs_w8_f32":
        print(json.dumps(other_workload(args.workload, args, rsx, wl, torch, np)), flush=True)
        return 0

    w = wl.WORKLOADS[2]
    world, n = w.world, w.n
    seg = n // world
    bytes_per_step = world * n * 4 + world * seg * 4

    log(f"generating inputs: W={world}, {n} fp32 per rank, layout {args.layout}")
    xs = wl.rank_inputs(2)
    if args.layout == "arena":
        arena_in = torch.empty(world * n, dtype=torch.float32, device="cuda:0")
        arena_out = torch.empty(world * seg, dtype=torch.float32, device="cuda:0")
        dev = [arena_in[r * n:(r + 1) * n] for r in range(world)]
        out = [arena_out[r * seg:(r + 1) * seg] for r in range(world)]
        for d, x in zip(dev, xs):
            d.copy_(torch.from_numpy(x))
    else:
        dev = [torch.from_numpy(x).to("cuda:0") for x in xs]
        out = [torch.empty(seg, dtype=torch.float32, device="cuda:0") for _ in range(world)]
    plan = rsx.ReduceScatter(dev, out, "sum")
    stream = torch.cuda.current_stream()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        plan()
    torch.cuda.synchronize()

    k = args.steps
    # Timed region: K launches back to back on the launch stream, bracketed by
    # one pair of HIP events (device time) and the host clock (wall time).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {k} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(k):
        plan()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    avg_launch_s = ev0.elapsed_time(ev1) / 1e3 / k
    value = bytes_per_step * k / elapsed / 1e9
    achieved = bytes_per_step / avg_launch_s / 1e9
    # Spread of single launches (each between its own pair of events), after the timed region.
    launch_ms = time_launches(plan, 20, 0, torch)
    log(f"wall {elapsed * 1e6 / k:.1f} us/step ({value:.0f} GB/s); kernel avg {avg_launch_s * 1e6:.1f} us "
        f"({achieved:.0f} GB/s); single launches median {statistics.median(launch_ms) * 1e3:.1f} us, "
        f"min {min(launch_ms) * 1e3:.1f} us")

    got = [o.cpu().numpy() for o in out]
    del dev, out

    result = {
        "metric": "reduce-scatter effective HBM GB/s and % of peak, W=8, 64Mi fp32/rank",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": k,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / k, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: N(0, 1e-3) fp32, numpy default_rng((2, rank)) per rank",
        "config": {
            "workload": "reduce_scatter sum fp32, W=8 virtual ranks, 67,108,864 elements/rank, "
                        "ring order",
            "world": world,
            "elements_per_rank": n,
            "recvcount": seg,
            "bytes_per_step": bytes_per_step,
            "parallelism": "one GPU; W ranks = W HBM buffers",
            "layout": ("W rank buffers consecutive in one allocation" if args.layout == "arena"
                       else "each rank buffer a separate PyTorch allocation"),
        },
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(),
            "kernel": "rsx::fold_kernel<F32T, RSX_SUM, 8, reduce-scatter, dwordx4, 1 tile per workgroup>",
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "single_launch_median_us": round(statistics.median(launch_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": bytes_per_step,
        },
    }

    if not args.no_cpu_baseline:
        log(f"oracle baseline on the host, ~{args.cpu_seconds:.0f} s")
        want, t_med, reps = cpu_baseline(xs, args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": round(bytes_per_step / t_med / 1e9, 3),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"the whole workload (one reduce-scatter of 8 x 67,108,864 fp32), "
                      f"{reps} passes, median {t_med:.2f} s; single-threaded NumPy",
            "cpu_model": cpu_model(),
        }
        log("oracle baseline on the host, threaded")
        want_t, t_thr, reps_t, threads = cpu_baseline_threaded(xs, max(2.0, args.cpu_seconds / 3))
        same_t = all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(want_t, want))
        result["cpu_baseline"]["threaded"] = {
            "value": round(bytes_per_step / t_thr / 1e9, 3), "unit": "GB/s", "cores": threads,
            "affinity_cores": cpu_threads()[1],
            "sample": f"the same workload, each segment's fold split over {threads} threads, "
                      f"{reps_t} passes, median {t_thr:.3f} s; bit-identical to the single-threaded "
                      f"oracle: {same_t}"}
        bad = sum(int(np.count_nonzero(g.view(np.uint32) != o.view(np.uint32)))
                  for g, o in zip(got, want))
        result["parity"] = {"checked_elements": int(sum(g.size for g in got)),
                            "mismatches": bad, "rule": "bit-exact fp32"}
        if bad:
            log(f"PARITY FAILURE: {bad} elements differ from the oracle")
    print(json.dumps(result), flush=True)
    return 1 if result.get("parity", {}).get("mismatches") else 0


if __name__ == "__main__":
    sys.exit(main())
