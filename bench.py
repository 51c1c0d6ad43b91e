"""Benchmark: GEMM TFLOP/s and fraction of the MI355X MFMA (or HBM) roofline
for each schedule (data-parallel, persistent, Stream-K, hybrid) on one GPU.

A step is one C = A.B of the workload through the C ABI (every MAC, every
Stream-K fixup, every store).  Each schedule is timed over --steps steps
after --warmup untimed ones; before every step a 512 MiB fill evicts L2 and
the Infinity Cache (outside the timed window), and HIP events on the launch
stream bracket the GEMM alone.

The line's value is the best schedule's TFLOP/s on the 4096^3 fp16 product;
"configs" holds the same measurement for every other workload (fp32 256^3,
fp16 1536x1536x8192, bf16 512x512x65536, bf16 8192x28672x8192 and, unless
--quick, the 16 seeded irregular bf16 shapes), each with an oracle check of
what was timed: every element against the full CPU oracle where it finishes
in seconds, seeded samples plus ragged edges otherwise.  The run exits
non-zero if any check fails.  "cpu_baseline" is the full oracle on the
4096^3 product, timed on the host's cores in the same run.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3, "i8": 5033.2}  # dense MFMA, 2.4 GHz
PEAK_HBM_GBS = 8000.0
SCHEDULES = ("dp", "persistent", "streamk", "hybrid")
METRIC = "GEMM TFLOP/s and % of MFMA peak per schedule (DP / persistent / Stream-K)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    from persistent_stream_tiling_amd.profiling import source_hash
    return source_hash()


def workload_table():
    from persistent_stream_tiling_amd import inputs
    return dict(inputs.WORKLOADS, **inputs.EXTRA_WORKLOADS, **inputs.irregular_workloads())


def to_device(bits, dtype):
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    elif dtype == "i8":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int8))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to("cuda")


def algorithmic_bytes(M, N, K, dtype, plan_info):
    """A and B read once, C written once (fp32, or the input dtype when the
    plan stores C in it); the callers add the Stream-K partials written and
    read once."""
    from persistent_stream_tiling_amd import FLAG_C_INPUT_DTYPE
    e = {"f32": 4, "i8": 1}.get(dtype, 2)
    ce = e if plan_info["flags"] & FLAG_C_INPUT_DTYPE else 4
    return (M * K + K * N) * e + M * N * ce


def partial_bytes(plan):
    """Bytes of Stream-K partial tiles written (and read back) by one run: every
    piece that does not start at k = 0, plus, with the split fixup, the head
    pieces of split tiles (which are parked too)."""
    info = plan.info
    parked = (1, 2) if info["split_fixup"] else (1,)
    n = 0
    for w in range(info["launch_grid"] if info["tiles_sk"] else 0):
        for (_, _, _, role, _) in plan.segments(w):
            if role in parked:
                n += 1
    return n * info["bm"] * info["bn"] * 4


def time_schedule(plan, a, b, c, ws, steps, warmup, flush):
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        plan.run(a, b, c, ws, check=False)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush.zero_()
        starts[i].record(stream)
        plan.run(a, b, c, ws, check=False)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return ms, wall


def oracle_threads():
    """Threads for the CPU oracle: the host's cores, capped by the CPU share
    this process was given (its affinity mask and OMP_NUM_THREADS)."""
    n = os.cpu_count() or 1
    try:
        n = min(n, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# Products up to this many multiply-adds are checked element by element
# against the full oracle (seconds of CPU time); larger ones on samples.
FULL_ORACLE_MACS = 4096 ** 3
TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3, "i8": 0.0}


def oracle_reference(name, wl, a_bits, b_bits, threads):
    """Oracle values to check the workload's GPU output against, and the
    oracle's own timing.  Full products up to FULL_ORACLE_MACS: every
    element.  Larger ones: 8192 seeded samples (timed, with the extrapolated
    full-product time) plus, except on the 8192x28672x8192 shape, every
    element of the last two rows and columns."""
    import oracle
    from persistent_stream_tiling_amd import inputs
    M, N, K, dt = wl["M"], wl["N"], wl["K"], wl["dtype"]
    checks = []
    if M * N * K <= FULL_ORACLE_MACS:
        t = time.perf_counter()
        ref, scale = oracle.gemm(a_bits, b_bits, dt, nthreads=threads)
        secs = time.perf_counter() - t
        checks.append(("all", None, ref, scale))
        timing = {"kind": "full", "elements": M * N, "seconds": round(secs, 3),
                  "gflops": round(2.0 * M * N * K / secs / 1e9, 2), "threads": threads}
    else:
        rows, cols = inputs.sample_positions(M, N, 8192, seed=wl["seed"] + 1000)
        t = time.perf_counter()
        ref, scale = oracle.gemm_sampled(a_bits, b_bits, dt, rows, cols, threads)
        secs = time.perf_counter() - t
        checks.append(("samples", (rows, cols), ref, scale))
        timing = {"kind": "sampled", "elements": int(rows.size), "seconds": round(secs, 3),
                  "gflops": round(2.0 * rows.size * K / secs / 1e9, 2), "threads": threads,
                  "extrapolated_full_seconds": round(secs * M * N / rows.size, 1)}
        if name != "bf16_8192x28672x8192":
            ref, scale = oracle.gemm(np.ascontiguousarray(a_bits[M - 2:]), b_bits, dt,
                                     nthreads=threads)
            checks.append(("last rows", (slice(M - 2, M), slice(None)), ref, scale))
            ref, scale = oracle.gemm(a_bits, np.ascontiguousarray(b_bits[:, N - 2:]), dt,
                                     nthreads=threads)
            checks.append(("last cols", (slice(None), slice(N - 2, N)), ref, scale))
    return checks, timing


def check_output(c, checks, dt):
    """max |C - C_ref| / S over every checked element, the element count, and
    whether all are within the workload's tolerance (bit-exact for int8)."""
    import torch
    worst, count, ok = 0.0, 0, True
    for _, idx, ref, scale in checks:
        if idx is None:
            got = c.cpu().numpy()
        elif isinstance(idx[0], np.ndarray):
            got = c[torch.from_numpy(idx[0]).cuda(), torch.from_numpy(idx[1]).cuda()].cpu().numpy()
        else:
            got = c[idx].cpu().numpy()
        got = got.astype(np.float64)
        err = np.abs(got - ref)
        count += int(ref.size)
        if dt == "i8":
            ok &= bool((err == 0).all())
        else:
            rel = err / np.maximum(scale, 1e-300)
            worst = max(worst, float(rel.max()) if rel.size else 0.0)
            ok &= bool((err <= TOL[dt] * scale).all())
    return worst, count, ok


TABLE_ROUNDS = 4


def schedule_table(args, out):
    """Median time of every schedule (tuned tiles, default grid) per workload.
    Each workload runs in a child process of its own (a workload's timing was
    seen to depend on what ran before it in the same process), its schedules
    interleaved round by round so that clock drift hits all alike."""
    import subprocess
    from persistent_stream_tiling_amd import inputs
    names = sorted(inputs.irregular_workloads()) if args.workload == "irregular" \
        else args.workload.split(",")
    per = max(1, args.steps // TABLE_ROUNDS)
    lines = [f"# Schedules per workload: `python bench.py --workload {args.workload} "
             f"--steps {args.steps} --table <file>`", "",
             f"Kernel source hash: {kernel_source_hash()}.  Median of {TABLE_ROUNDS * per} timed "
             "runs per schedule (rounds interleaved, 512 MiB cache flush before each run), each "
             "schedule in its tuned launch configuration (tuning.py: tile, order, copy hint, "
             "Stream-K partition; grid one workgroup per CU, or the library's default plan where "
             "the entry is empty); one process per workload.  'splits tiles' names the Stream-K "
             "partition: the pages' even split of all iterations over the workgroups, or each tile "
             "cut into its own pieces (GEMM_FLAG_TILE_SPLIT).", "",
             "| workload | M x N x K | tiles T | dp us | persistent us | Stream-K us | hybrid us "
             "| best | best TFLOP/s | Stream-K / DP | hybrid / DP | Stream-K splits tiles | "
             "hybrid T_sk (splits) |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in names:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--workload", name,
                            "--steps", str(args.steps), "--table-row"],
                           stdout=subprocess.PIPE, check=True, text=True)
        lines.append(r.stdout.strip().splitlines()[-1])
    text = "\n".join(lines) + "\n"
    open(out, "w").write(text)
    log(text)


def schedule_table_row(args):
    """One row of the schedule table, for one workload, on stdout."""
    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import inputs, tuning
    table = workload_table()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    rounds, per = TABLE_ROUNDS, max(1, args.steps // TABLE_ROUNDS)
    for name in [args.workload]:
        wl = table[name]
        M, N, K, dt = wl["M"], wl["N"], wl["K"], wl["dtype"]
        log(f"[table] {name}: {M}x{N}x{K} {dt}")
        a_bits, b_bits = inputs.operands(M, N, K, dt, wl["dist"], wl["seed"], wl["scale"])
        a, b = to_device(a_bits, dt), to_device(b_bits, dt)
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        runs = {}
        for sched in SCHEDULES:
            plan = gsk.GemmPlan(M, N, K, dt, sched, **tuning.bench_tiles(name, sched, dt))
            ws = plan.new_workspace()
            plan.run(a, b, c, ws)
            runs[sched] = (plan, ws, [])
        torch.cuda.synchronize()
        for _ in range(rounds):
            for sched, (plan, ws, times) in runs.items():
                ms, _ = time_schedule(plan, a, b, c, ws, per, 1, flush)
                times.extend(ms.tolist())
        med = {s: float(np.median(v[2])) * 1e3 for s, v in runs.items()}
        best = min(med, key=med.get)
        T = runs["dp"][0].info["tiles"]
        sk, hy = runs["streamk"][0].info, runs["hybrid"][0].info
        def how(i):  # Stream-K partition: the even split, or each tile in its own pieces
            return f"per-tile x{i['pieces_per_tile']}" if i["pieces_per_tile"] else "even split"
        sk_split = f"yes, {how(sk)}" if sk["max_pieces"] >= 2 else "no"
        hy_split = (f"{hy['tiles_sk']} (yes, {how(hy)})" if hy["tiles_sk"] and hy["max_pieces"] >= 2
                    else f"{hy['tiles_sk']} (no)")
        print(f"| {name} | {M} x {N} x {K} | {T} | " +
              " | ".join(f"{med[s]:.1f}" for s in SCHEDULES) +
              f" | {best} | {2.0 * M * N * K / (med[best] * 1e-6) / 1e12:.0f} | "
              f"{med['dp'] / med['streamk']:.2f} | {med['dp'] / med['hybrid']:.2f} | "
              f"{sk_split} | {hy_split} |", flush=True)


SWEEP_VARIANTS = (("streamk", 0), ("streamk", "tile_split"), ("hybrid", 0), ("hybrid", "tile_split"),
                  ("hybrid", "one_tile"), ("streamk", "two_kernel"))


def sweep_grids(name, T):
    """Stream-K grid sizes tried per workload: one workgroup per CU (the
    default), one per tile, 128, 64, a seeded random even size, and two per
    CU (only the two-kernel fixup allows grids beyond one resident workgroup
    per CU)."""
    import random
    rnd = random.Random(sum(map(ord, name)) + 20261202).randrange(2, 257, 2)
    out = []
    for g in (256, T, 128, 64, rnd, 512):
        if g not in out:
            out.append(g)
    return out


def grid_sweep(args, out):
    """Stream-K and hybrid (two-tile and one-tile) over several grid sizes g,
    against data-parallel, per workload; one child process per workload."""
    import subprocess
    from persistent_stream_tiling_amd import inputs
    names = sorted(inputs.irregular_workloads()) if args.workload == "irregular" \
        else args.workload.split(",")
    lines = [f"# Stream-K grid sweep: `python bench.py --workload {args.workload} "
             f"--steps {args.steps} --grid-sweep <file>`", "",
             f"Kernel source hash: {kernel_source_hash()}.  Median of {args.steps} timed runs per "
             "line and of as many data-parallel runs timed in alternating rounds with them "
             "(512 MiB cache flush before each), tuned tiles per schedule.  'splits tiles' says "
             "whether the plan does any Stream-K work (some tile cut over two or more "
             "workgroups); a plan that does not is a data-parallel run of whole tiles.  g = 256 is one "
             "workgroup per CU; g = T is one per tile; with g = s*T and s dividing the "
             "iterations per tile, Stream-K is a fixed split-K with s pieces per tile.  Grids "
             "above 256 are refused by the in-kernel fixups (they need every workgroup "
             "resident); `two_kernel` parks every piece and reduces the split tiles in a second "
             "kernel, which allows them.  `one_tile` is the hybrid without two_tiles (Stream-K "
             "over T mod g tiles only).  `tile_split` cuts each Stream-K tile into its own "
             "floor(g / T_sk) pieces (GEMM_FLAG_TILE_SPLIT) instead of splitting all the "
             "iterations evenly; the other lines use the even split.", "",
             "| workload | tiles T | schedule | g | T_sk | splits tiles | us | TFLOP/s | DP us "
             "(interleaved) | DP / this |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for name in names:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--workload", name,
                            "--steps", str(args.steps), "--grid-sweep-rows"],
                           stdout=subprocess.PIPE, check=True, text=True)
        lines += [ln for ln in r.stdout.splitlines() if ln.startswith("| ")]
    text = "\n".join(lines) + "\n"
    open(out, "w").write(text)
    log(text)


def grid_sweep_rows(args):
    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import (FLAG_FIXUP_TWO_KERNEL, FLAG_ONE_TILE, FLAG_TILE_SPLIT,
                                              inputs, tuning)
    wl = workload_table()[args.workload]
    M, N, K, dt = wl["M"], wl["N"], wl["K"], wl["dtype"]
    log(f"[sweep] {args.workload}: {M}x{N}x{K} {dt}")
    a_bits, b_bits = inputs.operands(M, N, K, dt, wl["dist"], wl["seed"], wl["scale"])
    a, b = to_device(a_bits, dt), to_device(b_bits, dt)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flops = 2.0 * M * N * K

    def interleaved(plan, ws, dp, dp_ws):
        """Medians of this plan and of data-parallel, timed in alternating
        rounds so that drift hits both alike."""
        ts, td = [], []
        half = max(1, args.steps // 2)
        for _ in range(2):
            ms, _ = time_schedule(plan, a, b, c, ws, half, 1, flush)
            ts.extend(ms.tolist())
            ms, _ = time_schedule(dp, a, b, c, dp_ws, half, 1, flush)
            td.extend(ms.tolist())
        if ws is not None and plan.workspace_status(ws) != 0:
            raise RuntimeError("a Stream-K fixup wait gave up")
        return float(np.median(ts)) * 1e3, float(np.median(td)) * 1e3

    dp = gsk.GemmPlan(M, N, K, dt, "dp", **tuning.bench_tiles(args.workload, "dp", dt))
    dp_ws = dp.new_workspace()
    for sched, variant in SWEEP_VARIANTS:
        tiles = tuning.bench_tiles(args.workload, sched, dt)
        # the partition is the variant's: Stream-K's even split unless tile_split
        tiles["flags"] = tiles.get("flags", 0) & ~FLAG_TILE_SPLIT
        if variant == "tile_split":
            tiles["flags"] |= FLAG_TILE_SPLIT
        if variant == "one_tile":
            tiles["flags"] = tiles.get("flags", 0) | FLAG_ONE_TILE
        if variant == "two_kernel":
            tiles["flags"] = tiles.get("flags", 0) | FLAG_FIXUP_TWO_KERNEL
        T = gsk.GemmPlan(M, N, K, dt, sched,
                         **dict(tiles, flags=tiles["flags"] & ~FLAG_TILE_SPLIT)).info["tiles"]
        label = sched + (f" {variant}" if variant else "")
        for g in sweep_grids(args.workload, T):
            try:
                plan = gsk.GemmPlan(M, N, K, dt, sched, grid=g, **tiles)
            except ValueError as e:
                print(f"| {args.workload} | {T} | {label} | {g} | | | refused: {str(e)[:60]} "
                      "| | | |", flush=True)
                continue
            info = plan.info
            # Stream-K work: tiles split over several workgroups (T_sk > 0 and
            # a tile with two or more pieces); otherwise the plan runs whole
            # tiles only and is data-parallel under another name
            splits = "yes" if info["tiles_sk"] > 0 and info["max_pieces"] >= 2 else "no"
            us, dp_us = interleaved(plan, plan.new_workspace(), dp, dp_ws)
            print(f"| {args.workload} | {T} | {label} | {g} | {info['tiles_sk']} | {splits} | "
                  f"{us:.1f} | {flops / (us * 1e-6) / 1e12:.0f} | {dp_us:.1f} | "
                  f"{dp_us / us:.2f} |", flush=True)


def log_sampled(args, out):
    """The pages' shape benchmark: fp16 GEMMs of log-sampled shapes, fp16 C.
    Per shape: data-parallel, Stream-K and hybrid (library default plans)
    and, as context only, torch.matmul (hipBLASLt) with the same fp16
    output; median of --steps rounds interleaved over the four, cache flush
    before every run."""
    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd.inputs import log_sampled_shapes
    shapes = log_sampled_shapes(args.log_sampled)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    rows = []

    for i, (M, N, K) in enumerate(shapes):
        a = torch.randn((M, K), device="cuda", generator=gen).half()
        b = torch.randn((K, N), device="cuda", generator=gen).half()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        err = 0.0
        ref = a[:64].float() @ b.float()
        sref = a[:64].float().abs() @ b.float().abs()
        runs = []
        for sched in ("dp", "streamk", "hybrid"):
            plan = gsk.GemmPlan(M, N, K, "f16", sched, flags=gsk.FLAG_C_INPUT_DTYPE)
            ws = plan.new_workspace()
            plan.run(a, b, c, ws)  # raises if a fixup wait gave up
            torch.cuda.synchronize()
            # sanity check on the first rows against an fp32 product (not a parity test:
            # parity is checked against the oracle by the test suite)
            err = max(err, float(((c[:64].float() - ref).abs() / sref.clamp_min(1e-30)).max()))
            runs.append((sched, (lambda p=plan, w=ws: p.run(a, b, c, w, check=False)), []))
        runs.append(("torch", lambda: torch.matmul(a, b, out=c), []))
        # rounds interleaved over the four: kernels of ~10 us vary by several us
        # with the state the GPU is in, and every line sees the same mixture of it
        for rnd in range(args.steps + 1):
            for _, fn, ts in runs:
                flush.zero_()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                fn()
                e.record()
                e.synchronize()
                if rnd:
                    ts.append(s.elapsed_time(e) * 1e3)
        us = {name: float(np.median(ts)) for name, _, ts in runs}
        T = -(-M // 256) * -(-N // 256)  # 256x256 tiles, for the summary by size
        if err > 4e-3 + 2.0 ** -11:
            raise RuntimeError(f"{(M, N, K)}: max |C - A.B| / S = {err:.2e}")
        rows.append((M, N, K, T, us))
        if i % 50 == 0:
            log(f"[log-sampled] {i}/{len(shapes)} {M}x{N}x{K}: " +
                " ".join(f"{k} {v:.1f}" for k, v in us.items()))
        del a, b, c, runs

    def gmean(x):
        return float(np.exp(np.mean(np.log(x))))
    best_sk = np.array([min(r[4]["streamk"], r[4]["hybrid"]) for r in rows])
    dp = np.array([r[4]["dp"] for r in rows])
    hy = np.array([r[4]["hybrid"] for r in rows])
    best = np.minimum(best_sk, dp)
    th = np.array([r[4]["torch"] for r in rows])
    lines = [f"# Log-sampled fp16 shapes: `python bench.py --log-sampled {args.log_sampled} "
             f"--steps {args.steps} --log-sampled-out <file>`", "",
             f"Kernel source hash: {kernel_source_hash()}.  {len(rows)} shapes (M, N, K) drawn "
             "log-uniformly in [256, 8192] and rounded to multiples of 256 (seeded); fp16 inputs "
             "N(0,1), fp16 C (fp32 accumulate); library default plans (tile and, for Stream-K "
             "and hybrid, g from the planner's cost model); median of "
             f"{args.steps} rounds interleaved over the four lines, 512 MiB cache flush before "
             "each run; T below counts "
             "256x256 tiles whatever tile the plan chose.  torch.matmul "
             "(hipBLASLt, same fp16 output) is context, not a target.", "",
             "| statistic | value |", "|---|---|",
             f"| mean DP time / hybrid time (the pages' statistic, over shapes) | "
             f"{float(np.mean(dp / hy)):.3f} |",
             f"| geomean DP / hybrid | {gmean(dp / hy):.3f} |",
             f"| geomean DP / best of Stream-K, hybrid | {gmean(dp / best_sk):.3f} |",
             f"| shapes where Stream-K or hybrid beats DP | {int((best_sk < dp).sum())} of {len(rows)} |",
             f"| geomean torch.matmul / best schedule | {gmean(th / best):.3f} |",
             f"| mean torch.matmul / hybrid | {float(np.mean(th / hy)):.3f} |",
             f"| shapes where the best schedule beats torch.matmul | {int((best < th).sum())} of {len(rows)} |",
             "", "By tile count T (256x256 tiles) relative to the 256 CUs:", "",
             "| T range | shapes | geomean DP / best SK-hybrid | geomean torch / best |",
             "|---|---|---|---|"]
    Ts = np.array([r[3] for r in rows])
    for lo_, hi_ in ((1, 64), (65, 192), (193, 256), (257, 512), (513, 4096)):
        m = (Ts >= lo_) & (Ts <= hi_)
        if m.any():
            lines.append(f"| {lo_}-{hi_} | {int(m.sum())} | {gmean(dp[m] / best_sk[m]):.3f} | "
                         f"{gmean(th[m] / best[m]):.3f} |")
    lines += ["", "First 40 shapes (us):", "",
              "| M | N | K | T | dp | Stream-K | hybrid | torch.matmul |", "|---|---|---|---|---|---|---|---|"]
    for (M, N, K, T, us) in rows[:40]:
        lines.append(f"| {M} | {N} | {K} | {T} | {us['dp']:.1f} | {us['streamk']:.1f} | "
                     f"{us['hybrid']:.1f} | {us['torch']:.1f} |")
    text = "\n".join(lines) + "\n"
    open(out, "w").write(text)
    log(text)


def load_traffic(workload, schedule):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        table = json.load(open(path))
    except ValueError:
        return None
    rec = table.get(f"{workload}/{schedule}")
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None  # counters were taken on another kernel build
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fp16_4096")
    ap.add_argument("--schedules", default=",".join(SCHEDULES))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle (its timing and every output check)")
    ap.add_argument("--c-dtype", choices=("f32", "input"), default="f32",
                    help="C as fp32 (the workloads' output type, the default) or in the input "
                         "dtype (the pages' fp16 output; fp16/bf16 workloads only)")
    ap.add_argument("--order", choices=("tuned", "bands", "hilbert", "rows"), default="tuned",
                    help="tile order of every plan: the tuned one, GROUP_M bands, the Hilbert "
                         "curve, or row-major")
    ap.add_argument("--kernel", choices=("tuned", "ring", "pingpong"), default="tuned",
                    help="fp16/bf16 256x256 kernel: the tuned one, the ring kernel, or the "
                         "wave-specialised ping-pong kernel")
    ap.add_argument("--configs", choices=("all", "standard", "none"), default="all",
                    help="after the --workload line, also measure the other standard workloads "
                         "(standard), plus the 16 irregular shapes (all, the default), or none")
    ap.add_argument("--report", default=None, help="also append per-schedule records here")
    ap.add_argument("--table", default=None, metavar="FILE",
                    help="no JSON line: time the four schedules on each of the workloads named by "
                         "--workload (comma-separated, or 'irregular' for the seeded irregular "
                         "shapes) and write a markdown table to FILE")
    ap.add_argument("--table-row", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--grid-sweep", default=None, metavar="FILE",
                    help="time Stream-K and hybrid over several grid sizes against DP for "
                         "each workload in --workload (comma list, or 'irregular'); write "
                         "a markdown table to FILE")
    ap.add_argument("--grid-sweep-rows", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--log-sampled", type=int, default=0, metavar="N",
                    help="the pages' shape benchmark: N log-sampled fp16 shapes (multiples of "
                         "256 in [256, 8192]), DP / Stream-K / hybrid and torch.matmul")
    ap.add_argument("--log-sampled-out", default="log_sampled.md", metavar="FILE")
    ap.add_argument("--traffic-run", default=None, metavar="SCHEDULE",
                    help="no timing: run a 256 MiB device copy, then this schedule's GEMM, "
                         "three times each (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    if args.table:
        schedule_table(args, args.table)  # children do the GPU work
        return
    if args.grid_sweep:
        grid_sweep(args, args.grid_sweep)
        return

    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import inputs, tuning

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.table_row:
        schedule_table_row(args)
        return
    if args.grid_sweep_rows:
        grid_sweep_rows(args)
        return
    if args.log_sampled:
        log_sampled(args, args.log_sampled_out)
        return
    if args.traffic_run:
        traffic_run(args)
        return

    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    threads = oracle_threads()
    failures = []

    head = measure_workload(args.workload, args, flush, threads, failures,
                            schedules=args.schedules.split(","), oracle=not args.no_cpu_baseline)
    configs = {}
    if args.configs != "none":
        names = [n for n in CONFIG_WORKLOADS if n != args.workload]
        if args.configs == "all":
            names += sorted(inputs.irregular_workloads())
        for name in names:
            configs[name] = measure_workload(name, args, flush, threads, failures,
                                             oracle=not args.no_cpu_baseline)

    dt = head["dtype"]
    best = head["best"]
    rec = head["schedules"][best]
    roof = dict(head["roofline"])
    roof["traffic"] = load_traffic(args.workload, best)
    cpu = None
    if head.get("cpu_oracle"):
        o = head["cpu_oracle"]
        M, N, K = head["M"], head["N"], head["K"]
        what = (f"every element of the {M}x{N}x{K} {dt} product" if o["kind"] == "full" else
                f"{o['elements']} seeded elements of the {M}x{N}x{K} {dt} product")
        cpu = {"value": round(2.0 * (M * N if o["kind"] == "full" else o["elements"]) * K
                              / o["seconds"] / 1e12, 6),
               "unit": "TOP/s" if dt == "i8" else "TFLOP/s", "cores": o["threads"],
               "kind": "oracle",
               "sample": f"{what}, each a {K}-term fp64 dot product in ascending k "
                         f"({o['seconds']:.1f} s on {o['threads']} threads)",
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    line = {
        "metric": METRIC,
        "value": rec["tflops"],
        "unit": "TOP/s" if dt == "i8" else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms"],
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": head["M"], "N": head["N"], "K": head["K"],
                   "distribution": head["distribution"], "c_dtype": head["c_dtype"],
                   "schedule": best, "tiles": rec["tiles"], "grid": rec["grid"]},
        "schedules": head["schedules"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "oracle_check": head.get("oracle_check"),
        "configs": {n: {k: v for k, v in r.items() if k not in ("dtype",)}
                    for n, r in configs.items()},
        "checks_failed": failures,
        "kernel_source": kernel_source_hash(),
    }
    if args.report:
        with open(args.report, "a") as f:
            f.write(json.dumps(line) + "\n")
    print(json.dumps(line), flush=True)
    if failures:
        log(f"[bench] FAILED oracle checks: {failures}")
        sys.exit(3)


# Workloads measured after the headline one (the 16 irregular shapes follow
# unless --configs standard).
CONFIG_WORKLOADS = ["fp16_4096", "fp32_256", "fp16_1536x1536x8192", "bf16_512x512x65536",
                    "bf16_8192x28672x8192", "i8_4096"]
HBM_BOUND = {"bf16_512x512x65536"}


def launch_tiles(name, schedule, dtype, args):
    """The tuned launch configuration of one workload and schedule, with the
    tile order and 256x256 kernel family the command line asks for."""
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import tuning
    t = tuning.bench_tiles(name, schedule, dtype)
    flags = t.get("flags", 0)
    order, kernel = getattr(args, "order", "tuned"), getattr(args, "kernel", "tuned")
    if order == "hilbert":
        flags |= gsk.FLAG_HILBERT_ORDER
    elif order in ("bands", "rows"):
        flags &= ~gsk.FLAG_HILBERT_ORDER
        t["group_m"] = t.get("group_m", 0) if order == "bands" else -1
    if kernel != "tuned" and (t.get("bm"), t.get("bn")) == (256, 256) and dtype in ("f16", "bf16"):
        if kernel == "pingpong":
            flags = (flags | gsk.FLAG_PING_PONG) & ~(gsk.FLAG_STREAM_COPIES | gsk.FLAG_RING_KERNEL)
            t.pop("wave_m", None)
            t.pop("wave_n", None)
        else:
            flags = (flags | gsk.FLAG_RING_KERNEL) & ~gsk.FLAG_PING_PONG
    t["flags"] = flags
    return t


def measure_workload(name, args, flush, threads, failures, schedules=SCHEDULES, oracle=True):
    """Time every schedule of one workload in its tuned launch configuration,
    check each schedule's output against the oracle, and return the record."""
    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import inputs, tuning
    wl = workload_table()[name]
    M, N, K, dt = wl["M"], wl["N"], wl["K"], wl["dtype"]
    log(f"[bench] {name}: {M}x{N}x{K} {dt} {wl['dist']} seed {wl['seed']}")
    a_bits, b_bits = inputs.operands(M, N, K, dt, wl["dist"], wl["seed"], wl["scale"])
    a, b = to_device(a_bits, dt), to_device(b_bits, dt)
    c_half = args.c_dtype == "input" and dt in ("f16", "bf16")
    c_type = torch.int32 if dt == "i8" else (a.dtype if c_half else torch.float32)
    c = torch.empty((M, N), dtype=c_type, device="cuda")
    flops = 2.0 * M * N * K
    unit = "TOP/s" if dt == "i8" else "TFLOP/s"
    checks, timing = (None, None)
    if oracle:
        checks, timing = oracle_reference(name, wl, a_bits, b_bits, threads)
        log(f"[bench] {name}: oracle ({timing['kind']}, {timing['elements']} elements) "
            f"{timing['seconds']:.2f} s on {threads} threads")
    del a_bits, b_bits
    results = {}
    worst_all, checked = 0.0, 0
    for sched in schedules:
        tiles = launch_tiles(name, sched, dt, args)
        if c_half:
            tiles["flags"] = tiles.get("flags", 0) | gsk.FLAG_C_INPUT_DTYPE
        plan = gsk.GemmPlan(M, N, K, dt, sched, **tiles)
        ws = plan.new_workspace()
        log(f"[bench] {sched}: {plan.describe()}")
        ms, wall = time_schedule(plan, a, b, c, ws, args.steps, args.warmup, flush)
        if ws is not None and plan.workspace_status(ws) != 0:
            failures.append(f"{name}/{sched}: a Stream-K fixup wait gave up")
        mean_ms = float(ms.mean())
        tflops = flops / (mean_ms * 1e-3) / 1e12
        compulsory = algorithmic_bytes(M, N, K, dt, plan.info)
        parked = 2 * partial_bytes(plan)
        rec = {"tflops": round(tflops, 2), "ms": round(mean_ms, 5),
               "ms_min": round(float(ms.min()), 5), "ms_median": round(float(np.median(ms)), 5),
               "frac_mfma": round(tflops / PEAK_TFLOPS[dt], 4),
               "hbm_gbs": round(compulsory / (mean_ms * 1e-3) / 1e9, 1),
               "compulsory_bytes": compulsory, "parked_bytes": parked,
               "tiles": tiles, "grid": plan.info["launch_grid"],
               "tiles_sk": plan.info["tiles_sk"], "wall_s": round(wall, 3)}
        if checks is not None:
            worst, count, ok = check_output(c, checks, dt)
            rec["oracle_max_err_over_S"] = worst
            worst_all, checked = max(worst_all, worst), count
            if not ok:
                failures.append(f"{name}/{sched}: outside the tolerance against the oracle")
        results[sched] = rec
        log(f"[bench] {sched}: {mean_ms:.4f} ms  {tflops:.1f} {unit}  "
            f"({100 * rec['frac_mfma']:.1f}% of MFMA peak), {rec['hbm_gbs']:.0f} GB/s compulsory")
        del plan, ws
    best = max(results, key=lambda s_: results[s_]["tflops"])
    r = results[best]
    if name in HBM_BOUND:
        roof = {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(r["hbm_gbs"] / PEAK_HBM_GBS, 4),
                "with_parked_gbs": round((r["compulsory_bytes"] + r["parked_bytes"])
                                         / (r["ms"] * 1e-3) / 1e9, 1)}
    else:
        roof = {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_TFLOPS[dt], "unit": unit,
                "frac": round(r["tflops"] / PEAK_TFLOPS[dt], 4)}
    out = {"M": M, "N": N, "K": K, "dtype": dt, "distribution": wl["dist"],
           "c_dtype": dt if c_half else ("i32" if dt == "i8" else "f32"), "best": best,
           "schedules": results, "roofline": roof}
    if checks is not None:
        out["oracle_check"] = {"elements": checked, "kind": timing["kind"],
                               "max_err_over_S": worst_all, "tolerance": TOL[dt],
                               "schedules_checked": len(results)}
        out["cpu_oracle"] = timing
    del a, b, c
    torch.cuda.empty_cache()
    return out


def traffic_run(args):
    """No timing: a 256 MiB device copy, then one schedule's GEMM, three times
    each (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import inputs, tuning
    from persistent_stream_tiling_amd.profiling import COPY_BYTES
    wl = workload_table()[args.workload]
    M, N, K, dt = wl["M"], wl["N"], wl["K"], wl["dtype"]
    a_bits, b_bits = inputs.operands(M, N, K, dt, wl["dist"], wl["seed"], wl["scale"])
    a, b = to_device(a_bits, dt), to_device(b_bits, dt)
    c_type = torch.int32 if dt == "i8" else torch.float32
    c = torch.empty((M, N), dtype=c_type, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    plan = gsk.GemmPlan(M, N, K, dt, args.traffic_run,
                        **launch_tiles(args.workload, args.traffic_run, dt, args))
    ws = plan.new_workspace()
    for _ in range(3):
        flush.zero_()
        dst.copy_(src)
    for _ in range(3):
        flush.zero_()
        plan.run(a, b, c, ws, check=False)
    torch.cuda.synchronize()
    alg = algorithmic_bytes(M, N, K, dt, plan.info) + 2 * partial_bytes(plan)
    print(json.dumps({"traffic_run": args.workload, "schedule": args.traffic_run,
                      "algorithmic_bytes": alg, "plan": plan.describe()}), flush=True)


if __name__ == "__main__":
    main()
