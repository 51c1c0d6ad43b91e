"""Turn rocprofv3 CSV output of bench.py runs into the short summaries kept
under profiles/ (kernel-time table, HBM traffic per launch).

  python -m persistent_stream_tiling_amd.profiling trace  --csv DIR --out FILE --cmd "..."
  python -m persistent_stream_tiling_amd.profiling traffic --fetch DIR --write DIR \
        --workload NAME --schedule NAME --out profiles/traffic.json --cmd "..."
  python -m persistent_stream_tiling_amd.profiling counters --csv DIR --workload NAME \
        --out profiles/FILE.md --cmd "..."
  python -m persistent_stream_tiling_amd.profiling l2 --csv-a DIR --csv-b DIR --out FILE
  python -m persistent_stream_tiling_amd.profiling tile-order --time F... --l2 DIR... \
        --fetch DIR... --workload NAME... --order NAME... --out FILE
  python -m persistent_stream_tiling_amd.profiling pack-share --csv DIR... \
        --workload NAME... --out FILE

`trace` with --bench-log also sets the traced bench run's own event timings
beside the kernel times.  `l2`, `tile-order` and `pack-share` summarise the
L2 counters of the 4096^3 kernel, the two tile orders, and the repack's share
of the repacked shapes' steps (the commands they expect are in their output).

`trace` reads a --kernel-trace --stats run of `bench.py` and reports, per
schedule, the mean duration of the GEMM kernel over the timed steps (the
bench runs the schedules one after the other: warm-up launches, then the
timed ones).  `traffic` reads two --pmc runs of `bench.py --traffic-run`
(FETCH_SIZE, then WRITE_SIZE), calibrates each counter against the plain
device copy of known size that run performs first, and stores the GEMM
kernel's HBM bytes per launch.  `counters` reads one --pmc run of
`bench.py --no-cpu-baseline` with COUNTERS and reports, per schedule, the
MFMA utilisation (MFMA-busy SIMD cycles over SIMDs x active GPU cycles), the
active clock (GPU-active cycles of one die over the dispatch's duration), LDS
bank-conflict and LDS-active fractions, and wait cycles on LDS results.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 256 << 20  # the copy in bench.py --traffic-run (read and written once)


def source_hash():
    """Hash of the device code (the kernels and the schedule arithmetic they
    run): counters and traffic taken on one build stay valid while it holds."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "kernels.h", "schedule.h"):
        with open(os.path.join(ROOT, "persistent_stream_tiling_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _find(dirname, suffix):
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirname}")
    return hits[0]


def _is_gemm(name):
    return "gsk::gemm_kernel" in name


def trace_summary(csv_dir, schedules, warmup, steps, cmd):
    rows = list(csv.DictReader(open(_find(csv_dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gemm = [r for r in rows if _is_gemm(r["Kernel_Name"])]
    per = warmup + steps
    lines = [f"# rocprofv3 kernel trace: `{cmd}`", "",
             f"Kernel source hash: {source_hash()}", "",
             "| schedule | kernel | launches | mean us (timed steps) | min us | max us |",
             "|---|---|---|---|---|---|"]
    out = {}
    for i, s in enumerate(schedules):
        block = gemm[i * per:(i + 1) * per]
        timed = block[warmup:]
        if not timed:
            break
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        name = timed[0]["Kernel_Name"].split("(")[0].replace("void ", "")
        out[s] = statistics.mean(d)
        lines.append(f"| {s} | `{name}` | {len(timed)} | {statistics.mean(d):.2f} | "
                     f"{min(d):.2f} | {max(d):.2f} |")
    stats_path = glob.glob(os.path.join(csv_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats_path:
        lines += ["", "rocprofv3 --stats (all launches of each kernel symbol, warm-ups included):",
                  "", "| kernel | calls | average us | percent |", "|---|---|---|---|"]
        for r in csv.DictReader(open(stats_path[0])):
            lines.append(f"| `{r['Name'][:80]}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(lines) + "\n", out


def _counter_per_dispatch(csv_dir, counter):
    rows = list(csv.DictReader(open(_find(csv_dir, "counter_collection.csv"))))
    vals = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
        vals[int(r["Dispatch_Id"])][1] += float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals)]


def traffic(fetch_dir, write_dir):
    res = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        disp = _counter_per_dispatch(d, counter)
        copies = [v for n, v in disp if not _is_gemm(n) and "copy" in n.lower()]
        gemms = [v for n, v in disp if _is_gemm(n)]
        if not copies or not gemms:
            raise RuntimeError(f"{counter}: need copy and gemm dispatches, got {[n for n, _ in disp]}")
        kib_copy = statistics.median(copies)
        factor = COPY_BYTES / (kib_copy * 1024.0)     # true bytes per counted byte
        res[key] = {"copy_kib": kib_copy, "factor": factor,
                    "gemm_kib": statistics.median(gemms),
                    "gemm_bytes": statistics.median(gemms) * 1024.0 * factor}
    return res


# One --pmc pass: 6 SQ counters and one GRBM counter (within one pass's limits).
COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT",
            "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS")
XCDS, CUS, SIMDS = 8, 256, 1024
SHORT_US = 50.0


def counters_summary(csv_dir, workload, schedules, warmup, steps, flops):
    """Per schedule: mean over the timed dispatches of each derived figure.
    GRBM_GUI_ACTIVE is summed over the dies by rocprofv3; all dies are busy
    for the whole dispatch, so one die's count is the sum over XCDS."""
    rows = list(csv.DictReader(open(_find(csv_dir, "counter_collection.csv"))))
    disp = {}
    for r in rows:
        if not _is_gemm(r["Kernel_Name"]):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                    "us": (int(r["End_Timestamp"]) -
                                                           int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    order = [disp[k] for k in sorted(disp)]
    per = warmup + steps
    out = []
    for i, s in enumerate(schedules):
        timed = order[i * per:(i + 1) * per][warmup:]
        if not timed:
            break
        def mean(f):
            return statistics.mean(f(d) for d in timed)
        gui = lambda d: d["GRBM_GUI_ACTIVE"] / XCDS  # noqa: E731
        out.append({
            "workload": workload, "schedule": s,
            "kernel": timed[0]["name"].split("(")[0].replace("void ", ""),
            "us": mean(lambda d: d["us"]),
            "tflops": mean(lambda d: flops / (d["us"] * 1e-6) / 1e12),
            "clock_ghz": mean(lambda d: gui(d) / (d["us"] * 1e3)),
            "mfma_util": mean(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui(d) * SIMDS)),
            "lds_bank_conflict": mean(lambda d: d["SQ_LDS_BANK_CONFLICT"] / (gui(d) * CUS)),
            "lds_active": mean(lambda d: d["SQ_LDS_IDX_ACTIVE"] / (gui(d) * CUS)),
            "lds_conflict_per_lds_instr": mean(
                lambda d: d["SQ_LDS_BANK_CONFLICT"] / max(d["SQ_INSTS_LDS"], 1.0)),
            "mfma_instrs": mean(lambda d: d["SQ_INSTS_MFMA"]),
            "lds_wait_per_lds_instr": mean(
                lambda d: d["SQ_WAIT_INST_LDS"] / max(d["SQ_INSTS_LDS"], 1.0)),
        })
    return out


def pmc_summary(csv_dir, schedules, warmup, steps):
    """Per schedule: the mean over the timed GEMM dispatches of every counter
    in a --pmc run of bench.py (one run of warm-up + timed steps per schedule,
    in order), and the dispatch duration."""
    rows = list(csv.DictReader(open(_find(csv_dir, "counter_collection.csv"))))
    disp = {}
    for r in rows:
        if not _is_gemm(r["Kernel_Name"]):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"us": (int(r["End_Timestamp"]) -
                                                           int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    seq = [disp[k] for k in sorted(disp)]
    per = warmup + steps
    out = {}
    for i, sched in enumerate(schedules):
        timed = seq[i * per:(i + 1) * per][warmup:]
        if timed:
            out[sched] = {k: statistics.mean(d.get(k, 0.0) for d in timed) for k in timed[0]}
    return out


def counters_table(records, cmd):
    lines = [f"# rocprofv3 counters per workload and schedule", "",
             f"Command per workload: `{cmd}`", "",
             f"Kernel source hash: {source_hash()}.  Means over the timed dispatches "
             "(counter collection serialises dispatches, so times are a little longer "
             "than in the bench).", "",
             "- MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE of one die) "
             "(rocprofv3's MfmaUtil);",
             "- clock = GRBM_GUI_ACTIVE of one die / dispatch duration;",
             "- peak at clock = 256 CUs x 4096 FLOP/clk x clock (fp16/bf16);",
             "- LDS bank conflict = SQ_LDS_BANK_CONFLICT / (256 CUs x GRBM_GUI_ACTIVE) "
             "(rocprofv3's LdsBankConflict), LDS active = SQ_LDS_IDX_ACTIVE / (256 x "
             "GRBM_GUI_ACTIVE) (LdsUtil).", "",
             "| workload | schedule | kernel | us | TFLOP/s | clock GHz | MFMA util | "
             "LDS bank conflict | LDS conflict cycles / LDS instr | LDS active |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    short = False
    for r in records:
        # GRBM_GUI_ACTIVE also counts the dispatch's own set-up: on a kernel of a
        # few microseconds it swamps the kernel, so clock and MFMA util are void
        if r["us"] < SHORT_US:
            short = True
            clock, util = "n/a*", "n/a*"
        else:
            clock, util = f"{r['clock_ghz']:.2f}", f"{100 * r['mfma_util']:.1f}%"
        lines.append(f"| {r['workload']} | {r['schedule']} | `{r['kernel']}` | {r['us']:.1f} | "
                     f"{r['tflops']:.0f} | {clock} | {util} | "
                     f"{100 * r['lds_bank_conflict']:.2f}% | "
                     f"{r['lds_conflict_per_lds_instr']:.3f} | {100 * r['lds_active']:.1f}% |")
    if short:
        lines += ["", f"\\* dispatches under {SHORT_US} us: the GPU-active count includes the "
                  "dispatch's set-up, so clock and MFMA util are not meaningful there."]
    return "\n".join(lines) + "\n"


def kernel_resources(out, cmd_note):
    """Per compiled kernel: registers, spills, scratch, occupancy and LDS, from
    the compiler's kernel-resource-usage remarks (device code of kernels.hip,
    compiled exactly as the library is)."""
    import re
    import subprocess
    import tempfile
    from . import _build
    src = os.path.join(_build.CSRC, "kernels.hip")
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [_build.hipcc(), f"--offload-arch={_build.ARCH}", "-O3", "-std=c++17",
               f"-I{_build.INCLUDE}", f"-I{_build.CSRC}", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-c",
               "-Rpass-analysis=kernel-resource-usage", src, "-o", os.path.join(tmp, "k.o")]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(res.stderr[-4000:])
    recs, cur = [], None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            recs.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)

    def pretty(mangled):
        m = re.match(r"_ZN3gsk\d+(\w+?)I(.*)EEvNS_10KernelArgsE", mangled)
        if not m:
            return mangled
        args = ", ".join(re.findall(r"Li(\d+)E|Lb(\d)E", m.group(2)) and
                         [x or y for x, y in re.findall(r"Li(\d+)E|Lb(\d)E", m.group(2))])
        return f"{m.group(1)}<{args}>"
    gemm = [r for r in recs if "KernelArgs" in r["name"]]
    lines = ["# Kernel resources (compiler remarks)", "",
             f"Command: `{cmd_note}`", "",
             f"Kernel source hash: {source_hash()}.  Template arguments: <dtype (0 fp32, 1 fp16, "
             "2 bf16, 3 int8), bm, bn, waves along M, waves along N[, non-temporal copies]>; "
             "gemm_kernel_pp<dtype> is 256x256 with 2x4 waves.  gemm_kernel_pp is the fp16/bf16/"
             "int8 default at 256x256 (wave-specialised ping-pong), gemm_kernel_pair the "
             "direct-to-LDS ring kernel (the other fp16/bf16 tiles), gemm_kernel the "
             "register-staged kernel (fp32, the other int8 tiles, fp16/bf16 64x64); "
             "fixup_kernel the two-kernel Stream-K fixup.", "",
             "| kernel | VGPRs | AGPRs | SGPRs | VGPR spills | SGPR spills | scratch B/lane | "
             "waves/SIMD | LDS B |", "|---|---|---|---|---|---|---|---|---|"]
    for r in gemm:
        lines.append(f"| `{pretty(r['name'])}` | {r.get('VGPRs')} | {r.get('AGPRs')} | "
                     f"{r.get('TotalSGPRs')} | {r.get('VGPRs Spill')} | {r.get('SGPRs Spill')} | "
                     f"{r.get('ScratchSize')} | {r.get('Occupancy')} | "
                     f"{r.get('LDS Size')} |")
    text = "\n".join(lines) + "\n"
    open(out, "w").write(text)
    return text


def pmc_table(dirs, labels, workloads, schedules, warmup, steps, title, cmds):
    """Markdown table of counter means per (workload, schedule, run label)."""
    groups = {}
    for d, lab, w in zip(dirs, labels, workloads):
        for sched, vals in pmc_summary(d, schedules, warmup, steps).items():
            groups.setdefault((w, sched), {})[lab] = vals
    counters = sorted({k for g in groups.values() for v in g.values() for k in v} - {"us"})
    hits = {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(counters)
    lines = [f"# {title}", "", "Commands (one rocprofv3 run per line; counters summed over "
             "dies and channels per dispatch, then averaged over the timed dispatches):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", f"Kernel source hash: {source_hash()}.", "",
              "| workload | schedule | run | us | " + " | ".join(counters) +
              (" | L2 hit rate |" if hits else " |"),
              "|---" * (4 + len(counters) + hits) + "|"]
    for (w, sched), labs in groups.items():
        for lab, v in labs.items():
            row = f"| {w} | {sched} | {lab} | {v['us']:.1f} | " + \
                  " | ".join(f"{v.get(c, 0.0):.4g}" for c in counters)
            if hits:
                h, mi = v.get("TCC_HIT_sum", 0.0), v.get("TCC_MISS_sum", 0.0)
                row += f" | {100 * h / max(h + mi, 1.0):.1f}%"
            lines.append(row + " |")
    return "\n".join(lines) + "\n"


def bench_line(log):
    """The JSON line a bench.py run printed (its last line starting with '{')."""
    return json.loads([ln for ln in open(log) if ln.startswith("{")][-1])


def trace_vs_events(means, line):
    """The traced run's own HIP-event timings next to the kernel times."""
    M, N, K = line["config"]["M"], line["config"]["N"], line["config"]["K"]
    flop, rl = 2.0 * M * N * K, line["roofline"]
    lines = ["", "## The same run's bench line (HIP events on the launch stream, one pair per step)",
             "", f"The traced command printed its JSON line: value {line['value']:.2f} "
             f"{line['unit']} ({line['config'].get('schedule')}), ms_per_step "
             f"{line['ms_per_step']:.5f}, roofline.frac {rl['frac']:.4f}, roofline.traffic "
             + (f"{rl['traffic'] / 1e6:.1f} MB per launch (from profiles/traffic.json)."
                if rl.get("traffic") else "null."), "",
             "| schedule | trace mean us (kernel only) | bench event mean us | events / trace | "
             "rate from the trace | rate from the events |", "|---|---|---|---|---|---|"]
    for sched, tr in means.items():
        ev = line["schedules"][sched]["ms"] * 1e3
        lines.append(f"| {sched} | {tr:.2f} | {ev:.2f} | {ev / tr:.3f} | "
                     f"{flop / tr / 1e6:.0f} | {flop / ev / 1e6:.0f} |")
    lines += ["", "The events also cover the kernel's dispatch after the cache flush and its "
              "completion signal, so the bench's event-based figures err low against the kernel "
              "time.", ""]
    return "\n".join(lines)


L2_CMDS = ["rocprofv3 --pmc TCC_READ_sum TCC_HIT_sum TCC_MISS_sum TCC_BUSY_sum GRBM_GUI_ACTIVE "
           "--output-format csv -d <dir> -o run -- python3 bench.py --schedules dp --steps 3 "
           "--warmup 1 --no-cpu-baseline --configs none",
           "rocprofv3 --pmc TCC_READ_SECTORS_sum TCC_REQ_sum GRBM_GUI_ACTIVE --output-format csv "
           "-d <dir> -o run -- python3 bench.py --schedules dp --steps 3 --warmup 1 "
           "--no-cpu-baseline --configs none"]


def l2_report(dir_a, dir_b):
    """L2 reads of the 4096^3 fp16 kernel (data-parallel): the two counter runs
    of L2_CMDS, then the derived rates."""
    text = pmc_table([dir_a, dir_b], ["a", "b"], ["fp16_4096"] * 2, ["dp"], 1, 3,
                     "L2 (TCC) reads of the 4096^3 fp16 ping-pong kernel, data-parallel schedule",
                     L2_CMDS)
    a = pmc_summary(dir_a, ["dp"], 1, 3)["dp"]
    b = pmc_summary(dir_b, ["dp"], 1, 3)["dp"]
    cyc = a["GRBM_GUI_ACTIVE"] / 8
    reads, sect = a["TCC_READ_sum"], b["TCC_READ_SECTORS_sum"] * 32
    hit = a["TCC_HIT_sum"] / max(a["TCC_HIT_sum"] + a["TCC_MISS_sum"], 1.0)
    bw = sect / (a["us"] * 1e-6) / 1e12
    lines = ["", "## Derived (from the table above)", "", "| quantity | value |", "|---|---|",
             f"| dispatch duration (under counter collection) | {a['us']:.1f} us |",
             f"| GPU-active cycles per die (GRBM_GUI_ACTIVE / 8) | {cyc:,.0f} (clock "
             f"{cyc / a['us'] / 1e3:.2f} GHz) |",
             f"| L2 read requests (TCC_READ_sum) | {reads:,.0f} |",
             f"| L2 read sectors x 32 B (TCC_READ_SECTORS_sum) | {sect / 1e9:.3f} GB "
             f"({b['TCC_READ_SECTORS_sum'] / reads:.2f} sectors = {sect / reads:.0f} B per "
             "request) |",
             f"| operand bytes the tiles copy into LDS (256 tiles x (256 + 256) x 4096 x 2 B) | "
             f"{256 * 512 * 4096 * 2 / 1e9:.3f} GB |",
             f"| L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)) | {100 * hit:.1f}% |",
             f"| L2 read bandwidth delivered | {bw:.2f} TB/s ({bw * 1e3 / 256:.0f} GB/s per CU) |",
             "| L2 channel cycles with a request pending (TCC_BUSY_sum / (8 dies x 16 channels) "
             f"/ die cycles) | {100 * a['TCC_BUSY_sum'] / 128 / cyc:.0f}% |", "",
             "Every L2 read is a whole 128-byte line, and the lines read equal the operand bytes "
             "the 256 tiles copy into LDS: the copies fetch nothing twice from L2.  The misses "
             "are the lines each die fetches for its own share of A and B from HBM or the "
             "Infinity Cache.", ""]
    return text + "\n".join(lines)


ORDER_CMD = ("python3 bench.py --workload <workload> --configs none --no-cpu-baseline "
             "--schedules dp,hybrid --order <bands|hilbert>")


def tile_order_report(times, l2_dirs, fetch_dirs, workloads, orders):
    """Bands against the Hilbert order: per (workload, order) one timed bench
    line, one L2 hit/miss counter run and one FETCH_SIZE run."""
    rec = {(w, o): bench_line(t) for t, w, o in zip(times, workloads, orders)}
    lines = ["# Tile order: GROUP_M bands against the Hilbert curve (L2 hits, HBM fetch, time)",
             "", "Each workload's tuned launch configuration (tuning.py), once with its band "
             "order (`--order bands`) and once with the Hilbert curve (`--order hilbert`, "
             "GEMM_FLAG_HILBERT_ORDER); the die remap flag is the tuned one.", "",
             "## Time (bench.py, mean of 20 cold runs)", "", f"    {ORDER_CMD} --steps 20", "",
             "| workload | schedule | bands us | hilbert us | bands TFLOP/s | hilbert TFLOP/s |",
             "|---|---|---|---|---|---|"]
    for w in dict.fromkeys(workloads):
        for sched in ("dp", "hybrid"):
            x = rec[(w, "bands")]["schedules"][sched]
            y = rec[(w, "hilbert")]["schedules"][sched]
            lines.append(f"| {w} | {sched} | {x['ms'] * 1e3:.1f} | {y['ms'] * 1e3:.1f} | "
                         f"{x['tflops']:.0f} | {y['tflops']:.0f} |")
    for title, dirs, counters in (("L2 hit rate", l2_dirs, "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE"),
                                  ("HBM fetch (FETCH_SIZE, KiB per dispatch, uncalibrated)",
                                   fetch_dirs, "FETCH_SIZE")):
        cmd = (f"rocprofv3 --pmc {counters} --output-format csv -d <dir> -o run -- "
               f"{ORDER_CMD} --steps 3 --warmup 1")
        t = pmc_table(dirs, orders, workloads, ["dp", "hybrid"], 1, 3, title, [cmd])
        lines += ["", "## " + t.split("\n", 1)[0][2:], t.split("\n", 1)[1].strip()]
    return "\n".join(lines) + "\n"


def pack_share(dirs, workloads):
    """The repack's share of the steps of repacked shapes, from --kernel-trace
    --stats runs of bench.py (one per workload)."""
    lines = ["# Repack share of the irregular bf16 shapes (rocprofv3 kernel trace)", "",
             f"Kernel source hash: {source_hash()}.  Rows whose byte length is not a multiple of "
             "16 are repacked into the workspace before the GEMM; both operands' repacks run as "
             "one launch (`pack_pair_kernel`, one thread per 16-byte destination chunk over a "
             "flat index of both operands).  The 512 MiB fill kernel "
             "(`vectorized_elementwise_kernel`) is the benchmark's cache flush, outside the "
             "timed window.  The bench times four schedules, each in its tuned configuration, "
             "so a workload's GEMM kernels can differ by schedule.", ""]
    for d, w in zip(dirs, workloads):
        rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
        lines += [f"## {w}", "", "    rocprofv3 --kernel-trace --stats --output-format csv -d "
                  f"<dir> -o tr -- python3 bench.py --workload {w} --configs none "
                  "--no-cpu-baseline --steps 5 --warmup 2", "",
                  "| kernel | calls | average us | percent |", "|---|---|---|---|"]
        pack = gemm = 0.0
        calls = 0
        for r in rows:
            name = r["Name"].split("(")[0].replace("void ", "")
            lines.append(f"| `{name[:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f} |")
            if "pack" in name:
                pack += float(r["TotalDurationNs"]) / 1e3
            elif "gemm_kernel" in name:
                gemm += float(r["TotalDurationNs"]) / 1e3
                calls += int(r["Calls"])
        p, g = pack / max(calls, 1), gemm / max(calls, 1)
        lines += ["", f"Per GEMM launch: pack {p:.1f} us + GEMM {g:.1f} us (mean over the "
                  f"schedules' kernels); the pack is {100 * p / max(p + g, 1e-9):.0f}% of a step.",
                  ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--schedules", default="dp,persistent,streamk,hybrid")
    t.add_argument("--warmup", type=int, default=5)
    t.add_argument("--steps", type=int, default=20)
    t.add_argument("--bench-log", default=None,
                   help="the traced command's output: add its event timings beside the trace")
    l2 = sub.add_parser("l2", help="L2 reads of the 4096^3 kernel (two --pmc runs)")
    l2.add_argument("--csv-a", required=True)
    l2.add_argument("--csv-b", required=True)
    l2.add_argument("--out", required=True)
    to = sub.add_parser("tile-order", help="bands against the Hilbert order")
    to.add_argument("--time", nargs="+", required=True, help="bench.py output per (workload, order)")
    to.add_argument("--l2", nargs="+", required=True, help="--pmc TCC_HIT/MISS run directories")
    to.add_argument("--fetch", nargs="+", required=True, help="--pmc FETCH_SIZE run directories")
    to.add_argument("--workload", nargs="+", required=True)
    to.add_argument("--order", nargs="+", required=True)
    to.add_argument("--out", required=True)
    ps = sub.add_parser("pack-share", help="the repack's share of repacked shapes' steps")
    ps.add_argument("--csv", nargs="+", required=True)
    ps.add_argument("--workload", nargs="+", required=True)
    ps.add_argument("--out", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--schedule", required=True)
    f.add_argument("--algorithmic-bytes", type=float, required=True)
    f.add_argument("--out", required=True)
    f.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True, nargs="+", help="one run directory per workload")
    c.add_argument("--workload", required=True, nargs="+")
    c.add_argument("--schedules", default="dp,persistent,streamk,hybrid")
    c.add_argument("--warmup", type=int, default=1)
    c.add_argument("--steps", type=int, default=3)
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", required=True)
    m = sub.add_parser("pmc", help="counter means per (label, workload, schedule) table")
    m.add_argument("--csv", required=True, nargs="+", help="one --pmc run directory each")
    m.add_argument("--label", required=True, nargs="+")
    m.add_argument("--workload", required=True, nargs="+")
    m.add_argument("--schedules", default="dp,persistent,streamk,hybrid")
    m.add_argument("--warmup", type=int, default=1)
    m.add_argument("--steps", type=int, default=3)
    m.add_argument("--title", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--cmd", required=True, nargs="+", help="the commands that made the runs")
    tt = sub.add_parser("traffic-table", help="markdown table of profiles/traffic.json records")
    tt.add_argument("--json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    tt.add_argument("--workload", required=True)
    tt.add_argument("--kernel", required=True, help="kernel name for the title")
    tt.add_argument("--out", required=True)
    h = sub.add_parser("ceilings", help="run the hardware-ceiling probes, write a table")
    h.add_argument("--out", required=True)
    r = sub.add_parser("resources")
    r.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd_name == "traffic-table":
        table = json.load(open(a.json))
        recs = {k.split("/", 1)[1]: v for k, v in table.items() if k.split("/", 1)[0] == a.workload}
        any_rec = next(iter(recs.values()))
        lines = [f"# HBM-side traffic per launch, {a.workload} (`{a.kernel}`)", "",
                 "Commands (one rocprofv3 run per counter, each on committed files), then the "
                 "table from `profiles/traffic.json`:", "",
                 "    " + any_rec["command"].replace("(then WRITE_SIZE) ", ""),
                 "    " + any_rec["command"].replace("FETCH_SIZE (then WRITE_SIZE)", "WRITE_SIZE"),
                 "    python3 -m persistent_stream_tiling_amd.profiling traffic --fetch <dir> "
                 "--write <dir> --workload <workload> --schedule <schedule> ...",
                 f"    python3 -m persistent_stream_tiling_amd.profiling traffic-table --workload "
                 f"{a.workload} --kernel ... --out <file>", "",
                 "Each run first copies 256 MiB device to device, then runs the GEMM three times; "
                 "a counter's calibration factor is 256 MiB over what it reads for that copy.  "
                 "Algorithmic bytes: A and B read once, C written once, plus every parked "
                 f"Stream-K piece written and read once.  Kernel source hash: "
                 f"{any_rec['source_hash']}.", "",
                 "| schedule | FETCH MB | WRITE MB | total MB | algorithmic MB | traffic / "
                 "algorithmic | FETCH factor | WRITE factor |", "|---|---|---|---|---|---|---|---|"]
        for sched in ("dp", "persistent", "streamk", "hybrid"):
            if sched in recs:
                r = recs[sched]
                lines.append(f"| {sched} | {r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} "
                             f"| {r['bytes_per_launch'] / 1e6:.1f} | {r['algorithmic_bytes'] / 1e6:.1f} "
                             f"| {r['traffic_over_algorithmic']:.3f} | {r['fetch_calibration']:.2f} | "
                             f"{r['write_calibration']:.2f} |")
        text = "\n".join(lines) + "\n"
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd_name == "ceilings":
        import subprocess
        from . import _build
        exe = os.path.join(_build.PROBES, "ceilings")
        if not os.path.exists(exe):
            raise RuntimeError(f"{exe} is missing: build it with _build.build_probes()")
        res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
        if res.returncode != 0:
            raise RuntimeError(res.stderr[-4000:])
        text = "\n".join([
            "# Hardware ceilings of the paths the GEMM kernels use (MI355X)", "",
            "Command: `python -m persistent_stream_tiling_amd.profiling ceilings --out <file>` "
            "(runs `persistent_stream_tiling_amd/probes/ceilings`, built from "
            "`probes/ceilings.hip` by `__graft_entry__.build()`; the probe kernels are "
            "described in that file's header).  A 512 MiB fill before every launch evicts "
            "L2 and the Infinity Cache; medians of 6 runs.", "",
            res.stdout.strip(), ""])
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd_name == "pmc":
        text = pmc_table(a.csv, a.label, a.workload, a.schedules.split(","), a.warmup, a.steps,
                         a.title, a.cmd)
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd_name in ("l2", "tile-order", "pack-share"):
        if a.cmd_name == "l2":
            text = l2_report(a.csv_a, a.csv_b)
        elif a.cmd_name == "tile-order":
            text = tile_order_report(a.time, a.l2, a.fetch, a.workload, a.order)
        else:
            text = pack_share(a.csv, a.workload)
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd_name == "resources":
        print(kernel_resources(a.out, "python -m persistent_stream_tiling_amd.profiling "
                                      "resources --out " + a.out))
    elif a.cmd_name == "counters":
        from . import inputs
        table = dict(inputs.WORKLOADS, **inputs.EXTRA_WORKLOADS, **inputs.irregular_workloads())
        recs = []
        for d, w in zip(a.csv, a.workload):
            wl = table[w]
            recs += counters_summary(d, w, a.schedules.split(","), a.warmup, a.steps,
                                     2.0 * wl["M"] * wl["N"] * wl["K"])
        text = counters_table(recs, a.cmd)
        open(a.out, "w").write(text)
        print(text)
    elif a.cmd_name == "trace":
        if a.bench_log:
            line = bench_line(a.bench_log)
            scheds = list(line["schedules"])
            text, means = trace_summary(a.csv, scheds, line["warmup"], line["steps"], a.cmd)
            text += trace_vs_events(means, line)
        else:
            text, _ = trace_summary(a.csv, a.schedules.split(","), a.warmup, a.steps, a.cmd)
        open(a.out, "w").write(text)
        print(text)
    else:
        r = traffic(a.fetch, a.write)
        table = json.load(open(a.out)) if os.path.exists(a.out) else {}
        total = r["fetch"]["gemm_bytes"] + r["write"]["gemm_bytes"]
        table[f"{a.workload}/{a.schedule}"] = {
            "bytes_per_launch": total, "fetch_bytes": r["fetch"]["gemm_bytes"],
            "write_bytes": r["write"]["gemm_bytes"],
            "fetch_calibration": r["fetch"]["factor"], "write_calibration": r["write"]["factor"],
            "algorithmic_bytes": a.algorithmic_bytes,
            "traffic_over_algorithmic": total / a.algorithmic_bytes,
            "source_hash": source_hash(), "command": a.cmd}
        json.dump(table, open(a.out, "w"), indent=1, sort_keys=True)
        print(json.dumps(table[f"{a.workload}/{a.schedule}"], indent=1))


if __name__ == "__main__":
    main()
