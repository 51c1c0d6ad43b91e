"""Turn rocprofv3 CSV output of bench.py runs into the short summaries kept
under profiles/ (kernel-time table, HBM traffic per launch).

  python -m persistent_stream_tiling_amd.profiling trace  --csv DIR --out FILE --cmd "..."
  python -m persistent_stream_tiling_amd.profiling traffic --fetch DIR --write DIR \
        --workload NAME --schedule NAME --out profiles/traffic.json --cmd "..."
  python -m persistent_stream_tiling_amd.profiling counters --csv DIR --workload NAME \
        --out profiles/FILE.md --cmd "..."

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
        groups = {}
        for d, lab, w in zip(a.csv, a.label, a.workload):
            for sched, vals in pmc_summary(d, a.schedules.split(","), a.warmup, a.steps).items():
                groups.setdefault((w, sched), {})[lab] = vals
        counters = sorted({k for g in groups.values() for v in g.values() for k in v} - {"us"})
        lines = [f"# {a.title}", "", "Commands (one rocprofv3 run per line; counters summed over "
                 "dies and channels per dispatch, then averaged over the timed dispatches):", ""]
        lines += [f"    {c}" for c in a.cmd]
        lines += ["", f"Kernel source hash: {source_hash()}.", "",
                  "| workload | schedule | run | us | " + " | ".join(counters) +
                  (" | L2 hit rate |" if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(counters) else " |"),
                  "|---" * (4 + len(counters) + ({"TCC_HIT_sum", "TCC_MISS_sum"} <= set(counters)))
                  + "|"]
        for (w, sched), labs in groups.items():
            for lab, v in labs.items():
                row = f"| {w} | {sched} | {lab} | {v['us']:.1f} | " + \
                      " | ".join(f"{v.get(c, 0.0):.4g}" for c in counters)
                if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(counters):
                    h, mi = v.get("TCC_HIT_sum", 0.0), v.get("TCC_MISS_sum", 0.0)
                    row += f" | {100 * h / max(h + mi, 1.0):.1f}%"
                lines.append(row + " |")
        text = "\n".join(lines) + "\n"
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
