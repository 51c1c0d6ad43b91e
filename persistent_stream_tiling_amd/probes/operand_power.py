"""How the operand values set the speed of a GEMM (measurement only).

The matrix cores draw more power the more operand bits toggle from one MFMA
to the next, and under sustained MFMA load the card's power limit sets the
clock.  This times the library's kernel in a benchmark workload's
data-parallel launch configuration (4096^3 fp16 by default) on the same shape
with four operand sets:

  normal     the benchmark's seeded operands
  exponents  the same values with their mantissa bits cleared (signs and
             exponents kept: powers of two; for int8, magnitudes rounded
             down to a power of two)
  ones       every element 1.0
  zeros      every element 0.0

Same kernel, same plan, same bytes moved; only the values differ.  Timing as
in the benchmark: a 512 MiB fill evicts L2 and the Infinity Cache before each
launch, HIP events on the launch stream, rounds interleaved across the sets,
median of 24 launches per set.

  python -m persistent_stream_tiling_amd.probes.operand_power --out FILE \
      [--workload bf16_8192x28672x8192]

Under `rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES` the same run
gives each set's clock and MFMA utilisation; `--counters DIR` turns that
run's counter CSV into a table (the dispatches come in the run's fixed order:
one warm-up launch per set, then the interleaved rounds).
"""
import argparse

import numpy as np

SETS = ("normal", "exponents", "ones", "zeros")
# per 16-bit dtype: the sign-and-exponent mask and the bits of 1.0 (as int16)
_BITS = {"f16": (-1024, 0x3C00), "bf16": (-128, 0x3F80)}  # 0xFC00, 0xFF80


def pow2_int8(v):
    """int8 values with their magnitude rounded down to a power of two (sign
    kept, 0 stays 0): the int8 counterpart of clearing a float's mantissa."""
    v = np.asarray(v, dtype=np.int8)
    mag = np.abs(v.astype(np.int16))
    p = np.zeros_like(mag)
    nz = mag > 0
    p[nz] = 1 << np.floor(np.log2(mag[nz])).astype(np.int16)
    return (np.sign(v.astype(np.int16)) * p).astype(np.int8)


def _operand_sets(dt, a_bits, b_bits):
    """Host arrays (int16 bit patterns, or int8 values) per operand set."""
    if dt == "i8":
        a, b = a_bits.view(np.int8), b_bits.view(np.int8)
        return {"normal": (a, b), "exponents": (pow2_int8(a), pow2_int8(b)),
                "ones": (np.ones_like(a), np.ones_like(b)),
                "zeros": (np.zeros_like(a), np.zeros_like(b))}
    mask, one = _BITS[dt]
    a, b = a_bits.view(np.int16), b_bits.view(np.int16)
    return {"normal": (a, b), "exponents": (a & np.int16(mask), b & np.int16(mask)),
            "ones": (np.full_like(a, one), np.full_like(b, one)),
            "zeros": (np.zeros_like(a), np.zeros_like(b))}


def run(workload="fp16_4096", rounds=6, per_round=4):
    import torch
    from .. import inputs, tuning
    from ..plan import GemmPlan
    w = dict(inputs.WORKLOADS, **inputs.EXTRA_WORKLOADS)[workload]
    M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
    if dt not in ("f16", "bf16", "i8"):
        raise ValueError(f"{workload}: fp16, bf16 or int8 workloads only")
    a_bits, b_bits = inputs.operands(M, N, K, dt, w["dist"], w["seed"], w["scale"])
    tt = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}[dt]
    ops = {}
    for k, (x, y) in _operand_sets(dt, a_bits, b_bits).items():
        x, y = torch.from_numpy(np.ascontiguousarray(x)), torch.from_numpy(np.ascontiguousarray(y))
        ops[k] = (x.cuda().view(tt), y.cuda().view(tt))
    tiles = tuning.bench_tiles(workload, "dp", dt)
    plan = GemmPlan(M, N, K, dt, "dp", **tiles)
    ws = plan.new_workspace()
    c = torch.empty((M, N), device="cuda", dtype=torch.int32 if dt == "i8" else torch.float32)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for x, y in ops.values():
        plan.run(x, y, c, ws)
    torch.cuda.synchronize()
    times = {k: [] for k in SETS}
    for _ in range(rounds):
        for k in SETS:
            x, y = ops[k]
            for _ in range(per_round):
                flush.zero_()
                s = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                s.record(stream)
                plan.run(x, y, c, ws, check=False)
                e.record(stream)
                e.synchronize()
                times[k].append(s.elapsed_time(e) * 1e3)
    flops = 2.0 * M * N * K
    return plan.describe(), {k: float(np.median(v)) for k, v in times.items()}, flops, dt


def counters(csv_dir, rounds=6, per_round=4):
    """Per operand set: mean dispatch time, clock (GRBM_GUI_ACTIVE of one die
    per microsecond) and MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES over 1024
    SIMDs x one die's GRBM_GUI_ACTIVE) over its timed GEMM dispatches."""
    import csv
    import statistics
    from ..profiling import SIMDS, XCDS, _find, _is_gemm
    disp = {}
    for r in csv.DictReader(open(_find(csv_dir, "counter_collection.csv"))):
        if not _is_gemm(r["Kernel_Name"]):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]),
                            {"us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    seq = [disp[k] for k in sorted(disp)]
    expected = len(SETS) * (1 + rounds * per_round)
    if len(seq) != expected:
        raise ValueError(f"{len(seq)} GEMM dispatches, expected {expected}")
    out = {}
    for i, d in enumerate(seq[len(SETS):]):
        out.setdefault(SETS[(i // per_round) % len(SETS)], []).append(d)
    res = {}
    for k, ds in out.items():
        gui = [d["GRBM_GUI_ACTIVE"] / XCDS for d in ds]
        res[k] = dict(us=statistics.mean(d["us"] for d in ds),
                      clock_ghz=statistics.mean(g / (d["us"] * 1e3) for g, d in zip(gui, ds)),
                      mfma_util=statistics.mean(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMDS)
                                                for g, d in zip(gui, ds)))
    return res


def counters_report(res, cmd, workload="fp16_4096"):
    lines = [f"# {workload} GEMM: clock and MFMA utilisation against operand values", "",
             f"Command: `{cmd}`, then `python -m persistent_stream_tiling_amd.probes."
             "operand_power --counters <dir> --out <file>`.  Means over each set's 24 timed "
             "dispatches (counter collection serialises dispatches).", "",
             "- clock = GRBM_GUI_ACTIVE of one die / dispatch duration;",
             "- MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE of one die).",
             "", "| operands | us | clock GHz | MFMA util |", "|---|---|---|---|"]
    for k in SETS:
        r = res[k]
        lines.append(f"| {k} | {r['us']:.1f} | {r['clock_ghz']:.2f} | {100 * r['mfma_util']:.1f}% |")
    return "\n".join(lines) + "\n"


def report(desc, med, flops, cmd, workload="fp16_4096", int8=False):
    unit, peak = ("TOP/s", 5033.2) if int8 else ("TFLOP/s", 2516.6)
    lines = [f"# {workload} GEMM: time against operand values", "",
             f"Command: `{cmd}` (`persistent_stream_tiling_amd/probes/operand_power.py`).", "",
             f"Plan: `{desc[:120]}`", "",
             f"| operands | us | {unit} | % of {peak} | time / normal |",
             "|---|---|---|---|---|"]
    for k in SETS:
        tf = flops / med[k] / 1e6
        lines.append(f"| {k} | {med[k]:.1f} | {tf:.1f} | {100 * tf / peak:.1f}% | "
                     f"{med[k] / med['normal']:.3f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="fp16_4096")
    ap.add_argument("--counters", default=None,
                    help="summarise this rocprofv3 --pmc output directory instead of timing")
    a = ap.parse_args(argv)
    if a.counters:
        cmd = ("rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES --output-format csv "
               "-d <dir> -o run -- python3 -m persistent_stream_tiling_amd.probes.operand_power "
               "--out <file>" + ("" if a.workload == "fp16_4096" else " --workload " + a.workload))
        text = counters_report(counters(a.counters), cmd, a.workload)
        open(a.out, "w").write(text)
        print(text)
        return
    desc, med, flops, dt = run(a.workload)
    cmd = "python -m persistent_stream_tiling_amd.probes.operand_power --out " + a.out
    if a.workload != "fp16_4096":
        cmd += " --workload " + a.workload
    text = report(desc, med, flops, cmd, a.workload, int8=dt == "i8")
    open(a.out, "w").write(text)
    print(text)


if __name__ == "__main__":
    main()
