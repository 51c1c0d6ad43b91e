"""How the operand values set the speed of an fp16/bf16 GEMM (measurement only).

The matrix cores draw more power the more operand bits toggle from one MFMA
to the next, and under sustained MFMA load the card's power limit sets the
clock.  This times the library's kernel in a benchmark workload's
data-parallel launch configuration (4096^3 fp16 by default) on the same shape
with four operand sets:

  normal     the benchmark's seeded operands
  exponents  the same values with their mantissa bits cleared (signs and
             exponents kept: powers of two)
  ones       every element 1.0
  zeros      every element 0.0

Same kernel, same plan, same bytes moved; only the values differ.  Timing as
in the benchmark: a 512 MiB fill evicts L2 and the Infinity Cache before each
launch, HIP events on the launch stream, rounds interleaved across the sets,
median of 24 launches per set.

  python -m persistent_stream_tiling_amd.probes.operand_power --out FILE \
      [--workload bf16_8192x28672x8192]
"""
import argparse

import numpy as np

SETS = ("normal", "exponents", "ones", "zeros")
# per dtype: the sign-and-exponent mask and the bits of 1.0 (as int16)
_BITS = {"f16": (-1024, 0x3C00), "bf16": (-128, 0x3F80)}  # 0xFC00, 0xFF80


def run(workload="fp16_4096", rounds=6, per_round=4):
    import torch
    from .. import inputs, tuning
    from ..plan import GemmPlan
    w = inputs.WORKLOADS[workload]
    M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
    if dt not in _BITS:
        raise ValueError(f"{workload}: fp16 or bf16 workloads only")
    a_bits, b_bits = inputs.operands(M, N, K, dt, w["dist"], w["seed"], w["scale"])
    a = torch.from_numpy(a_bits.view(np.int16)).cuda()
    b = torch.from_numpy(b_bits.view(np.int16)).cuda()
    mask, one = _BITS[dt]
    keep = torch.tensor(mask, dtype=torch.int16, device="cuda")
    ops = {"normal": (a, b), "exponents": (a & keep, b & keep),
           "ones": (torch.full_like(a, one), torch.full_like(b, one)),
           "zeros": (torch.zeros_like(a), torch.zeros_like(b))}
    tt = torch.float16 if dt == "f16" else torch.bfloat16
    ops = {k: (x.view(tt), y.view(tt)) for k, (x, y) in ops.items()}
    tiles = tuning.bench_tiles(workload, "dp", dt)
    plan = GemmPlan(M, N, K, dt, "dp", **tiles)
    ws = plan.new_workspace()
    c = torch.empty((M, N), device="cuda", dtype=torch.float32)
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
    return plan.describe(), {k: float(np.median(v)) for k, v in times.items()}, flops


def report(desc, med, flops, cmd, workload="fp16_4096"):
    lines = [f"# {workload} GEMM: time against operand values", "",
             f"Command: `{cmd}` (`persistent_stream_tiling_amd/probes/operand_power.py`).", "",
             f"Plan: `{desc[:120]}`", "",
             "| operands | us | TFLOP/s | % of 2516.6 | time / normal |",
             "|---|---|---|---|---|"]
    for k in SETS:
        tf = flops / med[k] / 1e6
        lines.append(f"| {k} | {med[k]:.1f} | {tf:.1f} | {100 * tf / 2516.6:.1f}% | "
                     f"{med[k] / med['normal']:.3f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="fp16_4096")
    a = ap.parse_args(argv)
    desc, med, flops = run(a.workload)
    cmd = "python -m persistent_stream_tiling_amd.probes.operand_power --out " + a.out
    if a.workload != "fp16_4096":
        cmd += " --workload " + a.workload
    text = report(desc, med, flops, cmd, a.workload)
    open(a.out, "w").write(text)
    print(text)


if __name__ == "__main__":
    main()
