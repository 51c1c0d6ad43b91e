"""The planner's default Stream-K plan for fp16/bf16: which tile and how many
workgroups g, from a cost model fitted to measurements.

  python -m persistent_stream_tiling_amd.grid_model --shapes 260 --out FILE   (GPU)

The Triton Stream-K issue's benchmark picks g per shape from a sweep (its
final revision reports the best of several g and two_tiles settings).  A
library call cannot sweep, so the planner (``gemm_plan_create`` with
schedule Stream-K or hybrid, no tile and grid 0) estimates the time of a few
candidate plans and takes the cheapest.  This module holds the same rule in
Python, the sweep that measures the candidates on log-sampled fp16 shapes,
the least-squares fit of the rule's coefficients, and the report that
compares the rule's picks with one workgroup per CU and with the best plan
measured.

Candidates, per tile (256x256, 256x128, 128x128, and 64x64 where it gives at
most one tile per CU) with T tiles of ipt 64-deep iterations:
  * aligned splits: g = s*T for s in CANDIDATE_S dividing ipt with g <= CUs.
    Each workgroup then runs one piece of exactly ipt/s iterations inside one
    tile (s = 1: one whole tile per workgroup, no fixup);
  * one workgroup per CU (g = CUs) when that does not split tiles evenly:
    Stream-K's even split of the T*ipt iterations, whose ranges cross tile
    boundaries, so some workgroups run two pieces.
Estimated time (us), with q the iterations of the longest range:
    c0 + it[tile] * q
       + [pieces > 1] * (split[tile] + c_log * area * log2(s))
       + [ranges cross tiles] * CROSS
where area = bm*bn / 65536.  The coefficients come from a least-squares fit
over the measured aligned splits; CROSS is then the median, over the measured
g = CUs plans that cross tiles, of what the fitted terms leave unexplained:
the cost of workgroups that run pieces of two tiles (a second pipeline fill
and a second parked piece, which the whole tile's fixup then waits for).
"""
import argparse
import json
import math
import os
import sys

import numpy as np

TILES = ((256, 256), (256, 128), (128, 128), (64, 64))
NT = len(TILES)
# 64x64 (the register-staged kernel) is a candidate only while it gives at
# most one tile per CU: it is slow per FLOP and wins only on the smallest
# shapes, where fixed per-tile costs dominate
SMALL_TILE = 3


def tile_allowed(ti, T, cus=256):
    return ti != SMALL_TILE or T <= cus
CANDIDATE_S = (1, 2, 3, 4, 6, 8, 16)
BK = 64
# Fitted by `python -m persistent_stream_tiling_amd.grid_model` on MI355X (the
# report is kept under profiles/); the planner in csrc/api.hip holds the same
# numbers (a CPU test checks that both pick the same plan).
COEF = dict(c0=13.31, it=(1.313, 0.979, 0.772, 0.929), split=(15.36, 9.15, 6.42, 2.35),
            c_log=0.08, cross=10.03)


def cdiv(a, b):
    return -(-a // b)


def estimate(coef, ti, T, ipt, g, cus=256):
    """Estimated us of Stream-K with tile TILES[ti], T tiles of ipt iterations,
    g workgroups (see the module docstring)."""
    bm, bn = TILES[ti]
    area = bm * bn / 65536.0
    aligned = g % T == 0 and ipt % (g // T) == 0
    if aligned:
        s, q, cross = g // T, ipt // (g // T), 0.0
    else:
        q, s, cross = cdiv(T * ipt, g), max(2, cdiv(g, T)), coef["cross"]
    est = coef["c0"] + coef["it"][ti] * q + cross
    if s > 1:
        est += coef["split"][ti] + coef["c_log"] * area * math.log2(s)
    return est


def choose(M, N, K, cus=256, coef=None):
    """(bm, bn, g) the planner picks for fp16/bf16 Stream-K/hybrid with no tile
    and grid 0, or None when no tile has at most `cus` tiles (then the
    planner keeps its one-workgroup-per-CU default)."""
    coef = coef or COEF
    ipt = cdiv(max(K, 1), BK)
    best, any_aligned = None, False
    for ti, (bm, bn) in enumerate(TILES):
        T = cdiv(M, bm) * cdiv(N, bn)
        if not tile_allowed(ti, T, cus):
            continue
        for s in CANDIDATE_S:
            if ipt % s or s * T > cus:
                continue
            any_aligned = True
            e = estimate(coef, ti, T, ipt, s * T, cus)
            if best is None or e < best[0]:
                best = (e, bm, bn, s * T)
        g = cus
        if T * ipt >= g and not (g % T == 0 and ipt % (g // T) == 0):
            e = estimate(coef, ti, T, ipt, g, cus)
            if best is None or e < best[0]:
                best = (e, bm, bn, g)
    return best[1:] if any_aligned else None


# -- the sweep (GPU) -------------------------------------------------------

def candidate_grids(T, cus=256):
    gs = {cus, 192, 128, 96, 64, 32}
    gs |= {s * T for s in (1, 2, 3, 4, 6, 8, 16)}
    return sorted(g for g in gs if 0 < g <= cus)


def sweep(shapes, steps, log=print):
    """Time data-parallel (library default tile) and Stream-K for every tile in
    TILES and every candidate grid; fp16 inputs N(0,1), fp16 C.  Per shape the
    configurations are timed in interleaved rounds (every configuration once
    per round, 512 MiB cache flush before each run; median over `steps`
    rounds after one untimed round): kernels of ~10 us vary by several us
    with the state the GPU is in, and interleaving gives every configuration
    the same mixture of it."""
    import torch
    import persistent_stream_tiling_amd as gsk
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    out = []
    for i, (M, N, K) in enumerate(shapes):
        a = torch.randn((M, K), device="cuda", generator=gen).half()
        b = torch.randn((K, N), device="cuda", generator=gen).half()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        runs = [("dp", gsk.GemmPlan(M, N, K, "f16", "dp", flags=gsk.FLAG_C_INPUT_DTYPE))]
        for ti, (bm, bn) in enumerate(TILES):
            T = cdiv(M, bm) * cdiv(N, bn)
            if not tile_allowed(ti, T):
                continue
            for g in candidate_grids(T):
                if g <= T * cdiv(K, BK) or g == 256:
                    runs.append((f"{bm}x{bn}/{g}",
                                 gsk.GemmPlan(M, N, K, "f16", "streamk", bm=bm, bn=bn, grid=g,
                                              flags=gsk.FLAG_C_INPUT_DTYPE)))
        runs = [(key, plan, plan.new_workspace(), []) for key, plan in runs]
        for rnd in range(steps + 1):
            for key, plan, ws, ts in runs:
                flush.zero_()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                plan.run(a, b, c, ws, check=rnd == 0)  # the untimed round checks the fixups
                e.record()
                e.synchronize()
                if rnd:
                    ts.append(s.elapsed_time(e) * 1e3)
        rec = dict(M=M, N=N, K=K, dp=None, sk={})
        for key, plan, ws, ts in runs:
            if key == "dp":
                rec["dp"] = float(np.median(ts))
            else:
                rec["sk"][key] = float(np.median(ts))
        out.append(rec)
        if i % 10 == 0:
            best = min(rec["sk"], key=rec["sk"].get)
            log(f"[grid-model] {i}/{len(shapes)} {M}x{N}x{K}: dp {rec['dp']:.1f} "
                f"best Stream-K {best} {rec['sk'][best]:.1f}")
        del a, b, c, runs
    return out


# -- fit and report (CPU) --------------------------------------------------

def _features(ti, T, ipt, s):
    bm, bn = TILES[ti]
    area = bm * bn / 65536.0
    q = ipt // s
    f = [1.0] + [q * (ti == i) for i in range(NT)]
    f += [float(s > 1 and ti == i) for i in range(NT)] + [(s > 1) * area * math.log2(s)]
    return f


def _parse(key):
    tile, g = key.split("/")
    bm, bn = map(int, tile.split("x"))
    return bm, bn, int(g)


def fit(records):
    """Least-squares coefficients over every measured aligned split, then the
    crossing cost from the measured one-workgroup-per-CU plans that cross."""
    X, y = [], []
    for r in records:
        ipt = cdiv(r["K"], BK)
        for key, us in r["sk"].items():
            bm, bn, g = _parse(key)
            T = cdiv(r["M"], bm) * cdiv(r["N"], bn)
            if g % T or ipt % (g // T):
                continue
            X.append(_features(TILES.index((bm, bn)), T, ipt, g // T))
            y.append(us)
    X, y = np.array(X), np.array(y)
    c, *_ = np.linalg.lstsq(X, y, rcond=None)
    rel = np.abs(X @ c - y) / y
    coef = dict(c0=float(c[0]), it=tuple(float(v) for v in c[1:1 + NT]),
                split=tuple(float(v) for v in c[1 + NT:1 + 2 * NT]), c_log=float(c[1 + 2 * NT]),
                cross=0.0)
    resid = []
    for r in records:
        ipt = cdiv(r["K"], BK)
        for key, us in r["sk"].items():
            bm, bn, g = _parse(key)
            T = cdiv(r["M"], bm) * cdiv(r["N"], bn)
            if g == 256 and T * ipt >= g and not (g % T == 0 and ipt % (g // T) == 0):
                resid.append(us - estimate(coef, TILES.index((bm, bn)), T, ipt, g))
    coef["cross"] = float(np.median(resid)) if resid else 0.0
    return coef, len(y), float(np.median(rel)), float(np.quantile(rel, 0.9))


def _old_default(M, N):
    """One workgroup per CU with the few-tiles tile rule (the planner's
    default before the model)."""
    t256 = cdiv(M, 256) * cdiv(N, 256)
    return 256, (256 if 2 * t256 >= 256 else 128), 256


def _measured(r, bm, bn, g):
    return r["sk"].get(f"{bm}x{bn}/{g}")


def report(records, coef, nfit, med_err, p90_err, cmd, kernel_source=None):
    def gmean(x):
        return float(np.exp(np.mean(np.log(x))))
    rows, changed = [], 0
    for r in records:
        M, N, K = r["M"], r["N"], r["K"]
        pick = choose(M, N, K)  # the library's coefficients
        changed += pick != choose(M, N, K, coef=coef)
        t_pick = _measured(r, *pick) if pick else None
        t_old = _measured(r, *_old_default(M, N))
        t_best = min(r["sk"].values())
        if t_pick is None or t_old is None:
            continue
        rows.append((M, N, K, r["dp"], t_old, t_pick, t_best, pick))
    dp = np.array([x[3] for x in rows])
    old = np.array([x[4] for x in rows])
    pick = np.array([x[5] for x in rows])
    best = np.array([x[6] for x in rows])
    c = coef
    lines = [f"# Stream-K default plan model: `{cmd}`", "",
             f"{len(records)} log-sampled fp16 shapes (M, N, K in [256, 8192], multiples of 256, "
             "seeded), fp16 C.  Per shape: data-parallel with the library's default tile, and "
             "Stream-K with 256x256, 256x128 and 128x128 tiles (and 64x64 where it gives at most "
             "256 tiles) at g in {256, 192, 128, 96, 64, "
             "32} and s*T for s in {1, 2, 3, 4, 6, 8, 16}; per shape, median over rounds "
             "interleaved across all these configurations, 512 MiB cache flush before each "
             "run." + (f"  Kernel source hash of the timed device code: {kernel_source}."
                       if kernel_source else ""), "",
             "## Fit", "",
             f"Least squares over the {nfit} measured aligned splits (g = s*T, s dividing the "
             "iterations per tile): median relative error "
             f"{med_err:.3f}, 90th percentile {p90_err:.3f}.", "",
             "| coefficient | " + " | ".join(f"{bm}x{bn}" for bm, bn in TILES) + " |",
             "|---|" + "---|" * NT,
             "| us per 64-deep iteration | " + " | ".join(f"{v:.3f}" for v in c["it"]) + " |",
             "| split tiles: us | " + " | ".join(f"{v:.2f}" for v in c["split"]) + " |", "",
             f"Constant {c['c0']:.2f} us; split tiles also "
             f"{c['c_log']:.2f} us x log2(s) x bm*bn/65536; ranges that cross tiles "
             f"{c['cross']:.1f} us (median residual of the measured g = 256 plans that cross).", "",
             "The library's planner (and COEF in this module) holds: " +
             ", ".join(f"{k} {v}" for k, v in COEF.items()) +
             f".  Those coefficients and the ones fitted to this run pick different plans for "
             f"{changed} of the {len(records)} shapes.", "",
             "## The library's picks against the measurements", "",
             "| statistic | one workgroup per CU (previous default) | planner's pick | best measured |",
             "|---|---|---|---|",
             f"| mean DP time / Stream-K time | {np.mean(dp / old):.3f} | {np.mean(dp / pick):.3f} | "
             f"{np.mean(dp / best):.3f} |",
             f"| geomean DP / Stream-K | {gmean(dp / old):.3f} | {gmean(dp / pick):.3f} | "
             f"{gmean(dp / best):.3f} |",
             f"| shapes where Stream-K beats DP | {int((old < dp).sum())} | {int((pick < dp).sum())} | "
             f"{int((best < dp).sum())} |",
             f"| geomean pick / best measured | {gmean(old / best):.3f} | {gmean(pick / best):.3f} | 1 |",
             "", f"({len(rows)} shapes where the model applies; on the other "
             f"{len(records) - len(rows)} every tile shape has more than 256 tiles: the planner "
             "keeps one workgroup per CU for Stream-K, and the hybrid one Stream-K wave cut per "
             "tile.)", "",
             "First 40 shapes (us):", "",
             "| M | N | K | dp | g = 256 (previous default) | planner's pick | pick | best measured |",
             "|---|---|---|---|---|---|---|---|"]
    for (M, N, K, d, o, p, b, pk) in rows[:40]:
        lines.append(f"| {M} | {N} | {K} | {d:.1f} | {o:.1f} | {p:.1f} | {pk[0]}x{pk[1]} g={pk[2]} | "
                     f"{b:.1f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", type=int, default=260)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--out", required=True, help="markdown report")
    ap.add_argument("--json", default=None, help="also keep the measurements here")
    ap.add_argument("--from-json", default=None, help="fit and report from kept measurements")
    args = ap.parse_args(argv)
    from .inputs import log_sampled_shapes
    kernel_source = None
    if args.from_json:
        kept = json.load(open(args.from_json))
        # {"kernel_source": hash, "records": [...]}, or a bare record list
        records = kept["records"] if isinstance(kept, dict) else kept
        kernel_source = kept.get("kernel_source") if isinstance(kept, dict) else None
    else:
        import torch
        if not torch.cuda.is_available():
            sys.exit("the sweep needs a GPU (or --from-json)")
        from .profiling import source_hash
        kernel_source = source_hash()
        records = sweep(log_sampled_shapes(args.shapes), args.steps,
                        log=lambda m: print(m, flush=True))
        if args.json:
            json.dump({"kernel_source": kernel_source, "records": records}, open(args.json, "w"))
    coef, nfit, med_err, p90 = fit(records)
    cmd = f"python -m persistent_stream_tiling_amd.grid_model --shapes {args.shapes} --out <file>"
    text = report(records, coef, nfit, med_err, p90, cmd, kernel_source)
    open(args.out, "w").write(text)
    print(text)


if __name__ == "__main__":
    main()
