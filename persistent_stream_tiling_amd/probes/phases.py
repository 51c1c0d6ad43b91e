"""Per-workgroup phase timing of the GEMM kernels (measurement only).

An instrumented copy of csrc/kernels.hip is built into probes/libphase.so
(`build()`, run by __graft_entry__.build() with the other probes).  Thread 0
of each workgroup stores wall-clock stamps (s_memrealtime, 100 MHz) into a
device buffer the host hands over with gemm_dbg_set():

  0 start of its work loop      4 end of the kernel (after any split fixup)
  1 end of its last MAC loop    5 end of its first MAC loop
  2 end of its last finish_tile 6 end of its first finish_tile
  3 split fixup: all of a tile's pieces seen (its wait done)
  7 ping-pong kernel: the first item's prologue done (first MFMA burst next)

The stamps sit outside the MAC loops, so the timed code is the library's.
The library itself carries none of this.

In the ping-pong kernel, wave 0 of each group also reads s_memtime at the
end of each of its MFMA bursts and after every phase barrier, and keeps, in
registers, the summed burst lengths and the summed lengths of its MFMA
phases (barrier exit to barrier exit); they are stored once, after its work
loop.  Their ratio is the share of an MFMA phase the burst takes: the rest
is the wait for the other group's memory work, the copies and the barrier.
(The clock read waits for the wave's outstanding LDS reads, which the next
MFMA needs anyway.)

  python -m persistent_stream_tiling_amd.probes.phases \\
      --case fp16_4096:dp:'{"bm":256,"bn":256,"group_m":4,"flags":2}' \\
      --case f16:4096x4096x64:dp:'{}'

A case is WORKLOAD:SCHEDULE:TILES_JSON, where WORKLOAD is a benchmark workload
name or DTYPE:MxNxK.  Per case it prints, over three runs after a warm-up
(warm caches), the span and the min / median / max over workgroups of each
phase, and the per-die means of the MAC-loop duration.
"""
import argparse
import ctypes
import json
import os
import re
import subprocess
import sys
import tempfile

from .. import _build

LIB = os.path.join(_build.PROBES, "libphase.so")

_HEADER = '''
constexpr size_t PS_BASE = PS_BASE_VALUE;
__device__ uint64_t *g_dbg;
extern "C" int gemm_dbg_set(void *p)
{
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_dbg), &p, sizeof(p));
}
__device__ __forceinline__ void dbg_stamp(int p, int i)
{
    if (g_dbg && threadIdx.x == 0)
        g_dbg[p * 8 + i] = wall_clock64();
}
__device__ __forceinline__ void dbg_stamp_first(int p, int i)
{
    if (g_dbg && threadIdx.x == 0 && g_dbg[p * 8 + i] == 0)
        g_dbg[p * 8 + i] = wall_clock64();
}
'''

# (what to find, what to put in its place); every pattern must occur
_PATCHES = [
    # ping-pong kernel: start, prologue, MAC end, finish end, kernel end
    ('''    WorkCursor cur = work_begin(P, p);
    WorkItem w;
    while (work_next(P, p, cur, w)) {
        int tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * 256, n0 = tn * 256;''',
     '''    WorkCursor cur = work_begin(P, p);
    WorkItem w;
    if (GRP == 0) dbg_stamp(p, 0);
    const bool ps_on = g_dbg != nullptr && q == 0;
    uint64_t ps_prev = 0, ps_burst = 0, ps_phase = 0;
    uint32_t ps_n = 0;
    bool ps_mfma = false;
    while (work_next(P, p, cur, w)) {
        int tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * 256, n0 = tn * 256;'''),
    # ping-pong kernel: MFMA burst and MFMA phase lengths
    ('''        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<8>();
            barrier_only();
            __builtin_amdgcn_sched_barrier(0);
        };''',
     '''        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<8>();
            barrier_only();
            if (ps_on) {
                const uint64_t t = __builtin_amdgcn_s_memtime();
                if (ps_mfma)
                    ps_phase += t - ps_prev;
                ps_prev = t;
                ps_mfma = false;
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto burst_end = [&]() {
            if (ps_on) {
                __builtin_amdgcn_sched_barrier(0);
                ps_burst += __builtin_amdgcn_s_memtime() - ps_prev;
                ps_mfma = true;
                ++ps_n;
            }
        };'''),
    ('''            if constexpr (GRP == 0) {
                multiply();
                phase_end();''',
     '''            if constexpr (GRP == 0) {
                multiply();
                burst_end();
                phase_end();'''),
    ('''                phase_end();
                multiply();
                phase_end();
            }
        }''',
     '''                phase_end();
                multiply();
                burst_end();
                phase_end();
            }
        }'''),
    ('''            read_frags(0);
        }
        phase_end();
''', '''            read_frags(0);
        }
        phase_end();
        if (GRP == 0) dbg_stamp_first(p, 7);
'''),
    ('''        wait_vmcnt<0>();  // zero-fill copies past the end have landed

        finish_tile<256, 256, MT, NT, DT == 3>(acc, args, w, p, m0, n0, wave, lane,
                                               GRP * Cfg::WTM, q * Cfg::WTN);''',
     '''        wait_vmcnt<0>();  // zero-fill copies past the end have landed
        if (GRP == 0) { dbg_stamp(p, 1); dbg_stamp_first(p, 5); }
        finish_tile<256, 256, MT, NT, DT == 3>(acc, args, w, p, m0, n0, wave, lane,
                                               GRP * Cfg::WTM, q * Cfg::WTN);
        if (GRP == 0) { dbg_stamp(p, 2); dbg_stamp_first(p, 6); }'''),
    ('''        reduce_split_tiles<256, 256, 2, 4, DT == 3>(args, p, wave, lane);
}''', '''        reduce_split_tiles<256, 256, 2, 4, DT == 3>(args, p, wave, lane);
    __syncthreads();
    dbg_stamp(p, 4);
}'''),
    # ring kernel: MAC end, finish end, kernel end (its start is inserted below)
    ('''        finish_tile<BM, BN, MT, NT>(acc, args, w, p, m0, n0, wave, lane, wy * Cfg::WTM,
                                    wx * Cfg::WTN);''',
     '''        dbg_stamp(p, 1);
        dbg_stamp_first(p, 5);
        finish_tile<BM, BN, MT, NT>(acc, args, w, p, m0, n0, wave, lane, wy * Cfg::WTM,
                                    wx * Cfg::WTN);
        dbg_stamp(p, 2);
        dbg_stamp_first(p, 6);'''),
    ('''    if (args.split_fixup == 1)
        reduce_split_tiles<BM, BN, WM, WN>(args, p, wave, lane);
}''', '''    if (args.split_fixup == 1)
        reduce_split_tiles<BM, BN, WM, WN>(args, p, wave, lane);
    __syncthreads();
    dbg_stamp(p, 4);
}'''),
    # split fixup: every piece of the tile seen
    ('''            wait_flags(args, pf, pl, [pf](int32_t q) { return split_slot(q, q == pf); }, false);
        __syncthreads();''',
     '''            wait_flags(args, pf, pl, [pf](int32_t q) { return split_slot(q, q == pf); }, false);
        __syncthreads();
        dbg_stamp(p, 3);'''),
]


# where the ping-pong group body ends (its work loop closed): store the sums
_PP_END = '''    }
}

template <int DT>
__global__ __launch_bounds__(512, 1) void gemm_kernel_pp(KernelArgs args)'''
_PP_SUMS = '''    }
    if (ps_on && (threadIdx.x & 63) == 0) {
        g_dbg[PS_BASE + ((size_t)p * 2 + GRP) * 4 + 0] = ps_burst;
        g_dbg[PS_BASE + ((size_t)p * 2 + GRP) * 4 + 1] = ps_phase;
        g_dbg[PS_BASE + ((size_t)p * 2 + GRP) * 4 + 2] = ps_n;
    }
}

template <int DT>
__global__ __launch_bounds__(512, 1) void gemm_kernel_pp(KernelArgs args)'''
# u64 offset of the per-group sums in the stamp buffer (8 stamps per
# workgroup come first)
PS_BASE = 65536


def instrument(src):
    """The instrumented text of kernels.hip."""
    i = src.index("namespace gsk {") + len("namespace gsk {")
    src = src[:i] + _HEADER.replace("PS_BASE_VALUE", str(PS_BASE)) + src[i:]
    for old, new in _PATCHES + [(_PP_END, _PP_SUMS)]:
        if src.count(old) != 1:
            raise RuntimeError("kernels.hip changed: a phase stamp no longer has its place:\n" + old)
        src = src.replace(old, new)
    # the ring kernel's work loop start
    m = re.search(r"void gemm_kernel_pair\(KernelArgs args\)\n\{", src)
    j = src.index("while (work_next(P, p, cur, w)) {", m.end())
    return src[:j] + "dbg_stamp(p, 0);\n    " + src[j:]


def build(out=LIB):
    """Compile the instrumented copy with api.hip into `out` (host-side hipcc)."""
    src = open(os.path.join(_build.CSRC, "kernels.hip")).read()
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "kernels_phase.hip")
        open(path, "w").write(instrument(src))
        cmd = [_build.hipcc(), f"--offload-arch={_build.ARCH}", "-O3", "-std=c++17", "-fPIC",
               "-shared", f"-I{_build.INCLUDE}", f"-I{_build.CSRC}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               path, os.path.join(_build.CSRC, "api.hip"), "-o", out + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
    os.replace(out + ".tmp", out)
    return out


def _operands(spec, torch, inputs):
    if ":" in spec:
        dt, shape = spec.split(":")
        M, N, K = map(int, shape.split("x"))
        w = dict(M=M, N=N, K=K, dtype=dt, dist="int8" if dt == "i8" else "normal", seed=5,
                 scale=1.0)
    else:
        w = dict(inputs.WORKLOADS, **inputs.EXTRA_WORKLOADS, **inputs.irregular_workloads())[spec]
    M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
    a, b = inputs.operands(M, N, K, dt, w["dist"], w["seed"], w["scale"])
    import numpy as np
    if dt == "i8":
        return M, N, K, dt, torch.from_numpy(a.view(np.int8)).cuda(), \
            torch.from_numpy(b.view(np.int8)).cuda()
    if dt == "f32":
        return M, N, K, dt, torch.from_numpy(a.view(np.float32)).cuda(), \
            torch.from_numpy(b.view(np.float32)).cuda()
    tt = torch.float16 if dt == "f16" else torch.bfloat16
    return M, N, K, dt, torch.from_numpy(a.view(np.int16)).view(tt).cuda(), \
        torch.from_numpy(b.view(np.int16)).view(tt).cuda()


def run(cases, runs=3):
    import numpy as np
    import torch
    from .. import _lib
    lib = _lib.load(LIB)
    lib.gemm_dbg_set.argtypes = [ctypes.c_void_p]
    lib.gemm_dbg_set.restype = ctypes.c_int
    from .. import inputs
    from ..plan import GemmPlan
    dbg = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    if lib.gemm_dbg_set(dbg.data_ptr()) != 0:
        raise RuntimeError("gemm_dbg_set failed")

    def q(x):
        return f"{np.min(x):7.1f} {np.median(x):7.1f} {np.max(x):7.1f}" if len(x) else "     --"
    for spec, sched, tiles in cases:
        M, N, K, dt, a, b = _operands(spec, torch, inputs)
        plan = GemmPlan(M, N, K, dt, sched, **tiles)
        g = plan.info["launch_grid"]
        if (PS_BASE + g * 8) * 8 > dbg.numel():
            raise ValueError(f"{g} workgroups exceed the stamp buffer")
        ws = plan.new_workspace()
        c = torch.empty((M, N), device="cuda",
                        dtype=torch.int32 if dt == "i8" else torch.float32)
        die = np.zeros(g, int)
        for hw in range(g):
            die[plan.logical_wg(hw)] = hw % 8
        print(f"{spec} {sched} {json.dumps(tiles)}: {plan.describe()[:160]}", flush=True)
        loops = []
        for rep in range(runs + 1):
            dbg.zero_()
            torch.cuda.synchronize()
            plan.run(a, b, c, ws, check=False)
            torch.cuda.synchronize()
            d = dbg[: g * 64].cpu().numpy().view(np.uint64).reshape(g, 8).astype(np.int64)
            if rep == 0:
                continue  # warm-up
            t0 = d[:, 0].min()
            st, mac, fin, wt, end, mac1, fin1, pro = ((d[:, i] - t0) / 100.0 for i in range(8))
            loops.append(mac - st)
            split = d[:, 3] > 0
            print(f"  run {rep}: span {end.max():.1f} us | start {q(st)} | MAC end {q(mac)} | "
                  f"finish end {q(fin)} | end {q(end)}")
            print(f"           first MAC end {q(mac1)} | first park/store {q(fin1 - mac1)}"
                  + (f" | prologue {q(pro[d[:, 7] > 0] - st[d[:, 7] > 0])}" if (d[:, 7] > 0).any()
                     else "")
                  + (f" | fixup wait {q(wt[split] - fin[split])} | reduce {q(end[split] - wt[split])}"
                     if split.any() else ""), flush=True)
        m = np.mean(loops, axis=0)
        print("  per-die mean (start to last MAC end) us: " +
              " ".join(f"{np.mean(m[die == x]):.1f}" for x in range(8) if (die == x).any()),
              flush=True)
        if plan.info["kernel_kind"] == 3:
            ps = dbg.cpu().numpy().view(np.uint64)[PS_BASE:PS_BASE + g * 8].reshape(g, 2, 4)
            ps = ps.astype(np.float64)
            for grp in range(2):
                nb = ps[:, grp, 2]
                ok = nb > 0
                if not ok.any():
                    continue
                burst = ps[ok, grp, 0] / nb[ok]
                phase = ps[ok, grp, 1] / nb[ok]
                print(f"  group {grp}, per MFMA phase (s_memtime ticks, median over workgroups): "
                      f"burst {np.median(burst):.0f}, phase {np.median(phase):.0f}, "
                      f"burst / phase {np.median(burst / phase):.3f}", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--case", action="append", required=True,
                    help="WORKLOAD:SCHEDULE:TILES_JSON (WORKLOAD may be DTYPE:MxNxK)")
    ap.add_argument("--runs", type=int, default=3)
    args = ap.parse_args(argv)
    cases = []
    for c in args.case:
        brace = c.find("{")
        head, tiles = (c[:brace].rstrip(":"), c[brace:]) if brace >= 0 else (c, "{}")
        spec, sched = head.rsplit(":", 1)
        cases.append((spec, sched, json.loads(tiles)))
    if not os.path.exists(LIB):
        sys.exit(f"{LIB} is missing: build it with persistent_stream_tiling_amd.probes.phases.build()")
    run(cases, args.runs)


if __name__ == "__main__":
    main()
