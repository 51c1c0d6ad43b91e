"""GPU parity: the gfx950 kernels through the C ABI against the CPU oracle.

Small shapes (several tiles plus ragged tails) are compared element by
element in full, for every compiled kernel variant.  The full-size
workloads, in the launch configuration the benchmark times, are compared
element by element where the full oracle takes seconds (every product up to
4096^3 multiply-adds), and on seeded samples plus their ragged edges above
that (the 8192x28672x8192 shape and the 16 irregular shapes).
Integer-valued inputs must match exactly; everything else must satisfy
|C - C_ref| <= tol * sum_k |a_ik||b_kj| (tol 1e-5 for fp32, 4e-3 for
fp16/bf16 inputs).
"""
import numpy as np
import pytest

import oracle
from gpu_util import compare, run_gemm, to_device
from persistent_stream_tiling_amd import inputs, tuning

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SCHEDULES = ("dp", "persistent", "streamk", "hybrid")

SMALL = [
    (320, 384, 512),   # whole 64-wide tiles, not whole 256-wide ones
    (300, 200, 704),   # ragged M and N; K a multiple of 8 (no repack)
    (257, 203, 701),   # ragged everything; rows not 16-byte multiples (repacked)
]
TILES = {"f16": [dict(bm=64, bn=64), dict(bm=128, bn=128), dict(bm=256, bn=128),
                 dict(bm=128, bn=256), dict(bm=256, bn=256)],
         "bf16": [dict(bm=64, bn=64), dict(bm=128, bn=128), dict(bm=256, bn=256),
                  dict(bm=256, bn=128, wave_m=4, wave_n=2)],
         "f32": [dict(bm=64, bn=64), dict(bm=128, bn=128)]}


def _small_case_id(v):
    return "x".join(map(str, v)) if isinstance(v, tuple) else str(v)


_ORACLE_CACHE = {}


def small_inputs(M, N, K, dtype, dist="normal"):
    key = (M, N, K, dtype, dist)
    if key not in _ORACLE_CACHE:
        a, b = inputs.operands(M, N, K, dtype, dist, seed=M * 7 + N * 3 + K)
        ref, scale = oracle.gemm(a, b, dtype)
        _ORACLE_CACHE[key] = (a, b, ref, scale)
    return _ORACLE_CACHE[key]


@pytest.mark.parametrize("shape", SMALL, ids=_small_case_id)
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_small_parity(shape, dtype, schedule):
    M, N, K = shape
    a, b, ref, scale = small_inputs(M, N, K, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    for tiles in TILES[dtype]:
        grids = [0, 37] if schedule in ("streamk", "hybrid") else [0]
        for g in grids:
            plan, ws, c = run_gemm(da, db, M, N, K, dtype, schedule, grid=g, **tiles)
            compare(c.cpu().numpy(), ref, scale, dtype, what=plan.describe())
            if ws is not None:
                assert plan.workspace_status(ws) == 0


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_integer_inputs_exact(dtype, schedule):
    # values in [-4, 4]: every partial sum is an integer below 2^24, exact in fp32
    M, N, K = 200, 136, 2050
    a, b = inputs.operands(M, N, K, dtype, "int4", seed=99)
    ref, _ = oracle.gemm(a, b, dtype, want_s=False)
    da, db = to_device(a, dtype), to_device(b, dtype)
    for tiles in TILES[dtype][:2]:
        plan, _, c = run_gemm(da, db, M, N, K, dtype, schedule, grid=0, **tiles)
        compare(c.cpu().numpy(), ref, None, dtype, exact=True, what=plan.describe())


def test_stream_k_long_k_integer_exact():
    # few tiles, long K: every tile split over many workgroups, fixed-order fixup
    M, N, K = 256, 256, 65536
    a, b = inputs.operands(M, N, K, "bf16", "int4", seed=5)
    rows, cols = inputs.sample_positions(M, N, 2048, seed=6, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    import persistent_stream_tiling_amd as gsk
    for tiles in (dict(bm=128, bn=128), dict(bm=64, bn=64), dict(bm=256, bn=256),
                  dict(bm=256, bn=128)):
        for g in (256, 100, 3):
            for flag in (gsk.FLAG_FIXUP_HEAD, gsk.FLAG_FIXUP_SPLIT):
                t = dict(tiles)
                t["flags"] = t.get("flags", 0) | flag
                plan, _, c = run_gemm(da, db, M, N, K, "bf16", "streamk", grid=g, **t)
                got = c.cpu().numpy()[rows, cols]
                compare(got, ref, None, "bf16", exact=True, what=plan.describe())


@pytest.mark.parametrize("tiles", [dict(bm=128, bn=128), dict(bm=256, bn=256), dict(bm=64, bn=64),
                                   dict(bm=256, bn=128)],
                         ids=lambda t: f"{t['bm']}x{t['bn']}")
def test_split_and_head_fixups_agree_bitwise(tiles):
    # both fixups add every element's pieces in ascending k order
    M, N, K = 512, 384, 16384
    a, b = inputs.operands(M, N, K, "bf16", "normal", seed=21)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    import persistent_stream_tiling_amd as gsk
    outs = {}
    for name, flag in (("head", gsk.FLAG_FIXUP_HEAD), ("split", gsk.FLAG_FIXUP_SPLIT)):
        t = dict(tiles)
        t["flags"] = t.get("flags", 0) | flag
        plan, ws, c = run_gemm(da, db, M, N, K, "bf16", "streamk", **t)
        assert plan.info["max_pieces"] >= 2
        assert plan.workspace_status(ws) == 0
        # flags and counters are left zero for the next run
        g = plan.info["g"]
        slots = 2 * g if plan.info["split_fixup"] else g
        flags_end = 256 + 4 * slots
        wsn = ws.cpu().numpy()
        assert not wsn[256:flags_end].any()
        if plan.info["split_fixup"]:
            counters = (flags_end + 255) // 256 * 256
            assert not wsn[counters:counters + 4 * plan.info["tiles_sk"]].any()
        outs[name] = c.cpu().numpy()
        # and a second run on the same workspace gives the same bits
        c2 = torch.empty_like(c)
        plan.run(da, db, c2, ws)
        torch.cuda.synchronize()
        assert np.array_equal(c2.cpu().numpy().view(np.uint32), outs[name].view(np.uint32))
    assert np.array_equal(outs["head"].view(np.uint32), outs["split"].view(np.uint32))
    rows, cols = inputs.sample_positions(M, N, 512, seed=1)
    ref, scale = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    compare(outs["split"][rows, cols], ref, scale, "bf16", what="split fixup")


@pytest.mark.parametrize("tiles", [dict(bm=128, bn=128), dict(bm=256, bn=256),
                                   dict(bm=256, bn=128, wave_m=4, wave_n=2), dict(bm=64, bn=64)],
                         ids=lambda t: f"{t['bm']}x{t['bn']}")
def test_two_kernel_fixup(tiles):
    # same additions in the same order as the split fixup, so the same bits;
    # and grids beyond one resident workgroup per CU, which only it allows
    import persistent_stream_tiling_amd as gsk
    M, N, K = 512, 384, 16384
    a, b = inputs.operands(M, N, K, "bf16", "normal", seed=21)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    rows, cols = inputs.sample_positions(M, N, 512, seed=1)
    ref, scale = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    for g in (0, 37):
        _, _, c_split = run_gemm(da, db, M, N, K, "bf16", "streamk", grid=g,
                                 flags=gsk.FLAG_FIXUP_SPLIT, **tiles)
        plan, ws, c_two = run_gemm(da, db, M, N, K, "bf16", "streamk", grid=g,
                                   flags=gsk.FLAG_FIXUP_TWO_KERNEL, **tiles)
        assert plan.info["split_fixup"] == 2
        assert torch.equal(c_split.view(torch.int32), c_two.view(torch.int32)), plan.describe()
        assert not ws[256:].cpu().numpy()[:4 * 2 * plan.info["g"]].any()  # no flag ever set
    ai, bi = inputs.operands(M, N, K, "bf16", "int4", seed=22)
    refi, _ = oracle.gemm_sampled(ai, bi, "bf16", rows, cols)
    dai, dbi = to_device(ai, "bf16"), to_device(bi, "bf16")
    for sched in ("streamk", "hybrid"):
        for g in (512, 1024):
            plan, ws, c = run_gemm(da, db, M, N, K, "bf16", sched, grid=g,
                                   flags=gsk.FLAG_FIXUP_TWO_KERNEL, **tiles)
            compare(c.cpu().numpy()[rows, cols], ref, scale, "bf16", what=plan.describe())
            plan, ws, c = run_gemm(dai, dbi, M, N, K, "bf16", sched, grid=g,
                                   flags=gsk.FLAG_FIXUP_TWO_KERNEL, **tiles)
            compare(c.cpu().numpy()[rows, cols], refi, None, "bf16", exact=True,
                    what=plan.describe())


@pytest.mark.parametrize("fixup", ["head", "split"])
def test_workspace_reuse_with_new_inputs(fixup):
    # partial slots are reused run after run; a stale copy of a slot in some
    # die's L2 would show up as a wrong result on the next run's new inputs
    import persistent_stream_tiling_amd as gsk
    flag = gsk.FLAG_FIXUP_HEAD if fixup == "head" else gsk.FLAG_FIXUP_SPLIT
    M, N, K = 384, 512, 12288
    plan = gsk.GemmPlan(M, N, K, "f16", "streamk", bm=128, bn=128, flags=flag)
    assert plan.info["max_pieces"] >= 3
    ws = plan.new_workspace()
    rows, cols = inputs.sample_positions(M, N, 1024, seed=2)
    for seed in (31, 32, 33, 34):
        a, b = inputs.operands(M, N, K, "f16", "int4", seed=seed)
        ref, _ = oracle.gemm_sampled(a, b, "f16", rows, cols)
        c = torch.full((M, N), float("nan"), device="cuda")
        plan.run(to_device(a, "f16"), to_device(b, "f16"), c, ws)
        torch.cuda.synchronize()
        compare(c.cpu().numpy()[rows, cols], ref, None, "f16", exact=True,
                what=f"{fixup} seed {seed}")
        assert plan.workspace_status(ws) == 0


@pytest.mark.parametrize("schedule", ["streamk", "hybrid"])
def test_deterministic_across_runs(schedule):
    M, N, K = 640, 640, 8192
    a, b = inputs.operands(M, N, K, "f16", "uniform", seed=11)
    da, db = to_device(a, "f16"), to_device(b, "f16")
    import persistent_stream_tiling_amd as gsk
    plan = gsk.GemmPlan(M, N, K, "f16", schedule, bm=128, bn=128)
    ws = plan.new_workspace()
    outs = []
    for _ in range(10):
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        plan.run(da, db, c, ws)
        outs.append(c)
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy().view(np.uint32)
    for o in outs[1:]:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), first)
    # flags are left clear: the workspace past the status word is all zero flags
    flags = ws[256:256 + 4 * plan.info["g"]].cpu().numpy()
    assert not flags.any() and plan.workspace_status(ws) == 0


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 300, 70), (300, 1, 70), (70, 90, 1),
                                   (33, 65, 17), (64, 64, 64), (5, 1000, 3)],
                         ids=_small_case_id)
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_edge_shapes(shape, schedule):
    M, N, K = shape
    for dtype in ("f16", "f32"):
        a, b = inputs.operands(M, N, K, dtype, "normal", seed=3)
        ref, scale = oracle.gemm(a, b, dtype)
        plan, _, c = run_gemm(to_device(a, dtype), to_device(b, dtype), M, N, K, dtype,
                              schedule)
        compare(c.cpu().numpy(), ref, scale, dtype, what=plan.describe())


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_stream_copies(schedule):
    # the non-temporal copy hint changes no value: same bits as without it
    import persistent_stream_tiling_amd as gsk
    for dtype in ("f16", "bf16"):
        M, N, K = 257, 203, 701
        a, b, ref, scale = small_inputs(M, N, K, dtype)
        da, db = to_device(a, dtype), to_device(b, dtype)
        for tiles in (dict(bm=256, bn=128, wave_m=4, wave_n=2), dict(bm=256, bn=256, wave_m=2, wave_n=4)):
            for g in ([0, 37] if schedule in ("streamk", "hybrid") else [0]):
                _, _, c0 = run_gemm(da, db, M, N, K, dtype, schedule, grid=g, **tiles)
                plan, _, c1 = run_gemm(da, db, M, N, K, dtype, schedule, grid=g,
                                       flags=gsk.FLAG_STREAM_COPIES, **tiles)
                assert plan.info["kernel_kind"] == 2
                assert torch.equal(c0.view(torch.int32), c1.view(torch.int32)), plan.describe()
                compare(c1.cpu().numpy(), ref, scale, dtype, what=plan.describe())


@pytest.mark.parametrize("schedule", ["streamk", "hybrid", "persistent"])
def test_degenerate_grids(schedule):
    # g = 1 (one workgroup walks everything), tiny g, g larger than the
    # iteration count (q = 0: workgroups past r get nothing) and g = T
    M, N, K = 257, 203, 701
    a, b, ref, scale = small_inputs(M, N, K, "bf16")
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    for tiles in (dict(bm=64, bn=64), dict(bm=128, bn=128), dict(bm=256, bn=256)):
        for g in (1, 2, 3, 250):
            plan, ws, c = run_gemm(da, db, M, N, K, "bf16", schedule, grid=g, **tiles)
            compare(c.cpu().numpy(), ref, scale, "bf16", what=plan.describe())
            if ws is not None:
                assert plan.workspace_status(ws) == 0


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_empty_shapes(schedule):
    import persistent_stream_tiling_amd as gsk
    # K = 0: C is the empty sum, all zeros
    plan = gsk.GemmPlan(37, 45, 0, "f16", schedule)
    a = torch.empty((37, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, 45), dtype=torch.float16, device="cuda")
    c = torch.full((37, 45), 7.0, device="cuda")
    plan.run(a, b, c, plan.new_workspace())
    torch.cuda.synchronize()
    assert (c == 0).all()
    # M = 0 or N = 0: nothing to do, nothing touched
    for M, N in ((0, 45), (37, 0)):
        plan = gsk.GemmPlan(M, N, 64, "f16", schedule)
        plan.run(torch.empty((M, 64), dtype=torch.float16, device="cuda"),
                 torch.empty((64, N), dtype=torch.float16, device="cuda"),
                 torch.empty((M, N), device="cuda"), plan.new_workspace())


@pytest.mark.parametrize("fixup", ["head", "split"])
def test_lost_signal_is_reported_and_workspace_recovers(fixup):
    # a piece whose flag never rises (forced from the host): every wait on it
    # is bounded, the kernel ends, and the workspace status says the run failed;
    # after a zero fill the same workspace serves a normal plan again
    import persistent_stream_tiling_amd as gsk
    flag = gsk.FLAG_FIXUP_HEAD if fixup == "head" else gsk.FLAG_FIXUP_SPLIT
    M, N, K = 256, 512, 16384
    a, b = inputs.operands(M, N, K, "bf16", "int4", seed=41)
    rows, cols = inputs.sample_positions(M, N, 1024, seed=42, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    bad = gsk.GemmPlan(M, N, K, "bf16", "streamk", bm=128, bn=128,
                       flags=flag | gsk.FLAG_DEBUG_DROP_SIGNAL)
    good = gsk.GemmPlan(M, N, K, "bf16", "streamk", bm=128, bn=128, flags=flag)
    assert bad.workspace_bytes == good.workspace_bytes and bad.info["max_pieces"] >= 2
    ws = good.new_workspace()
    c = torch.empty((M, N), device="cuda")
    assert bad.may_wait and good.may_wait
    # the binding reads the status after a run that can wait, and raises
    with pytest.raises(gsk.FixupError, match="gave up"):
        bad.run(da, db, c, ws)
    assert bad.workspace_status(ws) == 1
    # without the check the run stays asynchronous; the status is sticky
    bad.run(da, db, c, ws, check=False)
    torch.cuda.synchronize()
    assert bad.workspace_status(ws) == 1
    ws.zero_()
    good.run(da, db, c, ws)
    torch.cuda.synchronize()
    assert good.workspace_status(ws) == 0
    compare(c.cpu().numpy()[rows, cols], ref, None, "bf16", exact=True, what=good.describe())


def test_side_stream_and_reuse_across_plans():
    M, N, K = 300, 200, 704
    a, b, ref, scale = small_inputs(M, N, K, "f16")
    da, db = to_device(a, "f16"), to_device(b, "f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan, ws, c = run_gemm(da, db, M, N, K, "f16", "streamk", stream=s, bm=64, bn=64)
    compare(c.cpu().numpy(), ref, scale, "f16", what="side stream")


def test_rejects_misaligned_pointer():
    import persistent_stream_tiling_amd as gsk
    plan = gsk.GemmPlan(64, 64, 64, "f16", "dp")
    buf = torch.zeros(64 * 64 + 1, dtype=torch.float16, device="cuda")
    b = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    c = torch.zeros((64, 64), device="cuda")
    with pytest.raises(RuntimeError, match="aligned"):
        plan.run(buf.data_ptr() + 2, b, c)


# ---- full-size workloads, in the benchmark's launch configuration ----------

_FULL = {}


def full_case(name, n_samples, edges):
    """Device operands plus oracle values: every element where the product
    has at most 4096^3 multiply-adds, else seeded samples and (optionally)
    every element of the last two rows and last two columns."""
    if name not in _FULL:
        _FULL.clear()
        w = dict(inputs.WORKLOADS, **inputs.EXTRA_WORKLOADS, **inputs.irregular_workloads())[name]
        M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
        a, b = inputs.operands(M, N, K, dt, w["dist"], w["seed"], w["scale"])
        checks = []
        if M * N * K <= 4096 ** 3:
            ref, scale = oracle.gemm(a, b, dt)
            checks.append(("all", (slice(None), slice(None)), ref, scale))
        else:
            rows, cols = inputs.sample_positions(M, N, n_samples, seed=w["seed"] + 1000)
            ref, scale = oracle.gemm_sampled(a, b, dt, rows, cols)
            checks.append(("samples", (rows, cols), ref, scale))
            if edges:
                ref, scale = oracle.gemm(np.ascontiguousarray(a[M - 2:]), b, dt)
                checks.append(("last rows", (slice(M - 2, M), slice(None)), ref, scale))
                ref, scale = oracle.gemm(a, np.ascontiguousarray(b[:, N - 2:]), dt)
                checks.append(("last cols", (slice(None), slice(N - 2, N)), ref, scale))
        _FULL[name] = (w, to_device(a, dt), to_device(b, dt), checks)
    return _FULL[name]


def check_workload(name, n_samples, edges):
    w, da, db, checks = full_case(name, n_samples, edges)
    M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
    for schedule in SCHEDULES:
        tiles = tuning.bench_tiles(name, schedule, dt)
        plan, ws, c = run_gemm(da, db, M, N, K, dt, schedule, **tiles)
        for what, idx, ref, scale in checks:
            if isinstance(idx[0], np.ndarray):
                got = c[torch.from_numpy(idx[0]).cuda(), torch.from_numpy(idx[1]).cuda()]
            else:
                got = c[idx]
            compare(got.cpu().numpy(), ref, scale, dt, exact=dt == "i8",
                    what=f"{name} {what} {plan.describe()}")
        if ws is not None:
            assert plan.workspace_status(ws) == 0
        del c, ws


BIG = ["fp32_256", "fp16_4096", "fp16_1536x1536x8192", "bf16_512x512x65536",
       "bf16_8192x28672x8192", "i8_4096"]


@pytest.mark.parametrize("name", BIG)
def test_workload_parity(name):
    check_workload(name, 8192, edges=name != "bf16_8192x28672x8192")
    w, _, _, checks = full_case(name, 8192, True)
    # every element is compared for every product up to 4096^3 multiply-adds
    if w["M"] * w["N"] * w["K"] <= 4096 ** 3:
        assert checks[0][0] == "all" and checks[0][2].shape == (w["M"], w["N"])


@pytest.mark.parametrize("name", sorted(inputs.irregular_workloads()))
def test_irregular_sweep_parity(name):
    check_workload(name, 8192, edges=True)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_hilbert_tile_order(schedule):
    # the Hilbert order changes which tile a workgroup computes, never the
    # result's tolerance: ragged, repacked shapes at several tile sizes and
    # grids, against the oracle element by element
    import persistent_stream_tiling_amd as gsk
    for dtype, shape in (("f16", (257, 203, 701)), ("bf16", (1000, 777, 1500)),
                         ("f16", (320, 384, 512))):
        M, N, K = shape
        a, b, ref, scale = small_inputs(M, N, K, dtype)
        da, db = to_device(a, dtype), to_device(b, dtype)
        for tiles in (dict(bm=64, bn=64), dict(bm=128, bn=128), dict(bm=256, bn=256),
                      dict(bm=256, bn=256, flags=gsk.FLAG_PING_PONG)):
            for g in ([0, 37] if schedule in ("streamk", "hybrid") else [0]):
                t = dict(tiles)
                t["flags"] = t.get("flags", 0) | gsk.FLAG_HILBERT_ORDER
                plan, ws, c = run_gemm(da, db, M, N, K, dtype, schedule, grid=g, **t)
                assert "order=hilbert" in plan.describe()
                compare(c.cpu().numpy(), ref, scale, dtype, what=plan.describe())
