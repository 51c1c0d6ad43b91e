"""Every compiled kernel variant, launched through the C ABI, against the oracle.

The library exports its kernel table (gemm_variant_count / gemm_variant_get);
each entry is selected exactly (tile, wave layout, stages, copy hint) and run
in all four schedules on two shapes:

- 257 x 203 x 701: ragged M, N and K, and rows that are not 16-byte multiples
  (both operands repacked), every element compared;
- 320 x 200 x 9000 (a few tiles, long K): Stream-K and hybrid at g = 256 and
  g = 37 split every tile into pieces, in the in-kernel split fixup, the head
  fixup and the two-kernel fixup, with Stream-K's even split of all the
  iterations and with each tile cut into its own pieces (GEMM_FLAG_TILE_SPLIT);
  compared on seeded samples plus the ragged edges.

Integer-valued inputs (int8) must match exactly; the others within
tol * sum_k |a_ik||b_kj|.
"""
import numpy as np
import pytest

import oracle
from gpu_util import compare, run_gemm, to_device
from persistent_stream_tiling_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import persistent_stream_tiling_amd as gsk  # noqa: E402

DTYPE_NAMES = {0: "f32", 1: "f16", 2: "bf16", 3: "i8"}
SCHEDULES = ("dp", "persistent", "streamk", "hybrid")


def _variant_id(v):
    return (f"{DTYPE_NAMES[v['dtype']]}-{v['bm']}x{v['bn']}-w{v['wave_m']}x{v['wave_n']}"
            f"-k{v['kind']}" + ("-nt" if v["stream_copies"] else ""))


VARIANTS = gsk.variants()

_CASES = {}


def _case(M, N, K, dtype, sampled):
    key = (M, N, K, dtype, sampled)
    if key not in _CASES:
        dist = "int8" if dtype == "i8" else "normal"
        a, b = inputs.operands(M, N, K, dtype, dist, seed=M + 3 * N + 7 * K)
        if sampled:
            rows, cols = inputs.sample_positions(M, N, 2048, seed=17, tails=True)
            ref, scale = oracle.gemm_sampled(a, b, dtype, rows, cols)
            idx = (rows, cols)
        else:
            ref, scale = oracle.gemm(a, b, dtype)
            idx = None
        _CASES[key] = (to_device(a, dtype), to_device(b, dtype), idx, ref, scale)
    return _CASES[key]


def _tiles(v):
    t = dict(bm=v["bm"], bn=v["bn"], wave_m=v["wave_m"], wave_n=v["wave_n"],
             stages=v["stages"])
    if v["stream_copies"]:
        t["flags"] = gsk.FLAG_STREAM_COPIES
    if v["kind"] == 3:
        t["flags"] = t.get("flags", 0) | gsk.FLAG_PING_PONG
    elif v["kind"] == 2:
        t["flags"] = t.get("flags", 0) | gsk.FLAG_RING_KERNEL
    return t


def _check(plan, c, idx, ref, scale, dtype, v):
    info = plan.info
    # the plan runs exactly this kernel
    assert (info["bm"], info["bn"], info["wave_m"], info["wave_n"], info["kernel_kind"],
            info["stages"]) == (v["bm"], v["bn"], v["wave_m"], v["wave_n"], v["kind"],
                                v["stages"])
    got = c.cpu().numpy() if idx is None else c.cpu().numpy()[idx]
    if dtype == "i8":
        compare(got, ref, None, dtype, exact=True, what=plan.describe())
    else:
        compare(got, ref, scale, dtype, what=plan.describe())


def test_table_is_exported():
    assert len(VARIANTS) == gsk.load().gemm_variant_count() > 0
    for v in VARIANTS:
        assert v["threads"] == 64 * v["wave_m"] * v["wave_n"]
        assert 0 < v["lds_bytes"] <= 160 * 1024


@pytest.mark.parametrize("v", VARIANTS, ids=_variant_id)
def test_variant_ragged_repacked(v):
    dtype = DTYPE_NAMES[v["dtype"]]
    M, N, K = 257, 203, 701
    da, db, idx, ref, scale = _case(M, N, K, dtype, sampled=False)
    for sched in SCHEDULES:
        for g in ((0, 37) if sched in ("streamk", "hybrid") else (0,)):
            plan, ws, c = run_gemm(da, db, M, N, K, dtype, sched, grid=g, **_tiles(v))
            assert plan.info["pack_a"] and plan.info["pack_b"]
            _check(plan, c, idx, ref, scale, dtype, v)


@pytest.mark.parametrize("v", VARIANTS, ids=_variant_id)
def test_variant_split_long_k(v):
    dtype = DTYPE_NAMES[v["dtype"]]
    M, N, K = 320, 200, 9000
    da, db, idx, ref, scale = _case(M, N, K, dtype, sampled=True)
    for sched in SCHEDULES:
        if sched in ("dp", "persistent"):
            plan, _, c = run_gemm(da, db, M, N, K, dtype, sched, **_tiles(v))
            _check(plan, c, idx, ref, scale, dtype, v)
            continue
        for g in (0, 37):
            for fix in (gsk.FLAG_FIXUP_SPLIT, gsk.FLAG_FIXUP_HEAD, gsk.FLAG_FIXUP_TWO_KERNEL):
                for split in (0, gsk.FLAG_TILE_SPLIT):
                    t = _tiles(v)
                    t["flags"] = t.get("flags", 0) | fix | split
                    plan, ws, c = run_gemm(da, db, M, N, K, dtype, sched, grid=g, **t)
                    s = plan.info["pieces_per_tile"]
                    assert (s > 0) == (split != 0)
                    # (a per-tile split over fewer workgroups than twice the
                    # tiles leaves every tile whole)
                    assert plan.info["max_pieces"] >= 2 or s == 1, plan.describe()
                    _check(plan, c, idx, ref, scale, dtype, v)


PP_SHAPES = [(257, 203, 701), (512, 768, 1000), (300, 520, 4096), (1024, 1024, 2112)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", PP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ping_pong_matches_the_ring_kernel_bitwise(shape, dtype):
    # the wave-specialised kernel runs the same MFMAs in the same order per
    # element as the ring kernel with the same tile: identical bits in every
    # schedule (split tiles included), and within the oracle's bound
    M, N, K = shape
    a, b = inputs.operands(M, N, K, dtype, "normal", seed=M ^ N ^ K)
    ref, scale = oracle.gemm(a, b, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    for sched in SCHEDULES:
        for g in ((0, 37) if sched in ("streamk", "hybrid") else (0,)):
            ring, _, c_ring = run_gemm(da, db, M, N, K, dtype, sched, grid=g, bm=256, bn=256,
                                       flags=gsk.FLAG_RING_KERNEL)
            plan, _, c_pp = run_gemm(da, db, M, N, K, dtype, sched, grid=g, bm=256, bn=256)
            assert plan.info["kernel_kind"] == 3 and ring.info["kernel_kind"] == 2
            assert torch.equal(c_ring.view(torch.int32), c_pp.view(torch.int32)), plan.describe()
            compare(c_pp.cpu().numpy(), ref, scale, dtype, what=plan.describe())
