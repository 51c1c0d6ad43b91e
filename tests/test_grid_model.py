"""The planner's default Stream-K / hybrid plan (fp16/bf16, no tile, grid 0).

The C++ planner and persistent_stream_tiling_amd.grid_model hold the same
cost model; both must pick the same tile and grid.  Plans made for a
described device need no GPU.
"""
import random

import pytest

import persistent_stream_tiling_amd as gsk
from persistent_stream_tiling_amd import grid_model
from persistent_stream_tiling_amd.inputs import log_sampled_shapes


def _shapes():
    rnd = random.Random(5)
    shapes = list(log_sampled_shapes(300, seed=99))
    # ragged sizes, a single tile, one k iteration, very long K, many tiles
    shapes += [(rnd.randint(1, 9000), rnd.randint(1, 9000), rnd.randint(1, 20000)) for _ in range(200)]
    shapes += [(1, 1, 1), (256, 256, 64), (100, 3000, 65), (512, 512, 65536), (8192, 28672, 8192),
               (1536, 1536, 8192), (4096, 4096, 4096), (300, 200, 17)]
    return shapes


@pytest.mark.parametrize("schedule", ["streamk", "hybrid"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_planner_matches_the_python_rule(schedule, dtype):
    for (M, N, K) in _shapes():
        plan = gsk.plan_for_device(M, N, K, dtype, schedule)
        pick = grid_model.choose(M, N, K, cus=256)
        info = plan.info
        if pick is None:
            # no tile shape has at most 256 tiles: one workgroup per CU
            assert info["g"] == 256 and "(cost model)" not in plan.describe(), (M, N, K)
            continue
        bm, bn, g = pick
        assert (info["bm"], info["bn"], info["g"]) == (bm, bn, g), (M, N, K, plan.describe())
        assert "(cost model)" in plan.describe()
        # every candidate fits one workgroup per CU
        assert g <= 256


def test_candidates_are_aligned_splits_or_one_workgroup_per_cu():
    for (M, N, K) in _shapes():
        pick = grid_model.choose(M, N, K)
        if pick is None:
            continue
        bm, bn, g = pick
        T = -(-M // bm) * -(-N // bn)
        ipt = -(-K // 64)
        plan = gsk.plan_for_device(M, N, K, "f16", "streamk")
        info = plan.info
        if g == 256 and not (g % T == 0 and ipt % (g // T) == 0):
            continue  # Stream-K's even split over the CUs
        # an aligned split: every workgroup runs exactly one piece of one tile
        s = g // T
        assert g % T == 0 and ipt % s == 0 and s in grid_model.CANDIDATE_S
        assert info["r"] == 0 and info["q"] == ipt // s
        assert info["max_pieces"] == s
        for p in range(0, g, max(1, g // 17)):
            segs = plan.segments(p)
            assert len(segs) == 1 and segs[0][2] - segs[0][1] == ipt // s


def test_explicit_tile_or_grid_keeps_one_workgroup_per_cu():
    # the model applies only when neither a tile nor a grid is given
    p = gsk.plan_for_device(512, 256, 1536, "f16", "streamk", bm=256, bn=128)
    assert p.info["g"] == 256 and "(cost model)" not in p.describe()
    p = gsk.plan_for_device(512, 256, 1536, "f16", "streamk", grid=200)
    assert p.info["g"] == 200
    p = gsk.plan_for_device(512, 256, 1536, "f16", "streamk", flags=gsk.FLAG_PING_PONG)
    assert (p.info["bm"], p.info["bn"], p.info["g"]) == (256, 256, 256)
    # fp32 and int8 keep their defaults
    assert gsk.plan_for_device(512, 256, 1536, "f32", "streamk").info["g"] == 256
    assert gsk.plan_for_device(512, 256, 1536, "i8", "streamk").info["g"] == 256
    # data-parallel and persistent are unaffected
    assert "(cost model)" not in gsk.plan_for_device(512, 256, 1536, "f16", "dp").describe()


def test_fit_recovers_known_coefficients():
    # synthetic measurements made by the model itself: the fit returns the
    # coefficients it was given, and the crossing cost from the g = 256 plans
    coef = dict(c0=10.0, it=(1.3, 1.0, 0.75, 0.6), split=(23.0, 12.0, 6.75, 4.0), c_log=-3.0,
                cross=12.0)
    records = []
    # small shapes too, so that the 64x64 tile (at most 256 tiles) is measured
    shapes = list(log_sampled_shapes(60, seed=3)) + [(256 * i, 256 * j, 512 * k)
                                                      for i in (1, 2, 3) for j in (1, 2)
                                                      for k in (1, 3, 8)]
    for (M, N, K) in shapes:
        sk = {}
        for ti, (bm, bn) in enumerate(grid_model.TILES):
            T = -(-M // bm) * -(-N // bn)
            ipt = -(-K // 64)
            if not grid_model.tile_allowed(ti, T):
                continue
            for g in grid_model.candidate_grids(T):
                sk[f"{bm}x{bn}/{g}"] = grid_model.estimate(coef, ti, T, ipt, g)
        records.append(dict(M=M, N=N, K=K, dp=50.0, sk=sk))
    got, n, med_err, _ = grid_model.fit(records)
    assert n > 100 and med_err < 1e-9
    for k in ("c0", "c_log", "cross"):
        assert got[k] == pytest.approx(coef[k], abs=1e-6)
    for k in ("it", "split"):
        assert got[k] == pytest.approx(coef[k], abs=1e-6)


def test_default_hybrid_above_the_model_splits_per_tile():
    # more than 256 tiles for every tile shape: 256x256 tiles, g = 256, one
    # Stream-K wave (T_sk = T mod g) and its tiles cut into their own pieces
    for (M, N, K) in [(4608, 4352, 4096), (6144, 3072, 2048), (5120, 5120, 1024), (4352, 4352, 640),
                      (9000, 9000, 1000), (8192, 28672, 8192), (4160, 4224, 1000),
                      (6400, 6208, 320), (7680, 7168, 4096)]:
        assert grid_model.choose(M, N, K) is None
        for dtype in ("f16", "bf16"):
            info = gsk.plan_for_device(M, N, K, dtype, "hybrid").info
            T, ipt, g, t_sk = info["tiles"], -(-K // 64), info["g"], info["tiles_sk"]
            assert (info["bm"], info["bn"], g) == (256, 256, 256)
            assert t_sk == T % g
            if t_sk > 0:
                s = min(g // t_sk, ipt)
                assert info["pieces_per_tile"] == s and info["q"] == ipt // s
                assert info["r"] == ipt % s
            else:
                assert info["pieces_per_tile"] == 0, (M, N, K, t_sk)
            # an explicit tile or grid keeps the pages' even split
            assert gsk.plan_for_device(M, N, K, dtype, "hybrid", bm=256, bn=256).info["pieces_per_tile"] == 0
            assert gsk.plan_for_device(M, N, K, dtype, "hybrid", grid=256).info["pieces_per_tile"] == 0
        # Stream-K (T_sk = T > g) and data-parallel are unaffected
        assert gsk.plan_for_device(M, N, K, "f16", "streamk").info["pieces_per_tile"] == 0
