"""Host-side checks of the work decomposition (no GPU).

The planner and the kernel share one set of inline schedule functions, so
these checks cover exactly what the GPU executes:

* every (tile, k-iteration) pair is covered exactly once, for every schedule,
* Stream-K ranges are contiguous, ascending and balanced to within one
  iteration (issue #1393, the first-wave kernel's per-program range),
* the hybrid split follows the final revision's host formula,
* each split tile has exactly one owner (the workgroup holding k = 0); with
  the head fixup it waits only on later workgroups whose contribution is
  their first segment, so the waits cannot form a cycle; with the split
  fixup (where nobody waits before its MAC work is done) the walk is
  k-aligned: whole tiles, then the head piece, then the tail piece,
* the tile order and the die remap are bijections.
"""
import random

import numpy as np
import pytest

import persistent_stream_tiling_amd as gsk
from persistent_stream_tiling_amd import inputs

SCHEDULES = ("dp", "persistent", "streamk", "hybrid")


def plan(M, N, K, dtype="f16", schedule="hybrid", cus=256, wg_per_cu=1, **kw):
    return gsk.plan_for_device(M, N, K, dtype, schedule, cus=cus, xcds=8, wg_per_cu=wg_per_cu, **kw)


def all_segments(p):
    return [p.segments(w) for w in range(p.info["launch_grid"])]


def check_plan(p):
    info = p.info
    T, ipt, g = info["tiles"], info["iters_per_tile"], info["g"]
    T_sk, q, r = info["tiles_sk"], info["q"], info["r"]
    split = info["split_fixup"]
    segs = all_segments(p)
    cover = np.zeros((max(T, 1), max(ipt, 1)), dtype=np.int32)
    tile_workers = {}
    for w, ss in enumerate(segs):
        n_sk = len([s for s in ss if s[0] < T_sk])
        for i, (tile, kb, ke, role, peer_last) in enumerate(ss):
            assert 0 <= tile < T and 0 <= kb < ke <= ipt
            cover[tile, kb:ke] += 1
            tile_workers.setdefault(tile, []).append((w, kb, ke, role, peer_last, i))
            if role == gsk.ROLE_CONTRIB:
                assert kb > 0
                if split:  # k-aligned walk: whole tiles, head piece, then the tail piece
                    assert i == n_sk - 1, "the tail piece is the last Stream-K segment"
                else:
                    assert i == 0, "only a first segment may start inside a tile"
            if role == gsk.ROLE_OWNER:
                assert kb == 0 and ke < ipt
                if split:
                    assert all(s[3] == gsk.ROLE_FULL for s in ss[:i]), \
                        "the head piece follows the whole tiles"
                else:
                    assert i == n_sk - 1, "an owner segment is the last Stream-K segment"
            if role == gsk.ROLE_FULL:
                assert kb == 0 and ke == ipt
    if T and ipt:
        assert (cover == 1).all(), "every (tile, k-iteration) pair exactly once"

    # Stream-K ranges: contiguous, ascending, lengths q or q+1 (per-tile split:
    # each tile cut into s such ranges, workgroups past s * T_sk idle)
    s = info["pieces_per_tile"]

    def sk_begin(w):
        if s == 0:
            return w * q + min(w, r)
        t, j = divmod(w, s)
        return T_sk * ipt if t >= T_sk else t * ipt + j * q + min(j, r)
    if T_sk:
        if s:
            assert ipt == q * s + r and 1 <= s <= ipt and s * T_sk <= g
        else:
            assert info["iters_sk"] == T_sk * ipt == q * g + r
        prev_end = 0
        for w in range(g):
            its = [t * ipt + k for (t, kb, ke, _, _) in segs[w] if t < T_sk for k in range(kb, ke)]
            begin, end = sk_begin(w), sk_begin(w + 1)
            if s:
                # no range crosses a tile boundary
                assert begin == end or begin // ipt == (end - 1) // ipt
                if w >= s * T_sk:
                    assert begin == end
                    prev_end = end
                    continue
            # the walk may reorder whole segments (k-aligned mode), never iterations
            assert sorted(its) == list(range(begin, end))
            if not split:
                assert its == list(range(begin, end))
            assert begin == prev_end
            prev_end = end
            assert end - begin in (q, q + 1)
        assert prev_end == T_sk * ipt

    # fixup roles: one owner per split tile, peers = the later workgroups on it
    for tile, ws in tile_workers.items():
        if len(ws) == 1:
            assert ws[0][3] == gsk.ROLE_FULL
            continue
        owners = [x for x in ws if x[3] == gsk.ROLE_OWNER]
        assert len(owners) == 1
        ow, _, _, _, peer_last, _ = owners[0]
        contribs = sorted(x[0] for x in ws if x[3] == gsk.ROLE_CONTRIB)
        assert contribs == list(range(ow + 1, peer_last + 1))
        for x in ws:
            if x[3] == gsk.ROLE_CONTRIB:
                assert x[0] > ow
                if not split:
                    assert x[5] == 0  # head mode: signalled before the worker ever waits
    return segs


CONFIGS = [
    (256, 256, 256, "f32", dict(bm=64, bn=64)),
    (4096, 4096, 4096, "f16", {}),
    (4096, 4096, 4096, "f16", dict(bm=256, bn=128)),
    (4096, 4096, 4096, "f16", dict(bm=128, bn=128)),
    (1536, 1536, 8192, "f16", {}),
    (1536, 1536, 8192, "f16", dict(bm=128, bn=128)),
    (512, 512, 65536, "bf16", {}),
    (512, 512, 65536, "bf16", dict(bm=128, bn=128)),
    (2372, 5997, 6089, "bf16", {}),
    (1095, 6981, 15363, "bf16", dict(bm=128, bn=256)),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}")
def test_invariants_on_workloads(cfg, schedule):
    M, N, K, dt, kw = cfg
    check_plan(plan(M, N, K, dt, schedule, **kw))


TILE_SPLIT_CASES = [
    # (M, N, K, dtype, tiles, schedule, g): s = min(g // T_sk, ipt)
    (1536, 1536, 8192, "f16", dict(bm=256, bn=256), "streamk", 256),   # 36 tiles x 7, 4 idle
    (1536, 1536, 8192, "f16", dict(bm=256, bn=128), "streamk", 256),   # 72 tiles x 3
    (512, 512, 65536, "bf16", dict(bm=256, bn=128), "streamk", 256),   # 8 x 32: even split
    (300, 200, 704, "f16", dict(bm=64, bn=64), "streamk", 37),         # 20 tiles x 1: whole tiles
    (300, 200, 100, "f16", dict(bm=128, bn=128), "streamk", 256),      # s clamped to ipt = 2
    (257, 203, 701, "f32", dict(bm=64, bn=64), "streamk", 100),        # 20 tiles x 5, ragged
    (4000, 3000, 2000, "f16", dict(bm=256, bn=256), "hybrid", 256),    # one-tile hybrid below
    (2000, 900, 3000, "bf16", dict(bm=128, bn=128), "streamk", 201),   # odd g
]


@pytest.mark.parametrize("fixup", [0, gsk.FLAG_FIXUP_HEAD, gsk.FLAG_FIXUP_TWO_KERNEL])
@pytest.mark.parametrize("case", TILE_SPLIT_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{c[5]}-g{c[6]}")
def test_tile_split_partitions(case, fixup):
    M, N, K, dt, tiles, schedule, g = case
    flags = gsk.FLAG_TILE_SPLIT | fixup | (gsk.FLAG_ONE_TILE if schedule == "hybrid" else 0)
    p = plan(M, N, K, dt, schedule, grid=g, flags=flags, **tiles)
    i = p.info
    ipt, T_sk = i["iters_per_tile"], i["tiles_sk"]
    s = min(g // T_sk, ipt)
    assert i["pieces_per_tile"] == s and (i["q"], i["r"]) == divmod(ipt, s)
    assert i["max_pieces"] == s and "tile-split" in p.describe()
    check_plan(p)
    # every Stream-K tile has exactly s workgroups, t*s .. t*s + s - 1
    segs = all_segments(p)
    for t in range(T_sk):
        holders = sorted({w for w in range(g) for seg in segs[w] if seg[0] == t})
        assert holders == list(range(t * s, t * s + s))


def test_tile_split_needs_a_grid_of_at_least_the_stream_k_tiles():
    with pytest.raises(ValueError, match="TILE_SPLIT"):
        plan(1536, 1536, 8192, "f16", "streamk", bm=128, bn=128, grid=100,
             flags=gsk.FLAG_TILE_SPLIT)
    # two-tile hybrid: T_sk = T mod g + g can exceed g (192 tiles, g = 80: T_sk = 112)
    with pytest.raises(ValueError, match="TILE_SPLIT"):
        plan(4000, 3000, 2000, "f16", "hybrid", bm=256, bn=256, grid=80,
             flags=gsk.FLAG_TILE_SPLIT)
    # no Stream-K tiles: the flag changes nothing
    assert plan(4096, 4096, 4096, "f16", "dp", flags=gsk.FLAG_TILE_SPLIT).info["pieces_per_tile"] == 0


def test_invariants_large_mlp_shape():
    for schedule in SCHEDULES:
        check_plan(plan(8192, 28672, 8192, "bf16", schedule))


def test_invariants_random_sweep():
    # shapes and grids in the spirit of issue #1393's sweep: the CU count,
    # twice it, the tile count, and random even grids
    rnd = random.Random(1393)
    for _ in range(60):
        M, N = rnd.randint(1, 3000), rnd.randint(1, 3000)
        K = rnd.randint(1, 5000)
        bm, bn = rnd.choice([(64, 64), (128, 128), (256, 128), (128, 256), (256, 256)])
        tiles = -(-M // bm) * -(-N // bn)
        g = rnd.choice([256, 512, max(1, min(tiles, 511)), rnd.randrange(2, 512, 2), 1, 7])
        one_tile = rnd.random() < 0.5
        for schedule in SCHEDULES:
            p = plan(M, N, K, "bf16", schedule, wg_per_cu=2, bm=bm, bn=bn, grid=g,
                     flags=gsk.FLAG_ONE_TILE if one_tile else 0)
            check_plan(p)


def hybrid_split(T, g, two_tiles):
    # issue #1393, final revision's host wrapper, restated
    T_sk = T % g
    if two_tiles and T - T_sk > g:
        T_sk += g
    return T_sk


@pytest.mark.parametrize("T_shape", [(4096, 4096), (1536, 1536), (512, 512), (8192, 28672),
                                     (2372, 5997), (6620, 3734), (1000, 1000)])
@pytest.mark.parametrize("g", [256, 128, 200, 512])
@pytest.mark.parametrize("two_tiles", [True, False])
def test_hybrid_split_formula(T_shape, g, two_tiles):
    M, N = T_shape
    p = plan(M, N, 4096, "f16", "hybrid", wg_per_cu=2, grid=g,
             flags=0 if two_tiles else gsk.FLAG_ONE_TILE)
    T = p.info["tiles"]
    assert p.info["tiles_sk"] == hybrid_split(T, g, two_tiles)
    assert p.info["tiles_dp"] == T - p.info["tiles_sk"]
    if p.info["tiles_dp"]:
        assert p.info["tiles_dp"] % g == 0 or T < g, "data-parallel part is whole waves"


def test_pages_demo_partitions():
    # second revision's demo: 256 x 512 x 2048, 64^3 blocks, grid 82 -> 32 tiles of
    # 32 iterations; 1024 iterations over 82 programs: 12 each, the first 40 get 13
    p = plan(256, 512, 2048, "f16", "streamk", bm=64, bn=64, grid=82)
    i = p.info
    assert (i["tiles"], i["iters_per_tile"], i["iters_sk"], i["q"], i["r"]) == (32, 32, 1024, 12, 40)
    lengths = [sum(ke - kb for (_, kb, ke, _, _) in p.segments(w)) for w in range(82)]
    assert lengths == [13] * 40 + [12] * 42
    # first revision's demo: 256 x 512 x 32768, grid 32 -> one whole tile per program,
    # so Stream-K degenerates to data-parallel ("expected to have similar timings")
    p = plan(256, 512, 32768, "f16", "streamk", bm=64, bn=64, grid=32)
    assert (p.info["q"], p.info["r"], p.info["iters_per_tile"]) == (512, 0, 512)
    for w in range(32):
        assert [s[3] for s in p.segments(w)] == [gsk.ROLE_FULL]
    # under the final revision's hybrid formula the same case is all data-parallel
    assert plan(256, 512, 32768, "f16", "hybrid", bm=64, bn=64, grid=32).info["tiles_sk"] == 0
    # grid 0 in the pages means plain tiling; here that is the dp schedule
    assert plan(256, 512, 2048, "f16", "dp", bm=64, bn=64).info["tiles_sk"] == 0


def test_dp_is_one_tile_per_workgroup():
    p = plan(1000, 700, 300, "f16", "dp", bm=128, bn=128)
    assert p.info["launch_grid"] == p.info["tiles"]
    for w in range(p.info["launch_grid"]):
        assert p.segments(w) == [(w, 0, p.info["iters_per_tile"], gsk.ROLE_FULL, w)]


def test_persistent_strides_by_grid():
    p = plan(4096, 4096, 512, "f16", "persistent", bm=128, bn=128)
    g = p.info["launch_grid"]
    assert g == 256
    for w in (0, 5, 255):
        assert [s[0] for s in p.segments(w)] == [w + i * g for i in range(4)]


def test_tile_coords_bijection_and_grouping():
    p = plan(4096, 2048, 64, "f16", "dp", bm=128, bn=128)  # 32 x 16 tiles
    seen = {p.tile_coords(t) for t in range(p.info["tiles"])}
    assert seen == {(m, n) for m in range(32) for n in range(16)}
    assert [p.tile_coords(t) for t in range(10)] == [(m, 0) for m in range(8)] + [(0, 1), (1, 1)]
    # ragged last band: 10 tile rows, group 8 -> the last band has 2 rows
    p = plan(1280, 384, 64, "f16", "dp", bm=128, bn=128)
    coords = [p.tile_coords(t) for t in range(p.info["tiles"])]
    assert sorted(coords) == [(m, n) for m in range(10) for n in range(3)]
    assert coords[24:] == [(8, 0), (9, 0), (8, 1), (9, 1), (8, 2), (9, 2)]
    # linear order when grouping is off
    p = plan(1280, 384, 64, "f16", "dp", bm=128, bn=128, group_m=-1)
    assert [p.tile_coords(t) for t in range(4)] == [(0, 0), (0, 1), (0, 2), (1, 0)]


@pytest.mark.parametrize("grid", [1, 7, 8, 36, 255, 256, 1000, 3584])
def test_die_remap_is_a_bijection_with_contiguous_blocks(grid):
    p = plan(grid * 64, 64, 64, "f16", "dp", bm=64, bn=64)
    assert p.info["launch_grid"] == grid
    logical = [p.logical_wg(h) for h in range(grid)]
    assert sorted(logical) == list(range(grid))
    for die in range(8):
        block = [logical[h] for h in range(die, grid, 8)]
        assert block == list(range(block[0], block[0] + len(block))) if block else True


def test_streamk_grid_must_fit_resident_capacity():
    with pytest.raises(ValueError, match="resident"):
        plan(1536, 1536, 8192, "f16", "streamk", grid=300)
    plan(1536, 1536, 8192, "f16", "streamk", grid=300, wg_per_cu=2)
    plan(4096, 4096, 64, "f16", "persistent", grid=1000)  # no waits: any grid is fine


def test_rejects_bad_arguments():
    with pytest.raises(ValueError, match="negative"):
        plan(-1, 4, 4)
    with pytest.raises(ValueError, match="no kernel"):
        plan(64, 64, 64, "f16", "dp", bm=96, bn=96)
    with pytest.raises(ValueError, match="no kernel"):
        plan(64, 64, 64, "f16", "dp", bk=48)
    with pytest.raises(ValueError, match="unknown schedule"):
        plan(64, 64, 64, "f16", "zigzag")


def test_workspace_layout():
    p = plan(1536, 1536, 8192, "f16", "streamk")
    ws = p.workspace_bytes
    assert ws >= 256 + 4 * 256 + 4 * 256 * 256 * 256
    assert plan(4096, 4096, 4096, "f16", "dp").workspace_bytes == 0
    assert plan(4096, 4096, 4096, "f16", "persistent").workspace_bytes == 0
    # rows that are not 16-byte multiples are repacked: the workspace holds the copies
    p = plan(2372, 5997, 6089, "bf16", "dp")
    assert p.info["pack_a"] and p.info["pack_b"]
    assert p.workspace_bytes >= 2372 * 6096 * 2 + 6089 * 6000 * 2


def test_empty_shapes_plan():
    for M, N, K in ((0, 5, 5), (5, 0, 5), (5, 5, 0), (0, 0, 0)):
        for s in SCHEDULES:
            p = plan(M, N, K, "f16", s)
            assert p.info["tiles_sk"] == 0


def test_irregular_shape_list_is_reproducible():
    shapes = inputs.irregular_shapes()
    assert len(shapes) == 16
    assert shapes[0] == (2372, 5997, 6089) and shapes[-1] == (2108, 4087, 8760)
    for m, n, k in shapes:
        assert 1000 <= m <= 8192 and 1000 <= n <= 8192 and 1000 <= k <= 16384
        assert m % 128 and n % 128 and k % 128


def test_fixup_mode_choice_and_workspace():
    # 512 x 512 x 65536 at 128^2: 16 tiles, each cut into 16 pieces -> split by default
    p = plan(512, 512, 65536, "bf16", "streamk", bm=128, bn=128)
    assert p.info["max_pieces"] == 16 and p.info["split_fixup"] == 1
    g = p.info["g"]
    assert p.workspace_bytes >= 256 + 4 * 2 * g + 4 * p.info["tiles_sk"] + 2 * g * 128 * 128 * 4
    head = plan(512, 512, 65536, "bf16", "streamk", bm=128, bn=128, flags=gsk.FLAG_FIXUP_HEAD)
    assert head.info["split_fixup"] == 0 and head.workspace_bytes < p.workspace_bytes
    # second revision's demo: 13 or 12 iterations of 32-iteration tiles -> at most 4 pieces
    p = plan(256, 512, 2048, "f16", "streamk", bm=64, bn=64, grid=82)
    assert p.info["max_pieces"] == 4 and p.info["split_fixup"] == 1
    # two pieces per tile are split too
    p = plan(2372, 5997, 6089, "bf16", "streamk", bm=256, bn=256, grid=256)
    assert p.info["max_pieces"] == 2 and p.info["split_fixup"] == 1
    # whole tiles only: nothing to fix up
    p = plan(4096, 4096, 4096, "f16", "streamk")
    assert p.info["max_pieces"] == 1 and p.info["split_fixup"] == 0
    p = plan(1536, 1536, 8192, "f16", "streamk", bm=128, bn=128, flags=gsk.FLAG_FIXUP_SPLIT)
    assert p.info["split_fixup"] == 1


def test_split_tiles_per_workgroup_at_most_two():
    # every workgroup takes part in at most two split tiles (its first and
    # last); the split fixup relies on it for its two slots
    for (M, N, K, bm, g) in ((1536, 1536, 8192, 256, 256), (512, 512, 65536, 128, 256),
                             (300, 200, 704, 64, 37), (1000, 1000, 333, 128, 100)):
        p = plan(M, N, K, "f16", "streamk", bm=bm, bn=bm, grid=g, wg_per_cu=2)
        for w in range(p.info["launch_grid"]):
            pieces = [s for s in p.segments(w) if s[3] != gsk.ROLE_FULL]
            assert len(pieces) <= 2
            if len(pieces) == 2:
                if p.info["split_fixup"]:  # k-aligned walk: head piece, then tail piece
                    assert pieces[0][3] == gsk.ROLE_OWNER and pieces[1][3] == gsk.ROLE_CONTRIB
                else:
                    assert pieces[0][3] == gsk.ROLE_CONTRIB and pieces[1][3] == gsk.ROLE_OWNER


@pytest.mark.parametrize("shape,schedule,tile", [
    ((4096, 4096, 4096), "dp", (256, 256)),           # 256 tiles fill the CUs exactly
    ((8192, 28672, 8192), "persistent", (256, 256)),  # 14 full waves
    ((1536, 1536, 8192), "dp", (128, 128)),           # 36 big tiles would idle 86% of the CUs
    ((5376, 256, 512), "dp", (128, 128)),
    # Stream-K / hybrid: the planner's cost model (tests/test_grid_model.py)
    ((1536, 1536, 8192), "streamk", (256, 256)),      # one workgroup per CU, 18 iterations each
    ((512, 512, 65536), "hybrid", (128, 128)),        # 16 tiles in 16 pieces of 64 iterations
    ((4096, 4096, 4096), "streamk", (256, 256)),      # one whole tile per CU
])
def test_default_tile_follows_the_wave_model(shape, schedule, tile):
    M, N, K = shape
    plan = gsk.plan_for_device(M, N, K, "f16", schedule)
    assert (plan.info["bm"], plan.info["bn"]) == tile
    # an explicit tile always wins, and a layout only built at 256x256 keeps it
    assert gsk.plan_for_device(M, N, K, "f16", schedule, bm=64, bn=64).info["bm"] == 64
    p2 = gsk.plan_for_device(M, N, K, "bf16", schedule, wave_m=2, wave_n=4, stages=0)
    assert p2.info["wave_m"] == 2 and p2.info["wave_n"] == 4


def test_debug_drop_signal_needs_a_split_tile():
    drop = gsk.FLAG_DEBUG_DROP_SIGNAL
    # 8 tiles of 128x128 over 256 workgroups: every tile is split
    plan = gsk.plan_for_device(256, 512, 65536, "bf16", "streamk", bm=128, bn=128, flags=drop)
    assert plan.info["max_pieces"] >= 2
    for sched in ("dp", "persistent"):
        with pytest.raises(ValueError, match="splits some tile"):
            gsk.plan_for_device(256, 512, 65536, "bf16", sched, bm=128, bn=128, flags=drop)


def test_int8_plans():
    plan = gsk.plan_for_device(300, 200, 704, "i8", "hybrid")
    assert plan.info["bk"] == 128 and plan.info["kernel_kind"] == 0
    assert " C=i32 " in plan.describe()
    # a sum of 2^17 products of -128 * -128 would leave int32
    with pytest.raises(ValueError, match="overflow"):
        gsk.plan_for_device(64, 64, 1 << 17, "i8", "dp")
    assert gsk.plan_for_device(64, 64, (1 << 17) - 1, "i8", "dp").info["K"] == (1 << 17) - 1
    with pytest.raises(ValueError, match="int32"):
        gsk.plan_for_device(64, 64, 64, "i8", "dp", flags=gsk.FLAG_C_INPUT_DTYPE)
    # rows of 701 int8 values are not 16-byte multiples: both operands repacked
    p = gsk.plan_for_device(257, 203, 701, "i8", "dp")
    assert p.info["pack_a"] == 1 and p.info["pack_b"] == 1


def test_two_kernel_fixup_plans():
    two = gsk.FLAG_FIXUP_TWO_KERNEL
    # 8 tiles of 128x128 over 512 workgroups: more than can be resident at once
    with pytest.raises(ValueError, match="resident"):
        gsk.plan_for_device(256, 512, 65536, "bf16", "streamk", grid=512, bm=128, bn=128)
    plan = gsk.plan_for_device(256, 512, 65536, "bf16", "streamk", grid=512, bm=128, bn=128,
                               flags=two)
    assert plan.info["split_fixup"] == 2 and plan.info["g"] == 512
    assert "fixup=two-kernel" in plan.describe()
    # the coverage invariants hold for the grid beyond residency too
    check_plan(plan)
    with pytest.raises(ValueError, match="no signals"):
        gsk.plan_for_device(256, 512, 65536, "bf16", "streamk", grid=512, bm=128, bn=128,
                            flags=two | gsk.FLAG_DEBUG_DROP_SIGNAL)


def test_stream_copies_only_where_built():
    f = gsk.FLAG_STREAM_COPIES
    assert gsk.plan_for_device(512, 512, 65536, "bf16", "streamk", bm=256, bn=128,
                               flags=f).info["kernel_kind"] == 2
    with pytest.raises(ValueError, match="no kernel"):
        gsk.plan_for_device(512, 512, 4096, "bf16", "dp", bm=128, bn=128, flags=f)


def _page_swizzle(t, grid_m, grid_n, group_m):
    # the GROUP_M re-ordering of issue #1393's final revision (swizzle_tile),
    # restated: bands of group_m tile rows; the row is the global tile id mod
    # the band's height, the column the id within the band over that height
    width = group_m * grid_n
    group_id = t // width
    group_size = min(grid_m - group_id * group_m, group_m)
    return group_id * group_m + t % group_size, (t % width) // group_size


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [(11, 2, 8), (10, 3, 8), (13, 5, 4), (7, 7, 3),
                                                     (32, 16, 8), (5, 9, 8)])
def test_band_order_is_the_pages_swizzle(tiles_m, tiles_n, group_m):
    # on a short last band whose width is not a multiple of its height the
    # page's row index is a rotation of the within-band one
    p = plan(tiles_m * 64, tiles_n * 64, 64, "f16", "dp", bm=64, bn=64, group_m=group_m)
    assert (p.info["tiles_m"], p.info["tiles_n"]) == (tiles_m, tiles_n)
    T = tiles_m * tiles_n
    assert [p.tile_coords(t) for t in range(T)] == \
        [_page_swizzle(t, tiles_m, tiles_n, group_m) for t in range(T)]


def _hilbert_d2xy(order, d):
    # the textbook Hilbert index -> (x, y) map on a 2^order square (iterative,
    # bottom-up: rotate, then offset the quadrant)
    x = y = 0
    s, t = 1, d
    while s < (1 << order):
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


@pytest.mark.parametrize("tiles_m,tiles_n", [(1, 1), (2, 2), (4, 4), (8, 8), (16, 16), (3, 5),
                                             (7, 1), (1, 9), (11, 6), (17, 32), (32, 112), (23, 22)])
def test_hilbert_order(tiles_m, tiles_n):
    p = plan(tiles_m * 64, tiles_n * 64, 64, "f16", "dp", bm=64, bn=64,
             flags=gsk.FLAG_HILBERT_ORDER)
    assert "order=hilbert" in p.describe()
    T = tiles_m * tiles_n
    coords = [p.tile_coords(t) for t in range(T)]
    # the textbook curve on the enclosing power-of-two square, cells outside
    # the grid skipped (brute force over the whole square)
    order = max(tiles_m - 1, tiles_n - 1, 0).bit_length()
    want = [xy for xy in (_hilbert_d2xy(order, d) for d in range(4 ** order))
            if xy[0] < tiles_m and xy[1] < tiles_n]
    assert coords == want
    # on a power-of-two square each step moves to a neighbouring tile
    if tiles_m == tiles_n and tiles_m & (tiles_m - 1) == 0:
        assert all(abs(a[0] - b[0]) + abs(a[1] - b[1]) == 1 for a, b in zip(coords, coords[1:]))
    # every schedule still covers each (tile, k-iteration) pair exactly once
    for sched in ("streamk", "hybrid"):
        check_plan(plan(tiles_m * 64, tiles_n * 64, 1000, "f16", sched, bm=64, bn=64, grid=37,
                        flags=gsk.FLAG_HILBERT_ORDER))


def test_hilbert_textbook_pins():
    # d2xy pinned to hand-drawn curves: order 1 is the U (0,0) (0,1) (1,1) (1,0);
    # order 2 starts with a transposed U and ends with an anti-transposed one
    assert [_hilbert_d2xy(1, d) for d in range(4)] == [(0, 0), (0, 1), (1, 1), (1, 0)]
    assert [_hilbert_d2xy(2, d) for d in range(16)] == [
        (0, 0), (1, 0), (1, 1), (0, 1), (0, 2), (0, 3), (1, 3), (1, 2),
        (2, 2), (2, 3), (3, 3), (3, 2), (3, 1), (2, 1), (2, 0), (3, 0)]
