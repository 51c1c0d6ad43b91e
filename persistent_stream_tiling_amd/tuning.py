"""Launch configuration (tile shape, grid) per workload and schedule.

The benchmark times exactly these, and the full-size GPU parity tests run
exactly these, so what is measured is what is checked.  fp16/bf16 256x256
tiles in the default wave layout run the library's default kernel for that
tile, the wave-specialised ping-pong kernel.
"""
from ._lib import FLAG_NO_XCD_REMAP, FLAG_STREAM_COPIES, FLAG_TILE_SPLIT

SCHEDULES = ("dp", "persistent", "streamk", "hybrid")

_DEFAULTS = {
    "f32": dict(bm=64, bn=64),
    "f16": dict(bm=256, bn=256),
    "bf16": dict(bm=256, bn=256),
    "i8": dict(bm=256, bn=256),
}

# workload name -> schedule -> tiles; anything missing falls back to the dtype
# default.  Chosen from a sweep of tile shapes, wave grids and ring depths on
# MI355X (best mean time per schedule).
BENCH_TILES = {
    # 16 tiles of 64x64 (the configuration names this tile)
    "fp32_256": {s: dict(bm=64, bn=64) for s in SCHEDULES},
    # 256 tiles of 256x256: exactly one tile per CU; 4-row tile bands, hardware
    # workgroup order across the dies
    "fp16_4096": {s: dict(bm=256, bn=256, group_m=4, flags=FLAG_NO_XCD_REMAP) for s in SCHEDULES},
    # Tile-per-workgroup schedules: 144 tiles of 128x128 on 256 CUs.  Stream-K
    # and hybrid: 72 tiles of 256x128, each split over 3-4 workgroups, in the
    # hardware workgroup order (the pieces of one k range spread over the dies)
    "fp16_1536x1536x8192": dict(dp=dict(bm=128, bn=128), persistent=dict(bm=128, bn=128),
                                streamk=dict(bm=256, bn=128, wave_m=4, wave_n=2,
                                             flags=FLAG_NO_XCD_REMAP),
                                hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2,
                                            flags=FLAG_NO_XCD_REMAP)),
    # 64 tiles of 64x64 for the tile-per-workgroup schedules; Stream-K and
    # hybrid: 8 tiles of 256x128, each split over 32 workgroups; hardware
    # workgroup order, so each die holds one k range of all 8 tiles; operand
    # lines are read once per die at a time, so the copies skip cache reuse
    # (non-temporal: 55 against 73 us)
    "bf16_512x512x65536": dict(dp=dict(bm=64, bn=64), persistent=dict(bm=64, bn=64),
                               streamk=dict(bm=256, bn=128, wave_m=4, wave_n=2,
                                            flags=FLAG_NO_XCD_REMAP | FLAG_STREAM_COPIES),
                               hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2,
                                           flags=FLAG_NO_XCD_REMAP | FLAG_STREAM_COPIES)),
    # 3584 tiles of 256x256 (14 per CU)
    "bf16_8192x28672x8192": dict(dp=dict(bm=256, bn=256), persistent=dict(bm=256, bn=256, group_m=4),
                                 streamk=dict(bm=256, bn=256), hybrid=dict(bm=256, bn=256)),
}


# The 16 seeded irregular bf16 shapes: each schedule's fastest tile, wave layout,
# workgroup order, copy hint and Stream-K partition from a sweep on MI355X (median of
# 8 cold runs, rounds interleaved over every configuration of a shape; DP and
# persistent over 256x256, 256x128, 128x256, 128x128; Stream-K and hybrid over the
# library's default plan and 256x256 and 256x128 with die-contiguous or hardware
# order, plain or non-temporal copies, and Stream-K's even split or per-tile pieces
# (FLAG_TILE_SPLIT)).  dict() is the library's default plan.
IRREGULAR_TILES = {
    "bf16_irregular_00_2372x5997x6089": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_01_1095x6981x15363": dict(
        dp=dict(bm=128, bn=256),
        persistent=dict(bm=128, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2, flags=FLAG_TILE_SPLIT)),
    "bf16_irregular_02_2086x5147x4877": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_03_5477x2935x1139": dict(
        dp=dict(bm=128, bn=128),
        persistent=dict(bm=256, bn=128),
        streamk=dict(bm=256, bn=128, wave_m=4, wave_n=2, flags=FLAG_NO_XCD_REMAP),
        hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_04_3470x4884x10138": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=128, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_05_1295x7998x6460": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_06_6347x2237x3547": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_07_1613x5603x2096": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2, flags=FLAG_TILE_SPLIT)),
    "bf16_irregular_08_6620x3734x6086": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_09_6446x6520x7081": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict(bm=256, bn=256)),
    "bf16_irregular_10_5081x4376x4677": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=128, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_11_4622x6539x9711": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_12_3374x4491x2854": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict()),
    "bf16_irregular_13_4141x5473x12021": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=128, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=256, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
    "bf16_irregular_14_6262x5667x14876": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(bm=256, bn=256),
        hybrid=dict(bm=256, bn=256)),
    "bf16_irregular_15_2108x4087x8760": dict(
        dp=dict(bm=256, bn=256),
        persistent=dict(bm=256, bn=256),
        streamk=dict(),
        hybrid=dict(bm=256, bn=128, wave_m=4, wave_n=2, flags=FLAG_NO_XCD_REMAP | FLAG_TILE_SPLIT)),
}

BENCH_TILES.update(IRREGULAR_TILES)


def bench_tiles(workload, schedule, dtype):
    return dict(BENCH_TILES.get(workload, {}).get(schedule, _DEFAULTS[dtype]))
