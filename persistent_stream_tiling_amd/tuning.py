"""Launch configuration (tile shape, grid) per workload and schedule.

The benchmark times exactly these, and the full-size GPU parity tests run
exactly these, so what is measured is what is checked.
"""
SCHEDULES = ("dp", "persistent", "streamk", "hybrid")

_DEFAULTS = {
    "f32": dict(bm=64, bn=64),
    "f16": dict(bm=256, bn=256),
    "bf16": dict(bm=256, bn=256),
}

# workload name -> schedule -> tiles; anything missing falls back to the dtype default
BENCH_TILES = {
    "fp32_256": {s: dict(bm=64, bn=64) for s in SCHEDULES},
}


def bench_tiles(workload, schedule, dtype):
    return dict(BENCH_TILES.get(workload, {}).get(schedule, _DEFAULTS[dtype]))
