"""The Stream-K fixup protocol on host threads (no GPU).

tests/emulator/fixup_emulator.cpp runs one thread per workgroup over the
library's own schedule code and the kernels' workspace protocol (park a
piece, raise its flag; wait, add in ascending k; clear), with seeded random
start delays and pauses.  Checked here, for plans the library makes:
- no interleaving changes a bit of C, and the head, split and two-kernel
  fixups agree bitwise (all add every element's pieces in ascending k order);
- C matches the oracle: exactly for integer-valued inputs, otherwise within
  the bound of fp32 summation, (K + pieces) * 2^-24 * sum_k |a||b|;
- a clean run leaves every flag and counter zero;
- a piece whose signal never comes ends every wait on it after its bound,
  with the status word set, instead of hanging;
- ThreadSanitizer finds no data race in the protocol.
The oracle's C code also runs here under AddressSanitizer and
UndefinedBehaviorSanitizer (tests/emulator/oracle_sanitize_driver.c).
"""
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
import persistent_stream_tiling_amd as gsk
from persistent_stream_tiling_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "emulator", "fixup_emulator.cpp")
CSRC = os.path.join(ROOT, "persistent_stream_tiling_amd", "csrc")


def _compile(out, extra):
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-pthread", "-ffp-contract=off",
                    f"-I{CSRC}", *extra, SRC, "-o", out], check=True)
    return out


@pytest.fixture(scope="module")
def emulator(tmp_path_factory):
    return _compile(str(tmp_path_factory.mktemp("emu") / "fixup_emulator"), [])


@pytest.fixture(scope="module")
def emulator_tsan(tmp_path_factory):
    return _compile(str(tmp_path_factory.mktemp("emu_tsan") / "fixup_emulator"),
                    ["-fsanitize=thread"])


def emulate(exe, plan, a, b, tmp_path, seed, jitter_us=200, drop=-1, spin_limit=200000,
            split=None):
    i = plan.info
    M, N, K = plan.M, plan.N, plan.K
    split = i["split_fixup"] if split is None else split
    header = [M, N, K, i["bm"], i["bn"], i["bk"], i["tiles_m"], i["tiles_n"], i["tiles"],
              i["iters_per_tile"], i["tiles_sk"], i["g"], i["q"], i["r"], i["launch_grid"],
              i["group_m"], 1, split, split, drop, spin_limit, seed, jitter_us,
              i["pieces_per_tile"]]
    src, dst = tmp_path / f"in{seed}", tmp_path / f"out{seed}"
    with open(src, "wb") as f:
        f.write(struct.pack("<24i", *header))
        f.write(np.ascontiguousarray(a, dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(b, dtype=np.float32).tobytes())
    res = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = open(dst, "rb").read()
    status = struct.unpack("<i", raw[:4])[0]
    return status, np.frombuffer(raw[4:], dtype=np.float32).reshape(M, N), res.stderr


CASES = [
    # (M, N, K, schedule, tiles, grid): every tile split over several workgroups
    (200, 136, 2050, "streamk", dict(bm=64, bn=64), 37),
    (300, 200, 704, "hybrid", dict(bm=64, bn=64), 7),
    (128, 96, 4096, "streamk", dict(bm=64, bn=64), 23),
    (257, 203, 701, "hybrid", dict(bm=128, bn=128), 5),
    # each Stream-K tile cut into its own pieces (GEMM_FLAG_TILE_SPLIT)
    (200, 136, 2050, "streamk", dict(bm=64, bn=64, flags=gsk.FLAG_TILE_SPLIT), 37),
    (257, 203, 701, "hybrid", dict(bm=64, bn=64, flags=gsk.FLAG_TILE_SPLIT | gsk.FLAG_ONE_TILE), 17),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-g{c[5]}")
def test_interleavings_and_fixup_modes_agree_bitwise(case, emulator, tmp_path):
    M, N, K, sched, tiles, g = case
    a_bits, b_bits = inputs.operands(M, N, K, "f32", "uniform", seed=M + K)
    a, b = a_bits.view(np.float32), b_bits.view(np.float32)
    ref, scale = oracle.gemm(a_bits, b_bits, "f32")
    outs = []
    for flag in (gsk.FLAG_FIXUP_HEAD, gsk.FLAG_FIXUP_SPLIT, gsk.FLAG_FIXUP_TWO_KERNEL):
        t = dict(tiles)
        t["flags"] = t.get("flags", 0) | flag
        plan = gsk.plan_for_device(M, N, K, "f32", sched, grid=g, **t)
        assert plan.info["max_pieces"] >= 2
        for seed in (1, 2, 3):
            status, c, _ = emulate(emulator, plan, a, b, tmp_path, seed)
            assert status == 0
            outs.append(c)
    for c in outs[1:]:
        assert np.array_equal(c.view(np.uint32), outs[0].view(np.uint32))
    bound = (K + g) * 2.0 ** -24 * scale
    assert (np.abs(outs[0].astype(np.float64) - ref) <= bound).all()


def test_integer_inputs_are_exact(emulator, tmp_path):
    M, N, K = 160, 96, 3000
    a_bits, b_bits = inputs.operands(M, N, K, "f32", "int4", seed=8)
    ref, _ = oracle.gemm(a_bits, b_bits, "f32", want_s=False)
    plan = gsk.plan_for_device(M, N, K, "f32", "streamk", grid=29, bm=64, bn=64)
    status, c, _ = emulate(emulator, plan, a_bits.view(np.float32), b_bits.view(np.float32),
                           tmp_path, seed=5)
    assert status == 0 and np.array_equal(c.astype(np.float64), ref)


@pytest.mark.parametrize("flag", ["head", "split"])
def test_lost_signal_ends_every_wait(flag, emulator, tmp_path):
    M, N, K = 200, 136, 2050
    a_bits, b_bits = inputs.operands(M, N, K, "f32", "uniform", seed=9)
    f = gsk.FLAG_FIXUP_HEAD if flag == "head" else gsk.FLAG_FIXUP_SPLIT
    plan = gsk.plan_for_device(M, N, K, "f32", "streamk", grid=37, bm=64, bn=64, flags=f)
    # the last workgroup that parks a piece never raises its flag
    parked = (1, 2) if plan.info["split_fixup"] else (1,)
    drop = max(w for w in range(plan.info["g"]) for s in plan.segments(w) if s[3] in parked)
    status, _, _ = emulate(emulator, plan, a_bits.view(np.float32), b_bits.view(np.float32),
                           tmp_path, seed=4, drop=drop, spin_limit=400)
    assert status == 1


@pytest.mark.slow
@pytest.mark.parametrize("flag", ["head", "split"])
def test_no_data_race_under_thread_sanitizer(flag, emulator_tsan, tmp_path):
    M, N, K = 128, 96, 1024
    a_bits, b_bits = inputs.operands(M, N, K, "f32", "uniform", seed=10)
    f = gsk.FLAG_FIXUP_HEAD if flag == "head" else gsk.FLAG_FIXUP_SPLIT
    plan = gsk.plan_for_device(M, N, K, "f32", "streamk", grid=13, bm=64, bn=64, flags=f)
    status, _, err = emulate(emulator_tsan, plan, a_bits.view(np.float32),
                             b_bits.view(np.float32), tmp_path, seed=6, jitter_us=50)
    assert status == 0
    assert "ThreadSanitizer" not in err, err[-3000:]


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    # host-side sanitizers on the test oracle's C code (no GPU code involved)
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "emulator", "oracle_sanitize_driver.c"),
                    "-o", exe, "-lm", "-lpthread"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr[-3000:]
