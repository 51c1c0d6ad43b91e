"""GPU parity of the half-precision C epilogue (GEMM_FLAG_C_INPUT_DTYPE).

With the flag, C holds the input dtype (fp16 or bf16): every fp32 sum is
rounded to the nearest representable value, ties to even, as it is stored,
and Stream-K pieces stay fp32 until the finished sum is rounded.  So:
- the half C of a plan is bitwise the round-to-nearest-even of the fp32 C of
  the same plan without the flag;
- against the oracle, |C - C_ref| <= tol*S + u*(|C_ref| + tol*S), tol the
  fp32-accumulation bound (4e-3) and u the unit roundoff of the stored dtype
  (2^-11 for fp16, 2^-8 for bf16), since the stored value is within u
  relative of the fp32 sum (all values here are in the normal range);
- integer-valued products are exact in fp32, so C is bitwise the rounding of
  the exact (oracle) result.
"""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, to_device
from persistent_stream_tiling_amd import FLAG_C_INPUT_DTYPE, inputs, tuning

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SCHEDULES = ("dp", "persistent", "streamk", "hybrid")
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TILES = [dict(bm=64, bn=64), dict(bm=128, bn=128), dict(bm=256, bn=256),
         dict(bm=256, bn=128, wave_m=4, wave_n=2)]


def run_both(da, db, M, N, K, dtype, schedule, **tiles):
    """fp32 C and half C of the same plan (the flag only changes the store)."""
    import persistent_stream_tiling_amd as gsk
    out = []
    for half in (False, True):
        t = dict(tiles)
        if half:
            t["flags"] = t.get("flags", 0) | FLAG_C_INPUT_DTYPE
        plan = gsk.GemmPlan(M, N, K, dtype, schedule, **t)
        ws = plan.new_workspace()
        c = torch.full((M, N), float("nan"), device="cuda",
                       dtype=TORCH[dtype] if half else torch.float32)
        plan.run(da, db, c, ws)
        torch.cuda.synchronize()
        if ws is not None:
            assert plan.workspace_status(ws) == 0
        out.append((plan, c.cpu()))
    return out


def rounded(c32, dtype):
    # torch's CPU fp32 -> fp16 / bf16 conversion rounds to nearest even
    return c32.to(TORCH[dtype])


def check_half_against_oracle(ch, ref, scale, dtype, what):
    c = ch.to(torch.float64).numpy()
    assert not np.isnan(c).any(), f"{what}: NaN (element not written?)"
    bound = TOL[dtype] * scale + UNIT[dtype] * (np.abs(ref) + TOL[dtype] * scale)
    bad = np.abs(c - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound, first at " \
                          f"{np.argwhere(bad)[0]}"


@pytest.mark.parametrize("shape", [(320, 384, 512), (300, 200, 704), (257, 203, 701)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_half_c_small(shape, dtype, schedule):
    M, N, K = shape
    a, b = inputs.operands(M, N, K, dtype, "normal", seed=M + N + K)
    ref, scale = oracle.gemm(a, b, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    for tiles in TILES:
        for g in ([0, 37] if schedule in ("streamk", "hybrid") else [0]):
            (p32, c32), (ph, ch) = run_both(da, db, M, N, K, dtype, schedule, grid=g, **tiles)
            what = ph.describe()
            assert torch.equal(ch.view(torch.int16), rounded(c32, dtype).view(torch.int16)), what
            check_half_against_oracle(ch, ref, scale, dtype, what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_half_c_integer_inputs(dtype, schedule):
    # values in [-4, 4]: the fp32 sums are exact, so C is the rounded exact result
    M, N, K = 200, 136, 2050
    a, b = inputs.operands(M, N, K, dtype, "int4", seed=98)
    ref, _ = oracle.gemm(a, b, dtype, want_s=False)
    want = torch.from_numpy(ref).to(torch.float32).to(TORCH[dtype])  # exact -> rounded once
    da, db = to_device(a, dtype), to_device(b, dtype)
    for tiles in TILES[:2]:
        for g in ([0, 37] if schedule in ("streamk", "hybrid") else [0]):
            (_, _), (ph, ch) = run_both(da, db, M, N, K, dtype, schedule, grid=g, **tiles)
            assert torch.equal(ch.view(torch.int16), want.view(torch.int16)), ph.describe()


def test_half_c_split_tiles_and_zero_k():
    import persistent_stream_tiling_amd as gsk
    # long K, many pieces per tile: the fixup adds fp32 pieces, rounds once
    M, N, K = 512, 384, 16384
    a, b = inputs.operands(M, N, K, "bf16", "normal", seed=23)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    rows, cols = inputs.sample_positions(M, N, 1024, seed=4)
    ref, scale = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    for tiles in (dict(bm=128, bn=128), dict(bm=256, bn=128, wave_m=4, wave_n=2)):
        (_, c32), (ph, ch) = run_both(da, db, M, N, K, "bf16", "streamk", **tiles)
        assert ph.info["max_pieces"] >= 2
        assert torch.equal(ch.view(torch.int16), rounded(c32, "bf16").view(torch.int16))
        check_half_against_oracle(ch[rows, cols], ref, scale, "bf16", ph.describe())
    # K = 0: the empty sum, written as half-precision zeros
    plan = gsk.GemmPlan(37, 45, 0, "f16", "hybrid", flags=FLAG_C_INPUT_DTYPE)
    c = torch.full((37, 45), 7.0, dtype=torch.float16, device="cuda")
    plan.run(torch.empty((37, 0), dtype=torch.float16, device="cuda"),
             torch.empty((0, 45), dtype=torch.float16, device="cuda"), c, plan.new_workspace())
    torch.cuda.synchronize()
    assert (c.view(torch.int16) == 0).all()


def test_half_c_full_size_4096():
    # the 4096^3 fp16 product in the benchmark's launch configuration, fp16 C
    w = inputs.WORKLOADS["fp16_4096"]
    M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
    a, b = inputs.operands(M, N, K, dt, w["dist"], w["seed"], w["scale"])
    rows, cols = inputs.sample_positions(M, N, 4096, seed=w["seed"] + 2000)
    ref, scale = oracle.gemm_sampled(a, b, dt, rows, cols)
    da, db = to_device(a, dt), to_device(b, dt)
    ri, ci = torch.from_numpy(rows), torch.from_numpy(cols)
    for schedule in SCHEDULES:
        tiles = tuning.bench_tiles("fp16_4096", schedule, dt)
        (_, c32), (ph, ch) = run_both(da, db, M, N, K, dt, schedule, **tiles)
        assert torch.equal(ch.view(torch.int16), rounded(c32, dt).view(torch.int16))
        check_half_against_oracle(ch[ri, ci], ref, scale, dt, ph.describe())
