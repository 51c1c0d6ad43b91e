"""GPU parity of the int8 path: int8 inputs, exact int32 sums, int32 C.

Every int8 product is an integer of magnitude at most 2^14, so with K below
2^17 every sum is an exact int32 and the GPU result must equal the oracle's
exact sum bit for bit, in every schedule, including Stream-K tiles whose
pieces are added by the fixup (integer adds).
"""
import numpy as np
import pytest

import oracle
from gpu_util import to_device
from persistent_stream_tiling_amd import FLAG_FIXUP_HEAD, FLAG_FIXUP_SPLIT, inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SCHEDULES = ("dp", "persistent", "streamk", "hybrid")
TILES = [dict(bm=128, bn=128), dict(bm=256, bn=256)]


def run(da, db, M, N, K, schedule, **tiles):
    import persistent_stream_tiling_amd as gsk
    plan = gsk.GemmPlan(M, N, K, "i8", schedule, **tiles)
    ws = plan.new_workspace()
    c = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    plan.run(da, db, c, ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert plan.workspace_status(ws) == 0
    return plan, c.cpu().numpy()


def assert_exact(c, ref, what):
    bad = c.astype(np.float64) != ref
    assert not bad.any(), f"{what}: {bad.sum()} elements differ, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("shape", [(320, 384, 512), (300, 200, 704), (257, 203, 701)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_int8_small_exact(shape, schedule):
    M, N, K = shape
    a, b = inputs.operands(M, N, K, "i8", "int8", seed=M + N + K)
    ref, _ = oracle.gemm(a, b, "i8", want_s=False)
    da, db = to_device(a, "i8"), to_device(b, "i8")
    for tiles in TILES:
        for g in ([0, 37] if schedule in ("streamk", "hybrid") else [0]):
            plan, c = run(da, db, M, N, K, schedule, grid=g, **tiles)
            assert_exact(c, ref, plan.describe())


@pytest.mark.parametrize("flag", [FLAG_FIXUP_HEAD, FLAG_FIXUP_SPLIT], ids=["head", "split"])
def test_int8_long_k_split_tiles(flag):
    # few tiles, long K: every tile cut into many pieces, added as integers
    M, N, K = 256, 384, 16384
    a, b = inputs.operands(M, N, K, "i8", "int8", seed=71)
    rows, cols = inputs.sample_positions(M, N, 2048, seed=72, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "i8", rows, cols)
    da, db = to_device(a, "i8"), to_device(b, "i8")
    for tiles in TILES:
        for g in (256, 37):
            plan, c = run(da, db, M, N, K, "streamk", grid=g, flags=flag, **tiles)
            assert plan.info["max_pieces"] >= 2
            assert_exact(c[rows, cols], ref, plan.describe())


def test_int8_largest_k_does_not_overflow():
    # (-128)(-128) * 131071 = 2^31 - 2^14: the largest sum the plan allows
    M, N, K = 64, 96, 131071
    a = np.full((M, K), -128, dtype=np.int8)
    b = np.full((K, N), -128, dtype=np.int8)
    a[1::2, :] = 127  # odd rows: 127 * -128 per term
    da, db = to_device(a, "i8"), to_device(b, "i8")
    want = np.where(np.arange(M)[:, None] % 2 == 0, 16384 * K, -16256 * K) * np.ones((1, N))
    for schedule in ("dp", "streamk"):
        plan, c = run(da, db, M, N, K, schedule, bm=128, bn=128)
        assert_exact(c, want.astype(np.float64), plan.describe())


def test_int8_two_kernel_fixup_and_wide_grids():
    # the second kernel adds int32 pieces as integers too; grids past residency
    import persistent_stream_tiling_amd as gsk
    M, N, K = 256, 384, 16384
    a, b = inputs.operands(M, N, K, "i8", "int8", seed=73)
    rows, cols = inputs.sample_positions(M, N, 2048, seed=74, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "i8", rows, cols)
    da, db = to_device(a, "i8"), to_device(b, "i8")
    for g in (37, 256, 512, 1024):
        plan, c = run(da, db, M, N, K, "streamk", grid=g, flags=gsk.FLAG_FIXUP_TWO_KERNEL,
                      bm=128, bn=128)
        assert plan.info["split_fixup"] == 2
        assert_exact(c[rows, cols], ref, plan.describe())
