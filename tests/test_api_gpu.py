"""GPU checks of the flag combinations and the Python convenience call.

- the hybrid in its one-tile form (T_sk = T mod g) and in its two-tile form,
  each with the in-kernel split fixup and the two-kernel fixup, on a shape
  with more tiles than workgroups, against the oracle (ragged, repacked);
- ``matmul`` for every input dtype and output type, against the oracle.
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


@pytest.mark.parametrize("two_tiles", [True, False], ids=["two_tiles", "one_tile"])
@pytest.mark.parametrize("fixup", ["split", "two_kernel"])
def test_hybrid_forms_and_fixups(two_tiles, fixup):
    import persistent_stream_tiling_amd as gsk
    M, N, K = 1000, 777, 1500   # 128x128 tiles: 8 x 7 = 56 tiles on g = 20 or 24
    a, b = inputs.operands(M, N, K, "f16", "normal", seed=5)
    ref, scale = oracle.gemm(a, b, "f16")
    da, db = to_device(a, "f16"), to_device(b, "f16")
    flags = (0 if two_tiles else gsk.FLAG_ONE_TILE) | \
        (gsk.FLAG_FIXUP_SPLIT if fixup == "split" else gsk.FLAG_FIXUP_TWO_KERNEL)
    for g in (20, 24):
        plan, ws, c = run_gemm(da, db, M, N, K, "f16", "hybrid", grid=g, bm=128, bn=128,
                               flags=flags)
        T, T_sk = plan.info["tiles"], plan.info["tiles_sk"]
        want = T % g + (g if two_tiles and T - T % g > g else 0)
        assert T_sk == want and 0 < T_sk < T
        compare(c.cpu().numpy(), ref, scale, "f16", what=plan.describe())
        assert plan.workspace_status(ws) == 0


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_matmul_convenience_call(dtype):
    import persistent_stream_tiling_amd as gsk
    M, N, K = 300, 200, 704
    dist = "int8" if dtype == "i8" else "normal"
    a, b = inputs.operands(M, N, K, dtype, dist, seed=9)
    ref, scale = oracle.gemm(a, b, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    c = gsk.matmul(da, db, schedule="streamk", grid=37)
    if dtype == "i8":
        assert c.dtype == torch.int32
        compare(c.cpu().numpy(), ref, None, dtype, exact=True, what="matmul i8")
        return
    assert c.dtype == torch.float32
    compare(c.cpu().numpy(), ref, scale, dtype, what=f"matmul {dtype}")
    if dtype in ("f16", "bf16"):
        h = gsk.matmul(da, db, schedule="hybrid", out_dtype=da.dtype)
        assert h.dtype == da.dtype
        u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
        err = np.abs(h.float().cpu().numpy().astype(np.float64) - ref)
        assert (err <= 4e-3 * scale + u * (np.abs(ref) + 4e-3 * scale)).all()


def test_matmul_raises_when_a_fixup_wait_gives_up():
    # a piece whose flag never rises (forced from the host with the testing
    # flag; every wait stays bounded): matmul reads the status and raises,
    # and leaves its cached workspace clean for the next call
    import persistent_stream_tiling_amd as gsk
    M, N, K = 256, 512, 16384
    a, b = inputs.operands(M, N, K, "bf16", "int4", seed=43)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    bad = dict(bm=128, bn=128, flags=gsk.FLAG_FIXUP_SPLIT | gsk.FLAG_DEBUG_DROP_SIGNAL)
    with pytest.raises(gsk.FixupError):
        gsk.matmul(da, db, schedule="streamk", **bad)
    with pytest.raises(gsk.FixupError):  # the same cached plan fails the same way, again
        gsk.matmul(da, db, schedule="streamk", **bad)
    rows, cols = inputs.sample_positions(M, N, 512, seed=44, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    c = gsk.matmul(da, db, schedule="streamk", bm=128, bn=128, flags=gsk.FLAG_FIXUP_SPLIT)
    compare(c.cpu().numpy()[rows, cols], ref, None, "bf16", exact=True, what="after a failure")


def test_matmul_keeps_a_workspace_per_stream():
    # the same shape on two streams at once: each stream gets its own plan
    # and workspace, so the runs cannot share flags or partial slots
    import persistent_stream_tiling_amd as gsk
    from persistent_stream_tiling_amd import plan as plan_mod
    M, N, K = 384, 512, 12288
    a, b = inputs.operands(M, N, K, "f16", "int4", seed=45)
    rows, cols = inputs.sample_positions(M, N, 1024, seed=46, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "f16", rows, cols)
    da, db = to_device(a, "f16"), to_device(b, "f16")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(gsk.matmul(da, db, schedule="streamk", bm=128, bn=128))
    torch.cuda.synchronize()
    keys = [k for k in plan_mod._PLANS if k[:3] == (M, N, K)]
    assert {k[-1] for k in keys} >= {s1.cuda_stream, s2.cuda_stream}
    ws = [plan_mod._PLANS[k][1].data_ptr() for k in keys]
    assert len(set(ws)) == len(ws)
    for c in outs:
        compare(c.cpu().numpy()[rows, cols], ref, None, "f16", exact=True, what="per stream")
